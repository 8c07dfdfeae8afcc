// Paged decode attention that reads the quantized pages directly, for gfx950.
//
// The attention backend reads compressed KV pages as they are stored, without
// re-materializing fp16 K/V (aitrends.kr article 74976, TL;DR and the glossary
// entries on KV compression and the attention backend).
//
// Algebra (H = orthonormal Sylvester Hadamard, symmetric, H H = I):
//   key t restored:    x_t = H r_t,  r_tc = alpha_c (S_t k_tc + O_t)
//   score:             q . x_t = (H q) . r_t
//                          = S_t sum_c qt_c k_tc + O_t sum_c qt_c,  qt = (H q) * alpha_K
//   value output:      sum_t p_t x_t = H sum_t p_t r_t, with
//                      sum_t p_t r_tc = alpha_c (sum_t p_t S_t k_tc + sum_t p_t O_t)
// so the inverse rotation and the channel factors act on the query (once per
// tile) and on the accumulated output (once per sequence and head), never on
// the cached tokens.
//
// Work split: one workgroup of 4 waves per (sequence, kv head, partition of
// 64-token chunks); both contractions run on v_mfma_f32_4x4x4_16b_f16 with
// the cached codes as one operand and the query fold (QK) or the
// probabilities (PV) as the other, in groups of 4 query rows (the kernel's
// own comment below gives the lane layouts).  Codes enter the MFMA as fp16
// denormals: a field masked in place in its 16-bit half reads as
// (code * 2^e) * 2^-24, exactly, with e fixed by the field's position; the
// matching 2^-e rides on the query (K side), on the probabilities (V tokens)
// or on the output fold (V channels).  Unpacking is one AND per two codes.
// Online softmax runs per chunk; partitions are merged by a second kernel
// that also applies the final Hadamard.
//
// Query rows: a decode step has one row per query head of the GQA group.
// With several queries per sequence (the newest n_q tokens, already cached,
// each attending causally to the tokens up to its own position) the rows are
// (query, head) pairs, 8 at most per workgroup, and a row's scores past its
// position are masked.
#pragma once
#include <type_traits>

#include "kvq_internal.h"
#include "kvq_tile.h"

namespace kvq {
namespace {


typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32); }

// max of two floats as one v_max_f32.  fmaxf on a value that arrives from
// another lane gets a canonicalizing v_max (x, x) first (NaN quieting); the
// reductions here never see a NaN (finite inputs, -inf for masked scores).
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max(|a|, |b|, c) as one v_max3_f32 with absolute-value operands
__device__ __forceinline__ float vmax3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// v_permlane16_swap / v_permlane32_swap with both operands a copy of v return
// a pair whose two members are v and the value of lane l^16 (resp. l^32) in
// some order, so a symmetric op over the pair reduces over that lane pair in
// the VALU (no LDS round trip).
__device__ __forceinline__ float sum16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float sum32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float max16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return vmax(__int_as_float(p[0]), __int_as_float(p[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return vmax(__int_as_float(p[0]), __int_as_float(p[1]));
}

// Reductions over the 4 lanes l, l^16, l^32, l^48 (one query head's lanes).
__device__ __forceinline__ float group_max(float v) { return max32(max16(v)); }
__device__ __forceinline__ float group_sum(float v) { return sum32(sum16(v)); }

constexpr int kWaves = 4;             // waves per decode workgroup
constexpr int kChunk = 64;            // tokens per wave step (4 pages)
constexpr int kMaxChunksPerPart = 64;
// Slot pointers staged per partition: its pages, then those of one 128-token
// tile past any partition (the loads a wave issues after its last chunk read
// there: chunk c_begin + kMaxChunksPerPart, pages up to 8 on).
constexpr int kSlotEntries = 4 * kMaxChunksPerPart + 8;
// A slot-sized block that those loads read in place of pool pages (the values
// are never used; one small block stays in cache, where a reload of pool pages
// would be fetched from memory again).
static __device__ __align__(256) uint8_t g_spare_slot[4096];

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Code fields of one 32-bit word (two 16-bit halves), masked in place so that
// each half reads as the fp16 denormal m * 2^-24 whose mantissa m is the code
// times the power of two fixed by the field's bit position (the field's
// weight: 16^(X mod 2) at 4 bits, 4^(X mod 4) at 2 bits, 1 at 8 bits, where
// X = 0 takes fields 0, 2 and X = 1 fields 1, 3).
// Fields in bits 8..15 of a half are taken from y = x >> 8.  One AND per pair
// of codes, no conversion and no offset term.
template <int BITS, int X>
__device__ __forceinline__ unsigned code_field(unsigned x, unsigned y) {
  if constexpr (BITS == 8) {
    return (X == 0 ? x : y) & 0x00FF00FFu;
  } else if constexpr (BITS == 4) {
    constexpr unsigned m = (X & 1) ? 0x00F000F0u : 0x000F000Fu;
    return ((X < 2) ? x : y) & m;
  } else {
    constexpr unsigned m = 0x00030003u << (2 * (X & 3));
    return ((X < 4) ? x : y) & m;
  }
}
// Channel of operand element k (< 4) of QK step s (< 32): the step takes
// fields X, X + 1 of a code word, each from both 16-bit halves (K codes in
// unit order: field m of unit u holds channel u + 16 m; a unit is a 32-bit
// word at 4 bits, a 16-bit half at 2 bits, two words at 8 bits).
template <int BITS>
__host__ __device__ constexpr int qk_channel(int s, int k) {
  if constexpr (BITS == 8) {
    // word s = half s % 2 of unit s / 2; elements: fields 0, 2, 1, 3 of the word
    const int m = 4 * (s & 1) + 2 * (k & 1) + (k >> 1);
    return (s >> 1) + 16 * m;
  } else if constexpr (BITS == 4) {
    // word s / 2; even s: fields 0, 4 | 1, 5; odd s: 2, 6 | 3, 7
    const int m = 2 * (s & 1) + 4 * (k & 1) + (k >> 1);
    return (s >> 1) + 16 * m;
  } else {
    // word s / 4 = units 2 (s / 4) (low half), + 1 (high half); fields 2 (s % 4) + k / 2
    return 2 * (s >> 2) + (k & 1) + 16 * (2 * (s & 3) + (k >> 1));
  }
}
// Inverse: the step / element of channel c, as 4 s + k.
template <int BITS>
__host__ __device__ constexpr int qk_slot(int c) {
  const int u = c & 15, m = c >> 4;
  if constexpr (BITS == 8) return 4 * (2 * u + (m >> 2)) + 2 * (m & 1) + ((m >> 1) & 1);
  else if constexpr (BITS == 4) return 4 * (2 * u + ((m >> 1) & 1)) + 2 * (m & 1) + (m >> 2);
  else return 4 * (4 * (u >> 1) + (m >> 1)) + 2 * (m & 1) + (u & 1);
}
// Weight of channel c's K code field as read in place (16^(m mod 2) at 4 bits,
// 4^(m mod 4) at 2 bits, 1 at 8 bits, m = c / 16).
template <int BITS>
__host__ __device__ constexpr float k_field_weight(int c) {
  if (BITS == 8) return 1.f;
  return BITS == 4 ? (((c >> 4) & 1) ? 16.f : 1.f) : (float)(1 << (2 * ((c >> 4) & 3)));
}

// fp16x4 MFMA operand from two code-field words
__device__ __forceinline__ f16x4 as_f16x4(unsigned a, unsigned b) {
  return __builtin_bit_cast(f16x4, u32x2{a, b});
}

// fp32 pair -> fp16 pair hi, x = v * s rounded (nearest even) to a multiple
// of 1/w, and the fp16 pair lo = x - hi (the subtraction is exact; lo is
// rounded).  m = 1.5 * 2^23 / w: adding it leaves 1/w as the ulp, so
// (x + m) - m is the rounded x for |x| w < 2^22; the product v * s enters
// both through an fma, unrounded.  With w the code field's weight and
// |x| w <= 2^11, hi is exact in fp16 and every product hi * (code w 2^-24)
// is an integer multiple of 2^-24: an MFMA chain over hi then sums exactly
// (its partial sums stay below 2^24 units), where products of unrelated
// exponents would lose low bits in the MFMA's adder.  lo runs in a chain of
// its own, 2^-11 smaller.
__device__ __forceinline__ void split_grid(float v0, float v1, float s0, float s1, float m0, float m1, unsigned& hi,
                                           unsigned& lo) {
  const float h0 = __builtin_fmaf(v0, s0, m0) - m0, h1 = __builtin_fmaf(v1, s1, m1) - m1;
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{h0, h1}, f16x2));
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{__builtin_fmaf(v0, s0, -h0),
                                                                  __builtin_fmaf(v1, s1, -h1)}, f16x2));
}
constexpr float kGrid = 12582912.f;   // 1.5 * 2^23

// Another lane's value through a DPP permutation of the VALU operand (no LDS
// round trip): quad_perm [1,0,3,2] is lane ^ 1 and [2,3,0,1] lane ^ 2;
// row_half_mirror is 7 - lane within each 8, row_mirror 15 - lane within each
// 16 (on values already equal within each quad, resp. each 8, these pair the
// same groups as lane ^ 4 and lane ^ 8); row_ror:n is lane - n within each 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140, kRor4 = 0x124, kRor8 = 0x128;

__device__ __forceinline__ float wave_max(float v) {
  v = vmax(v, dpp<kXor1>(v));
  v = vmax(v, dpp<kXor2>(v));
  v = vmax(v, dpp<kHalfMirror>(v));
  v = vmax(v, dpp<kMirror>(v));
  return group_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kXor1>(v);
  v += dpp<kXor2>(v);
  v += dpp<kHalfMirror>(v);
  v += dpp<kMirror>(v);
  return group_sum(v);
}
// Sum / max over the lanes of one MFMA row index i = lane & 3 within groups of
// NB blocks (NB = 8: each 32-lane half; NB = 16: the wave).  The sum keeps the
// xor pairing (lane ^ 4, then ^ 8, ^ 16, ^ 32): the query sum it forms meets a
// term it nearly cancels in short heavy-tailed tiles, where a different
// association of the same terms was measurably less accurate.  The max is
// exact in any order: two rotations cover the 4 lanes of the class in each 16.
template <int NB>
__device__ __forceinline__ float blocks_sum(float v) {
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  v += lane_xor<16>(v);
  if (NB == 16) v += xor32(v);
  return v;
}
template <int NB>
__device__ __forceinline__ float blocks_max(float v) {
  v = vmax(v, dpp<kRor4>(v));
  v = vmax(v, dpp<kRor8>(v));
  v = max16(v);
  if (NB == 16) v = max32(v);
  return v;
}

template <int T, int HG>
struct alignas(16) DecodeSmem {
  // the partition's K and V slots (this kv head), kept as global-memory
  // pointers: loads through them are global loads (a generic pointer read
  // back from LDS would make every slot load a flat load, which also counts
  // against the LDS counter and makes LDS waits wait for memory)
  const __attribute__((address_space(1))) uint8_t* kp[kSlotEntries];
  const __attribute__((address_space(1))) uint8_t* vp[kSlotEntries];
  union {
    struct {
      float hq[4 * HG][kHeadDim];                // (H q)_c / weight of c's K field, at qk_slot(c)
      float pt[kWaves][4 * HG][kChunk];          // per-wave transpose of the probabilities
    } loop;
    struct {
      float acc[kWaves][4 * HG][kHeadDim];
      float m[kWaves][4 * HG];
      float l[kWaves][4 * HG];
    } merge;
  };
};

// Decode attention over quantized pages; one workgroup of 4 waves per
// (partition of 64-token chunks, kv head, sequence); wave w takes chunks
// begin + w, begin + w + 4, ...  Both contractions run on
// v_mfma_f32_4x4x4_16b_f16 (16 blocks of 4 x 4, K = 4), so that the lane
// layouts fit a group of 4 query heads with no padding:
//   QK:  D[b][head i][token j] = sum_k qt[i][c_k] K[4b + j][c_k] over 32 steps
//        of 4 channels.  Lane 4b + j feeds its own token's codes (B); the
//        query operand A is the same for every block and is broadcast from
//        one block (CBSZ/ABID), so 16 steps' worth of qt sit in one register
//        set spread over the 16 blocks.  Output: lane = token, 4 heads.
//   PV:  D[b][head i][channel 4b + j] = sum_k P[t_k][i] V[t_k][4b + j] over 16
//        steps of 4 tokens; A = probabilities (transposed once through LDS,
//        broadcast from block = step), B = the lane's channel's codes.
//        Output: lane = channel l (and 64 + l), 4 heads.
// Groups of more than 4 heads run 4 at a time (HG groups) on the same codes.
// Shared memory of the decode kernel; with FUSED, the tile quantizer's
// buffers (one per concurrent quantizer group of 2T threads) overlay it.
template <int T, int HG, bool FUSED>
struct alignas(16) DecodeSmemU {
  static constexpr int QG = FUSED ? (64 * kWaves) / (2 * T) : 0;
  union {
    DecodeSmem<T, HG> dec;
    std::conditional_t<FUSED, TileSmem<T>, char> q[QG > 0 ? QG : 1];   // (the append's buffers)
  };
};

// FUSED: the same decode step preceded by the append of one token per
// sequence (A.seq_lens then holds the lengths before it; the attention covers
// one more token).  The append re-quantizes the token's (partial) tile, whose
// pages only the last partition of each (sequence, kv head) reads, so that
// workgroup does it first (K and V tiles side by side, 2T threads each) and
// the write-to-read order stays inside one workgroup.
// Grid: x = kv head + kv_heads * (row block + blocks * sequence), y =
// partition.  The partition index varies slowest, so the short last
// partitions of every (sequence, kv head) are dispatched after the full ones
// and do not hold back full ones behind them when the grid exceeds what the
// chip holds at once.
// MQ: several queries per sequence (A.n_q of them, the newest cached tokens);
// row blocks of NH rows, row r = query r / G, head r % G, and query i sees
// the tokens before L - n_q + i + 1.
// Groups of up to 8 heads keep 2 waves per SIMD (at most 256 registers in all,
// VGPRs and AGPRs); 16 heads need more registers and run 1 wave per SIMD.
// M16: slots with fp16 metadata (scales, offsets and channel factors read as
// fp16 and widened to fp32; the arithmetic is the same).
// KCH: K slots rounded per channel: the fold takes the channel scales A in
// place of alpha_K, both per-token factors are beta, and the offset term is
// sum_c qt_c M_c over the represented query (the zero offsets M of the tile).
template <int T, int BK, int BV, int HG, bool FUSED, bool MQ = false, bool M16 = false, bool KCH = false>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(HG <= 2 ? 2 : 1)))
void decode_kernel(DecodeArgs A, QuantArgs Q) {
  constexpr int NH = 4 * HG;
  constexpr int SETS = (T == 32) ? 4 : 2;        // QK A register sets
  constexpr int BLK = 32 / SETS;                 // steps per set = blocks per broadcast group
  constexpr int CB = (T == 32) ? 3 : 4;          // CBSZ of the QK broadcast
  constexpr int TPC = (T == 32) ? 2 : 1;         // tiles per chunk
  constexpr int PPT = T / kPage;                 // pages per tile
  constexpr int SLOT_K = slot_bytes(BK, T, M16, KCH), SLOT_V = slot_bytes(BV, T, M16);
  constexpr int CODE_K = slot_code_bytes(BK), CODE_V = slot_code_bytes(BV);
  constexpr int OFF_K = slot_offset_at(BK, M16), OFF_V = slot_offset_at(BV, M16);
  constexpr int ALPHA_K = KCH ? slot_chan_scale_at(BK) : slot_alpha_at(BK, M16), ALPHA_V = slot_alpha_at(BV, M16);
  constexpr int ZP_K = slot_chan_zp_at(BK, T);
  constexpr int AL = slot_alpha_len(T);
  // V fields of tokens 2 and 3 of a quad weigh kTok times those of tokens 0, 1;
  // their probabilities enter the MFMA divided by kTok.
  constexpr float kTok = (BV == 8) ? 1.f : (BV == 4) ? 16.f : 4.f;
  // Exponents that bound the MFMA operands' hi parts (the query fold below
  // 2^(QE+1), p S_V below 2^(PE+1)): with codes below 2^BITS every product
  // and every chain's partial sum stays an integer of at most 22 bits in
  // units of 2^-24 (as at 4 bits with QE = PE = 10), so the chains sum exactly.
  constexpr int QE = (BK == 8) ? 6 : 10, PE = (BV == 8) ? 6 : 10;
  constexpr int KQ = (BK == 8) ? 8 : 4, VQ = (BV == 8) ? 8 : 4;   // code registers (u32x4)
  constexpr float kTwo24 = 16777216.f;
  __shared__ DecodeSmemU<T, HG, FUSED> smu;
  auto& sm = smu.dec;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  const int bq = lane >> 2, iq = lane & 3;       // MFMA block and row/column of this lane
  const int H = A.kv_heads;
  const int G = A.group;
  const int RB = MQ ? (A.n_q * G + NH - 1) / NH : 1;     // row blocks per (sequence, kv head)
  const int part = blockIdx.y;
  const int seq = (int)blockIdx.x / (H * RB);
  const int hb = (int)blockIdx.x - seq * H * RB;
  const int kvh = hb % H;
  const int r0 = MQ ? (hb / H) * NH : 0;                  // first query row of this workgroup
  const int nrows = MQ ? min(NH, A.n_q * G - r0) : G;   // its real rows
  const int L = A.seq_lens[seq] + (FUSED ? 1 : 0);
  const int nchunks = min((L + kChunk - 1) / kChunk, A.max_tiles);
  const int c_begin = part * A.tiles_per_part;
  const int c_end = min(nchunks, c_begin + A.tiles_per_part);
  if (c_begin >= c_end) return;  // uniform over the workgroup
  // the query rows wave 0 folds below, loaded first so that their memory
  // latency overlaps that of the block table and the first chunk
  // (rows past the real ones load row 0 and are zeroed at the fold: no
  // branch around the loads, so nothing has to wait for them before the fold)
  u32x4 qraw[4];
  const bool q_real = (lane & 15) < nrows;
  if (wave == 0) {
    const int n16 = lane & 15, grp = lane >> 4;
    const bool real = q_real;
    size_t qix;
    if constexpr (MQ) {
      const int r = r0 + (real ? n16 : 0);
      qix = ((size_t)seq * A.n_q + r / G) * A.q_heads + kvh * G + r % G;
    } else {
      qix = (size_t)seq * A.q_heads + kvh * G + (real ? n16 : 0);
    }
    const uint16_t* qrow = A.q + qix * kHeadDim + 32 * grp;
#pragma unroll
    for (int v = 0; v < 4; ++v) qraw[v] = *reinterpret_cast<const u32x4*>(qrow + 8 * v);
  }
  // MQ: tokens visible to row h (causal: up to its query's position)
  int vis[MQ ? NH : 1];
  if constexpr (MQ) {
#pragma unroll
    for (int h = 0; h < NH; ++h) vis[h] = min(L, L - A.n_q + 1 + (r0 + h) / G);   // padding rows: L
  }
  if constexpr (FUSED) {
    if (c_end == nchunks) {   // the last partition: append, then attend
      const int tile_idx = (L - 1) / T;
      if ((tile_idx + 1) * (T / kPage) <= Q.max_blocks) {
        constexpr int QG = DecodeSmemU<T, HG, FUSED>::QG;
        const int g = threadIdx.x / (2 * T), tid = threadIdx.x % (2 * T);
        if constexpr (QG == 1) {
          quantize_tile_body<T, BK, false, kAppend, M16, kPathBoth, KCH>(Q, smu.q[0].f, &smu.q[0].s, 0, kvh, seq, tile_idx, tid);
          __syncthreads();
          quantize_tile_body<T, BV, true, kAppend, M16>(Q, smu.q[0].f, &smu.q[0].s, 1, kvh, seq, tile_idx, tid);
        } else {
          // groups 2j and 2j + 1 quantize K and V; with 4 groups (tile 32) the
          // second pair repeats the first, writing the same bytes, so that every
          // wave meets the quantizer's barriers (with K rounded per channel the
          // V body passes the K body's extra barriers too)
          if ((g & 1) == 0)
            quantize_tile_body<T, BK, false, kAppend, M16, kPathBoth, KCH>(Q, smu.q[g].f, &smu.q[g].s, 0, kvh, seq, tile_idx, tid);
          else quantize_tile_body<T, BV, true, kAppend, M16, kPathBoth, false, KCH>(Q, smu.q[g].f, &smu.q[g].s, 1, kvh, seq, tile_idx, tid);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  const int npages = ((L + T - 1) / T) * PPT;   // pages the sequence owns (whole tiles)
  // the partition's K and V slot addresses (up to the end of its last tile), staged once in LDS
  {
    const int32_t* row = A.block_table + (size_t)seq * A.max_blocks + 4 * c_begin;
    const int last = min(npages, ((4 * c_end + PPT - 1) / PPT) * PPT);
    const int n = last - 4 * c_begin;
    static_assert(SLOT_K <= (int)sizeof(g_spare_slot) && SLOT_V <= (int)sizeof(g_spare_slot), "spare slot size");
    for (int i = threadIdx.x; i < kSlotEntries; i += 64 * kWaves) {
      if (i < n) {
        const size_t slot = (size_t)row[i] * H + kvh;
        sm.kp[i] = (const __attribute__((address_space(1))) uint8_t*)(A.pool_k + slot * SLOT_K);
        sm.vp[i] = (const __attribute__((address_space(1))) uint8_t*)(A.pool_v + slot * SLOT_V);
      } else {
        sm.kp[i] = (const __attribute__((address_space(1))) uint8_t*)g_spare_slot;
        sm.vp[i] = (const __attribute__((address_space(1))) uint8_t*)g_spare_slot;
      }
    }
  }
  __syncthreads();
  // LDS index of page pj of the sequence; a T = 32 chunk whose second tile
  // was never started reads its first tile's pages instead (every token there
  // is past the end and masked)
  auto page_ix = [&](int pj) { return (pj < npages ? pj : pj - 2) - 4 * c_begin; };
  auto kslot = [&](int pj) { return (const uint8_t*)sm.kp[page_ix(pj)]; };   // K slot of page pj of the sequence
  auto vslot = [&](int pj) { return (const uint8_t*)sm.vp[page_ix(pj)]; };

  // ------------------------------------------------ per-chunk operands (loaded one chunk ahead,
  // each right after its last use in the current chunk)
  u32x4 kq[KQ];           // K codes of token `lane`, in unit order (the 4 blocks of its slot)
  float sk, ok;           // its scale and offset
  u32x4 vq[VQ];           // V codes of run `lane` (channels lane, 64 + lane), 4 pages
  f32x4 svq, ovq;         // V scale / offset of tokens 4 bq .. 4 bq + 3
  f32x4 ak[SETS];         // alpha_K of this lane's QK steps (fold layout)
  f32x4 mk[KCH ? SETS : 1];   // KCH: the zero offsets M of the same channels
  float av[TPC][2];       // alpha_V of channels lane, 64 + lane
  auto tile_page = [&](int c, int tile_in_chunk) {   // first page (in the sequence) of a tile of chunk c
    return (T == 128) ? 4 * (c & ~1) : 4 * c + PPT * tile_in_chunk;
  };
  auto load_k = [&](int c) {
    const uint8_t* sl = kslot(4 * c + (lane >> 4));
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      if (BK == 8) {
        kq[2 * blk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 512 * blk + 32 * (lane & 15)));
        kq[2 * blk + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 512 * blk + 32 * (lane & 15) + 16));
      } else if (BK == 4) kq[blk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 256 * blk + 16 * (lane & 15)));
      else { const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sl + 128 * blk + 8 * (lane & 15))); kq[blk] = u32x4{x[0], x[1], 0u, 0u}; }
    }
    sk = load_meta<M16>(sl + CODE_K, lane & 15);
    ok = KCH ? sk : load_meta<M16>(sl + OFF_K, lane & 15);   // KCH: beta for both
  };
  auto load_v = [&](int c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint8_t* sl = vslot(4 * c + p);
      if (BV == 8) {
        vq[2 * p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 32 * lane));
        vq[2 * p + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 32 * lane + 16));
      } else if (BV == 4) vq[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sl + 16 * lane));
      else { const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sl + 8 * lane)); vq[p] = u32x4{x[0], x[1], 0u, 0u}; }
    }
    const uint8_t* sl = vslot(4 * c + (bq >> 2));
    if constexpr (M16) {
      const u32x2 sw = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sl + CODE_V + 8 * (bq & 3)));
      const u32x2 ow = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sl + OFF_V + 8 * (bq & 3)));
      svq = f32x4{half_bits_to_float((uint16_t)sw[0]), half_bits_to_float((uint16_t)(sw[0] >> 16)),
                  half_bits_to_float((uint16_t)sw[1]), half_bits_to_float((uint16_t)(sw[1] >> 16))};
      ovq = f32x4{half_bits_to_float((uint16_t)ow[0]), half_bits_to_float((uint16_t)(ow[0] >> 16)),
                  half_bits_to_float((uint16_t)ow[1]), half_bits_to_float((uint16_t)(ow[1] >> 16))};
    } else {
      svq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sl + CODE_V + 16 * (bq & 3)));
      ovq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sl + OFF_V + 16 * (bq & 3)));
    }
  };
  auto load_alpha = [&](int c) {
    // QK steps of this lane: s = BLK st + bq % BLK; element k is channel qk_channel(s, k)
    const int tp = tile_page(c, (T == 32) ? (bq >> 3) : 0);
#pragma unroll
    for (int st = 0; st < SETS; ++st) {
      const int s = BLK * st + (bq % BLK);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ch = qk_channel<BK>(s, k);
        ak[st][k] = load_meta<M16>(kslot(tp + ch / AL) + ALPHA_K, ch % AL);
        if constexpr (KCH) mk[st][k] = load_meta<false>(kslot(tp + ch / AL) + ZP_K, ch % AL);
      }
    }
  };
  auto load_av = [&](int c) {
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int tpv = tile_page(c, tt);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = lane + 64 * h;
        av[tt][h] = load_meta<M16>(vslot(tpv + ch / AL) + ALPHA_V, ch % AL);
      }
    }
  };
  // At tile 128 a wave takes the two chunks of a tile back to back (partitions
  // cover whole tiles, c_begin is even), so the query fold and its channel
  // factors serve both; otherwise wave w takes chunks begin + w, + 4, ...
  constexpr bool PAIRS = (T == 128);
  auto next_chunk = [&](int c) { return PAIRS ? (((c - c_begin) & 1) ? c + 2 * kWaves - 1 : c + 1) : c + kWaves; };
  auto new_tile = [&](int c) { return !PAIRS || ((c - c_begin) & 1) == 0; };
  int chunk = c_begin + (PAIRS ? 2 * wave : wave);
  if (chunk < c_end) {
    load_alpha(chunk);
    load_k(chunk);
    load_v(chunk);
    load_av(chunk);
  }

  // ------------------------------------------------ H q of the group (wave 0), to LDS
  // stored divided by the weight of channel c's K code field (a power of two)
  if (wave == 0) {
    const int n16 = lane & 15, grp = lane >> 4;
    float hq[32];
    const unsigned sgw = sign_word(A.signs, grp);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x4 w = q_real ? qraw[v] : u32x4{0u, 0u, 0u, 0u};
      // randomized rotation: q's channels take the signs before H (keys are H s k)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] ^= sign_pair_mask_w(sgw, 8 * v, i);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hq[8 * v + 2 * i] = half_bits_to_float((uint16_t)(w[i] & 0xFFFF));
        hq[8 * v + 2 * i + 1] = half_bits_to_float((uint16_t)(w[i] >> 16));
      }
    }
#pragma unroll
    for (int bit = 1; bit < 32; bit <<= 1)
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i & bit) continue;
        const float lo = hq[i], hi = hq[i | bit];
        hq[i] = lo + hi;
        hq[i | bit] = lo - hi;
      }
    const float s16 = (grp & 1) ? -1.f : 1.f, s32 = (grp & 2) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) hq[i] = __builtin_fmaf(hq[i], s16, lane_xor<16>(hq[i]));
#pragma unroll
    for (int i = 0; i < 32; ++i) hq[i] = __builtin_fmaf(hq[i], s32, xor32(hq[i]));
    if (n16 < NH) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {   // channel 32 grp + i, stored in QK step order
        const int c = 32 * grp + i;
        sm.loop.hq[n16][qk_slot<BK>(c)] = hq[i] * (kInvSqrtD / k_field_weight<BK>(c));
      }
    }
  }
  __syncthreads();

  const float c0 = A.sm_scale_log2;
  float m_run[NH], l_run[NH];     // per head: running max (wave-uniform), partial sum (this lane's tokens)
  float acc[2][NH];               // [channel half][head]: channels lane, 64 + lane
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
    acc[0][h] = 0.f;
    acc[1][h] = 0.f;
  }

  // query fold, in the QK A layout: lane (bq, iq) holds qt[head 4 hg + iq]
  // [channels of step BLK st + bq % BLK] as fp16 hi / lo; qsum and the
  // power-of-two scale per (head, tile)
  f16x4 qa_hi[HG][SETS], qa_lo[HG][SETS];
  float cA[HG], cB[HG];
  // field weights of this lane's steps: elements 0, 1 weigh w0 and 2, 3 w1
  // (8 bits: 1 and 1; 4 bits: 1 and 16; 2 bits: w0 = 16 on odd steps, else 1,
  // and w1 = 4 w0; a step's parity is bq's)
  const float w0 = (BK != 2) ? 1.f : ((bq & 1) ? 16.f : 1.f);
  const float w1 = (BK == 8) ? 1.f : (BK == 4) ? 16.f : w0 * 4.f;
  // the split grids' constants kGrid / w (powers of two: exact products)
  const float g0 = w0 == 1.f ? kGrid : kGrid * (1.f / 16.f);
  const float g1 = (BK == 8) ? kGrid : (BK == 4) ? kGrid * (1.f / 16.f) : g0 * 0.25f;

  for (; chunk < c_end; chunk = next_chunk(chunk)) {
    const int next = next_chunk(chunk);
    const bool more = next < c_end;   // uniform
    // the chunk whose operands load into the registers this one frees: the
    // next, or past the last the spare slot, so that every load is issued
    // unconditionally and no register copy at the loop's end waits for them.
    // At tile 128 (waves of 16 chunks and more, alpha_K once per two chunks)
    // the loads stay conditional: there the extra loads cost more than the
    // copy's wait (same-box A/B at 6 x 128K: 192.6 against 203.7 us).
    constexpr bool UNCOND = (T != 128);
    const int ld = more ? next : c_begin + kMaxChunksPerPart;   // (past the last: the spare slot)

    // -------------------------------------------- query fold (once per tile)
    if (new_tile(chunk)) {
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int hh = 4 * hg + iq;
        float x[SETS][4];
        float qm0 = 0.f, qm1 = 0.f, qsum = 0.f;   // |x| maxima of the elements of weight w0 and w1
#pragma unroll
        for (int st = 0; st < SETS; ++st) {
          const int s = BLK * st + (bq % BLK);
          const f32x4 hv = *reinterpret_cast<const f32x4*>(&sm.loop.hq[hh][4 * s]);
#pragma unroll
          for (int k = 0; k < 4; ++k) x[st][k] = hv[k] * ak[st][k];
          qm0 = vmax3_abs(x[st][0], x[st][1], qm0);
          qm1 = vmax3_abs(x[st][2], x[st][3], qm1);
        }
        // the bound is on qt itself: x times the field weight
        float qmax = vmax(qm0 * w0, qm1 * w1);
        qmax = blocks_max<BLK>(qmax);
        int ex = (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127;
        ex = min(max(ex, -100), 100);
        // scaled qt below 2^(QE+1): its hi part is an integer of at most QE + 1 bits
        const float qscale = __uint_as_float((unsigned)(127 + QE - ex) << 23);    // 2^(QE-ex)
        const float qunscale = __uint_as_float((unsigned)(127 - QE + ex) << 23);  // 2^(ex-QE)
        // The offset term takes the sum of the query as the MFMA sees it (hi + lo):
        // the split's rounding then enters each score as sum_c err_c (S k_c + O),
        // in proportion to the restored key.  (With the exact sum it would leave
        // S sum_c err_c k_c against O sum_c qt_c, and in tiles of a few tokens,
        // where S and O reach 1e4..1e5 and nearly cancel, that costs ~1e-3.)
        // The pairs enter the sum through v_dot2 (fp16 products with the field
        // weights are exact in fp32).
        const f16x2 wp0{(_Float16)w0, (_Float16)w0}, wp1{(_Float16)w1, (_Float16)w1};
#pragma unroll
        for (int st = 0; st < SETS; ++st) {
          unsigned h01, l01, h23, l23;
          split_grid(x[st][0], x[st][1], qscale, qscale, g0, g0, h01, l01);
          split_grid(x[st][2], x[st][3], qscale, qscale, g1, g1, h23, l23);
          qa_hi[hg][st] = as_f16x4(h01, h23);
          qa_lo[hg][st] = as_f16x4(l01, l23);
          if constexpr (KCH) {   // sum_c qt_c M_c over the represented query
            const f16x2 a = __builtin_bit_cast(f16x2, h01), b = __builtin_bit_cast(f16x2, l01);
            const f16x2 c = __builtin_bit_cast(f16x2, h23), e = __builtin_bit_cast(f16x2, l23);
            const float z0 = w0 * mk[KCH ? st : 0][0], z1 = w0 * mk[KCH ? st : 0][1];
            const float z2 = w1 * mk[KCH ? st : 0][2], z3 = w1 * mk[KCH ? st : 0][3];
            qsum = __builtin_fmaf((float)a[0], z0, qsum);
            qsum = __builtin_fmaf((float)b[0], z0, qsum);
            qsum = __builtin_fmaf((float)a[1], z1, qsum);
            qsum = __builtin_fmaf((float)b[1], z1, qsum);
            qsum = __builtin_fmaf((float)c[0], z2, qsum);
            qsum = __builtin_fmaf((float)e[0], z2, qsum);
            qsum = __builtin_fmaf((float)c[1], z3, qsum);
            qsum = __builtin_fmaf((float)e[1], z3, qsum);
          } else {
            qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h01), wp0, qsum, false);
            qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, l01), wp0, qsum, false);
            qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h23), wp1, qsum, false);
            qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, l23), wp1, qsum, false);
          }
        }
        qsum = blocks_sum<BLK>(qsum) * qunscale;
        cA[hg] = c0 * kTwo24 * qunscale;   // score = S D cA + O cB
        cB[hg] = c0 * qsum;
      }
    }
    if (UNCOND || (more && new_tile(next))) load_alpha(ld);

    // -------------------------------------------- QK: lane = token, 4 heads per group
    f32x4 d[HG], dl[HG];   // hi chain (exact) and lo chain
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      d[hg] = f32x4{0.f, 0.f, 0.f, 0.f};
      dl[hg] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    static_for<0, 32>([&](auto S_) {
      constexpr int s = decltype(S_)::value;
      f16x4 b;
      if constexpr (BK == 8) {
        const unsigned x = kq[s >> 2][s & 3], y = x >> 8;
        b = as_f16x4(code_field<8, 0>(x, y), code_field<8, 1>(x, y));
      } else if constexpr (BK == 4) {
        const unsigned x = kq[s >> 3][(s >> 1) & 3], y = x >> 8;
        if constexpr ((s & 1) == 0) b = as_f16x4(code_field<4, 0>(x, y), code_field<4, 1>(x, y));
        else b = as_f16x4(code_field<4, 2>(x, y), code_field<4, 3>(x, y));
      } else {
        const unsigned x = kq[s >> 3][(s >> 2) & 1], y = x >> 8;
        constexpr int X0 = 2 * (s & 3);
        b = as_f16x4(code_field<2, X0>(x, y), code_field<2, X0 + 1>(x, y));
      }
      constexpr int st = s / BLK, abid = s % BLK;
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        d[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(qa_hi[hg][st], b, d[hg], CB, abid, 0);
        dl[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(qa_lo[hg][st], b, dl[hg], CB, abid, 0);
      }
    });
    // per-head score factors of this token's tile: lane iq of its broadcast group
    float sc[HG][4];
    const int tok = chunk * kChunk + lane;
    const bool past = tok >= L;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float fa, fb;
        if constexpr (T == 32) {
          fa = __shfl(cA[hg], (lane & 32) + i);
          fb = __shfl(cB[hg], (lane & 32) + i);
        } else {
          fa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cA[hg]), i));
          fb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cB[hg]), i));
        }
        const bool masked = MQ ? tok >= vis[4 * hg + i] : past;
        sc[hg][i] = masked ? -INFINITY : __builtin_fmaf(fa * sk, d[hg][i] + dl[hg][i], fb * ok);
      }
    if (UNCOND || more) load_k(ld);

    // -------------------------------------------- online softmax (base 2), per head
    // the running max moves only when a chunk's scores pass it: a test in
    // each lane and one vote over the wave decide, and only then are the
    // chunk's maxima reduced over the wave (m_run is the same in every lane)
    bool pass = false;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int i = 0; i < 4; ++i) pass |= sc[hg][i] > m_run[4 * hg + i];
    if (__builtin_amdgcn_ballot_w64(pass) != 0) {   // wave-uniform
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float m_new = fmaxf(m_run[h], wave_max(sc[h >> 2][h & 3]));
        // (MQ: a row may have seen no visible token yet; -inf - -inf is no number)
        const float corr = (MQ && m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
        m_run[h] = m_new;
        l_run[h] *= corr;
        acc[0][h] *= corr;
        acc[1][h] *= corr;
      }
    }
    // probabilities scaled by 2^k per chunk so that P = p S_V stays below 2^(PE+1)
    // (its hi part is an integer of at most PE + 1 bits)
    float smax = fmaxf(fmaxf(svq[0], svq[1]), fmaxf(svq[2], svq[3]));
    smax = wave_max(smax);   // scales are >= 0
    int pe = (int)((__float_as_uint(smax) >> 23) & 0xFF) - 127;
    pe = min(max(pe, -100), 100);
    const float pk = (float)(PE - pe);
    const float pinv = __uint_as_float((unsigned)(127 - PE + pe) << 23);  // 2^-k
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * hg + i;
        const float mb = (MQ && m_run[h] == -INFINITY) ? 0.f : m_run[h];   // masked rows: p = 0
        const float p = __builtin_amdgcn_exp2f(sc[hg][i] - (mb - pk));
        l_run[h] = __builtin_fmaf(p, pinv, l_run[h]);
        sm.loop.pt[wave][h][lane] = p;
      }
    asm volatile("" ::: "memory");  // the reads below see this wave's writes (LDS keeps order)

    // -------------------------------------------- PV A operands: P^T, lane (bq, iq) = tokens 4 bq.., head iq
    f16x4 pa_hi[HG], pa_lo[HG];
    float spo[HG];
    {
      // As on the K side, the offset term sum_t p_t O_t is taken through the
      // represented P (hi + lo): p_t O_t = P_t (O_t / sw_t); a row of zero range
      // (sw = 0, P = 0) keeps its exact p_t O_t.
      const f32x4 sw{svq[0], svq[1], svq[2] * (1.f / kTok), svq[3] * (1.f / kTok)};
      f32x4 zr;   // O / sw, nearest (reciprocal refined by one Newton step)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float rc = __builtin_amdgcn_rcpf(sw[k]);
        const float z0 = ovq[k] * rc;
        zr[k] = sw[k] > 0.f ? __builtin_fmaf(__builtin_fmaf(-sw[k], z0, ovq[k]), rc, z0) : 0.f;
      }
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&sm.loop.pt[wave][4 * hg + iq][4 * bq]);
        unsigned h01, l01, h23, l23;
        split_grid(p4[0], p4[1], sw[0], sw[1], kGrid, kGrid, h01, l01);
        split_grid(p4[2], p4[3], sw[2], sw[3], kGrid / kTok, kGrid / kTok, h23, l23);
        pa_hi[hg] = as_f16x4(h01, h23);
        pa_lo[hg] = as_f16x4(l01, l23);
        const f16x2 a = __builtin_bit_cast(f16x2, h01), b = __builtin_bit_cast(f16x2, l01);
        const f16x2 c = __builtin_bit_cast(f16x2, h23), e = __builtin_bit_cast(f16x2, l23);
        float po = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (!(sw[k] > 0.f)) po = __builtin_fmaf(p4[k], ovq[k], po);
        po = __builtin_fmaf((float)a[0], zr[0], po);
        po = __builtin_fmaf((float)b[0], zr[0], po);
        po = __builtin_fmaf((float)a[1], zr[1], po);
        po = __builtin_fmaf((float)b[1], zr[1], po);
        po = __builtin_fmaf((float)c[0], zr[2], po);
        po = __builtin_fmaf((float)e[0], zr[2], po);
        po = __builtin_fmaf((float)c[1], zr[3], po);
        po = __builtin_fmaf((float)e[1], zr[3], po);
        spo[hg] = blocks_sum<(T == 32) ? 8 : 16>(po) * pinv;   // per tile: sum_t p_t O_t, head iq
      }
    }

    // -------------------------------------------- PV: lane = channel, 4 heads per group
    // one tile at a time (a T = 32 chunk holds two, each with its own alpha_V)
    f32x4 vh[2][HG], vl[2][HG];   // [channel half][group]: hi chain (exact) and lo chain
    auto pv_tile = [&](auto TT_) {
      constexpr int tt = decltype(TT_)::value;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          vh[h][hg] = f32x4{0.f, 0.f, 0.f, 0.f};
          vl[h][hg] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      static_for<tt * (16 / TPC), (tt + 1) * (16 / TPC)>([&](auto S_) {
        constexpr int s = decltype(S_)::value;   // tokens 4 s .. 4 s + 3: page s / 4, quad g = s % 4
        constexpr int g = s & 3;
        f16x4 b[2];
        if constexpr (BV == 8) {
          // word 2 g + h of the page's run: tokens 4 g .. 4 g + 3 in fields 0, 2, 1, 3
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const unsigned x = vq[2 * (s >> 2) + (g >> 1)][2 * (g & 1) + h], y = x >> 8;
            b[h] = as_f16x4(code_field<8, 0>(x, y), code_field<8, 1>(x, y));
          }
        } else if constexpr (BV == 4) {
          const unsigned x = vq[s >> 2][g], y = x >> 8;
          b[0] = as_f16x4(code_field<4, 0>(x, y), code_field<4, 1>(x, y));
          b[1] = as_f16x4(code_field<4, 2>(x, y), code_field<4, 3>(x, y));
        } else {
          const unsigned x = vq[s >> 2][g >> 1], y = x >> 8;
          constexpr int X0 = 4 * (g & 1);
          b[0] = as_f16x4(code_field<2, X0>(x, y), code_field<2, X0 + 1>(x, y));
          b[1] = as_f16x4(code_field<2, X0 + 2>(x, y), code_field<2, X0 + 3>(x, y));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            vh[h][hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa_hi[hg], b[h], vh[h][hg], 4, s, 0);
            vl[h][hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa_lo[hg], b[h], vl[h][hg], 4, s, 0);
          }
      });
    };
    // acc += alpha_V (sum_t p_t S_t k_t + sum_t p_t O_t) over the tile
    // (vh, vl carry 2^(k-24) times the channel half's V field weight)
    auto pv_fold = [&](int tt) {
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float so = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(spo[hg]), 32 * tt + i));
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float cf = kTwo24 * pinv * ((BV == 2 && h == 1) ? (1.f / 16.f) : 1.f);
            const float y = __builtin_fmaf(vl[h][hg][i], cf, __builtin_fmaf(vh[h][hg][i], cf, so));
            acc[h][4 * hg + i] = __builtin_fmaf(av[tt][h], y, acc[h][4 * hg + i]);
          }
        }
    };
    pv_tile(std::integral_constant<int, 0>{});
    if constexpr (TPC == 2) {
      pv_fold(0);
      pv_tile(std::integral_constant<int, 1>{});
    }
    if (UNCOND || more) load_v(ld);
    pv_fold(TPC - 1);
    if (UNCOND || more) load_av(ld);
  }

  // ------------------------------------------------ merge the waves, write the partition's partial
#pragma unroll
  for (int h = 0; h < NH; ++h) l_run[h] = wave_sum(l_run[h]);
  __syncthreads();  // every wave is done with the loop buffers
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    sm.merge.acc[wave][h][lane] = acc[0][h];
    sm.merge.acc[wave][h][64 + lane] = acc[1][h];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      sm.merge.m[wave][h] = m_run[h];
      sm.merge.l[wave][h] = l_run[h];
    }
  }
  __syncthreads();
  // thread -> (head, 4 channels)
  for (int it = threadIdx.x; it < nrows * 32; it += 64 * kWaves) {
    const int h = it >> 5, c = 4 * (it & 31);
    float M = sm.merge.m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.merge.m[w][h]);
    float wt[kWaves], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.merge.m[w][h];
      wt[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      lsum = __builtin_fmaf(wt[w], sm.merge.l[w][h], lsum);
    }
    f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.merge.acc[w][h][c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(wt[w], y[e], x[e]);
    }
    size_t pidx;
    if constexpr (MQ) {
      const int r = r0 + h;
      pidx = (((size_t)seq * A.n_q + r / G) * A.q_heads + kvh * G + r % G) * A.max_parts + part;
    } else {
      pidx = ((size_t)seq * A.q_heads + kvh * G + h) * A.max_parts + part;
    }
    *reinterpret_cast<f32x4*>(A.ws_acc + pidx * kHeadDim + c) = x;
    if (c == 0) {
      A.ws_ml[2 * pidx] = M;
      A.ws_ml[2 * pidx + 1] = lsum;
    }
  }
}

template <typename F>
hipError_t by_tile(int tile, F&& f) {
  switch (tile) {
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
  }
  return hipErrorInvalidValue;
}
// Slot formats: fp32 metadata (code widths 2 and 4 in any pairing, 8 for
// both), fp16 metadata or K rounded per channel (2 and 4 only).
template <int FMT, typename F>
hipError_t by_format(int bits_k, int bits_v, F&& f) {
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  if constexpr (FMT == kFmtFp32) {
    if (bits_k == 8 && bits_v == 8) return f(I8{}, I8{});
  }
  if (bits_k == 4 && bits_v == 4) return f(I4{}, I4{});
  if (bits_k == 4 && bits_v == 2) return f(I4{}, I2{});
  if (bits_k == 2 && bits_v == 4) return f(I2{}, I4{});
  if (bits_k == 2 && bits_v == 2) return f(I2{}, I2{});
  return hipErrorInvalidValue;
}
// K and V code widths: 2 and 4 in any pairing, 8 for both
template <typename F>
hipError_t by_bits_pair(int bits_k, int bits_v, F&& f) {
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  if (bits_k == 8 && bits_v == 8) return f(I8{}, I8{});
  if (bits_k == 4 && bits_v == 4) return f(I4{}, I4{});
  if (bits_k == 4 && bits_v == 2) return f(I4{}, I2{});
  if (bits_k == 2 && bits_v == 4) return f(I2{}, I4{});
  if (bits_k == 2 && bits_v == 2) return f(I2{}, I2{});
  return hipErrorInvalidValue;
}

// Launchers of the decode kernel for one metadata format (each translation
// unit instantiates one format); the partition merge follows.
template <int FMT>
hipError_t launch_decode_fmt(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format<FMT>(bits_k, bits_v, [&](auto BK, auto BV) {
      constexpr bool M16 = FMT == kFmtM16, KCH = FMT == kFmtKch;
      dim3 grid(a.kv_heads * a.num_seqs, a.max_parts);
      const QuantArgs q{};
      if (a.group <= 4)
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 1, false, false, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      else if (a.group <= 8)
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 2, false, false, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      else
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 4, false, false, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_combine(a, kChunk, true, s);
    });
  });
}

template <int FMT>
hipError_t launch_append_decode_fmt(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                    hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format<FMT>(bits_k, bits_v, [&](auto BK, auto BV) {
      constexpr bool M16 = FMT == kFmtM16, KCH = FMT == kFmtKch;
      dim3 grid(a.kv_heads * a.num_seqs, a.max_parts);
      if (a.group <= 4)
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 1, true, false, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      else if (a.group <= 8)
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 2, true, false, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      else
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 4, true, false, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      DecodeArgs b = a;
      b.seq_lens_plus_one = 1;
      return launch_combine(b, kChunk, true, s);
    });
  });
}

// Several queries per sequence: rows beyond 4 run in blocks of 8 (two groups
// of 4 heads); blocks of 16 read the pages once but measured slower (a
// 4-token verify at 4 x 16K, 8 kv / 32 query heads: 97 us against 67 us), as
// did blocks of 4 (88 us).
template <int FMT>
hipError_t launch_multi_query_fmt(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format<FMT>(bits_k, bits_v, [&](auto BK, auto BV) {
      constexpr bool M16 = FMT == kFmtM16, KCH = FMT == kFmtKch;
      const int rows = a.n_q * a.group;
      const QuantArgs q{};
      if (rows <= 4) {
        dim3 grid(a.kv_heads * a.num_seqs, a.max_parts);
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 1, false, true, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      } else {
        dim3 grid(a.kv_heads * ((rows + 7) / 8) * a.num_seqs, a.max_parts);
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 2, false, true, M16, KCH>), grid, dim3(64 * kWaves), 0, s, a, q);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_combine(a, 64, true, s);
    });
  });
}

}  // namespace
}  // namespace kvq
