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
// tiles).  The group of G query heads sharing the kv head is padded to 16
// MFMA columns and both contractions run on v_mfma_f32_16x16x32_f16:
//   QK:  S^T[t][g] = sum_c K[t][c] W[c][g]: A = 16 tokens of codes, B = qt
//        split into fp16 hi + lo (two MFMAs into one accumulator).
//   PV:  O^T[c][g] = sum_t V[t][c] P[t][g]: A = codes of 2 pages (32 tokens),
//        B = p_t S_t split into fp16 hi + lo.
// Codes enter the MFMA as fp16 denormals: a field masked in place in its
// 16-bit half reads as (code * 2^e) * 2^-24, exactly, with e fixed by the
// field's position; the matching 2^-e rides on the query (K side), on the
// probabilities (V tokens) or on the output fold (V channels).  Unpacking is
// one AND per two codes.  The QK output layout (lane = query head, 4 tokens
// per lane) is exactly the B layout PV needs, so no shuffle sits between the
// two.  Online softmax runs per tile; partitions are merged by a second
// kernel that also applies the final Hadamard.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x8 as_f16x8(unsigned a, unsigned b, unsigned c, unsigned d) {
  u32x4 v{a, b, c, d};
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32); }

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
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}

// Reductions over the 4 lanes l, l^16, l^32, l^48 (one query head's lanes).
__device__ __forceinline__ float group_max(float v) { return max32(max16(v)); }
__device__ __forceinline__ float group_sum(float v) { return sum32(sum16(v)); }

constexpr int kWaves = 4;  // waves per decode workgroup

// Metadata of one tile as staged in LDS: the slots' (scale, offset, alpha
// slice) areas, K pages then V pages, each META bytes.
template <int T>
struct TileMeta {
  static constexpr int NP = T / kPage;
  static constexpr int META = 8 * kPage + 4 * slot_alpha_len(T);  // bytes per slot
  static constexpr int BYTES = 2 * NP * META;
  static constexpr int PIECES = BYTES / 16;                     // 16-byte loads
  static constexpr int PER_LANE = (PIECES + 63) / 64;
};

constexpr int kMaxTilesPerPart = 64;

// Code fields of one 32-bit word (two 16-bit halves), masked in place so that
// each half reads as the fp16 denormal m * 2^-24 whose mantissa m is the code
// times the power of two fixed by the field's bit position (field_weight).
// Fields in bits 8..15 of a half are taken from y = x >> 8.  One AND per pair
// of codes, no conversion and no offset term.
template <int BITS, int X>
__device__ __forceinline__ unsigned code_field(unsigned x, unsigned y) {
  if (BITS == 4) {
    constexpr unsigned m = (X & 1) ? 0x00F000F0u : 0x000F000Fu;
    return ((X < 2) ? x : y) & m;
  } else {
    constexpr unsigned m = 0x00030003u << (2 * (X & 3));
    return ((X < 4) ? x : y) & m;
  }
}
template <int BITS>
__host__ __device__ constexpr float field_weight(int x) {
  return BITS == 4 ? ((x & 1) ? 16.f : 1.f) : (float)(1 << (2 * (x & 3)));
}

template <int T, int U>
struct alignas(16) DecodeSmem {
  int32_t pages[kMaxTilesPerPart * (T / kPage)];  // the partition's page ids
  union {
    struct {
      float hq[4 * U][kHeadDim];                       // (H q)_c / weight of channel c's K field
      uint8_t meta[kWaves][2][TileMeta<T>::BYTES];     // per-wave double buffer
      u32x4 qb[kWaves][2][4 * U][16];                  // per-wave QK B operands [hi/lo][head][unit]
      float cab[kWaves][4 * U][2];                     // per-wave, per head: score factors
    } loop;
    struct {
      float acc[kWaves][16][kHeadDim];
      float m[kWaves][16];
      float l[kWaves][16];
    } merge;
  };
};

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, lane_xor<1>(v));
  v = fmaxf(v, lane_xor<2>(v));
  v = fmaxf(v, lane_xor<4>(v));
  v = fmaxf(v, lane_xor<8>(v));
  return group_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += lane_xor<1>(v);
  v += lane_xor<2>(v);
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  return group_sum(v);
}

// Sum / max over aligned groups of N lanes (N <= 16).
template <int N>
__device__ __forceinline__ float span_sum(float v) {
  if (N > 1) v += lane_xor<1>(v);
  if (N > 2) v += lane_xor<2>(v);
  if (N > 4) v += lane_xor<4>(v);
  if (N > 8) v += lane_xor<8>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float span_max(float v) {
  if (N > 1) v = fmaxf(v, lane_xor<1>(v));
  if (N > 2) v = fmaxf(v, lane_xor<2>(v));
  if (N > 4) v = fmaxf(v, lane_xor<4>(v));
  if (N > 8) v = fmaxf(v, lane_xor<8>(v));
  return v;
}

// fp32 pair -> fp16 pair hi (nearest even) and the fp16 pair lo of what is
// left (x - hi is exact in fp32; v_fma_mix_f32 reads hi's halves as fp16).
// hi + lo carries x to ~2^-22 relative, without bias.
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
  const unsigned hb = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x0, x1}, f16x2));
  float r0, r1;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r0) : "v"(hb), "v"(x0));
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r1) : "v"(hb), "v"(x1));
  hi = hb;
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, f16x2));
}

// One workgroup of 4 waves per (partition of tiles, kv head, sequence); wave
// w takes tiles begin + w, begin + w + 4, ...  Each wave prefetches its next
// tile's codes (registers) and metadata (registers, then LDS) while it works
// on the current one; the 4 waves' softmax states are merged in LDS at the end.
//
// U = 1, 2, 4 for groups of up to 4, 8, 16 query heads.  Per tile, the query
// fold qt = (H q) * alpha_K runs in a compact layout (lane = head, 8U
// channels) and reaches the MFMA B layout through LDS; MFMA column n reads
// head n mod 4U, so columns past the group repeat real heads and need no mask.
template <int T, int BK, int BV, int U>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs A) {
  using TM = TileMeta<T>;
  constexpr int NP = TM::NP;
  constexpr int META = TM::META;
  constexpr int SLOT_K = slot_bytes(BK, T), SLOT_V = slot_bytes(BV, T);
  constexpr int CODE_K = slot_code_bytes(BK), CODE_V = slot_code_bytes(BV);
  constexpr int AL = slot_alpha_len(T);
  constexpr int NH = 4 * U;      // heads laid out per kv head
  constexpr int LPH = 16 / U;    // fold lanes per head
  // V fields of tokens 2 and 3 of a quad weigh kTok times those of tokens 0, 1:
  // their probabilities enter the B operand divided by kTok (2^-kL2Tok).
  constexpr float kTok = (BV == 4) ? 16.f : 4.f;
  constexpr float kL2Tok = (BV == 4) ? 4.f : 2.f;
  constexpr float kTwo24 = 16777216.f;
  __shared__ DecodeSmem<T, U> sm;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int part = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int G = A.group;
  const int L = A.seq_lens[seq];
  const int ntiles = min((L + T - 1) / T, A.max_tiles);
  const int tile_begin = part * A.tiles_per_part;
  const int tile_end = min(ntiles, tile_begin + A.tiles_per_part);
  if (tile_begin >= tile_end) return;  // uniform over the workgroup
  const int H = A.kv_heads;
  const int head = n16 % NH;           // query head of this lane's MFMA column
  // the partition's page ids, staged once in LDS
  {
    const int32_t* row = A.block_table + (size_t)seq * A.max_blocks + tile_begin * NP;
    const int n = (tile_end - tile_begin) * NP;
    for (int i = threadIdx.x; i < n; i += 64 * kWaves) sm.pages[i] = row[i];
  }
  __syncthreads();

  // ------------------------------------------------ prefetch of one tile
  u32x4 ck[NP], cv[NP], mpre[TM::PER_LANE];
  auto issue = [&](int tl) {
    const int32_t* tp = sm.pages + (tl - tile_begin) * NP;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const size_t pg = (size_t)__builtin_amdgcn_readfirstlane(tp[p]) * H + kvh;
      const uint8_t* sk = A.pool_k + pg * SLOT_K;
      const uint8_t* sv = A.pool_v + pg * SLOT_V;
      if (BK == 4) ck[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sk + 16 * lane));
      else { const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sk + 8 * lane)); ck[p] = u32x4{x[0], x[1], 0u, 0u}; }
      if (BV == 4) cv[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sv + 16 * lane));
      else { const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sv + 8 * lane)); cv[p] = u32x4{x[0], x[1], 0u, 0u}; }
    }
#pragma unroll
    for (int j = 0; j < TM::PER_LANE; ++j) {
      const int i = lane + 64 * j;
      if (i < TM::PIECES) {
        const int role = i / (NP * META / 16);
        const int rem = i % (NP * META / 16);
        const int p = rem / (META / 16), off = 16 * (rem % (META / 16));
        const size_t pg = (size_t)tp[p] * H + kvh;
        const uint8_t* src = role == 0 ? A.pool_k + pg * SLOT_K + CODE_K : A.pool_v + pg * SLOT_V + CODE_V;
        mpre[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off));
      }
    }
  };
  int tile = tile_begin + wave;
  if (tile < tile_end) issue(tile);

  // ------------------------------------------------ H q of the group (wave 0), to LDS
  // stored divided by the weight of channel c's K code field (a power of two)
  if (wave == 0) {
    const bool real = n16 < G;
    float hq[32];
    const uint16_t* qrow = A.q + ((size_t)seq * A.q_heads + kvh * G + (real ? n16 : 0)) * kHeadDim + 32 * grp;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4 w = real ? *reinterpret_cast<const u32x4*>(qrow + 8 * v) : u32x4{0u, 0u, 0u, 0u};
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
      for (int v = 0; v < 8; ++v) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = hq[4 * v + e] * (kInvSqrtD / field_weight<BK>(e));
        *reinterpret_cast<f32x4*>(&sm.loop.hq[n16][32 * grp + 4 * v]) = x;
      }
    }
  }
  __syncthreads();

  const float c0 = A.sm_scale_log2;
  // fold layout: lane -> head fh, units fu0 .. fu0 + U - 1 (unit = chunk + 4 lane group)
  const int fh = lane / LPH;
  const int fu0 = (lane % LPH) * U;
  float m_run = -INFINITY, l_run = 0.f;
  float acc[8][4];  // [block i][r]: channel 32 grp + 8 r + i, query head of column n16
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;

  int buf = 0;
  for (; tile < tile_end; tile += kWaves) {
    // stage this tile's metadata, then start loading the next tile
    uint8_t* mb = sm.loop.meta[wave][buf];
#pragma unroll
    for (int j = 0; j < TM::PER_LANE; ++j) {
      const int i = lane + 64 * j;
      if (i < TM::PIECES) *reinterpret_cast<u32x4*>(mb + 16 * i) = mpre[j];
    }
    u32x4 kc[NP], vc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) { kc[p] = ck[p]; vc[p] = cv[p]; }
    if (tile + kWaves < tile_end) issue(tile + kWaves);
    const uint8_t* mK = mb;              // page p: S at +0, O at +64, alpha slice at +128
    const uint8_t* mV = mb + NP * META;

    // -------------------------------------------- query fold: qt = (H q) * alpha_K (compact)
    {
      constexpr int D1 = (BK == 4) ? 4 : 8;   // slot j -> channel cb + (j >> 1) + D1 (j & 1)
      float qv[U][8];
      float qsum = 0.f, qmax = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int unit = fu0 + u, ch = unit & 3, g4 = unit >> 2;
        const int cb = (BK == 4) ? 32 * g4 + 8 * ch : 32 * g4 + 16 * (ch >> 1) + 4 * (ch & 1);
        const f32x4 h0 = *reinterpret_cast<const f32x4*>(&sm.loop.hq[fh][cb]);
        const f32x4 h1 = *reinterpret_cast<const f32x4*>(&sm.loop.hq[fh][cb + D1]);
        const uint8_t* ap = mK + (cb / AL) * META + 8 * kPage + 4 * (cb % AL);
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(ap);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(ap + 4 * D1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (j & 1) ? h1[j >> 1] * a1[j >> 1] : h0[j >> 1] * a0[j >> 1];
          qv[u][j] = x;
          qmax = fmaxf(qmax, fabsf(x));
        }
      }
      qmax = span_max<LPH>(qmax);
      // a power-of-two scale per head keeps the fp16 split in range
      int ex = (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127;
      ex = min(max(ex, -100), 100);
      const float qscale = __uint_as_float((unsigned)(127 + 14 - ex) << 23);    // 2^(14-ex)
      const float qunscale = __uint_as_float((unsigned)(127 - 14 + ex) << 23);  // 2^(ex-14)
      // The offset term uses the sum of the query exactly as the MFMA sees it
      // (hi + lo), so that the split's rounding enters every score as
      // sum_c err_c (S k_c + O), proportional to the restored key, instead of
      // leaving S sum_c err_c k_c against O sum_c qt_c uncancelled.
#pragma unroll
      for (int u = 0; u < U; ++u) {
        u32x4 hi, lo;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          unsigned h, l;
          split_pair(qv[u][2 * m] * qscale, qv[u][2 * m + 1] * qscale, h, l);
          hi[m] = h;
          lo[m] = l;
          const f16x2 hh = __builtin_bit_cast(f16x2, h), ll = __builtin_bit_cast(f16x2, l);
          const float w = field_weight<BK>(m);   // slots 2m, 2m + 1 share field m
          qsum = __builtin_fmaf((float)hh[0], w, qsum);
          qsum = __builtin_fmaf((float)ll[0], w, qsum);
          qsum = __builtin_fmaf((float)hh[1], w, qsum);
          qsum = __builtin_fmaf((float)ll[1], w, qsum);
        }
        sm.loop.qb[wave][0][fh][fu0 + u] = hi;
        sm.loop.qb[wave][1][fh][fu0 + u] = lo;
      }
      qsum = span_sum<LPH>(qsum) * qunscale;
      if ((lane % LPH) == 0) {
        sm.loop.cab[wave][fh][0] = c0 * kTwo24 * qunscale;  // score = S D cab0 + O cab1
        sm.loop.cab[wave][fh][1] = c0 * qsum;
      }
    }
    asm volatile("" ::: "memory");  // the reads below see this wave's writes (LDS keeps order)
    f16x8 bq_hi[4], bq_lo[4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      bq_hi[ch] = __builtin_bit_cast(f16x8, sm.loop.qb[wave][0][head][ch + 4 * grp]);
      bq_lo[ch] = __builtin_bit_cast(f16x8, sm.loop.qb[wave][1][head][ch + 4 * grp]);
    }
    const float sA = sm.loop.cab[wave][head][0];
    const float sB = sm.loop.cab[wave][head][1];

    // -------------------------------------------- scores of the tile's pages
    // chunk-major order: the NP pages' accumulation chains interleave
    f32x4 d[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) d[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        f16x8 a;
        if (BK == 4) {
          const unsigned x = kc[p][ch], y = x >> 8;
          a = as_f16x8(code_field<4, 0>(x, y), code_field<4, 1>(x, y), code_field<4, 2>(x, y),
                       code_field<4, 3>(x, y));
        } else {
          const unsigned x = kc[p][ch >> 1], y = x >> 8;
          if (ch & 1)
            a = as_f16x8(code_field<2, 4>(x, y), code_field<2, 5>(x, y), code_field<2, 6>(x, y),
                         code_field<2, 7>(x, y));
          else
            a = as_f16x8(code_field<2, 0>(x, y), code_field<2, 1>(x, y), code_field<2, 2>(x, y),
                         code_field<2, 3>(x, y));
        }
        d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq_hi[ch], d[p], 0, 0, 0);
        d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq_lo[ch], d[p], 0, 0, 0);
      }
    }
    float s[NP][4];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const f32x4 S = *reinterpret_cast<const f32x4*>(mK + p * META + 16 * grp);
      const f32x4 O = *reinterpret_cast<const f32x4*>(mK + p * META + 4 * kPage + 16 * grp);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[p][r] = __builtin_fmaf(sA * S[r], d[p][r], sB * O[r]);
    }
    if (tile == ntiles - 1 && (L % T) != 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile * T + p * kPage + 4 * grp + r >= L) s[p][r] = -INFINITY;
    }

    // -------------------------------------------- online softmax (base 2)
    // the running max moves only when some score passes it; otherwise the
    // accumulators need no rescale (checked for the whole wave at once)
    float tmax = s[0][0];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[p][r]);
    tmax = group_max(tmax);
    if (__builtin_amdgcn_ballot_w64(tmax > m_run) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][r] *= corr;
    }
    // P = p S enters the MFMA as fp16 hi + lo; a power of two 2^k per tile,
    // carried by the exponent of p, puts max P at 2^14..2^15 so that lo stays
    // a normal fp16 (its 11 bits are what make hi + lo nearly fp32-exact)
    float smax = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const f32x4 S = *reinterpret_cast<const f32x4*>(mV + p * META + 16 * grp);
      smax = fmaxf(smax, fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])));
    }
    smax = group_max(smax);   // scales are >= 0
    int pe = (int)((__float_as_uint(smax) >> 23) & 0xFF) - 127;
    pe = min(max(pe, -100), 100);
    const float pk = (float)(14 - pe);                                   // k
    const float pinv = __uint_as_float((unsigned)(127 - 14 + pe) << 23);  // 2^-k
    const float m_lo = m_run - pk, m_hi = m_lo + kL2Tok;
    float psa = 0.f, psb = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[p][r] = __builtin_amdgcn_exp2f(s[p][r] - (r < 2 ? m_lo : m_hi));
        if (r < 2) psa += s[p][r];
        else psb += s[p][r];
      }
    l_run = __builtin_fmaf(pinv, __builtin_fmaf(kTok, psb, psa), l_run);

    // -------------------------------------------- values of the tile's pages
    float vacc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) vacc[i][r] = 0.f;
    float spa = 0.f, spb = 0.f;
#pragma unroll
    for (int pp = 0; pp < NP; pp += 2) {
      unsigned bh[4], bl[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f32x4 S = *reinterpret_cast<const f32x4*>(mV + (pp + h2) * META + 16 * grp);
        const f32x4 O = *reinterpret_cast<const f32x4*>(mV + (pp + h2) * META + 4 * kPage + 16 * grp);
        float pw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pw[r] = s[pp + h2][r] * S[r];
          if (r < 2) spa = __builtin_fmaf(s[pp + h2][r], O[r], spa);
          else spb = __builtin_fmaf(s[pp + h2][r], O[r], spb);
        }
        split_pair(pw[0], pw[1], bh[2 * h2], bl[2 * h2]);
        split_pair(pw[2], pw[3], bh[2 * h2 + 1], bl[2 * h2 + 1]);
      }
      const f16x8 ph = as_f16x8(bh[0], bh[1], bh[2], bh[3]);
      const f16x8 pl = as_f16x8(bl[0], bl[1], bl[2], bl[3]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        unsigned u[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          if (BV == 4) {
            const unsigned x = vc[pp + h2][i >> 1], y = x >> 8;
            if (i & 1) { u[2 * h2] = code_field<4, 2>(x, y); u[2 * h2 + 1] = code_field<4, 3>(x, y); }
            else { u[2 * h2] = code_field<4, 0>(x, y); u[2 * h2 + 1] = code_field<4, 1>(x, y); }
          } else {
            const unsigned x = vc[pp + h2][i >> 2], y = x >> 8;
            switch (i & 3) {
              case 0: u[2 * h2] = code_field<2, 0>(x, y); u[2 * h2 + 1] = code_field<2, 1>(x, y); break;
              case 1: u[2 * h2] = code_field<2, 2>(x, y); u[2 * h2 + 1] = code_field<2, 3>(x, y); break;
              case 2: u[2 * h2] = code_field<2, 4>(x, y); u[2 * h2 + 1] = code_field<2, 5>(x, y); break;
              default: u[2 * h2] = code_field<2, 6>(x, y); u[2 * h2 + 1] = code_field<2, 7>(x, y); break;
            }
          }
        }
        const f16x8 a = as_f16x8(u[0], u[1], u[2], u[3]);
        f32x4 dv{vacc[i][0], vacc[i][1], vacc[i][2], vacc[i][3]};
        dv = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ph, dv, 0, 0, 0);
        dv = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pl, dv, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) vacc[i][r] = dv[r];
      }
    }
    const float spo = group_sum(__builtin_fmaf(kTok, spb, spa)) * pinv;   // sum_t p_t O_t

    // -------------------------------------------- fold: acc += alpha_V (sum_t p_t S_t k_t + sum_t p_t O_t)
    // (vacc carries 2^(k-24) times the V field weight of block i)
    const float cf0 = kTwo24 * pinv, cf1 = (BV == 2) ? cf0 * (1.f / 16.f) : cf0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 32 * grp + 8 * r;
      const uint8_t* ap = mV + (c / AL) * META + 8 * kPage + 4 * (c % AL);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(ap);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(ap + 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float al = (i < 4) ? a0[i] : a1[i - 4];
        const float t = __builtin_fmaf(vacc[i][r], (i & 1) ? cf1 : cf0, spo);
        acc[i][r] = __builtin_fmaf(al, t, acc[i][r]);
      }
    }
    buf ^= 1;
  }

  // ------------------------------------------------ merge the waves, write the partition's partial
  l_run = group_sum(l_run);
  __syncthreads();  // every wave is done with the loop buffers
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* dst = &sm.merge.acc[wave][n16][32 * grp + 8 * r];
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
  }
  if (grp == 0) {
    sm.merge.m[wave][n16] = m_run;
    sm.merge.l[wave][n16] = l_run;
  }
  __syncthreads();
  if (wave != 0 || n16 >= G) return;
  float M = sm.merge.m[0][n16];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.merge.m[w][n16]);
  float wt[kWaves], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm.merge.m[w][n16];
    wt[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    lsum = __builtin_fmaf(wt[w], sm.merge.l[w][n16], lsum);
  }
  const size_t pidx = ((size_t)seq * A.q_heads + kvh * G + n16) * A.max_parts + part;
  float* dst = A.ws_acc + pidx * kHeadDim + 32 * grp;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.merge.acc[w][n16][32 * grp + 4 * v]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(wt[w], y[e], x[e]);
    }
    *reinterpret_cast<f32x4*>(dst + 4 * v) = x;
  }
  if (grp == 0) {
    A.ws_ml[2 * pidx] = M;
    A.ws_ml[2 * pidx + 1] = lsum;
  }
}

// Merge the partitions of one (sequence, query head):
// out = s H (sum_p w_p acc_p) / (sum_p w_p l_p), w_p = 2^(m_p - max m), with
// the Hadamard H applied for pages quantized in the rotated basis (ROT) and
// s = A.out_scale.
template <bool ROT>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs A) {
  __shared__ float wts[1024];
  const int lane = threadIdx.x;
  const int seq = blockIdx.x / A.q_heads;
  const int L = A.seq_lens[seq];
  const int T = A.unit_tokens;
  const int ntiles = min((L + T - 1) / T, A.max_tiles);
  const int nparts = min((ntiles + A.tiles_per_part - 1) / A.tiles_per_part, A.max_parts);
  const size_t base = (size_t)blockIdx.x * A.max_parts;
  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, A.ws_ml[2 * (base + p)]);
  M = wave_max(M);
  float den = 0.f;
  for (int p = lane; p < nparts; p += 64) {
    const float w = __builtin_amdgcn_exp2f(A.ws_ml[2 * (base + p)] - M);
    wts[p] = w;
    den = __builtin_fmaf(w, A.ws_ml[2 * (base + p) + 1], den);
  }
  den = wave_sum(den);
  __syncthreads();
  float x0 = 0.f, x1 = 0.f;
  const float* src = A.ws_acc + base * kHeadDim;
  int p = 0;
  for (; p + 4 <= nparts; p += 4) {
    const float a0 = src[(p + 0) * kHeadDim + lane], b0 = src[(p + 0) * kHeadDim + lane + 64];
    const float a1 = src[(p + 1) * kHeadDim + lane], b1 = src[(p + 1) * kHeadDim + lane + 64];
    const float a2 = src[(p + 2) * kHeadDim + lane], b2 = src[(p + 2) * kHeadDim + lane + 64];
    const float a3 = src[(p + 3) * kHeadDim + lane], b3 = src[(p + 3) * kHeadDim + lane + 64];
    x0 = __builtin_fmaf(wts[p], a0, x0); x1 = __builtin_fmaf(wts[p], b0, x1);
    x0 = __builtin_fmaf(wts[p + 1], a1, x0); x1 = __builtin_fmaf(wts[p + 1], b1, x1);
    x0 = __builtin_fmaf(wts[p + 2], a2, x0); x1 = __builtin_fmaf(wts[p + 2], b2, x1);
    x0 = __builtin_fmaf(wts[p + 3], a3, x0); x1 = __builtin_fmaf(wts[p + 3], b3, x1);
  }
  for (; p < nparts; ++p) {
    x0 = __builtin_fmaf(wts[p], src[p * kHeadDim + lane], x0);
    x1 = __builtin_fmaf(wts[p], src[p * kHeadDim + lane + 64], x1);
  }
  float* o = A.out + (size_t)blockIdx.x * kHeadDim;
  if (!ROT) {
    const float inv = den > 0.f ? A.out_scale / den : 0.f;   // an empty sequence gives zeros
    o[lane] = x0 * inv;
    o[lane + 64] = x1 * inv;
    return;
  }
  const float inv = den > 0.f ? A.out_scale * kInvSqrtD / den : 0.f;
  // channels lane (bit 6 = 0) and lane + 64 (bit 6 = 1)
  float y0 = x0 + x1, y1 = x0 - x1;
  auto stage = [&](float& v, float partner, int bit) {
    v = __builtin_fmaf(v, (lane & bit) ? -1.f : 1.f, partner);
  };
  stage(y0, lane_xor<1>(y0), 1);   stage(y1, lane_xor<1>(y1), 1);
  stage(y0, lane_xor<2>(y0), 2);   stage(y1, lane_xor<2>(y1), 2);
  stage(y0, lane_xor<4>(y0), 4);   stage(y1, lane_xor<4>(y1), 4);
  stage(y0, lane_xor<8>(y0), 8);   stage(y1, lane_xor<8>(y1), 8);
  stage(y0, lane_xor<16>(y0), 16); stage(y1, lane_xor<16>(y1), 16);
  stage(y0, xor32(y0), 32);        stage(y1, xor32(y1), 32);
  o[lane] = y0 * inv;
  o[lane + 64] = y1 * inv;
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
template <typename F>
hipError_t by_bits(int bits, F&& f) {
  switch (bits) {
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, int unit_tokens, bool rotate, hipStream_t s) {
  DecodeArgs b = a;
  b.unit_tokens = unit_tokens;
  if (rotate) hipLaunchKernelGGL(combine_kernel<true>, dim3(a.num_seqs * a.q_heads), dim3(64), 0, s, b);
  else hipLaunchKernelGGL(combine_kernel<false>, dim3(a.num_seqs * a.q_heads), dim3(64), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_bits(bits_k, [&](auto BK) {
      return by_bits(bits_v, [&](auto BV) {
        dim3 grid(a.max_parts, a.kv_heads, a.num_seqs);
        if (a.group <= 4) hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 1>), grid, dim3(64 * kWaves), 0, s, a);
        else if (a.group <= 8) hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 2>), grid, dim3(64 * kWaves), 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 4>), grid, dim3(64 * kWaves), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_combine(a, T(), true, s);
      });
    });
  });
}

}  // namespace kvq
