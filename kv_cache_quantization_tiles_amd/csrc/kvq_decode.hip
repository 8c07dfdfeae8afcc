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
// Work split: one wave per (sequence, kv head, partition of tiles).  The
// group of G query heads sharing the kv head is padded to 16 and both
// contractions run on v_mfma_f32_16x16x32_f16:
//   QK:  S^T[t][g] = sum_c K[t][c] W[c][g]: A = 16 tokens of codes (each code
//        k as the exact fp16 1 + k/64), B = qt split into fp16 hi + lo.
//   PV:  O^T[c][g] = sum_t V[t][c] P[t][g]: A = codes of 2 pages (32 tokens),
//        B = p_t S_t split into fp16 hi + lo.
// The QK output layout (lane = query head, 4 tokens per lane) is exactly the
// B layout PV needs, so no shuffle sits between the two.  Codes unpack with
// two integer ops per pair of codes (shift, and-or) and no conversion.
// Online softmax runs per tile; partitions are merged by a second kernel that
// also applies the final Hadamard.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr unsigned kOne = 0x3C003C00u;  // fp16 1.0 in both halves

// Pair of codes from nibble/field position x of both 16-bit halves, moved to
// mantissa bits 4.. so that the fp16 value is 1 + code/64.  The mask and the
// fp16 one are passed in VGPRs so that one v_and_or_b32 does the masking.
template <int BITS, int X>
__device__ __forceinline__ unsigned code_pair(unsigned w, unsigned mask, unsigned one) {
  constexpr int shift = 4 - BITS * X;  // > 0: left, < 0: right
  const unsigned s = (shift >= 0) ? (w << (shift >= 0 ? shift : 0)) : (w >> (shift < 0 ? -shift : 0));
  unsigned r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(s), "v"(mask), "v"(one));
  return r;
}

__device__ __forceinline__ f16x8 as_f16x8(unsigned a, unsigned b, unsigned c, unsigned d) {
  u32x4 v{a, b, c, d};
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (unsigned)__builtin_bit_cast(uint16_t, a) | ((unsigned)__builtin_bit_cast(uint16_t, b) << 16);
}

// hi/lo fp16 split of two fp32 values, returned as (hi pair, lo pair).
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
  const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
  const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
  hi = (unsigned)__builtin_bit_cast(uint16_t, h0) | ((unsigned)__builtin_bit_cast(uint16_t, h1) << 16);
  lo = (unsigned)__builtin_bit_cast(uint16_t, l0) | ((unsigned)__builtin_bit_cast(uint16_t, l1) << 16);
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

// Channel of A-operand slot (chunk ch, lane group grp, slot j) for K codes.
template <int BITS>
__device__ __forceinline__ int k_channel(int ch, int grp, int j) {
  const int m = j >> 1, hi = j & 1;
  if (BITS == 4) return 32 * grp + 8 * ch + m + 4 * hi;
  return 32 * grp + 16 * (ch >> 1) + 4 * (ch & 1) + m + 8 * hi;
}

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

template <int T>
struct alignas(16) DecodeSmem {
  int32_t pages[kMaxTilesPerPart * (T / kPage)];  // the partition's page ids
  union {
    struct {
      float hq[16][kHeadDim];                                  // H q of the group, orthonormal
      uint8_t meta[kWaves][2][TileMeta<T>::BYTES];             // per-wave double buffer
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

// One workgroup of 4 waves per (partition of tiles, kv head, sequence); wave
// w takes tiles begin + w, begin + w + 4, ...  Each wave prefetches its next
// tile's codes (registers) and metadata (registers, then LDS) while it works
// on the current one; the 4 waves' softmax states are merged in LDS at the end.
template <int T, int BK, int BV>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs A) {
  using TM = TileMeta<T>;
  constexpr int NP = TM::NP;
  constexpr int META = TM::META;
  constexpr int SLOT_K = slot_bytes(BK, T), SLOT_V = slot_bytes(BV, T);
  constexpr int CODE_K = slot_code_bytes(BK), CODE_V = slot_code_bytes(BV);
  constexpr int AL = slot_alpha_len(T);
  __shared__ DecodeSmem<T> sm;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  // code-unpack constants, kept in VGPRs (see code_pair)
  unsigned m4 = 0x00F000F0u, m2 = 0x00300030u, one = kOne;
  asm volatile("" : "+v"(m4), "+v"(m2), "+v"(one));
  const int n16 = lane & 15, grp = lane >> 4;
  const int part = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int G = A.group;
  const int L = A.seq_lens[seq];
  const int ntiles = min((L + T - 1) / T, A.max_tiles);
  const int tile_begin = part * A.tiles_per_part;
  const int tile_end = min(ntiles, tile_begin + A.tiles_per_part);
  if (tile_begin >= tile_end) return;  // uniform over the workgroup
  const int H = A.kv_heads;
  const bool real = n16 < G;
  // the partition's page ids, staged once in LDS (a scalar load per tile would
  // make every later LDS wait also wait for global memory)
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
      const size_t pg = (size_t)tp[p] * H + kvh;
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
  if (wave == 0) {
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
    for (int i = 0; i < 32; ++i) hq[i] = __builtin_fmaf(hq[i], s32, xor32(hq[i])) * kInvSqrtD;
#pragma unroll
    for (int v = 0; v < 8; ++v)
      *reinterpret_cast<f32x4*>(&sm.loop.hq[n16][32 * grp + 4 * v]) =
          f32x4{hq[4 * v], hq[4 * v + 1], hq[4 * v + 2], hq[4 * v + 3]};
  }
  __syncthreads();

  const float c0 = A.sm_scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  float acc[8][4];  // [block i][r]: channel 32 grp + 8 r + i, query head g = n16
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

    // -------------------------------------------- query fold: qt = (H q) * alpha_K
    float qt[32];
    float qsum = 0.f, qmax = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int c = 32 * grp + 4 * v;
      const f32x4 h4 = *reinterpret_cast<const f32x4*>(&sm.loop.hq[n16][c]);
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(mK + (c / AL) * META + 8 * kPage + 4 * (c % AL));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qt[4 * v + e] = h4[e] * a4[e];
        qsum += qt[4 * v + e];
        qmax = fmaxf(qmax, fabsf(qt[4 * v + e]));
      }
    }
    qsum = group_sum(qsum);
    qmax = group_max(qmax);
    // a power-of-two scale per query head keeps the fp16 split of qt in range
    int ex = (int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127;
    ex = min(max(ex, -100), 100);
    const float qscale = __uint_as_float((unsigned)(127 + 14 - ex) << 23);    // 2^(14-ex)
    const float qunscale = __uint_as_float((unsigned)(127 - 14 + ex) << 23);  // 2^(ex-14)
    f16x8 bq_hi[4], bq_lo[4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      unsigned hi[4], lo[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i0 = k_channel<BK>(ch, 0, 2 * m), i1 = k_channel<BK>(ch, 0, 2 * m + 1);
        split_pair(qt[i0] * qscale, qt[i1] * qscale, hi[m], lo[m]);
      }
      bq_hi[ch] = as_f16x8(hi[0], hi[1], hi[2], hi[3]);
      bq_lo[ch] = as_f16x8(lo[0], lo[1], lo[2], lo[3]);
    }
    const float sA = c0 * 64.f * qunscale;   // score = sA S (D) + c0 qsum (O - 64 S)
    const float sB = c0 * qsum;

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
          const unsigned x = kc[p][ch];
          a = as_f16x8(code_pair<4, 0>(x, m4, one), code_pair<4, 1>(x, m4, one), code_pair<4, 2>(x, m4, one),
                       code_pair<4, 3>(x, m4, one));
        } else {
          const unsigned x = kc[p][ch >> 1];
          if (ch & 1)
            a = as_f16x8(code_pair<2, 4>(x, m2, one), code_pair<2, 5>(x, m2, one), code_pair<2, 6>(x, m2, one),
                         code_pair<2, 7>(x, m2, one));
          else
            a = as_f16x8(code_pair<2, 0>(x, m2, one), code_pair<2, 1>(x, m2, one), code_pair<2, 2>(x, m2, one),
                         code_pair<2, 3>(x, m2, one));
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
      for (int r = 0; r < 4; ++r) s[p][r] = __builtin_fmaf(sA * S[r], d[p][r], sB * __builtin_fmaf(-64.f, S[r], O[r]));
    }
    if (tile == ntiles - 1 && (L % T) != 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile * T + p * kPage + 4 * grp + r >= L) s[p][r] = -INFINITY;
    }

    // -------------------------------------------- online softmax (base 2)
    float tmax = s[0][0];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[p][r]);
    tmax = group_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[p][r] = __builtin_amdgcn_exp2f(s[p][r] - m_new);
        psum += s[p][r];
      }
    l_run = __builtin_fmaf(l_run, corr, psum);

    // -------------------------------------------- values of the tile's pages
    float vacc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) vacc[i][r] = 0.f;
    float sp = 0.f, spo = 0.f;
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
          sp += pw[r];
          spo = __builtin_fmaf(s[pp + h2][r], O[r], spo);
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
            const unsigned x = vc[pp + h2][i >> 1];
            if (i & 1) { u[2 * h2] = code_pair<4, 2>(x, m4, one); u[2 * h2 + 1] = code_pair<4, 3>(x, m4, one); }
            else { u[2 * h2] = code_pair<4, 0>(x, m4, one); u[2 * h2 + 1] = code_pair<4, 1>(x, m4, one); }
          } else {
            const unsigned x = vc[pp + h2][i >> 2];
            switch (i & 3) {
              case 0: u[2 * h2] = code_pair<2, 0>(x, m2, one); u[2 * h2 + 1] = code_pair<2, 1>(x, m2, one); break;
              case 1: u[2 * h2] = code_pair<2, 2>(x, m2, one); u[2 * h2 + 1] = code_pair<2, 3>(x, m2, one); break;
              case 2: u[2 * h2] = code_pair<2, 4>(x, m2, one); u[2 * h2 + 1] = code_pair<2, 5>(x, m2, one); break;
              default: u[2 * h2] = code_pair<2, 6>(x, m2, one); u[2 * h2 + 1] = code_pair<2, 7>(x, m2, one); break;
            }
          }
        }
        const f16x8 a = as_f16x8(u[0], u[1], u[2], u[3]);
        f32x4 d{vacc[i][0], vacc[i][1], vacc[i][2], vacc[i][3]};
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ph, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pl, d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) vacc[i][r] = d[r];
      }
    }
    sp = group_sum(sp);
    spo = group_sum(spo);

    // -------------------------------------------- fold: acc = acc corr + alpha_V (64 (D - sp) + spo)
    const float kv = __builtin_fmaf(-64.f, sp, spo);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 32 * grp + 8 * r;
      const uint8_t* ap = mV + (c / AL) * META + 8 * kPage + 4 * (c % AL);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(ap);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(ap + 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float al = (i < 4) ? a0[i] : a1[i - 4];
        const float val = al * __builtin_fmaf(64.f, vacc[i][r], kv);
        acc[i][r] = __builtin_fmaf(acc[i][r], corr, val);
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
  if (wave != 0 || !real) return;
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
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV()>), grid, dim3(64 * kWaves), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_combine(a, T(), true, s);
      });
    });
  });
}

}  // namespace kvq
