// Tile quantizer kernels for gfx950: Hadamard rotation along channels, then
// Sinkhorn-like alternating channel/token variance normalization, then
// per-token asymmetric round-to-nearest to packed 2- or 4-bit codes.
//
// Method: page "Huawei's KVarN boosts vLLM KV-cache capacity by 5x without
// accuracy loss" (axbrief.com), section "기존 방식과 달라진 지점" (the
// four-step tile quantizer); restore: page "화웨이가 공개한 KVarN" (ttj.kr),
// section "양자화로 캐시를 다이어트시킨다".
//
// One workgroup quantizes one tile of T tokens x 128 channels with 2T
// threads.  Thread (tq, cg) holds the 4 tokens 4tq..4tq+3 and the 16
// channels 8cg+j and 64+8cg+j (j < 8) in registers for the whole kernel:
//   * the fp16 rows are read once (two 16-byte loads per token, the 8 cg
//     threads of a token covering its 256-byte row);
//   * the Hadamard butterfly runs 4 stages in registers (channel bits 0,1,2,6)
//     and 3 stages across the 8 cg lanes with ds_swizzle (channel bits 3,4,5);
//     it is left unnormalized and the 1/sqrt(128) is folded into the factors;
//   * the normalization never rewrites the tile: with weights b = 1/beta and
//     a = 1/alpha, the channel step needs the spread over t of u = b_t R_tc
//     and the token step that over c of u = a_c R_tc.  Each is one pass of
//     d = u - ref (ref: the first token's, resp. channel 0's, value of u),
//     sum d and sum d^2 (three VALU ops per element); the shift keeps
//     E[d^2] - E[d]^2 accurate when a mean dwarfs the spread.  Partial sums
//     go through LDS and one thread per channel (token) finalizes the
//     variance, the guard and the reciprocal std;
//   * the last token step is skipped: its factor cancels exactly in the
//     stored scale, offset and codes (rounding is per token row);
//   * codes: z = R * a, per-row min/max through LDS, v = (z - min) / step,
//     round half to even, packed and stored straight into the output layout.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace {

enum Mode { kDense = 0, kPaged = 1, kAppend = 2 };

typedef unsigned int qt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int qt_u32x2 __attribute__((ext_vector_type(2)));
typedef float qt_f32x4 __attribute__((ext_vector_type(4)));

// fp16 pair (low, high half of w) -> fp32 (low + high, low - high): the
// conversion rides on the first butterfly stage, one v_fma_mix_f32 each (the
// mixed-precision FMA reads the two fp16 halves directly; low * 1 + high is
// rounded once, as the fp32 sum of the converted values would be).
__device__ __forceinline__ void first_stage(unsigned w, float& y0, float& y1) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(y0) : "v"(w));
  asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(y1) : "v"(w));
}

// Shared memory of one workgroup.
template <int T>
struct alignas(16) Smem {
  float red[2][T / 4][kHeadDim];  // channel partials; token partials and row min/max alias it
  float a[kHeadDim];              // 1/alpha in unnormalized units
  float alpha[kHeadDim];          // channel factors (normalized units)
  float ref_c[kHeadDim];          // R of the tile's first token (channel-step shift)
  float b[T];                     // 1/beta
  float ref_t[T];                 // R of channel 0 of each token (token-step shift)
  float inv[T];                   // levels / range per row (0 for empty rows)
  float nmi[T];                   // -min * inv per row
};

// Packs N codes into one 32-bit word: field f (bits [BITS*f, BITS*(f+1)))
// takes v[f] rounded to nearest even by v_cvt_pk_u8_f32.
template <int BITS, int N>
__device__ __forceinline__ unsigned pack_fields(const float (&v)[N]) {
  constexpr int PER = 8 / BITS;  // fields per byte
  unsigned acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0u;
#pragma unroll
  for (int f = 0; f < N; ++f) acc[f % PER] = __builtin_amdgcn_cvt_pk_u8_f32(v[f], f / PER, acc[f % PER]);
  unsigned w = acc[0];
#pragma unroll
  for (int p = 1; p < PER; ++p) w |= acc[p] << (BITS * p);
  return w;
}

template <int T, int BITS, bool VLAYOUT, int MODE>
__device__ __forceinline__ void quantize_tile_body(const QuantArgs& A, Smem<T>& sm, int role,
                                                   int head, int seq, int tile_idx, int tid) {
  constexpr int NT = 2 * T;
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const int cg = tid & 7;
  const int tq = tid >> 3;

  // ---------------------------------------------------------------- rows of this tile
  const int t0 = tile_idx * T;
  int n_valid;
  const uint16_t* rows_base = nullptr;  // row t at rows_base + t * row_stride
  int r_new = -1;                       // append: the row taken from the new token
  const int H = (MODE == kDense) ? A.heads : A.kv_heads;
  const size_t row_stride = (size_t)H * kHeadDim;
  if (MODE == kDense) {
    n_valid = min(T, A.n_tokens - t0);
    rows_base = A.x + ((size_t)t0 * H + head) * kHeadDim;
  } else if (MODE == kPaged) {
    const int a0 = A.cu_seqlens[seq];
    n_valid = min(T, A.cu_seqlens[seq + 1] - a0 - t0);
    rows_base = A.src[role] + ((size_t)(a0 + t0) * H + head) * kHeadDim;
  } else {
    r_new = A.lens_before[seq] % T;
    n_valid = r_new + 1;
    rows_base = A.staging[role] + ((size_t)seq * T * H + head) * kHeadDim;
  }

  // ---------------------------------------------------------------- load fp16 rows
  // Rows past the tile's end load row 0 again: their values are then exact
  // copies of row 0, which the statistics below exclude exactly.
  qt_u32x4 raw[4][2];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * tq + r;
    const int src_t = (t < n_valid) ? t : 0;
    const uint16_t* row = rows_base + (size_t)src_t * row_stride;
    if (MODE == kAppend && src_t == r_new) row = A.src[role] + ((size_t)seq * H + head) * kHeadDim;
    raw[r][0] = __builtin_nontemporal_load(reinterpret_cast<const qt_u32x4*>(row + 8 * cg));
    raw[r][1] = __builtin_nontemporal_load(reinterpret_cast<const qt_u32x4*>(row + 64 + 8 * cg));
  }
  // Keep the fp16 rows of a partial tile for later appends.
  if (MODE != kDense && A.staging[role] != nullptr) {
    uint16_t* stg = A.staging[role] + ((size_t)seq * T * H + head) * kHeadDim;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      const bool write = (MODE == kPaged) ? (n_valid < T && t < n_valid) : (t == r_new);
      if (write) {
        *reinterpret_cast<qt_u32x4*>(stg + (size_t)t * row_stride + 8 * cg) = raw[r][0];
        *reinterpret_cast<qt_u32x4*>(stg + (size_t)t * row_stride + 64 + 8 * cg) = raw[r][1];
      }
    }
  }

  // ---------------------------------------------------------------- Hadamard (unnormalized)
  // register index k = 8*half + j  <->  channel 64*half + 8*cg + j
  float R[4][16];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 4; ++i) first_stage(raw[r][half][i], R[r][8 * half + 2 * i], R[r][8 * half + 2 * i + 1]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int bit = 2; bit < 16; bit <<= 1) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k & bit) continue;
        const float lo = R[r][k], hi = R[r][k | bit];
        R[r][k] = lo + hi;
        R[r][k | bit] = lo - hi;
      }
    }
  }
  {
    const float s1 = (cg & 1) ? -1.f : 1.f;
    const float s2 = (cg & 2) ? -1.f : 1.f;
    const float s4 = (cg & 4) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 16; ++k) R[r][k] = __builtin_fmaf(R[r][k], s1, lane_xor<1>(R[r][k]));
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 16; ++k) R[r][k] = __builtin_fmaf(R[r][k], s2, lane_xor<2>(R[r][k]));
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 16; ++k) R[r][k] = __builtin_fmaf(R[r][k], s4, lane_xor<4>(R[r][k]));
  }

  // ---------------------------------------------------------------- normalization
  // Spread sums are taken over values shifted by a reference (channel step:
  // the tile's first token; token step: the token's channel 0), so that
  // E[d^2] - E[d]^2 does not cancel when a mean dwarfs the spread.
  if (tq == 0) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      *reinterpret_cast<qt_f32x4*>(&sm.ref_c[64 * half + 8 * cg]) =
          qt_f32x4{R[0][8 * half], R[0][8 * half + 1], R[0][8 * half + 2], R[0][8 * half + 3]};
      *reinterpret_cast<qt_f32x4*>(&sm.ref_c[64 * half + 8 * cg + 4]) =
          qt_f32x4{R[0][8 * half + 4], R[0][8 * half + 5], R[0][8 * half + 6], R[0][8 * half + 7]};
    }
  }
  if (cg == 0)
    *reinterpret_cast<qt_f32x4*>(&sm.ref_t[4 * tq]) = qt_f32x4{R[0][0], R[1][0], R[2][0], R[3][0]};
  for (int c = tid; c < kHeadDim; c += NT) {
    sm.a[c] = kInvSqrtD;
    sm.alpha[c] = 1.0f;
  }
  if (tid < T) sm.b[tid] = 1.0f;
  __syncthreads();
  float a[16], b[4], refc[16], reft[4];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const qt_f32x4 lo = *reinterpret_cast<const qt_f32x4*>(&sm.ref_c[64 * half + 8 * cg]);
    const qt_f32x4 hi = *reinterpret_cast<const qt_f32x4*>(&sm.ref_c[64 * half + 8 * cg + 4]);
#pragma unroll
    for (int i = 0; i < 4; ++i) { refc[8 * half + i] = lo[i]; refc[8 * half + 4 + i] = hi[i]; }
  }
  {
    const qt_f32x4 rt = *reinterpret_cast<const qt_f32x4*>(&sm.ref_t[4 * tq]);
#pragma unroll
    for (int r = 0; r < 4; ++r) reft[r] = rt[r];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = kInvSqrtD;
#pragma unroll
  for (int r = 0; r < 4; ++r) b[r] = 1.0f;
  const float inv_n = 1.0f / (float)n_valid;
  const float n_copies = (float)(T - n_valid);  // rows that are copies of row 0
  const int iters = A.iters;
  float b0 = 1.0f;

  for (int it = 0; it < iters; ++it) {
    // channel step: spread over the tile's valid tokens of u = b_t R_tc
    {
      float s1[16], s2[16], kc[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) kc[k] = b0 * refc[k];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float d = __builtin_fmaf(b[0], R[0][k], -kc[k]);
        s1[k] = d;
        s2[k] = d * d;
      }
#pragma unroll
      for (int r = 1; r < 4; ++r) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float d = __builtin_fmaf(b[r], R[r][k], -kc[k]);
          s1[k] += d;
          s2[k] = __builtin_fmaf(d, d, s2[k]);
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c0 = 64 * half + 8 * cg;
        *reinterpret_cast<qt_f32x4*>(&sm.red[0][tq][c0]) =
            qt_f32x4{s1[8 * half], s1[8 * half + 1], s1[8 * half + 2], s1[8 * half + 3]};
        *reinterpret_cast<qt_f32x4*>(&sm.red[0][tq][c0 + 4]) =
            qt_f32x4{s1[8 * half + 4], s1[8 * half + 5], s1[8 * half + 6], s1[8 * half + 7]};
        *reinterpret_cast<qt_f32x4*>(&sm.red[1][tq][c0]) =
            qt_f32x4{s2[8 * half], s2[8 * half + 1], s2[8 * half + 2], s2[8 * half + 3]};
        *reinterpret_cast<qt_f32x4*>(&sm.red[1][tq][c0 + 4]) =
            qt_f32x4{s2[8 * half + 4], s2[8 * half + 5], s2[8 * half + 6], s2[8 * half + 7]};
      }
    }
    __syncthreads();
    for (int c = tid; c < kHeadDim; c += NT) {
      float S1 = 0.f, S2 = 0.f;
#pragma unroll
      for (int g = 0; g < T / 4; ++g) {
        S1 += sm.red[0][g][c];
        S2 += sm.red[1][g][c];
      }
      // copies of row 0 each added row 0's own shifted value rho (the fma
      // residual of the shift); take them out
      const float rc = sm.ref_c[c];
      const float kcc = b0 * rc;
      const float rho = __builtin_fmaf(b0, rc, -kcc);
      S1 = __builtin_fmaf(-n_copies, rho, S1);
      S2 = __builtin_fmaf(-n_copies, rho * rho, S2);
      const float m = S1 * inv_n;                                   // mean of the shifted values
      const float var = fmaxf(__builtin_fmaf(-m, m, S2 * inv_n), 0.f);
      const float mu = m + kcc;                                     // mean of u
      const float ms = __builtin_fmaf(mu, mu, var);                 // mean square of u
      if (var > kGuard2 * ms) {
        sm.a[c] = __builtin_amdgcn_rsqf(var);
        sm.alpha[c] = __builtin_sqrtf(var * (1.0f / kHeadDim));
      }
    }
    __syncthreads();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const qt_f32x4 lo = *reinterpret_cast<const qt_f32x4*>(&sm.a[64 * half + 8 * cg]);
      const qt_f32x4 hi = *reinterpret_cast<const qt_f32x4*>(&sm.a[64 * half + 8 * cg + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[8 * half + i] = lo[i]; a[8 * half + 4 + i] = hi[i]; }
    }
    if (it + 1 == iters) break;  // the final token step cancels in every stored value

    // token step: spread over the 128 channels of u = a_c R_tc
    const float a0 = sm.a[0];
    {
      float t1[4], t2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float kt = a0 * reft[r];
        float x1, x2;
        {
          const float d = __builtin_fmaf(a[0], R[r][0], -kt);
          x1 = d;
          x2 = d * d;
        }
#pragma unroll
        for (int k = 1; k < 16; ++k) {
          const float d = __builtin_fmaf(a[k], R[r][k], -kt);
          x1 += d;
          x2 = __builtin_fmaf(d, d, x2);
        }
        t1[r] = x1;
        t2[r] = x2;
      }
      float* tr = &sm.red[0][0][0];  // [2][8][T] view
      *reinterpret_cast<qt_f32x4*>(&tr[(0 * 8 + cg) * T + 4 * tq]) = qt_f32x4{t1[0], t1[1], t1[2], t1[3]};
      *reinterpret_cast<qt_f32x4*>(&tr[(1 * 8 + cg) * T + 4 * tq]) = qt_f32x4{t2[0], t2[1], t2[2], t2[3]};
    }
    __syncthreads();
    if (tid < T) {
      const float* tr = &sm.red[0][0][0];
      float T1 = 0.f, T2 = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        T1 += tr[(0 * 8 + g) * T + tid];
        T2 += tr[(1 * 8 + g) * T + tid];
      }
      const float m = T1 * (1.0f / kHeadDim);
      const float var = fmaxf(__builtin_fmaf(-m, m, T2 * (1.0f / kHeadDim)), 0.f);
      const float mu = __builtin_fmaf(a0, sm.ref_t[tid], m);
      const float ms = __builtin_fmaf(mu, mu, var);
      if (var > kGuard2 * ms) sm.b[tid] = __builtin_amdgcn_rsqf(var);
    }
    __syncthreads();
    {
      b0 = sm.b[0];
      const qt_f32x4 bb = *reinterpret_cast<const qt_f32x4*>(&sm.b[4 * tq]);
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = (4 * tq + r < n_valid) ? bb[r] : b0;  // copies weigh as row 0
    }
  }

  // ---------------------------------------------------------------- rounding
  float zmin[4], zmax[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int k = 0; k < 16; ++k) R[r][k] *= a[k];
    float mn = fminf(R[r][0], R[r][1]), mx = fmaxf(R[r][0], R[r][1]);
#pragma unroll
    for (int k = 2; k < 16; k += 2) {
      mn = fminf(mn, fminf(R[r][k], R[r][k + 1]));
      mx = fmaxf(mx, fmaxf(R[r][k], R[r][k + 1]));
    }
    zmin[r] = mn;
    zmax[r] = mx;
  }
  {
    float* tr = &sm.red[0][0][0];
    *reinterpret_cast<qt_f32x4*>(&tr[(0 * 8 + cg) * T + 4 * tq]) = qt_f32x4{zmin[0], zmin[1], zmin[2], zmin[3]};
    *reinterpret_cast<qt_f32x4*>(&tr[(1 * 8 + cg) * T + 4 * tq]) = qt_f32x4{zmax[0], zmax[1], zmax[2], zmax[3]};
  }
  __syncthreads();

  // Output addressing (paged): the tile's pages.
  uint8_t* pool = nullptr;
  const int32_t* pages = nullptr;
  constexpr int SLOT = slot_bytes(BITS, T);
  constexpr int CODE_BYTES = slot_code_bytes(BITS);
  if (MODE != kDense) {
    pool = A.pool[role];
    pages = A.block_table + (size_t)seq * A.max_blocks + (t0 / kPage);
  }
  auto slot_ptr = [&](int page_in_tile) -> uint8_t* {
    return pool + ((size_t)pages[page_in_tile] * H + head) * SLOT;
  };

  if (tid < T) {
    const float* tr = &sm.red[0][0][0];
    float mn = tr[(0 * 8) * T + tid], mx = tr[(1 * 8) * T + tid];
#pragma unroll
    for (int g = 1; g < 8; ++g) {
      mn = fminf(mn, tr[(0 * 8 + g) * T + tid]);
      mx = fmaxf(mx, tr[(1 * 8 + g) * T + tid]);
    }
    float step = 0.f, off = 0.f, inv = 0.f, nmi = 0.f;
    if (tid < n_valid) {
      const float range = mx - mn;
      step = range * (1.0f / LEVELS);
      off = mn;
      if (range > 0.f) {
        inv = LEVELS * __builtin_amdgcn_rcpf(range);
        nmi = -mn * inv;
      }
    }
    sm.inv[tid] = inv;
    sm.nmi[tid] = nmi;
    if (MODE == kDense) {
      if (tid < n_valid) {
        A.scale[(size_t)(t0 + tid) * H + head] = step;
        A.offset[(size_t)(t0 + tid) * H + head] = off;
      }
    } else {
      uint8_t* slot = slot_ptr(tid / kPage);
      reinterpret_cast<float*>(slot + CODE_BYTES)[tid % kPage] = step;
      reinterpret_cast<float*>(slot + CODE_BYTES + 4 * kPage)[tid % kPage] = off;
    }
  }
  for (int c = tid; c < kHeadDim; c += NT) {
    const float al = sm.alpha[c];
    if (MODE == kDense) {
      A.alpha[((size_t)tile_idx * H + head) * kHeadDim + c] = al;
    } else {
      constexpr int AL = slot_alpha_len(T);
      reinterpret_cast<float*>(slot_ptr(c / AL) + CODE_BYTES + 8 * kPage)[c % AL] = al;
    }
  }
  __syncthreads();

  // values before rounding: v = (z - min) * levels / range, in [0, levels]
  {
    const qt_f32x4 iv = *reinterpret_cast<const qt_f32x4*>(&sm.inv[4 * tq]);
    const qt_f32x4 nm = *reinterpret_cast<const qt_f32x4*>(&sm.nmi[4 * tq]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 16; ++k) R[r][k] = __builtin_fmaf(R[r][k], iv[r], nm[r]);
  }

  if (MODE == kDense || !VLAYOUT) {
    // natural packing, 8 channels of one token per 8*BITS bits
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      if (MODE == kDense && t >= n_valid) continue;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = R[r][8 * half + j];
        unsigned w;
        if (BITS == 4) {
          // fields in order 0..7; bytes take fields (0,1), (2,3), ...
          float o[8] = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
          w = pack_fields<4>(o);
        } else {
          w = pack_fields<2>(v);
        }
        if (MODE == kDense) {
          uint8_t* row = A.codes + ((size_t)(t0 + t) * H + head) * (kHeadDim * BITS / 8);
          if (BITS == 4) *reinterpret_cast<uint32_t*>(row + BITS * (8 * half + cg)) = w;
          else *reinterpret_cast<uint16_t*>(row + BITS * (8 * half + cg)) = (uint16_t)w;
        } else {
          // K slot: 4 blocks of 32 channels, token after token
          constexpr int CB = 4 * BITS;  // bytes per token per block
          uint8_t* dst = slot_ptr((4 * tq) / kPage) + (2 * half + (cg >> 2)) * (kPage * CB) +
                         ((4 * tq) % kPage + r) * CB + BITS * (cg & 3);
          if (BITS == 4) *reinterpret_cast<uint32_t*>(dst) = w;
          else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
        }
      }
    }
  } else {
    // V slot: run l (4*BITS bytes at 4*BITS*l) holds channels l and 64 + l of
    // the page's 16 tokens; token 4g + r of half h is pair p = 2g + h, in word
    // p / (F/4) of the run, field 2m + (r>>1) + (F/2)(r&1), m = p mod (F/4).
    // This thread holds quad g (its 4 tokens) of the runs 8 cg + j (its
    // channels j and 8 + j), so it builds its pairs' fields of every run.
    constexpr int F = 32 / BITS;
    uint8_t* slot = slot_ptr((4 * tq) / kPage);
    const int g = tq % (kPage / 4);
    unsigned w8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float o[F];
#pragma unroll
      for (int f = 0; f < F; ++f) o[f] = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[2 * h + (r >> 1) + (F / 2) * (r & 1)] = R[r][8 * h + j];
      w8[j] = pack_fields<BITS>(o);   // fields of m = h; m = 2 (g & 1) + h for 2-bit is a shift
    }
    if (BITS == 4) {
      // one word per (run, quad): this thread's alone
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(slot + 16 * (8 * cg + j) + 4 * g) = w8[j];
    } else {
      // one word per (run, quad pair): merge with the thread of quad g ^ 1
      // (lane ^ 8); the even quad's thread writes runs j < 4, the odd one j >= 4
      const bool odd = (g & 1) != 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned mine = (odd ? w8[j + 4] : w8[j]) << (odd ? 8 : 0);
        const unsigned give = (odd ? w8[j] : w8[j + 4]) << (odd ? 8 : 0);
        const unsigned got = (unsigned)__float_as_int(lane_xor<8>(__int_as_float((int)give)));
        *reinterpret_cast<uint32_t*>(slot + 8 * (8 * cg + j + (odd ? 4 : 0)) + 4 * (g >> 1)) = mine | got;
      }
    }
  }
}

}  // namespace
}  // namespace kvq
