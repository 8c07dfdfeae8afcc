// Tile quantizer for gfx950: Hadamard rotation along channels, then
// Sinkhorn-like alternating channel/token variance normalization, then
// per-token asymmetric round-to-nearest to packed 2-, 4- or 8-bit codes.
//
// Method: page "Huawei's KVarN boosts vLLM KV-cache capacity by 5x without
// accuracy loss" (axbrief.com), section "기존 방식과 달라진 지점" (the
// four-step tile quantizer); restore: page "화웨이가 공개한 KVarN" (ttj.kr),
// section "양자화로 캐시를 다이어트시킨다".
//
// One workgroup (or one group of 2T threads inside the fused decode kernel)
// quantizes one tile of T tokens x 128 channels, T/32 waves.  Wave w takes
// tokens 32w..32w+31 as two 16-token blocks; lane l = 16 g + j ends up
// holding, for the whole kernel, the 8 tokens 32w + 16 bb + 4g + r (bb < 2,
// r < 4) of the 8 channels j + 16 m (m < 8), in registers:
//   * rotation on the matrix cores: with channel c = 32p + k (k < 32), one
//     v_mfma_f32_16x16x32_f16 per (block, p, sign) multiplies 16 fp16 rows
//     by [H16; +-H16], which is the Sylvester transform over channel bits
//     0..4 (the fp16 input enters the MFMA as loaded; every product is exact
//     and a single instruction sums 32 of them); the transform over bits 5, 6
//     (the four p) is a 4-point butterfly in registers.  Lane 16g + j then
//     holds rows 4g..4g+3 of output channels j + 16 sigma + 32 p'.  The
//     transform is left unnormalized, the 1/sqrt(128) folded into the factors;
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
//     round half to even; a lane's 8 codes of a token are one unit of the
//     stored unit order (channel u + 16 m in field m of unit u), so K codes
//     and dense codes are stored straight from registers, and V runs (channels
//     l and 64 + l) are built from the lane's own quad of tokens.
// Tiles of fewer than 16 valid tokens take a float64 path instead (the
// partial tiles every append rewrites, and short sequence ends): their
// statistics come from a handful of values, and alternating normalization of
// such a tile can amplify fp32 rounding of the rotated values several
// hundredfold into the stored factors.  In float64 the rotation of fp16
// input is exact (sums of 128 fp16 values need at most 47 bits) and the
// normalization follows the plain definition (two-pass mean and spread,
// factors applied to the data); the first wave does it, 4 lanes per token.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace {

enum Mode { kDense = 0, kPaged = 1, kAppend = 2 };

typedef unsigned int qt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int qt_u32x2 __attribute__((ext_vector_type(2)));
typedef float qt_f32x4 __attribute__((ext_vector_type(4)));

// Shared memory of one workgroup.  Per-channel arrays marked "lane order"
// keep channel j + 16 m at index 8 j + m (a lane's 8 channels side by side).
// Partial sums are laid out so that the 16 lanes of a row group write to
// distinct banks: channel step [row][half h][j][4] (channels j + 16 (4h + m)),
// token step and row min / max [j][token] with rows of T + 4 floats.
template <int T>
constexpr int kRedStride = T + 4;
template <int T>
struct alignas(16) Smem {
  float red[2][16 * kRedStride<T>];   // partial sums (channel step: [s][row 4w+g][h][j][4];
                                      // token step and row min / max: [s][j][token])
  float a[kHeadDim];      // 1/alpha in unnormalized units (lane order)
  float alpha[kHeadDim];  // channel factors, normalized units (natural order)
  float ref_c[kHeadDim];  // R of the tile's first token (lane order)
  float b[T];             // 1/beta
  float ref_t[T];         // R of channel 0 of each token (token-step shift)
  float inv[T];           // levels / range per row (0 for empty rows)
  float nmi[T];           // -min * inv per row
};

// Buffers of the float64 path for tiles of fewer than 16 tokens.  Only the
// kernels that run that path hold them (overlaid on the fp32 buffers, which
// a short tile never uses); the bulk prefill kernels keep their small
// footprint.
constexpr int kShortTile = 16;
struct alignas(16) ShortSmem {
  double col[kShortTile][kHeadDim + 2];   // the tile [token][channel]
  double inv_g[kHeadDim];                 // 1 / (factor of the current channel step); KCH: levels / range
  double alpha[kHeadDim];                 // channel factors
  double zmin[kHeadDim];                  // KCH: each channel's minimum over the tile
};
template <int T>
union TileSmem {
  Smem<T> f;
  ShortSmem s;
};

typedef _Float16 qt_f16x8 __attribute__((ext_vector_type(8)));

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

// min / max of three floats as one v_min3_f32 / v_max3_f32 (fminf / fmaxf
// add canonicalizing ops around values that may be signaling NaNs; the tile's
// values are finite)
__device__ __forceinline__ float vmin3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// A double's value in lane l ^ 1 (QX1) or l ^ 2 (QX2): DPP quad permutations
// of its two halves (VALU, no LDS round trip).
constexpr int kQuadX1 = 0xB1, kQuadX2 = 0x4E;
template <int CTRL>
__device__ __forceinline__ double quad_dpp(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, 0xF, 0xF, true);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// The float64 path for a tile of n < 16 valid tokens.  Lanes (t, k) =
// (tid >> 2, tid & 3) of the group's first wave hold token t, channels
// 32k + i (i < 32), in registers; per-channel statistics go through the
// tile's copy in LDS, one thread per channel.  Writes the tile's scales,
// offsets and channel factors, and leaves in R the integer codes of the
// lane's rows in the fp32 path's layout (zeros past the tile's end), ready
// for the code store.
template <int T, int BITS, int MODE, bool M16, bool KCH = false, bool PADK = false>
__device__ __forceinline__ void short_tile(const QuantArgs& A, ShortSmem& sh, int role, int head, int seq,
                                           int t0, int n, const uint16_t* rows_base, size_t row_stride,
                                           int r_new, int tid, float (&R)[8][8], uint8_t* pool,
                                           const int32_t* pages) {
  constexpr double LEVELS = (double)((1 << BITS) - 1);
  constexpr int NT = 2 * T;
  constexpr int CODE_BYTES = slot_code_bytes(BITS);
  constexpr int AL = slot_alpha_len(T);
  constexpr int SLOT = slot_bytes(BITS, T, M16, KCH);
  constexpr int OFF_AT = slot_offset_at(BITS, M16), ALPHA_AT = slot_alpha_at(BITS, M16);
  constexpr double kInvSqrtD64 = 0.088388347648318440550;   // 1/sqrt(128)
  const int H = (MODE == kDense) ? A.heads : A.kv_heads;
  const bool act = tid < 64;
  const int t = tid >> 2, k = tid & 3;
  const double dn = (double)n;
  auto page_slot = [&](int p) -> uint8_t* { return pool + ((size_t)pages[p] * H + head) * SLOT; };

  double y[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = 0.0;
  if (act && t < n) {
    const uint16_t* row = rows_base + (size_t)t * row_stride;
    if (MODE == kAppend && t == r_new) row = A.src[role] + ((size_t)seq * H + head) * kHeadDim;
    const unsigned sg = A.signs[k];   // randomized rotation: bit i = channel 32k + i negated
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const qt_u32x4 w = *reinterpret_cast<const qt_u32x4*>(row + 32 * k + 8 * v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * v + e;
        const double x = (double)half_bits_to_float((uint16_t)(w[e >> 1] >> (16 * (e & 1))));
        y[i] = ((sg >> i) & 1u) ? -x : x;
      }
    }
  }
  for (int c = tid; c < kHeadDim; c += NT) sh.alpha[c] = 1.0;
  // Hadamard: channel bits 0..4 in registers, bits 5, 6 across the token's 4
  // lanes (exact in float64), then the orthonormal scale
#pragma unroll
  for (int bit = 1; bit < 32; bit <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & bit) continue;
      const double lo = y[i], hi = y[i | bit];
      y[i] = lo + hi;
      y[i | bit] = lo - hi;
    }
  {
    const bool up1 = (k & 1) != 0, up2 = (k & 2) != 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double o = quad_dpp<kQuadX1>(y[i]);
      y[i] = up1 ? o - y[i] : y[i] + o;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double o = quad_dpp<kQuadX2>(y[i]);
      y[i] = (up2 ? o - y[i] : y[i] + o) * kInvSqrtD64;
    }
  }

  double beta = 1.0;
  const int iters = A.iters;
  for (int it = 0; it < iters; ++it) {
    // channel step: mean, spread and RMS of each channel over the n tokens
    if (act) {
#pragma unroll
      for (int i = 0; i < 32; i += 2)
        *reinterpret_cast<double2*>(&sh.col[t][32 * k + i]) = double2{y[i], y[i + 1]};
    }
    __syncthreads();
    for (int c = tid; c < kHeadDim; c += NT) {
      double s1 = 0.0, s2 = 0.0;
      for (int r = 0; r < n; ++r) {
        const double v = sh.col[r][c];
        s1 += v;
        s2 = __builtin_fma(v, v, s2);
      }
      const double mean = s1 / dn;
      double c2 = 0.0;
      for (int r = 0; r < n; ++r) {
        const double d = sh.col[r][c] - mean;
        c2 = __builtin_fma(d, d, c2);
      }
      const double sd = __builtin_sqrt(c2 / dn), rms = __builtin_sqrt(s2 / dn);
      const double g = (sd > kGuard * rms) ? sd : 1.0;
      sh.inv_g[c] = 1.0 / g;
      sh.alpha[c] *= g;
    }
    __syncthreads();
    if (act) {
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        const double2 ig = *reinterpret_cast<const double2*>(&sh.inv_g[32 * k + i]);
        y[i] *= ig.x;
        y[i + 1] *= ig.y;
      }
    }
    // the final token step cancels in every stored value of a row-rounded
    // tile; per-channel rounding needs it
    if (it + 1 == iters && !KCH) break;
    // token step: mean, spread and RMS of each token over its 128 channels
    if (act) {
      double s1 = 0.0, s2 = 0.0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        s1 += y[i];
        s2 = __builtin_fma(y[i], y[i], s2);
      }
      s1 += quad_dpp<kQuadX1>(s1);
      s2 += quad_dpp<kQuadX1>(s2);
      s1 += quad_dpp<kQuadX2>(s1);
      s2 += quad_dpp<kQuadX2>(s2);
      const double mean = s1 * (1.0 / kHeadDim);
      double c2 = 0.0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const double d = y[i] - mean;
        c2 = __builtin_fma(d, d, c2);
      }
      c2 += quad_dpp<kQuadX1>(c2);
      c2 += quad_dpp<kQuadX2>(c2);
      const double sd = __builtin_sqrt(c2 * (1.0 / kHeadDim)), rms = __builtin_sqrt(s2 * (1.0 / kHeadDim));
      const double g = (sd > kGuard * rms) ? sd : 1.0;
      const double ig = 1.0 / g;
      beta *= g;
#pragma unroll
      for (int i = 0; i < 32; ++i) y[i] *= ig;
    }
  }

  if constexpr (KCH) {
    // rounding per channel over the n tokens: zero-point = min, step =
    // range / levels, ties to even; the slot keeps beta per token, A = alpha
    // step and M = min / step per channel (a zero-range channel: A = alpha min,
    // M = 1, codes 0)
    __syncthreads();   // every thread is done with the channel step's col reads
    if (act && t < n) {
#pragma unroll
      for (int i = 0; i < 32; i += 2)
        *reinterpret_cast<double2*>(&sh.col[t][32 * k + i]) = double2{y[i], y[i + 1]};
    }
    __syncthreads();
    for (int c = tid; c < kHeadDim; c += NT) {
      double lo = sh.col[0][c], hi = lo;
      for (int r = 1; r < n; ++r) {
        lo = fmin(lo, sh.col[r][c]);
        hi = fmax(hi, sh.col[r][c]);
      }
      const double st = (hi - lo) / LEVELS;
      sh.zmin[c] = lo;
      sh.inv_g[c] = st > 0.0 ? 1.0 / st : 0.0;
      const double al = sh.alpha[c];
      uint8_t* slot = page_slot(c / AL);
      store_meta<false>(slot + slot_chan_scale_at(BITS), c % AL, (float)(st > 0.0 ? al * st : al * lo));
      store_meta<false>(slot + slot_chan_zp_at(BITS, T), c % AL, (float)(st > 0.0 ? lo / st : 1.0));
    }
    if (act && k == 0) store_meta<false>(page_slot(0) + CODE_BYTES, t, t < n ? (float)beta : 0.f);
    if (tid >= kShortTile && tid < T) store_meta<false>(page_slot(tid / kPage) + CODE_BYTES, tid % kPage, 0.f);
    __syncthreads();
    unsigned cw[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      unsigned wd = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 32 * k + 4 * v + e;
        const double cd = (act && t < n) ? fmin(fmax(__builtin_rint((y[4 * v + e] - sh.zmin[c]) * sh.inv_g[c]), 0.0), LEVELS) : 0.0;
        wd |= (unsigned)cd << (8 * e);
      }
      cw[v] = wd;
    }
    __syncthreads();   // every thread is done reading col
    uint8_t* code8 = reinterpret_cast<uint8_t*>(&sh.col[0][0]);
    if (act) {
      *reinterpret_cast<qt_u32x4*>(code8 + kHeadDim * t + 32 * k) = qt_u32x4{cw[0], cw[1], cw[2], cw[3]};
      *reinterpret_cast<qt_u32x4*>(code8 + kHeadDim * t + 32 * k + 16) = qt_u32x4{cw[4], cw[5], cw[6], cw[7]};
    }
    __syncthreads();
    const int lane = tid & 63, w = tid >> 6, j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int m = 0; m < 8; ++m)
        R[q][m] = (w == 0 && q < 4) ? (float)code8[kHeadDim * (4 * g + q) + j + 16 * m] : 0.f;
    return;
  }

  // rounding: per token, zero-point = min, step = range / levels, ties to even
  double mn = y[0], mx = y[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fmin(mn, y[i]);
    mx = fmax(mx, y[i]);
  }
  mn = fmin(mn, quad_dpp<kQuadX1>(mn));
  mx = fmax(mx, quad_dpp<kQuadX1>(mx));
  mn = fmin(mn, quad_dpp<kQuadX2>(mn));
  mx = fmax(mx, quad_dpp<kQuadX2>(mx));
  const double step = (mx - mn) / LEVELS;
  const bool real = act && t < n;
  const double inv = (real && step > 0.0) ? 1.0 / step : 0.0;   // empty and zero-range rows: codes 0
  unsigned cw[8];   // the lane's 32 codes, one byte each
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    unsigned w = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double c = fmin(fmax(__builtin_rint((y[4 * v + e] - mn) * inv), 0.0), LEVELS);
      w |= (unsigned)c << (8 * e);
    }
    cw[v] = w;
  }
  // scales and offsets: S = beta * step, O = beta * min (0 past the tile's end)
  double bs = real ? beta * step : 0.0, bo = real ? beta * mn : 0.0;
  double ea = 1.0;   // fp16 metadata: the power of two moved into the channel factors
  if constexpr (M16) {
    double m = (k == 0) ? fmax(fabs(bs), fabs(bo)) : 0.0;   // the tile's largest |S|, |O| (wave 0 holds it)
#pragma unroll
    for (int sb = 1; sb < 64; sb <<= 1) m = fmax(m, __shfl_xor(m, sb));
    const int ex = (int)((__double_as_longlong(m) >> 52) & 0x7FF);
    const int e = (ex == 0 || ex == 0x7FF) ? 0 : ex - 1023 - 10;
    ea = __longlong_as_double((long long)(1023 + e) << 52);
    bs /= ea;
    bo /= ea;
    if (tid == 0) sh.inv_g[0] = ea;   // for the channel factors' writers (after the barrier below)
  }
  const float S = (float)bs, O = (float)bo;
  if (MODE == kDense) {
    if (act && k == 0 && t < n) {
      A.scale[(size_t)(t0 + t) * H + head] = S;
      A.offset[(size_t)(t0 + t) * H + head] = O;
    }
  } else {
    if (act && k == 0) {
      if constexpr (M16) {
        store_meta<true>(page_slot(0) + CODE_BYTES, t, (float)(_Float16)bs);
        store_meta<true>(page_slot(0) + OFF_AT, t, (float)(_Float16)bo);
      } else {
        store_meta<false>(page_slot(0) + CODE_BYTES, t, S);
        store_meta<false>(page_slot(0) + OFF_AT, t, O);
      }
    }
    if (tid >= kShortTile && tid < T) {   // rows of the tile's later pages
      store_meta<M16>(page_slot(tid / kPage) + CODE_BYTES, tid % kPage, 0.f);
      store_meta<M16>(page_slot(tid / kPage) + OFF_AT, tid % kPage, 0.f);
    }
  }
  // codes to the fp32 path's register layout through LDS ([token][channel] bytes over col)
  __syncthreads();   // every thread is done reading col
  uint8_t* code8 = reinterpret_cast<uint8_t*>(&sh.col[0][0]);
  if (act) {
    *reinterpret_cast<qt_u32x4*>(code8 + kHeadDim * t + 32 * k) = qt_u32x4{cw[0], cw[1], cw[2], cw[3]};
    *reinterpret_cast<qt_u32x4*>(code8 + kHeadDim * t + 32 * k + 16) = qt_u32x4{cw[4], cw[5], cw[6], cw[7]};
  }
  if constexpr (M16) ea = sh.inv_g[0];
  for (int c = tid; c < kHeadDim; c += NT) {
    if (MODE == kDense) A.alpha[((size_t)(t0 / T) * H + head) * kHeadDim + c] = (float)sh.alpha[c];
    else if constexpr (M16) store_meta<true>(page_slot(c / AL) + ALPHA_AT, c % AL, (float)(_Float16)(sh.alpha[c] * ea));
    else store_meta<false>(page_slot(c / AL) + ALPHA_AT, c % AL, (float)sh.alpha[c]);
  }
  __syncthreads();
  const int lane = tid & 63, w = tid >> 6, j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int m = 0; m < 8; ++m)
      R[q][m] = (w == 0 && q < 4) ? (float)code8[kHeadDim * (4 * g + q) + j + 16 * m] : 0.f;
  if constexpr (PADK) {   // the per-channel K body beside this one passes three more barriers
    __syncthreads();
    __syncthreads();
    __syncthreads();
  }
}

// Which tiles a quantizer instantiation handles: the fp32 path only (tiles of
// fewer than 16 tokens return at once: the bulk prefill kernels, kept free of
// the float64 path's registers), the float64 path only (its own small launch
// over the sequences' last tiles), or both by a runtime branch (appends).
enum TilePath { kPathFp32 = 0, kPathShort = 1, kPathBoth = 2 };

// KCH: a K tile rounded per channel (fp32 metadata, paged layouts): all
// normalization half-steps run, and the slot takes beta per token and the
// channel scales and zero offsets in place of S, O and alpha.
// PADK: a body that runs beside a per-channel K body in one workgroup (the
// fused append + decode) and passes the same number of workgroup barriers.
template <int T, int BITS, bool VLAYOUT, int MODE, bool M16 = false,
          int PATH = (MODE == kAppend) ? kPathBoth : kPathFp32, bool KCH = false, bool PADK = false>
__device__ __forceinline__ void quantize_tile_body(const QuantArgs& A, Smem<T>& sm, ShortSmem* sh, int role,
                                                   int head, int seq, int tile_idx, int tid) {
  static_assert(!KCH || (!VLAYOUT && !M16 && MODE != kDense), "per-channel rounding: paged K slots, fp32 metadata");
  static_assert(!(KCH && PADK), "a per-channel body is not padded");
  constexpr int NT = 2 * T;
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  // token (in the tile) of register row q = 4 bb + r
  auto tok = [&](int q) { return 32 * w + 16 * (q >> 2) + 4 * g + (q & 3); };

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

  // (uniform over the group)
  if (PATH == kPathFp32 && n_valid < kShortTile) return;
  if (PATH == kPathShort && (n_valid >= kShortTile || n_valid <= 0)) return;

  // ---------------------------------------------------------------- load fp16 rows (MFMA A layout)
  // raw[bb][p]: row j of block bb, channels 32p + 8g .. 32p + 8g + 7.
  // Rows past the tile's end load row 0 again: their values are then exact
  // copies of row 0, which the statistics below exclude exactly.
  qt_u32x4 raw[2][4];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int t = 32 * w + 16 * bb + j;
    const int src_t = (t < n_valid) ? t : 0;
    const uint16_t* row = rows_base + (size_t)src_t * row_stride;
    if (MODE == kAppend && src_t == r_new) row = A.src[role] + ((size_t)seq * H + head) * kHeadDim;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      raw[bb][p] = __builtin_nontemporal_load(reinterpret_cast<const qt_u32x4*>(row + 32 * p + 8 * g));
  }
  // Keep the fp16 rows of a partial tile for later appends.
  if (MODE != kDense && A.staging[role] != nullptr) {
    uint16_t* stg = A.staging[role] + ((size_t)seq * T * H + head) * kHeadDim;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int t = 32 * w + 16 * bb + j;
      const bool write = (MODE == kPaged) ? (n_valid < T && t < n_valid) : (t == r_new);
      if (write) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          *reinterpret_cast<qt_u32x4*>(stg + (size_t)t * row_stride + 32 * p + 8 * g) = raw[bb][p];
      }
    }
  }

  // randomized rotation: channel c negated first (the fp16 sign bits of the
  // MFMA operand; the staged rows above stay as given)
  if (any_sign(A.signs)) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[bb][p][i] ^= sign_pair_mask(A.signs, 32 * p + 8 * g, i);
  }

  // Output addressing (paged): the tile's pages.
  uint8_t* pool = nullptr;
  const int32_t* pages = nullptr;
  constexpr int SLOT = slot_bytes(BITS, T, M16, KCH);
  constexpr int CODE_BYTES = slot_code_bytes(BITS);
  constexpr int OFF_AT = slot_offset_at(BITS, M16), ALPHA_AT = slot_alpha_at(BITS, M16);
  if (MODE != kDense) {
    pool = A.pool[role];
    pages = A.block_table + (size_t)seq * A.max_blocks + (t0 / kPage);
  }
  auto slot_ptr = [&](int page_in_tile) -> uint8_t* {
    return pool + ((size_t)pages[page_in_tile] * H + head) * SLOT;
  };

  float R[8][8];   // [q = 4 bb + r][m = sigma + 2 p']: token tok(q), channel j + 16 m
  if (PATH != kPathFp32 && (PATH == kPathShort || n_valid < kShortTile)) {   // uniform over the group
    short_tile<T, BITS, MODE, M16, KCH, PADK>(A, *sh, role, head, seq, t0, n_valid, rows_base, row_stride, r_new,
                                              tid, R, pool, pages);
  } else {
    // ---------------------------------------------------------------- Hadamard (unnormalized)
    // B+ = [H16; H16], B- = [H16; -H16] in the MFMA B layout: lane (g, j) holds
    // rows 8g..8g+7 of column j, H16[k][j] = (-1)^popcount(k & j).
    // Bit a of hrow is the sign of H16[a][j]: the parity of a & j, the XOR of
    // the patterns of a's bits 0..3 over the bits set in j.
    const unsigned jb = (unsigned)j;
    const unsigned hrow = ((0u - (jb & 1u)) & 0xAAAAu) ^ ((0u - ((jb >> 1) & 1u)) & 0xCCCCu) ^
                          ((0u - ((jb >> 2) & 1u)) & 0xF0F0u) ^ ((0u - ((jb >> 3) & 1u)) & 0xFF00u);
    const unsigned sp = (hrow >> (8 * (g & 1))) & 0xFFu;   // rows 8g..8g+7 (mod 16)
    const unsigned sn = sp ^ ((g >= 2) ? 0xFFu : 0u);
    qt_u32x4 bpw, bnw;   // fp16 pairs of +-1.0 (0x3C00, sign in bit 15 of each half)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bpw[i] = 0x3C003C00u | ((sp << (15 - 2 * i)) & 0x8000u) | ((sp << (30 - 2 * i)) & 0x80000000u);
      bnw[i] = 0x3C003C00u | ((sn << (15 - 2 * i)) & 0x8000u) | ((sn << (30 - 2 * i)) & 0x80000000u);
    }
    const qt_f16x8 bpos = __builtin_bit_cast(qt_f16x8, bpw), bneg = __builtin_bit_cast(qt_f16x8, bnw);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      qt_f32x4 zp[4], zn[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const qt_f16x8 x = __builtin_bit_cast(qt_f16x8, raw[bb][p]);
        zp[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, bpos, qt_f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        zn[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, bneg, qt_f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
      // channel bits 5, 6: y[p'] = sum_p (-1)^popcount(p & p') z[p]
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
          const qt_f32x4* z = sg ? zn : zp;
          const float e0 = z[0][r] + z[1][r], e1 = z[0][r] - z[1][r];
          const float e2 = z[2][r] + z[3][r], e3 = z[2][r] - z[3][r];
          R[4 * bb + r][sg + 0] = e0 + e2;
          R[4 * bb + r][sg + 4] = e0 - e2;
          R[4 * bb + r][sg + 2] = e1 + e3;
          R[4 * bb + r][sg + 6] = e1 - e3;
        }
    }

    // ---------------------------------------------------------------- normalization
    // Spread sums are taken over values shifted by a reference (channel step:
    // the tile's first token; token step: the token's channel 0), so that
    // E[d^2] - E[d]^2 does not cancel when a mean dwarfs the spread.
    if (w == 0 && g == 0) {
      *reinterpret_cast<qt_f32x4*>(&sm.ref_c[8 * j]) = qt_f32x4{R[0][0], R[0][1], R[0][2], R[0][3]};
      *reinterpret_cast<qt_f32x4*>(&sm.ref_c[8 * j + 4]) = qt_f32x4{R[0][4], R[0][5], R[0][6], R[0][7]};
    }
    if (j == 0) {
      *reinterpret_cast<qt_f32x4*>(&sm.ref_t[tok(0)]) = qt_f32x4{R[0][0], R[1][0], R[2][0], R[3][0]};
      *reinterpret_cast<qt_f32x4*>(&sm.ref_t[tok(4)]) = qt_f32x4{R[4][0], R[5][0], R[6][0], R[7][0]};
    }
    for (int c = tid; c < kHeadDim; c += NT) {
      sm.a[c] = kInvSqrtD;
      sm.alpha[c] = 1.0f;
    }
    if (tid < T) sm.b[tid] = 1.0f;
    __syncthreads();
    // (the references are re-read from LDS in each step, to keep registers free)
    float a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = kInvSqrtD;
      b[i] = 1.0f;
    }
    const float inv_n = __builtin_amdgcn_rcpf((float)n_valid);   // the hardware reciprocal (within an ulp)
    const float n_copies = (float)(T - n_valid);  // rows that are copies of row 0
    const int iters = A.iters;
    float b0 = 1.0f;
    float* red0 = sm.red[0];
    float* red1 = sm.red[1];

    for (int it = 0; it < iters; ++it) {
      // channel step: spread over the tile's valid tokens of u = b_t R_tc
      {
        float s1[8], s2[8], kc[8];
        {
          const qt_f32x4 r0 = *reinterpret_cast<const qt_f32x4*>(&sm.ref_c[8 * j]);
          const qt_f32x4 r1 = *reinterpret_cast<const qt_f32x4*>(&sm.ref_c[8 * j + 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            kc[i] = b0 * r0[i];
            kc[4 + i] = b0 * r1[i];
          }
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float d = __builtin_fmaf(b[0], R[0][m], -kc[m]);
          s1[m] = d;
          s2[m] = d * d;
        }
#pragma unroll
        for (int q = 1; q < 8; ++q) {
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const float d = __builtin_fmaf(b[q], R[q][m], -kc[m]);
            s1[m] += d;
            s2[m] = __builtin_fmaf(d, d, s2[m]);
          }
        }
        float* p1 = red0 + (4 * w + g) * kHeadDim + 4 * j;
        float* p2 = red1 + (4 * w + g) * kHeadDim + 4 * j;
        *reinterpret_cast<qt_f32x4*>(p1) = qt_f32x4{s1[0], s1[1], s1[2], s1[3]};
        *reinterpret_cast<qt_f32x4*>(p1 + 64) = qt_f32x4{s1[4], s1[5], s1[6], s1[7]};
        *reinterpret_cast<qt_f32x4*>(p2) = qt_f32x4{s2[0], s2[1], s2[2], s2[3]};
        *reinterpret_cast<qt_f32x4*>(p2 + 64) = qt_f32x4{s2[4], s2[5], s2[6], s2[7]};
      }
      __syncthreads();
      // The finalize is a short dependent chain that the group's other waves
      // wait for at the next barrier: its waves go first meanwhile (wave
      // priority), the other workgroups' element passes fill the issue slots.
      __builtin_amdgcn_s_setprio(2);
      for (int i = tid; i < kHeadDim; i += NT) {   // lane-order index i: channel (i >> 3) + 16 (i & 7)
        float S1 = 0.f, S2 = 0.f;
        const int at = 64 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);   // its place in a row of partials
#pragma unroll
        for (int row = 0; row < T / 8; ++row) {
          S1 += red0[row * kHeadDim + at];
          S2 += red1[row * kHeadDim + at];
        }
        // copies of row 0 each added row 0's own shifted value rho (the fma
        // residual of the shift); take them out
        const float rc = sm.ref_c[i];
        const float kcc = b0 * rc;
        const float rho = __builtin_fmaf(b0, rc, -kcc);
        S1 = __builtin_fmaf(-n_copies, rho, S1);
        S2 = __builtin_fmaf(-n_copies, rho * rho, S2);
        const float mn = S1 * inv_n;                                  // mean of the shifted values
        const float var = fmaxf(__builtin_fmaf(-mn, mn, S2 * inv_n), 0.f);
        const float mu = mn + kcc;                                    // mean of u
        const float ms = __builtin_fmaf(mu, mu, var);                 // mean square of u
        if (var > kGuard2 * ms) {
          sm.a[i] = __builtin_amdgcn_rsqf(var);
          // the stored factor only (codes use a): the hardware square root,
          // within an ulp, in place of the correctly rounded expansion
          sm.alpha[(i >> 3) + 16 * (i & 7)] = __builtin_amdgcn_sqrtf(var * (1.0f / kHeadDim));
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      {
        const qt_f32x4 lo = *reinterpret_cast<const qt_f32x4*>(&sm.a[8 * j]);
        const qt_f32x4 hi = *reinterpret_cast<const qt_f32x4*>(&sm.a[8 * j + 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = lo[i]; a[4 + i] = hi[i]; }
      }
      // the final token step cancels in every stored value of a row-rounded
      // tile; per-channel rounding needs it
      if (it + 1 == iters && !KCH) {
        if constexpr (PADK) {   // the per-channel K body beside this one runs the token step's two barriers
          __syncthreads();
          __syncthreads();
        }
        break;
      }

      // token step: spread over the 128 channels of u = a_c R_tc
      const float a0 = sm.a[0];   // channel 0
      {
        float t1[8], t2[8];
        const qt_f32x4 u0 = *reinterpret_cast<const qt_f32x4*>(&sm.ref_t[tok(0)]);
        const qt_f32x4 u1 = *reinterpret_cast<const qt_f32x4*>(&sm.ref_t[tok(4)]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float kt = a0 * ((q < 4) ? u0[q] : u1[q - 4]);
          float x1, x2;
          {
            const float d = __builtin_fmaf(a[0], R[q][0], -kt);
            x1 = d;
            x2 = d * d;
          }
#pragma unroll
          for (int m = 1; m < 8; ++m) {
            const float d = __builtin_fmaf(a[m], R[q][m], -kt);
            x1 += d;
            x2 = __builtin_fmaf(d, d, x2);
          }
          t1[q] = x1;
          t2[q] = x2;
        }
        *reinterpret_cast<qt_f32x4*>(&red0[j * kRedStride<T> + tok(0)]) = qt_f32x4{t1[0], t1[1], t1[2], t1[3]};
        *reinterpret_cast<qt_f32x4*>(&red0[j * kRedStride<T> + tok(4)]) = qt_f32x4{t1[4], t1[5], t1[6], t1[7]};
        *reinterpret_cast<qt_f32x4*>(&red1[j * kRedStride<T> + tok(0)]) = qt_f32x4{t2[0], t2[1], t2[2], t2[3]};
        *reinterpret_cast<qt_f32x4*>(&red1[j * kRedStride<T> + tok(4)]) = qt_f32x4{t2[4], t2[5], t2[6], t2[7]};
      }
      __syncthreads();
      __builtin_amdgcn_s_setprio(2);   // (as in the channel step's finalize)
      if (tid < T) {
        float T1 = 0.f, T2 = 0.f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          T1 += red0[jj * kRedStride<T> + tid];
          T2 += red1[jj * kRedStride<T> + tid];
        }
        const float mn = T1 * (1.0f / kHeadDim);
        const float var = fmaxf(__builtin_fmaf(-mn, mn, T2 * (1.0f / kHeadDim)), 0.f);
        const float mu = __builtin_fmaf(a0, sm.ref_t[tid], mn);
        const float ms = __builtin_fmaf(mu, mu, var);
        if (var > kGuard2 * ms) sm.b[tid] = __builtin_amdgcn_rsqf(var);
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      {
        b0 = sm.b[0];
        const qt_f32x4 u0 = *reinterpret_cast<const qt_f32x4*>(&sm.b[tok(0)]);
        const qt_f32x4 u1 = *reinterpret_cast<const qt_f32x4*>(&sm.b[tok(4)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {   // copies weigh as row 0
          b[i] = (tok(i) < n_valid) ? u0[i] : b0;
          b[4 + i] = (tok(4 + i) < n_valid) ? u1[i] : b0;
        }
      }
    }

    // ---------------------------------------------------------------- rounding
    if constexpr (KCH) {
      // per channel over the tile's tokens of y = R a b (copies of row 0 weigh
      // as row 0 and leave the minima and maxima alone); the slot takes beta =
      // 1 / b per token, A = alpha step and M = min / step per channel (a
      // zero-range channel: A = alpha min, M = 1, codes 0)
      float cmin[8], cmax[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int m = 0; m < 8; ++m) R[q][m] *= a[m] * b[q];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        cmin[m] = vmin3f(vmin3f(vmin3f(R[0][m], R[1][m], R[2][m]), R[3][m], R[4][m]), R[5][m], vmin3f(R[6][m], R[7][m], R[7][m]));
        cmax[m] = vmax3f(vmax3f(vmax3f(R[0][m], R[1][m], R[2][m]), R[3][m], R[4][m]), R[5][m], vmax3f(R[6][m], R[7][m], R[7][m]));
      }
      float* p1 = red0 + (4 * w + g) * kHeadDim + 8 * j;   // [row 4w + g][lane order]
      float* p2 = red1 + (4 * w + g) * kHeadDim + 8 * j;
      *reinterpret_cast<qt_f32x4*>(p1) = qt_f32x4{cmin[0], cmin[1], cmin[2], cmin[3]};
      *reinterpret_cast<qt_f32x4*>(p1 + 4) = qt_f32x4{cmin[4], cmin[5], cmin[6], cmin[7]};
      *reinterpret_cast<qt_f32x4*>(p2) = qt_f32x4{cmax[0], cmax[1], cmax[2], cmax[3]};
      *reinterpret_cast<qt_f32x4*>(p2 + 4) = qt_f32x4{cmax[4], cmax[5], cmax[6], cmax[7]};
      __syncthreads();
      for (int i = tid; i < kHeadDim; i += NT) {   // lane-order index i: channel (i >> 3) + 16 (i & 7)
        float mn = red0[i], mx = red1[i];
#pragma unroll
        for (int row = 1; row < T / 8; ++row) {
          mn = fminf(mn, red0[row * kHeadDim + i]);
          mx = fmaxf(mx, red1[row * kHeadDim + i]);
        }
        const float range = mx - mn;
        const float inv = range > 0.f ? LEVELS * __builtin_amdgcn_rcpf(range) : 0.f;
        sm.a[i] = inv;             // (the channel factors' reciprocals are in registers)
        sm.ref_c[i] = -mn * inv;   // (the channel-step references are no longer needed)
        const int c = (i >> 3) + 16 * (i & 7);
        const float al = sm.alpha[c];
        const float st = range * (1.0f / LEVELS);
        constexpr int AL = slot_alpha_len(T);
        uint8_t* slot = slot_ptr(c / AL);
        store_meta<false>(slot + slot_chan_scale_at(BITS), c % AL, range > 0.f ? al * st : al * mn);
        store_meta<false>(slot + slot_chan_zp_at(BITS, T), c % AL, range > 0.f ? mn / st : 1.f);
      }
      if (tid < T) store_meta<false>(slot_ptr(tid / kPage) + CODE_BYTES, tid % kPage, tid < n_valid ? 1.f / sm.b[tid] : 0.f);
      __syncthreads();
      const qt_f32x4 i0 = *reinterpret_cast<const qt_f32x4*>(&sm.a[8 * j]);
      const qt_f32x4 i1 = *reinterpret_cast<const qt_f32x4*>(&sm.a[8 * j + 4]);
      const qt_f32x4 n0 = *reinterpret_cast<const qt_f32x4*>(&sm.ref_c[8 * j]);
      const qt_f32x4 n1 = *reinterpret_cast<const qt_f32x4*>(&sm.ref_c[8 * j + 4]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool real = tok(q) < n_valid;   // rows past the tile's end get code 0
#pragma unroll
        for (int m = 0; m < 8; ++m)
          R[q][m] = real ? __builtin_fmaf(R[q][m], m < 4 ? i0[m] : i1[m - 4], m < 4 ? n0[m] : n1[m - 4]) : 0.f;
      }
    } else {
    {
      float zmin[8], zmax[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int m = 0; m < 8; ++m) R[q][m] *= a[m];
        float mn = vmin3f(R[q][0], R[q][1], R[q][2]), mx = vmax3f(R[q][0], R[q][1], R[q][2]);
        mn = vmin3f(mn, R[q][3], R[q][4]);
        mx = vmax3f(mx, R[q][3], R[q][4]);
        mn = vmin3f(mn, R[q][5], R[q][6]);
        mx = vmax3f(mx, R[q][5], R[q][6]);
        mn = vmin3f(mn, R[q][7], R[q][7]);
        mx = vmax3f(mx, R[q][7], R[q][7]);
        zmin[q] = mn;
        zmax[q] = mx;
      }
      *reinterpret_cast<qt_f32x4*>(&red0[j * kRedStride<T> + tok(0)]) = qt_f32x4{zmin[0], zmin[1], zmin[2], zmin[3]};
      *reinterpret_cast<qt_f32x4*>(&red0[j * kRedStride<T> + tok(4)]) = qt_f32x4{zmin[4], zmin[5], zmin[6], zmin[7]};
      *reinterpret_cast<qt_f32x4*>(&red1[j * kRedStride<T> + tok(0)]) = qt_f32x4{zmax[0], zmax[1], zmax[2], zmax[3]};
      *reinterpret_cast<qt_f32x4*>(&red1[j * kRedStride<T> + tok(4)]) = qt_f32x4{zmax[4], zmax[5], zmax[6], zmax[7]};
    }
    __syncthreads();

    float step = 0.f, off = 0.f;
    if (tid < T) {
      float mn = red0[tid], mx = red1[tid];
#pragma unroll
      for (int jj = 1; jj < 15; jj += 2) {
        mn = vmin3f(mn, red0[jj * kRedStride<T> + tid], red0[(jj + 1) * kRedStride<T> + tid]);
        mx = vmax3f(mx, red1[jj * kRedStride<T> + tid], red1[(jj + 1) * kRedStride<T> + tid]);
      }
      mn = vmin3f(mn, red0[15 * kRedStride<T> + tid], red0[15 * kRedStride<T> + tid]);
      mx = vmax3f(mx, red1[15 * kRedStride<T> + tid], red1[15 * kRedStride<T> + tid]);
      float inv = 0.f, nmi = 0.f;
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
      } else if (!M16) {
        uint8_t* slot = slot_ptr(tid / kPage);
        store_meta<false>(slot + CODE_BYTES, tid % kPage, step);
        store_meta<false>(slot + OFF_AT, tid % kPage, off);
      }
    }
    float ea = 1.f;   // fp16 metadata: the power of two moved into the channel factors
    if constexpr (M16 && MODE != kDense) {
      float m = fmaxf(fabsf(step), fabsf(off));   // the tile's largest |S|, |O| (0 past its end)
#pragma unroll
      for (int sb = 1; sb < 64; sb <<= 1) m = fmaxf(m, __shfl_xor(m, sb));
      if (lane == 0) sm.ref_t[w] = m;   // (the token-step references are no longer needed)
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) m = fmaxf(m, sm.ref_t[i]);
      const int e = meta_exponent(m);
      ea = pow2f(e);
      if (tid < T) {
        uint8_t* slot = slot_ptr(tid / kPage);
        store_meta<true>(slot + CODE_BYTES, tid % kPage, step * pow2f(-e));
        store_meta<true>(slot + OFF_AT, tid % kPage, off * pow2f(-e));
      }
    }
    for (int c = tid; c < kHeadDim; c += NT) {
      const float al = sm.alpha[c];
      if (MODE == kDense) {
        A.alpha[((size_t)tile_idx * H + head) * kHeadDim + c] = al;
      } else {
        constexpr int AL = slot_alpha_len(T);
        store_meta<M16>(slot_ptr(c / AL) + ALPHA_AT, c % AL, al * ea);
      }
    }
    __syncthreads();

    // values before rounding: v = (z - min) * levels / range, in [0, levels]
    {
      const qt_f32x4 i0 = *reinterpret_cast<const qt_f32x4*>(&sm.inv[tok(0)]);
      const qt_f32x4 i1 = *reinterpret_cast<const qt_f32x4*>(&sm.inv[tok(4)]);
      const qt_f32x4 n0 = *reinterpret_cast<const qt_f32x4*>(&sm.nmi[tok(0)]);
      const qt_f32x4 n1 = *reinterpret_cast<const qt_f32x4*>(&sm.nmi[tok(4)]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float iv = (q < 4) ? i0[q] : i1[q - 4];
        const float nm = (q < 4) ? n0[q] : n1[q - 4];
#pragma unroll
        for (int m = 0; m < 8; ++m) R[q][m] = __builtin_fmaf(R[q][m], iv, nm);
      }
    }
    }   // per-token rounding

  }

  // the slots of the lane's two pages (its tokens 32 w + 16 bb + ...), taken
  // once: the byte stores below could alias the block table, so an address
  // formed per store would reload the page id from memory each time
  uint8_t* lane_slot[2] = {nullptr, nullptr};
  if (MODE != kDense) {
    lane_slot[0] = slot_ptr(2 * w);
    lane_slot[1] = slot_ptr(2 * w + 1);
  }
  if (MODE == kDense || !VLAYOUT) {
    // unit j of each of the lane's tokens: field m <- channel j + 16 m
    // (a unit is BITS bytes: half a word at 2 bits, a word at 4, two words at 8)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int t = tok(q);
      if (MODE == kDense && t >= n_valid) continue;
      uint8_t* dst;
      if (MODE == kDense) dst = A.codes + ((size_t)(t0 + t) * H + head) * (kHeadDim * BITS / 8) + BITS * j;
      else   // K slot: 4 blocks of 4 units (4 BITS bytes per token), token after token
        dst = lane_slot[q >> 2] + (j >> 2) * (kPage * 4 * BITS) + (t % kPage) * (4 * BITS) + BITS * (j & 3);
      if constexpr (BITS == 8) {
        const float lo[4] = {R[q][0], R[q][1], R[q][2], R[q][3]};
        const float hi[4] = {R[q][4], R[q][5], R[q][6], R[q][7]};
        *reinterpret_cast<qt_u32x2*>(dst) = qt_u32x2{pack_fields<8>(lo), pack_fields<8>(hi)};
      } else {
        const unsigned wd = pack_fields<BITS>(R[q]);
        if (BITS == 4) *reinterpret_cast<uint32_t*>(dst) = wd;
        else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)wd;
      }
    }
  } else if constexpr (BITS == 8) {
    // V slot at 8 bits: run l (32 bytes) holds word p = 2g + h per token quad g and
    // channel half h, field (r >> 1) + 2 (r & 1) for token 4g + r
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      uint8_t* slot = lane_slot[bb];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        unsigned wd[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[(r >> 1) + 2 * (r & 1)] = R[4 * bb + r][m + 4 * h];
          wd[h] = pack_fields<8>(o);
        }
        *reinterpret_cast<qt_u32x2*>(slot + 32 * (j + 16 * m) + 8 * g) = qt_u32x2{wd[0], wd[1]};
      }
    }
  } else {
    // V slot: run l (4*BITS bytes at 4*BITS*l) holds channels l and 64 + l of
    // the page's 16 tokens; token 4g + r of half h is pair p = 2g + h, in word
    // p / (F/4) of the run, field 2m' + (r>>1) + (F/2)(r&1), m' = p mod (F/4).
    // The lane holds quad g of page 2w + bb for the runs j + 16 m (m < 4),
    // channels j + 16 m (h = 0) and j + 16 (m + 4) (h = 1).
    constexpr int F = 32 / BITS;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      uint8_t* slot = lane_slot[bb];
      unsigned part[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float o[F];
#pragma unroll
        for (int f = 0; f < F; ++f) o[f] = 0.f;
        const int mq = (BITS == 4) ? 0 : 2 * (g & 1);   // m' = 2 (g mod 2) + h at 2 bits
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[2 * h + (r >> 1) + (F / 2) * (r & 1)] = R[4 * bb + r][m + 4 * h];
        // fields 2 m' + ... with m' = mq + h: the mq part is a shift of the word
        part[m] = pack_fields<BITS>(o) << (BITS * 2 * mq);
      }
      if (BITS == 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) *reinterpret_cast<uint32_t*>(slot + 16 * (j + 16 * m) + 4 * g) = part[m];
      } else {
        // one word per (run, quad pair): merge with the lane of quad g ^ 1
        // (lane ^ 16); the even quad's lane writes runs m < 2, the odd one m >= 2
        const bool odd = (g & 1) != 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const unsigned mine = odd ? part[k + 2] : part[k];
          const unsigned give = odd ? part[k] : part[k + 2];
          const unsigned got = (unsigned)__shfl_xor((int)give, 16);
          *reinterpret_cast<uint32_t*>(slot + 8 * (j + 16 * (k + (odd ? 2 : 0))) + 4 * (g >> 1)) = mine | got;
        }
      }
    }
  }
}

}  // namespace
}  // namespace kvq
