// Baselines for the long-context comparison: paged decode attention on fp16
// pages and on fp8 (OCP E4M3, one scale per tensor) pages, and the cache
// fills that write those pages.  The aitrends.kr page (article 74976, TL;DR)
// runs fp16, fp8 and compressed KV side by side on the same workload.
//
// Page layouts per (page, kv head): K [16 tokens][128 channels], V [128
// channels][16 tokens] (channel-major), fp16 or E4M3 bytes; rows past the
// sequence end are 0.  Decode: one workgroup of 4 waves per (partition of
// 64-token blocks, kv head, sequence); each wave walks its blocks page by
// page with the next page prefetched.  QK^T runs on mfma_f32_16x16x32_f16
// (A = 16 tokens x 32 channels of K as stored, B = the fp16 query, exact
// products); PV on mfma_f32_16x16x16_f16 (A = 16 channels x 4 tokens of V as
// stored, B = probabilities as fp16 hi + lo), whose B layout is the QK output
// layout.  Partitions are merged by the shared combine kernel.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kBlock = 64;                   // tokens per partition unit
constexpr int kPagesPerBlock = kBlock / kPage;
constexpr int kMaxBlocksPerPart = 64;

__device__ __forceinline__ float max16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}
__device__ __forceinline__ float sum16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float sum32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float group_max(float v) { return max32(max16(v)); }
__device__ __forceinline__ float group_sum(float v) { return sum32(sum16(v)); }

// two E4M3 bytes (low or high 16 bits of w) -> two fp16, exact
template <bool HI>
__device__ __forceinline__ unsigned e4m3x2_to_f16x2(unsigned w) {
  const f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(unsigned, h);
}

__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
  const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
  const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
  hi = (unsigned)__builtin_bit_cast(uint16_t, h0) | ((unsigned)__builtin_bit_cast(uint16_t, h1) << 16);
  lo = (unsigned)__builtin_bit_cast(uint16_t, l0) | ((unsigned)__builtin_bit_cast(uint16_t, l1) << 16);
}

// ---------------------------------------------------------------- cache fill
// grid: x = page index in the sequence, y = kv head, z = sequence; 256 threads.
template <bool FP8>
__global__ __launch_bounds__(256) void fill_kernel(BaseFillArgs A) {
  __shared__ uint16_t tile[2][kPage][kHeadDim + 2];  // K and V rows of the page
  const int seq = blockIdx.z, head = blockIdx.y, pj = blockIdx.x;
  const int a0 = A.cu_seqlens[seq];
  const int len = A.cu_seqlens[seq + 1] - a0;
  const int t0 = pj * kPage;
  if (t0 >= len || (pj + 1) > A.max_blocks) return;
  const int n = min(kPage, len - t0);
  const int H = A.kv_heads;
  const int tid = threadIdx.x;
  const int row = tid >> 4, col = (tid & 15) * 8;
  const size_t page = (size_t)A.block_table[(size_t)seq * A.max_blocks + pj] * H + head;
  constexpr int EB = FP8 ? 1 : 2;  // bytes per element
  uint8_t* pk = A.pool_k + page * (kPage * kHeadDim * EB);
  uint8_t* pv = A.pool_v + page * (kPage * kHeadDim * EB);
  u32x4 kw{0u, 0u, 0u, 0u}, vw{0u, 0u, 0u, 0u};
  if (row < n) {
    const size_t off = ((size_t)(a0 + t0 + row) * H + head) * kHeadDim + col;
    kw = *reinterpret_cast<const u32x4*>(A.k + off);
    vw = *reinterpret_cast<const u32x4*>(A.v + off);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tile[0][row][col + 2 * i] = (uint16_t)(kw[i] & 0xFFFF);
    tile[0][row][col + 2 * i + 1] = (uint16_t)(kw[i] >> 16);
    tile[1][row][col + 2 * i] = (uint16_t)(vw[i] & 0xFFFF);
    tile[1][row][col + 2 * i + 1] = (uint16_t)(vw[i] >> 16);
  }
  __syncthreads();
  // K: [token][channel], row-major like the input
  if (!FP8) {
    *reinterpret_cast<u32x4*>(pk + (row * kHeadDim + col) * 2) = kw;
  } else {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = half_bits_to_float(tile[0][row][col + i]) / A.k_scale;
    unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0u, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    unsigned hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0u, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
    if (row >= n) { lo = 0u; hi = 0u; }
    *reinterpret_cast<u32x2*>(pk + row * kHeadDim + col) = u32x2{lo, hi};
  }
  // V: [channel][token]; thread -> channel tid / 2, tokens 8 (tid & 1) .. +8
  {
    const int c = tid >> 1, tb = 8 * (tid & 1);
    uint16_t hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) hv[i] = tile[1][tb + i][c];
    if (!FP8) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (unsigned)hv[2 * i] | ((unsigned)hv[2 * i + 1] << 16);
      *reinterpret_cast<u32x4*>(pv + (c * kPage + tb) * 2) = w;
    } else {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (tb + i < n) ? half_bits_to_float(hv[i]) / A.v_scale : 0.f;
      unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0u, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
      unsigned hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0u, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
      *reinterpret_cast<u32x2*>(pv + c * kPage + tb) = u32x2{lo, hi};
    }
  }
}

// ---------------------------------------------------------------- append
// One decode token per sequence written into its page (K row p % 16, V
// column p % 16 of the page holding position p = lens_before[s]), encoded as
// the fill encodes.  grid: x = kv head, y = sequence; 128 threads = channels.
template <bool FP8>
__global__ __launch_bounds__(128) void append_base_kernel(BaseFillArgs A, const int32_t* lens_before) {
  const int head = blockIdx.x, seq = blockIdx.y, c = threadIdx.x;
  const int p = lens_before[seq];
  if (p / kPage >= A.max_blocks) return;   // no page for this position
  const int H = A.kv_heads;
  const size_t page = (size_t)A.block_table[(size_t)seq * A.max_blocks + p / kPage] * H + head;
  const int r = p % kPage;
  const size_t src = ((size_t)seq * H + head) * kHeadDim + c;
  const uint16_t kh = A.k[src], vh = A.v[src];
  if (!FP8) {
    reinterpret_cast<uint16_t*>(A.pool_k)[page * (kPage * kHeadDim) + r * kHeadDim + c] = kh;
    reinterpret_cast<uint16_t*>(A.pool_v)[page * (kPage * kHeadDim) + c * kPage + r] = vh;
  } else {
    const unsigned kb = __builtin_amdgcn_cvt_pk_fp8_f32(half_bits_to_float(kh) / A.k_scale, 0.f, 0u, false);
    const unsigned vb = __builtin_amdgcn_cvt_pk_fp8_f32(half_bits_to_float(vh) / A.v_scale, 0.f, 0u, false);
    A.pool_k[page * (kPage * kHeadDim) + r * kHeadDim + c] = (uint8_t)(kb & 0xFFu);
    A.pool_v[page * (kPage * kHeadDim) + c * kPage + r] = (uint8_t)(vb & 0xFFu);
  }
}

// ---------------------------------------------------------------- decode
struct alignas(16) BaseSmem {
  int32_t pages[kMaxBlocksPerPart * kPagesPerBlock];
  float acc[kWaves][16][kHeadDim];
  float m[kWaves][16];
  float l[kWaves][16];
};

template <bool FP8>
__global__ __launch_bounds__(64 * kWaves) void decode_base_kernel(DecodeArgs A) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int PAGE_BYTES = kPage * kHeadDim * EB;
  __shared__ BaseSmem sm;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int part = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int G = A.group;
  const int L = min(A.seq_lens[seq], A.max_blocks * kPage);   // stays inside the block table
  const int nblocks = min((L + kBlock - 1) / kBlock, A.max_tiles);
  const int blk_begin = part * A.tiles_per_part;
  const int blk_end = min(nblocks, blk_begin + A.tiles_per_part);
  if (blk_begin >= blk_end) return;
  const int H = A.kv_heads;
  const bool real = n16 < G;
  {
    const int32_t* row = A.block_table + (size_t)seq * A.max_blocks + blk_begin * kPagesPerBlock;
    const int np = min((blk_end - blk_begin) * kPagesPerBlock, (L + kPage - 1) / kPage - blk_begin * kPagesPerBlock);
    for (int i = threadIdx.x; i < np; i += 64 * kWaves) sm.pages[i] = row[i];
  }
  __syncthreads();
  const int last_page = (L + kPage - 1) / kPage - 1;   // page index in the sequence

  // query as the QK B operand: lane (g, grp), chunk ch -> channels 32 ch + 8 grp .. + 8
  f16x8 qb[4];
  {
    const uint16_t* qrow = A.q + ((size_t)seq * A.q_heads + kvh * G + (real ? n16 : 0)) * kHeadDim;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const u32x4 w = real ? *reinterpret_cast<const u32x4*>(qrow + 32 * ch + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
      qb[ch] = __builtin_bit_cast(f16x8, w);
    }
  }

  // per page: K chunks (A operand of QK) and V blocks (A operand of PV)
  u32x4 kr[4];
  u32x2 vr[8];
  auto issue = [&](int page_in_seq) {
    const size_t pg = (size_t)sm.pages[page_in_seq - blk_begin * kPagesPerBlock] * H + kvh;
    const uint8_t* pk = A.pool_k + pg * PAGE_BYTES;
    const uint8_t* pv = A.pool_v + pg * PAGE_BYTES;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int off = (n16 * kHeadDim + 32 * ch + 8 * grp) * EB;
      if (!FP8) kr[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pk + off));
      else { const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pk + off)); kr[ch] = u32x4{x[0], x[1], 0u, 0u}; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = ((16 * i + n16) * kPage + 4 * grp) * EB;
      if (!FP8) vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pv + off));
      else vr[i] = u32x2{__builtin_nontemporal_load(reinterpret_cast<const unsigned*>(pv + off)), 0u};
    }
  };

  const float cs = A.sm_scale_log2;  // includes the K scale
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's pages, in order: pages 4 blk .. 4 blk + 3 of blocks
  // blk = blk_begin + wave + 4 b, stopping at the sequence's last page
  auto page_of = [&](int j) { return kPagesPerBlock * (blk_begin + wave + kWaves * (j >> 2)) + (j & 3); };
  auto valid = [&](int j) {
    return blk_begin + wave + kWaves * (j >> 2) < blk_end && page_of(j) <= last_page;
  };
  if (valid(0)) issue(page_of(0));
  for (int j = 0; valid(j); ++j) {
    u32x4 kc[4];
    u32x2 vc[8];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) kc[ch] = kr[ch];
#pragma unroll
    for (int i = 0; i < 8; ++i) vc[i] = vr[i];
    const int cur = page_of(j);
    if (valid(j + 1)) issue(page_of(j + 1));

    // scores
    f32x4 d{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      f16x8 a;
      if (!FP8) {
        a = __builtin_bit_cast(f16x8, kc[ch]);
      } else {
        const u32x4 w{e4m3x2_to_f16x2<false>(kc[ch][0]), e4m3x2_to_f16x2<true>(kc[ch][0]),
                      e4m3x2_to_f16x2<false>(kc[ch][1]), e4m3x2_to_f16x2<true>(kc[ch][1])};
        a = __builtin_bit_cast(f16x8, w);
      }
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[ch], d, 0, 0, 0);
    }
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = cur * kPage + 4 * grp + r;
      s[r] = (t < L) ? cs * d[r] : -INFINITY;
    }
    // online softmax (base 2), per page
    float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    tmax = group_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = __builtin_amdgcn_exp2f(s[r] - m_new);
      psum += s[r];
    }
    l_run = __builtin_fmaf(l_run, corr, psum);
    unsigned h01, l01, h23, l23;
    split_pair(s[0], s[1], h01, l01);
    split_pair(s[2], s[3], h23, l23);
    const f16x4 ph = __builtin_bit_cast(f16x4, u32x2{h01, h23});
    const f16x4 pl = __builtin_bit_cast(f16x4, u32x2{l01, l23});
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f16x4 a;
      if (!FP8) a = __builtin_bit_cast(f16x4, vc[i]);
      else a = __builtin_bit_cast(f16x4, u32x2{e4m3x2_to_f16x2<false>(vc[i][0]), e4m3x2_to_f16x2<true>(vc[i][0])});
      f32x4 x = acc[i] * corr;
      x = __builtin_amdgcn_mfma_f32_16x16x16f16(a, ph, x, 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pl, x, 0, 0, 0);
    }
  }

  // merge the waves; lane (g, grp) holds channels 16 i + 4 grp + r
  l_run = group_sum(l_run);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<f32x4*>(&sm.acc[wave][n16][16 * i + 4 * grp]) = acc[i];
  if (grp == 0) {
    sm.m[wave][n16] = m_run;
    sm.l[wave][n16] = l_run;
  }
  __syncthreads();
  if (wave != 0 || !real) return;
  float M = sm.m[0][n16];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.m[w][n16]);
  float wt[kWaves], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm.m[w][n16];
    wt[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    lsum = __builtin_fmaf(wt[w], sm.l[w][n16], lsum);
  }
  const size_t pidx = ((size_t)seq * A.q_heads + kvh * G + n16) * A.max_parts + part;
  float* dst = A.ws_acc + pidx * kHeadDim;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int c = 32 * grp + 4 * v;   // this lane writes channels 32 grp .. +32
    f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.acc[w][n16][c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(wt[w], y[e], x[e]);
    }
    *reinterpret_cast<f32x4*>(dst + c) = x;
  }
  if (grp == 0) {
    A.ws_ml[2 * pidx] = M;
    A.ws_ml[2 * pidx + 1] = lsum;
  }
}

}  // namespace

hipError_t launch_fill_baseline(const BaseFillArgs& a, bool fp8, int num_seqs, int max_seq_len, hipStream_t s) {
  dim3 grid((max_seq_len + kPage - 1) / kPage, a.kv_heads, num_seqs);
  if (fp8) hipLaunchKernelGGL(fill_kernel<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fill_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_baseline(const BaseFillArgs& a, const int32_t* lens_before, bool fp8, int num_seqs,
                                  hipStream_t s) {
  dim3 grid(a.kv_heads, num_seqs);
  if (fp8) hipLaunchKernelGGL(append_base_kernel<true>, grid, dim3(128), 0, s, a, lens_before);
  else hipLaunchKernelGGL(append_base_kernel<false>, grid, dim3(128), 0, s, a, lens_before);
  return hipGetLastError();
}

hipError_t launch_decode_baseline(const DecodeArgs& a, bool fp8, hipStream_t s) {
  dim3 grid(a.max_parts, a.kv_heads, a.num_seqs);
  if (fp8) hipLaunchKernelGGL(decode_base_kernel<true>, grid, dim3(64 * kWaves), 0, s, a);
  else hipLaunchKernelGGL(decode_base_kernel<false>, grid, dim3(64 * kWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(a, kBlock, false, s);
}

}  // namespace kvq
