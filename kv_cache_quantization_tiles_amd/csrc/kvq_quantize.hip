// Tile quantizer kernels for gfx950 (the tile body is in kvq_tile.h):
// Hadamard rotation along channels (one v_mfma_f32_16x16x32_f16 per 16-token
// block, 32-channel group and sign for channel bits 0..4, a register
// butterfly for bits 5, 6), Sinkhorn-like alternating channel/token variance
// normalization on one-pass shifted sums, per-token asymmetric round-to-
// nearest to packed 2-, 4- or 8-bit codes stored in unit order (dense codes,
// K slots) or as V runs; tiles of fewer than 16 tokens in float64.  Also the
// dense restore, the restore into fp16 pages and a copy kernel that
// calibrates bandwidth and byte counters.
//
// Method: page "Huawei's KVarN boosts vLLM KV-cache capacity by 5x without
// accuracy loss" (axbrief.com), section "기존 방식과 달라진 지점" (the
// four-step tile quantizer); restore: page "화웨이가 공개한 KVarN" (ttj.kr),
// section "양자화로 캐시를 다이어트시킨다".
#include "kvq_tile.h"

namespace kvq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int T, int BITS>
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(4))) void quantize_dense_kernel(QuantArgs A) {
  __shared__ Smem<T> sm;
  quantize_tile_body<T, BITS, false, kDense>(A, sm, nullptr, 0, blockIdx.y, 0, blockIdx.x, threadIdx.x);
}

// the last tile of each head's run when it holds fewer than 16 tokens (float64 path)
template <int T, int BITS>
__global__ __launch_bounds__(2 * T) void quantize_dense_short_kernel(QuantArgs A) {
  __shared__ TileSmem<T> sm;
  quantize_tile_body<T, BITS, false, kDense, false, kPathShort>(A, sm.f, &sm.s, 0, blockIdx.x, 0, (A.n_tokens - 1) / T,
                                                         threadIdx.x);
}

// grid: x = tile slot, y = head + Hkv * role (0 K, 1 V).  Sequence s owns
// the slots from floor(cu[s] / T) + s up to the next sequence's start; the
// starts rise by at least ceil(len / T) (and at most one more), so
// total_tokens / T + num_seqs slots hold every tile
// of any length mix with at most one idle slot per sequence (a grid sized by
// the longest sequence leaves most workgroups idle when lengths vary).  A
// wave finds its sequence with one load of cu_seqlens per 64 sequences and
// a ballot: the starts increase, so the sequences starting at or before the
// slot are a prefix and the last one holds it.
template <int T, int BK, int BV, bool M16, bool KCH>
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(4))) void quantize_paged_kernel(QuantArgs A) {
  __shared__ Smem<T> sm;
  const int f = blockIdx.x;
  const int lane = threadIdx.x & 63;
  int seq = -1, a0 = 0, a1 = 0;
  for (int b = 0; b < A.num_seqs; b += 64) {   // uniform
    const int i = b + lane;
    int c0 = 0, c1 = 0;
    bool before = false;
    if (i < A.num_seqs) {
      c0 = A.cu_seqlens[i];
      c1 = A.cu_seqlens[i + 1];
      before = c0 / T + i <= f;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(before);
    if (m != 0) {
      const int l = 63 - __builtin_clzll(m);
      seq = b + l;
      a0 = __builtin_amdgcn_readlane(c0, l);
      a1 = __builtin_amdgcn_readlane(c1, l);
    }
  }
  if (seq < 0) return;   // uniform over the workgroup from here on
  const int tile = f - (a0 / T + seq);
  if (tile * T >= a1 - a0 || (tile + 1) * (T / kPage) > A.max_blocks) return;
  const int role = blockIdx.y / A.kv_heads;
  const int head = blockIdx.y % A.kv_heads;
  if (role == 0) quantize_tile_body<T, BK, false, kPaged, M16, kPathFp32, KCH>(A, sm, nullptr, 0, head, seq, tile, threadIdx.x);
  else quantize_tile_body<T, BV, true, kPaged, M16>(A, sm, nullptr, 1, head, seq, tile, threadIdx.x);
}

// grid: x = head + Hkv * role, y = sequence: the sequence's last tile when it
// holds fewer than 16 tokens (float64 path)
template <int T, int BK, int BV, bool M16, bool KCH>
__global__ __launch_bounds__(2 * T) void quantize_paged_short_kernel(QuantArgs A) {
  __shared__ TileSmem<T> sm;
  const int seq = blockIdx.y;
  const int len = A.cu_seqlens[seq + 1] - A.cu_seqlens[seq];
  if (len <= 0) return;
  const int role = blockIdx.x / A.kv_heads;
  const int head = blockIdx.x % A.kv_heads;
  const int tile = (len - 1) / T;
  if ((tile + 1) * (T / kPage) > A.max_blocks) return;   // no pages for this tile
  if (role == 0) quantize_tile_body<T, BK, false, kPaged, M16, kPathShort, KCH>(A, sm.f, &sm.s, 0, head, seq, tile, threadIdx.x);
  else quantize_tile_body<T, BV, true, kPaged, M16, kPathShort>(A, sm.f, &sm.s, 1, head, seq, tile, threadIdx.x);
}

// grid: x = head, y = role, z = sequence
template <int T, int BK, int BV, bool M16, bool KCH>
__global__ __launch_bounds__(2 * T) void append_kernel(QuantArgs A) {
  __shared__ TileSmem<T> sm;
  const int seq = blockIdx.z;
  const int tile_idx = A.lens_before[seq] / T;
  if ((tile_idx + 1) * (T / kPage) > A.max_blocks) return;  // no page for this tile
  if (blockIdx.y == 0)
    quantize_tile_body<T, BK, false, kAppend, M16, kPathBoth, KCH>(A, sm.f, &sm.s, 0, blockIdx.x, seq, tile_idx, threadIdx.x);
  else quantize_tile_body<T, BV, true, kAppend, M16>(A, sm.f, &sm.s, 1, blockIdx.x, seq, tile_idx, threadIdx.x);
}

// ---------------------------------------------------------------- dequantize (dense)
// 128 threads = 16 rows (token, head) x 8 channel groups; same register
// layout and butterfly as the quantizer.
template <int T, int BITS>
__global__ __launch_bounds__(128) void dequantize_kernel(DequantArgs A) {
  const int tid = threadIdx.x;
  const int cg = tid & 7;
  const long row = (long)blockIdx.x * 16 + (tid >> 3);
  const long nrows = (long)A.n_tokens * A.heads;
  const bool valid = row < nrows;
  const long rr = valid ? row : 0;
  const int t = (int)(rr / A.heads), h = (int)(rr % A.heads);
  const uint8_t* crow = A.codes + rr * (kHeadDim * BITS / 8);
  const float* al = A.alpha + ((size_t)(t / T) * A.heads + h) * kHeadDim;
  const float S = A.scale[rr], O = A.offset[rr];
  // Codes in unit order (channel u + 16 m in field m of unit u): this
  // thread's channels 64 half + 8 cg + j are field 4 half + (cg >> 1) of the
  // units 8 (cg & 1) + j.
  unsigned units[8];       // fields 0..3 of the unit (fields 4..7 in units8_hi at 8 bits)
  unsigned units8_hi[8];
  if (BITS == 8) {
    // a unit is 8 bytes: word 2j holds fields 0..3, word 2j + 1 fields 4..7
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(crow + 64 * (cg & 1) + 16 * v4);
      units[2 * v4] = w[0];
      units8_hi[2 * v4] = w[1];
      units[2 * v4 + 1] = w[2];
      units8_hi[2 * v4 + 1] = w[3];
    }
  } else if (BITS == 4) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(crow + 32 * (cg & 1));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(crow + 32 * (cg & 1) + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      units[i] = lo[i];
      units[4 + i] = hi[i];
    }
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>(crow + 16 * (cg & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      units[2 * i] = v[i] & 0xFFFFu;
      units[2 * i + 1] = v[i] >> 16;
    }
  }
  float x[16];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int m = 4 * half + (cg >> 1);
    const int c0 = 64 * half + 8 * cg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const unsigned u = (BITS == 8 && m >= 4) ? units8_hi[j] : units[j];
      const int mm = (BITS == 8) ? (m & 3) : m;
      const float q = (float)((u >> (BITS * mm)) & ((1u << BITS) - 1u));
      x[8 * half + j] = al[c0 + j] * __builtin_fmaf(S, q, O);
    }
  }
#pragma unroll
  for (int bit = 1; bit < 16; bit <<= 1)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k & bit) continue;
      const float lo = x[k], hi = x[k | bit];
      x[k] = lo + hi;
      x[k | bit] = lo - hi;
    }
  const float s1 = (cg & 1) ? -1.f : 1.f, s2 = (cg & 2) ? -1.f : 1.f, s4 = (cg & 4) ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], s1, lane_xor<1>(x[k]));
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], s2, lane_xor<2>(x[k]));
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], s4, lane_xor<4>(x[k]));
  if (any_sign(A.signs)) {   // randomized rotation: the restore ends with the signs
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c0 = 64 * half + 8 * cg;
      const unsigned b = (sign_word(A.signs, c0 >> 5) >> (c0 & 31)) & 0xFFu;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[8 * half + j] = ((b >> j) & 1u) ? -x[8 * half + j] : x[8 * half + j];
    }
  }
  if (!valid) return;
  uint16_t* orow = A.out + rr * kHeadDim;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned)float_to_half_bits(x[8 * half + 2 * i] * kInvSqrtD) |
             ((unsigned)float_to_half_bits(x[8 * half + 2 * i + 1] * kInvSqrtD) << 16);
    *reinterpret_cast<u32x4*>(orow + 64 * half + 8 * cg) = w;
  }
}

// ---------------------------------------------------------------- quantized pages -> fp16 pages
// The re-materializing read path's restore: every token of a quantized page
// rebuilt as H (alpha (S code + O)) / sqrt(128) in fp32 and stored as fp16 in
// the fp16 pool's page of the same id (K token-major, V channel-major), as
// kvq_fill_pages_fp16 lays them out.  128 threads = 16 tokens x 8 channel
// groups, the dense restore's register layout and butterfly.
template <int T, int BITS, bool VL, bool M16, bool KCH = false>
__device__ __forceinline__ void restore_page(const RematArgs& A, int seq, int pj, int head, int n,
                                             uint16_t (*vt)[kPage + 2]) {
  constexpr int PPT = T / kPage, AL = slot_alpha_len(T);
  constexpr int SLOT = slot_bytes(BITS, T, M16, KCH), CODE = slot_code_bytes(BITS);
  constexpr int OFF_AT = slot_offset_at(BITS, M16);
  // KCH (K rounded per channel): the channel scales A stand where alpha does
  // and the restore is beta A (code + M)
  constexpr int ALPHA_AT = KCH ? slot_chan_scale_at(BITS) : slot_alpha_at(BITS, M16);
  constexpr unsigned MASK = (1u << BITS) - 1u;
  const int H = A.kv_heads;
  const int tid = threadIdx.x, t = tid >> 3, cg = tid & 7;
  const int32_t* row_tab = A.block_table + (size_t)seq * A.max_blocks;
  const uint8_t* pool = VL ? A.pool_v : A.pool_k;
  const int pid = row_tab[pj];
  const uint8_t* slot = pool + ((size_t)pid * H + head) * SLOT;
  // channel factors of the page's tile: channel c sits in the tile's page c / AL
  const int pt0 = (pj / PPT) * PPT;
  float al[16];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int c0 = 64 * half + 8 * cg;   // 8 channels inside one page's slice (AL is a multiple of 16)
    const uint8_t* ap = pool + ((size_t)row_tab[pt0 + c0 / AL] * H + head) * SLOT + ALPHA_AT;
#pragma unroll
    for (int i = 0; i < 8; ++i) al[8 * half + i] = load_meta<M16>(ap, c0 % AL + i);
  }
  float mz[KCH ? 16 : 1];   // KCH: the zero offsets of the lane's channels
  if constexpr (KCH) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c0 = 64 * half + 8 * cg;
      const uint8_t* zp = pool + ((size_t)row_tab[pt0 + c0 / AL] * H + head) * SLOT + slot_chan_zp_at(BITS, T);
#pragma unroll
      for (int i = 0; i < 8; ++i) mz[8 * half + i] = load_meta<false>(zp, c0 % AL + i);
    }
  }
  const float S = load_meta<M16>(slot + CODE, t);   // KCH: beta
  const float O = KCH ? 0.f : load_meta<M16>(slot + OFF_AT, t);
  float x[16];
  if (!VL) {
    // unit order: channel 64 half + 8 cg + j is field 4 half + (cg >> 1) of unit
    // 8 (cg & 1) + j; block b of token t at 4 BITS (16 b + t)
    unsigned units[8], units8_hi[8];   // at 8 bits a unit is two words (fields 0..3, 4..7)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const uint8_t* bp = slot + (16 * (2 * (cg & 1) + bb) + t) * 4 * BITS;
      if (BITS == 8) {
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(bp + 16 * v2);
          units[4 * bb + 2 * v2] = w[0];
          units8_hi[4 * bb + 2 * v2] = w[1];
          units[4 * bb + 2 * v2 + 1] = w[2];
          units8_hi[4 * bb + 2 * v2 + 1] = w[3];
        }
      } else if (BITS == 4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(bp);
#pragma unroll
        for (int i = 0; i < 4; ++i) units[4 * bb + i] = w[i];
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(bp);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          units[4 * bb + 2 * i] = w[i] & 0xFFFFu;
          units[4 * bb + 2 * i + 1] = w[i] >> 16;
        }
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int m = 4 * half + (cg >> 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned u = (BITS == 8 && m >= 4) ? units8_hi[j] : units[j];
        const int mm = (BITS == 8) ? (m & 3) : m;
        const float code = (float)((u >> (BITS * mm)) & MASK);
        if constexpr (KCH) x[8 * half + j] = al[8 * half + j] * S * (code + mz[KCH ? 8 * half + j : 0]);
        else x[8 * half + j] = al[8 * half + j] * __builtin_fmaf(S, code, O);
      }
    }
  } else {
    // runs: run l = 8 cg + j holds channels l (h = 0) and 64 + l (h = 1); token
    // t = 4g + r of half h is pair p = 2g + h: word p / (F/4), field
    // 2 (p mod F/4) + (r >> 1) + (F/2)(r & 1)
    constexpr int F = 32 / BITS;
    const int g = t >> 2, r = t & 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int l = 8 * cg + j;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = 2 * g + h;
        const unsigned w = *reinterpret_cast<const uint32_t*>(slot + 4 * BITS * l + 4 * (p / (F / 4)));
        const int f = 2 * (p % (F / 4)) + (r >> 1) + (F / 2) * (r & 1);
        x[8 * h + j] = al[8 * h + j] * __builtin_fmaf(S, (float)((w >> (BITS * f)) & MASK), O);
      }
    }
  }
#pragma unroll
  for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k & bit) continue;
      const float lo = x[k], hi = x[k | bit];
      x[k] = lo + hi;
      x[k | bit] = lo - hi;
    }
#pragma unroll
  for (int k = 0; k < 8; ++k) {   // channel bit 6: the two halves
    const float lo = x[k], hi = x[k + 8];
    x[k] = lo + hi;
    x[k + 8] = lo - hi;
  }
  const float s1 = (cg & 1) ? -1.f : 1.f, s2 = (cg & 2) ? -1.f : 1.f, s4 = (cg & 4) ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], s1, lane_xor<1>(x[k]));
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], s2, lane_xor<2>(x[k]));
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], s4, lane_xor<4>(x[k]));
  if (any_sign(A.signs)) {   // randomized rotation: the restore ends with the signs
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c0 = 64 * half + 8 * cg;
      const unsigned b = (sign_word(A.signs, c0 >> 5) >> (c0 & 31)) & 0xFFu;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[8 * half + j] = ((b >> j) & 1u) ? -x[8 * half + j] : x[8 * half + j];
    }
  }
  uint16_t hv[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) hv[k] = (t < n) ? float_to_half_bits(x[k] * kInvSqrtD) : (uint16_t)0;
  const size_t page = ((size_t)pid * H + head) * (kPage * kHeadDim);
  if (!VL) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (unsigned)hv[8 * half + 2 * i] | ((unsigned)hv[8 * half + 2 * i + 1] << 16);
      *reinterpret_cast<u32x4*>(A.base_k + page + t * kHeadDim + 64 * half + 8 * cg) = w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) vt[64 * (k >> 3) + 8 * cg + (k & 7)][t] = hv[k];
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {   // 256 chunks of 8 tokens of one channel
      const int i = tid + 128 * it, c = i >> 1, t0 = 8 * (i & 1);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (unsigned)vt[c][t0 + 2 * e] | ((unsigned)vt[c][t0 + 2 * e + 1] << 16);
      *reinterpret_cast<u32x4*>(A.base_v + page + c * kPage + t0) = w;
    }
  }
}

// grid: x = page of the sequence, y = head + Hkv * role (0 K, 1 V), z = sequence
template <int T, int BK, int BV, bool M16, bool KCH>
__global__ __launch_bounds__(128) void rematerialize_kernel(RematArgs A) {
  __shared__ uint16_t vt[kHeadDim][kPage + 2];
  const int seq = blockIdx.z, pj = blockIdx.x;
  const int role = blockIdx.y / A.kv_heads, head = blockIdx.y % A.kv_heads;
  const int L = A.seq_lens[seq];
  if (pj * kPage >= L) return;   // uniform over the workgroup
  const int n = min(kPage, L - pj * kPage);
  if (role == 0) restore_page<T, BK, false, M16, KCH>(A, seq, pj, head, n, vt);
  else restore_page<T, BV, true, M16>(A, seq, pj, head, n, vt);
}

// ---------------------------------------------------------------- bandwidth probe
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (; i < n; i += stride) dst[i] = __builtin_nontemporal_load(&src[i]);
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
    case 8: return f(std::integral_constant<int, 8>{});
  }
  return hipErrorInvalidValue;
}

// Slot formats: K and V code widths 2 and 4 in any pairing, 8 for both; fp16
// metadata (M16) with 2 and 4 only.
template <typename F>
hipError_t by_format(int bits_k, int bits_v, int fmt, F&& f) {
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using B0 = std::integral_constant<bool, false>;
  using B1 = std::integral_constant<bool, true>;
  if (fmt == kFmtFp32) {
    if (bits_k == 8 && bits_v == 8) return f(I8{}, I8{}, B0{}, B0{});
    if (bits_k == 4 && bits_v == 4) return f(I4{}, I4{}, B0{}, B0{});
    if (bits_k == 4 && bits_v == 2) return f(I4{}, I2{}, B0{}, B0{});
    if (bits_k == 2 && bits_v == 4) return f(I2{}, I4{}, B0{}, B0{});
    if (bits_k == 2 && bits_v == 2) return f(I2{}, I2{}, B0{}, B0{});
  } else if (fmt == kFmtM16) {
    if (bits_k == 4 && bits_v == 4) return f(I4{}, I4{}, B1{}, B0{});
    if (bits_k == 4 && bits_v == 2) return f(I4{}, I2{}, B1{}, B0{});
    if (bits_k == 2 && bits_v == 4) return f(I2{}, I4{}, B1{}, B0{});
    if (bits_k == 2 && bits_v == 2) return f(I2{}, I2{}, B1{}, B0{});
  } else if (fmt == kFmtKch) {
    if (bits_k == 4 && bits_v == 4) return f(I4{}, I4{}, B0{}, B1{});
    if (bits_k == 4 && bits_v == 2) return f(I4{}, I2{}, B0{}, B1{});
    if (bits_k == 2 && bits_v == 4) return f(I2{}, I4{}, B0{}, B1{});
    if (bits_k == 2 && bits_v == 2) return f(I2{}, I2{}, B0{}, B1{});
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize_dense(const QuantArgs& a, int tile, int bits, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_bits(bits, [&](auto B) {
      dim3 grid((a.n_tokens + T() - 1) / T(), a.heads);
      hipLaunchKernelGGL((quantize_dense_kernel<T(), B()>), grid, dim3(2 * T()), 0, s, a);
      const int tail = a.n_tokens % T();
      if (tail > 0 && tail < kShortTile)
        hipLaunchKernelGGL((quantize_dense_short_kernel<T(), B()>), dim3(a.heads), dim3(2 * T()), 0, s, a);
      return hipGetLastError();
    });
  });
}

hipError_t launch_quantize_paged(const QuantArgs& a, int tile, int bits_k, int bits_v, int fmt,
                                 int num_seqs, int total_tokens, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format(bits_k, bits_v, fmt, [&](auto BK, auto BV, auto M, auto KC) {
      dim3 grid(total_tokens / T() + num_seqs, 2 * a.kv_heads);
      hipLaunchKernelGGL((quantize_paged_kernel<T(), BK(), BV(), M(), KC()>), grid, dim3(2 * T()), 0, s, a);
      hipLaunchKernelGGL((quantize_paged_short_kernel<T(), BK(), BV(), M(), KC()>), dim3(2 * a.kv_heads, num_seqs),
                         dim3(2 * T()), 0, s, a);
      return hipGetLastError();
    });
  });
}

hipError_t launch_append(const QuantArgs& a, int tile, int bits_k, int bits_v, int fmt, int num_seqs,
                         hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format(bits_k, bits_v, fmt, [&](auto BK, auto BV, auto M, auto KC) {
      dim3 grid(a.kv_heads, 2, num_seqs);
      hipLaunchKernelGGL((append_kernel<T(), BK(), BV(), M(), KC()>), grid, dim3(2 * T()), 0, s, a);
      return hipGetLastError();
    });
  });
}

hipError_t launch_dequantize(const DequantArgs& a, int tile, int bits, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_bits(bits, [&](auto B) {
      const long rows = (long)a.n_tokens * a.heads;
      dim3 grid((unsigned)((rows + 15) / 16));
      hipLaunchKernelGGL((dequantize_kernel<T(), B()>), grid, dim3(128), 0, s, a);
      return hipGetLastError();
    });
  });
}

hipError_t launch_rematerialize(const RematArgs& a, int tile, int bits_k, int bits_v, int fmt, int num_seqs,
                                int max_seq_len, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_format(bits_k, bits_v, fmt, [&](auto BK, auto BV, auto M, auto KC) {
      dim3 grid((max_seq_len + kPage - 1) / kPage, 2 * a.kv_heads, num_seqs);
      hipLaunchKernelGGL((rematerialize_kernel<T(), BK(), BV(), M(), KC()>), grid, dim3(128), 0, s, a);
      return hipGetLastError();
    });
  });
}

hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(copy_kernel, dim3(256 * 16), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace kvq
