// Launchers of the quantized-page decode attention (the kernel itself is in
// kvq_decode_kernel.h) and the kernel that merges its partitions.
#include "kvq_decode_kernel.h"

namespace kvq {
namespace {

// Merge the partitions of one (sequence, query, query head):
// out = s H (sum_p w_p acc_p) / (sum_p w_p l_p), w_p = 2^(m_p - max m), with
// the Hadamard H applied for pages quantized in the rotated basis (ROT) and
// s = A.out_scale.
template <bool ROT>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs A) {
  __shared__ float wts[1024];
  const int lane = threadIdx.x;
  const int seq = blockIdx.x / (A.q_heads * A.n_q);   // rows [S][n_q][Hq]
  const int L = A.seq_lens[seq] + A.seq_lens_plus_one;
  const int T = A.unit_tokens;
  const int ntiles = min((L + T - 1) / T, A.max_tiles);
  const int nparts = min((ntiles + A.tiles_per_part - 1) / A.tiles_per_part, A.max_parts);
  const size_t base = (size_t)blockIdx.x * A.max_parts;
  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, A.ws_ml[2 * (base + p)]);
  M = wave_max(M);
  float den = 0.f;
  for (int p = lane; p < nparts; p += 64) {
    // a row that sees no token at all (M = -inf) gets zeros
    const float w = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(A.ws_ml[2 * (base + p)] - M);
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
  // randomized rotation: the restore ends with the sign of each channel
  const float s0 = ((A.signs[lane >> 5] >> (lane & 31)) & 1u) ? -inv : inv;
  const float s1 = ((A.signs[2 + (lane >> 5)] >> (lane & 31)) & 1u) ? -inv : inv;
  o[lane] = y0 * s0;
  o[lane + 64] = y1 * s1;
}

}  // namespace


hipError_t launch_combine(const DecodeArgs& a, int unit_tokens, bool rotate, hipStream_t s) {
  DecodeArgs b = a;
  b.unit_tokens = unit_tokens;
  if (rotate) hipLaunchKernelGGL(combine_kernel<true>, dim3(a.num_seqs * a.n_q * a.q_heads), dim3(64), 0, s, b);
  else hipLaunchKernelGGL(combine_kernel<false>, dim3(a.num_seqs * a.n_q * a.q_heads), dim3(64), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int tile, int bits_k, int bits_v, int fmt, hipStream_t s) {
  if (fmt == kFmtM16) return launch_decode_m16(a, tile, bits_k, bits_v, s);
  if (fmt == kFmtKch) return launch_decode_kch(a, tile, bits_k, bits_v, s);
  return launch_decode_fmt<kFmtFp32>(a, tile, bits_k, bits_v, s);
}

hipError_t launch_append_decode(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                int fmt, hipStream_t s) {
  if (fmt == kFmtM16) return launch_append_decode_m16(a, q, tile, bits_k, bits_v, s);
  if (fmt == kFmtKch) return launch_append_decode_kch(a, q, tile, bits_k, bits_v, s);
  return launch_append_decode_fmt<kFmtFp32>(a, q, tile, bits_k, bits_v, s);
}

}  // namespace kvq
