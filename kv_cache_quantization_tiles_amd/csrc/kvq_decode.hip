// Launchers of the quantized-page decode attention (the kernel itself is in
// kvq_decode_kernel.h) and the kernel that merges its partitions.
#include "kvq_decode_kernel.h"

namespace kvq {
namespace {

// Merge the partitions of one (sequence, query, query head):
// out = s H (sum_p w_p acc_p) / (sum_p w_p l_p), w_p = 2^(m_p - max m), with
// the Hadamard H applied for pages quantized in the rotated basis (ROT) and
// s = A.out_scale.  One wave per row; the row's partials are read with every
// load in flight at once (16 partitions per round): lanes 32h + i take
// channels 4i..4i+3 of the partitions of parity h and keep a running maximum
// (rescaling their sums when it grows), and the two halves merge at the end.
// The Hadamard then runs over channel bits 0, 1 in registers and bits 2..6
// across the lanes.
template <bool ROT>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs A) {
  constexpr int U = 8;   // float4 loads in flight per lane and round
  const int lane = threadIdx.x, half = lane >> 5, c4 = lane & 31;
  const int seq = blockIdx.x / (A.q_heads * A.n_q);   // rows [S][n_q][Hq]
  const int L = A.seq_lens[seq] + A.seq_lens_plus_one;
  const int T = A.unit_tokens;
  const int ntiles = min((L + T - 1) / T, A.max_tiles);
  const int nparts = min((ntiles + A.tiles_per_part - 1) / A.tiles_per_part, A.max_parts);
  const size_t base = (size_t)blockIdx.x * A.max_parts;
  const float2* ml = reinterpret_cast<const float2*>(A.ws_ml) + base;
  const f32x4* acc = reinterpret_cast<const f32x4*>(A.ws_acc) + base * (kHeadDim / 4);
  float m = -INFINITY, den = 0.f;
  f32x4 x{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < nparts; p0 += 2 * U) {
    float2 s[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + 2 * u + half;
      const bool ok = p < nparts;
      s[u] = ok ? ml[p] : float2{-INFINITY, 0.f};
      v[u] = ok ? acc[(size_t)p * (kHeadDim / 4) + c4] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mc = fmaxf(mc, s[u].x);
    // a partition that sees no token (m = -inf) weighs 0
    const float r = (mc == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mc);
    den *= r;
    x *= r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = (s[u].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[u].x - mc);
      den = __builtin_fmaf(w, s[u].y, den);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(w, v[u][e], x[e]);
    }
    m = mc;
  }
  {   // the two halves (partitions of either parity)
    const float mm = fmaxf(m, xor32(m));
    const float r = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mm);
    den *= r;
    den += xor32(den);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] *= r;
      x[e] += xor32(x[e]);
    }
  }
  f32x4* o = reinterpret_cast<f32x4*>(A.out + (size_t)blockIdx.x * kHeadDim) + c4;
  if (!ROT) {
    const float inv = den > 0.f ? A.out_scale / den : 0.f;   // an empty sequence gives zeros
    if (half == 0) *o = x * inv;
    return;
  }
  const float inv = den > 0.f ? A.out_scale * kInvSqrtD / den : 0.f;
  // channel c = 4 c4 + e: bits 0, 1 in registers
  float y[4];
  {
    const float a0 = x[0] + x[1], a1 = x[0] - x[1], a2 = x[2] + x[3], a3 = x[2] - x[3];
    y[0] = a0 + a2;
    y[2] = a0 - a2;
    y[1] = a1 + a3;
    y[3] = a1 - a3;
  }
  // bits 2..6 across lanes c4 ^ 1 .. c4 ^ 16
  auto stage = [&](float& v, float partner, int bit) {
    v = __builtin_fmaf(v, (c4 & bit) ? -1.f : 1.f, partner);
  };
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    stage(y[e], lane_xor<1>(y[e]), 1);
    stage(y[e], lane_xor<2>(y[e]), 2);
    stage(y[e], lane_xor<4>(y[e]), 4);
    stage(y[e], lane_xor<8>(y[e]), 8);
    stage(y[e], lane_xor<16>(y[e]), 16);
  }
  // randomized rotation: the restore ends with the sign of each channel
  const unsigned sg = (sign_word(A.signs, c4 >> 3) >> (4 * (c4 & 7))) & 0xFu;
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = y[e] * (((sg >> e) & 1u) ? -inv : inv);
  if (half == 0) *o = r;
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
