// Several queries per sequence over the quantized pages: the newest n_q
// tokens of each sequence (already in the cache) attend causally to the
// cached tokens up to their own positions, reading the compressed pages
// directly as the decode step does (aitrends.kr article 74976, TL;DR: the
// attention backend reads compressed KV pages without re-materializing fp16).
// It is the decode kernel with (query, head) rows in place of heads; rows come
// in blocks of up to 8 per workgroup, and every block reads the partition's
// pages (a block's re-read of the same pages is served mostly from cache).
#include "kvq_decode_kernel.h"

namespace kvq {

hipError_t launch_multi_query(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return by_tile(tile, [&](auto T) {
    return by_bits_pair(bits_k, bits_v, [&](auto BK, auto BV) {
      const int rows = a.n_q * a.group;
      const QuantArgs q{};
      // rows beyond 8 run in blocks of 8 (two groups of 4 heads); blocks of
      // 16 read the pages once but measured slower (a 4-token verify at
      // 4 x 16K, 8 kv / 32 query heads: 97 us against 67 us), as did blocks
      // of 4 (88 us)
      if (rows <= 4) {
        dim3 grid(a.kv_heads * a.num_seqs, a.max_parts);
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 1, false, true>), grid, dim3(64 * kWaves), 0, s, a, q);
      } else {
        dim3 grid(a.kv_heads * ((rows + 7) / 8) * a.num_seqs, a.max_parts);
        hipLaunchKernelGGL((decode_kernel<T(), BK(), BV(), 2, false, true>), grid, dim3(64 * kWaves), 0, s, a, q);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_combine(a, 64, true, s);
    });
  });
}

}  // namespace kvq
