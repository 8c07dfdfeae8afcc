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

hipError_t launch_multi_query(const DecodeArgs& a, int tile, int bits_k, int bits_v, bool m16, hipStream_t s) {
  if (m16) return launch_multi_query_m16(a, tile, bits_k, bits_v, s);
  return launch_multi_query_fmt<false>(a, tile, bits_k, bits_v, s);
}

}  // namespace kvq
