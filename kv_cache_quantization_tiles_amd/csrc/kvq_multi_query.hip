// Several queries per sequence over the quantized pages: the newest n_q
// tokens of each sequence (already in the cache) attend causally to the
// cached tokens up to their own positions, reading the compressed pages
// directly as the decode step does (aitrends.kr article 74976, TL;DR: the
// attention backend reads compressed KV pages without re-materializing fp16).
// With 16 or more (query, head) rows per sequence and kv head the rows go
// to the 16-row MFMA kernel (kvq_mq_dense.h) in blocks of up to 64, each
// block reading the partition's pages once; fewer rows run on the decode
// kernel with (query, head) rows in place of heads, in blocks of up to 8.
#include "kvq_mq_dense.h"

namespace kvq {

hipError_t launch_multi_query(const DecodeArgs& a, int tile, int bits_k, int bits_v, int fmt, hipStream_t s) {
  if (fmt == kFmtM16) return launch_multi_query_m16(a, tile, bits_k, bits_v, s);
  if (fmt == kFmtKch) return launch_multi_query_kch(a, tile, bits_k, bits_v, s);
  if (mq_dense(a.n_q, a.group)) return launch_mq_dense_fmt<kFmtFp32>(a, tile, bits_k, bits_v, s);
  return launch_multi_query_fmt<kFmtFp32>(a, tile, bits_k, bits_v, s);
}

}  // namespace kvq
