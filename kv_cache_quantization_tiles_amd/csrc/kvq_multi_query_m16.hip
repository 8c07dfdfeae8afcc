// Multi-query launcher for slots with fp16 metadata (see kvq_multi_query.hip;
// a translation unit of its own so that the two formats compile in parallel).
#include "kvq_mq_dense.h"

namespace kvq {

hipError_t launch_multi_query_m16(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  if (mq_dense(a.n_q, a.group)) return launch_mq_dense_fmt<kFmtM16>(a, tile, bits_k, bits_v, s);
  return launch_multi_query_fmt<kFmtM16>(a, tile, bits_k, bits_v, s);
}

}  // namespace kvq
