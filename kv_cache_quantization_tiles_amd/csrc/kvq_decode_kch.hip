// Decode, fused append + decode and multi-query launchers for K slots rounded
// per channel (the kernels are in kvq_decode_kernel.h and kvq_mq_dense.h; a
// translation unit of its own so that the slot formats compile in parallel).
#include "kvq_mq_dense.h"

namespace kvq {

hipError_t launch_decode_kch(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return launch_decode_fmt<kFmtKch>(a, tile, bits_k, bits_v, s);
}

hipError_t launch_append_decode_kch(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                    hipStream_t s) {
  return launch_append_decode_fmt<kFmtKch>(a, q, tile, bits_k, bits_v, s);
}

hipError_t launch_multi_query_kch(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  if (mq_dense(a.n_q, a.group)) return launch_mq_dense_fmt<kFmtKch>(a, tile, bits_k, bits_v, s);
  return launch_multi_query_fmt<kFmtKch>(a, tile, bits_k, bits_v, s);
}

}  // namespace kvq
