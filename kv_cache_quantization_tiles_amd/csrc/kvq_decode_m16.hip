// Decode launchers for slots with fp16 metadata (the kernel is in
// kvq_decode_kernel.h; a translation unit of its own so that the two
// metadata formats compile in parallel).
#include "kvq_decode_kernel.h"

namespace kvq {

hipError_t launch_decode_m16(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s) {
  return launch_decode_fmt<kFmtM16>(a, tile, bits_k, bits_v, s);
}

hipError_t launch_append_decode_m16(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                    hipStream_t s) {
  return launch_append_decode_fmt<kFmtM16>(a, q, tile, bits_k, bits_v, s);
}

}  // namespace kvq
