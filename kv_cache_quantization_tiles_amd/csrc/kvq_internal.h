// Internal declarations shared by the HIP translation units of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
// A channel (token) whose spread is at most 1e-2 of its RMS keeps factor 1:
// var > kGuard2 * meansq  <=>  std > 1e-2 * rms.
constexpr float kGuard2 = 1e-4f;
constexpr double kGuard = 1e-2;   // the same test in float64: std > kGuard * rms
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// Slot layout: codes | scale[16] | offset[16] | alpha slice[2048 / T], the
// metadata fp32 (4 bytes each) or, with fp16 metadata (M16), fp16 (2 bytes).
__host__ __device__ constexpr int slot_code_bytes(int bits) { return kPage * kHeadDim * bits / 8; }
__host__ __device__ constexpr int slot_alpha_len(int tile) { return kPage * kHeadDim / tile; }
__host__ __device__ constexpr int meta_bytes(bool m16) { return m16 ? 2 : 4; }
// K slots rounded per channel (KCH, fp32 metadata): codes | beta[16] |
// channel-scale slice A[2048 / T] | zero-offset slice M[2048 / T].
__host__ __device__ constexpr int slot_bytes(int bits, int tile, bool m16 = false, bool kch = false) {
  return kch ? slot_code_bytes(bits) + 4 * kPage + 8 * slot_alpha_len(tile)
             : slot_code_bytes(bits) + meta_bytes(m16) * (2 * kPage + slot_alpha_len(tile));
}
__host__ __device__ constexpr int slot_chan_scale_at(int bits) { return slot_code_bytes(bits) + 4 * kPage; }
__host__ __device__ constexpr int slot_chan_zp_at(int bits, int tile) {
  return slot_code_bytes(bits) + 4 * kPage + 4 * slot_alpha_len(tile);
}
__host__ __device__ constexpr int slot_offset_at(int bits, bool m16) {   // byte of offset[0]
  return slot_code_bytes(bits) + meta_bytes(m16) * kPage;
}
__host__ __device__ constexpr int slot_alpha_at(int bits, bool m16) {    // byte of alpha slice[0]
  return slot_code_bytes(bits) + meta_bytes(m16) * 2 * kPage;
}

// Arguments of the tile-quantizer kernels (dense, paged prefill, append).
struct QuantArgs {
  // dense layout
  const uint16_t* x;
  uint8_t* codes;
  float* alpha;
  float* scale;
  float* offset;
  int n_tokens;
  int heads;
  // paged layouts: index 0 = K, 1 = V
  const uint16_t* src[2];     // prefill rows [total][Hkv][D] or new rows [S][Hkv][D]
  uint8_t* pool[2];
  uint16_t* staging[2];       // [S][T][Hkv][D] or null
  const int32_t* cu_seqlens;  // prefill
  int num_seqs;               // prefill: sequences in cu_seqlens
  const int32_t* lens_before; // append
  const int32_t* block_table;
  int max_blocks;
  int kv_heads;
  int iters;
  uint32_t signs[4];          // randomized rotation (bit c = channel c negated); all 0 = plain
};

struct DequantArgs {
  const uint8_t* codes;
  const float* alpha;
  const float* scale;
  const float* offset;
  int n_tokens;
  int heads;
  uint16_t* out;
  uint32_t signs[4];
};

struct DecodeArgs {
  const uint16_t* q;          // [S][Hq][D]
  const int32_t* block_table; // [S][max_blocks]
  const int32_t* seq_lens;    // [S]
  const uint8_t* pool_k;
  const uint8_t* pool_v;
  float* out;                 // [S][Hq][D]
  float* ws_acc;              // [S][Hq][P][D]
  float* ws_ml;               // [S][Hq][P][2]
  int num_seqs;
  int q_heads;
  int kv_heads;
  int group;
  int max_blocks;
  int tiles_per_part;
  int max_parts;
  int max_tiles;               // ceil(max_seq_len / T): no tile past it is read
  float sm_scale_log2;        // sm_scale * log2(e) (times the K scale for fp8 pages)
  int unit_tokens;            // tokens per partition unit (tile, or 64 for the baselines)
  float out_scale;            // output multiplier (the V scale for fp8 pages, else 1)
  int seq_lens_plus_one;      // 1: seq_lens are the lengths before an appended token
  int n_q;                    // queries per sequence (1 for a decode step); q, out: [S][n_q][Hq][D]
  uint32_t signs[4];          // randomized rotation of the quantized pages (0 for the baselines)
};

struct BaseFillArgs {
  const uint16_t* k;          // [total][Hkv][D] fp16
  const uint16_t* v;
  const int32_t* cu_seqlens;
  const int32_t* block_table;
  int max_blocks;
  int kv_heads;
  uint8_t* pool_k;            // [pages][Hkv][16][D] fp16 or E4M3
  uint8_t* pool_v;            // [pages][Hkv][D][16]
  float k_scale;
  float v_scale;
};

struct RematArgs {
  const uint8_t* pool_k;      // quantized page pools
  const uint8_t* pool_v;
  const int32_t* block_table; // [S][max_blocks]
  int max_blocks;
  const int32_t* seq_lens;    // [S]
  int kv_heads;
  uint16_t* base_k;           // fp16 pools: K [pages][Hkv][16][D], V [pages][Hkv][D][16]
  uint16_t* base_v;
  uint32_t signs[4];
};

// Slot formats of the paged pools: fp32 metadata, fp16 metadata, or K slots
// rounded per channel (fp32 metadata; V as with kFmtFp32).
constexpr int kFmtFp32 = 0, kFmtM16 = 1, kFmtKch = 2;

hipError_t launch_quantize_dense(const QuantArgs& a, int tile, int bits, hipStream_t s);
hipError_t launch_quantize_paged(const QuantArgs& a, int tile, int bits_k, int bits_v, int fmt,
                                 int num_seqs, int total_tokens, hipStream_t s);
hipError_t launch_append(const QuantArgs& a, int tile, int bits_k, int bits_v, int fmt, int num_seqs,
                         hipStream_t s);
hipError_t launch_dequantize(const DequantArgs& a, int tile, int bits, hipStream_t s);
hipError_t launch_rematerialize(const RematArgs& a, int tile, int bits_k, int bits_v, int fmt, int num_seqs,
                                int max_seq_len, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int tile, int bits_k, int bits_v, int fmt, hipStream_t s);
hipError_t launch_decode_m16(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s);
hipError_t launch_decode_kch(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s);
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_combine(const DecodeArgs& a, int unit_tokens, bool rotate, hipStream_t s);
// Several queries per sequence: with at least 16 (query, head) rows per
// sequence and kv head the 16-row MFMA kernel takes them in blocks of up to
// 64 rows; fewer rows (and one query, which must equal the decode step bit
// for bit) run on the decode kernel in blocks of up to 8.
inline bool mq_dense(int n_q, int group) { return n_q > 1 && (long)n_q * group >= 16; }
inline int mq_row_blocks(int n_q, int group) {
  const long rows = (long)n_q * group;
  return (int)(mq_dense(n_q, group) ? (rows + 63) / 64 : (rows + 7) / 8);
}
hipError_t launch_multi_query(const DecodeArgs& a, int tile, int bits_k, int bits_v, int fmt, hipStream_t s);
hipError_t launch_multi_query_m16(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s);
hipError_t launch_multi_query_kch(const DecodeArgs& a, int tile, int bits_k, int bits_v, hipStream_t s);
hipError_t launch_append_decode(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                int fmt, hipStream_t s);
hipError_t launch_append_decode_m16(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                    hipStream_t s);
hipError_t launch_append_decode_kch(const DecodeArgs& a, const QuantArgs& q, int tile, int bits_k, int bits_v,
                                    hipStream_t s);
hipError_t launch_fill_baseline(const BaseFillArgs& a, bool fp8, int num_seqs, int max_seq_len, hipStream_t s);
hipError_t launch_decode_baseline(const DecodeArgs& a, bool fp8, hipStream_t s);
hipError_t launch_append_baseline(const BaseFillArgs& a, const int32_t* lens_before, bool fp8, int num_seqs,
                                  hipStream_t s);

// ---------------------------------------------------------------- device helpers

// Sign flips of the randomized rotation: the 8 sign bits of channels c0..c0+7
// (c0 a multiple of 8) spread to the fp16 sign bits of 4 words of fp16 pairs
// (channel c0 + 2w in the low half of word w, c0 + 2w + 1 in the high half).
__device__ __forceinline__ unsigned sign_pair_mask(const uint32_t* signs, int c0, int w) {
  const unsigned b = (signs[c0 >> 5] >> (c0 & 31)) & 0xFFu;
  return ((b << (15 - 2 * w)) & 0x8000u) | ((b << (30 - 2 * w)) & 0x80000000u);
}
// The sign word of channels 32 k .. 32 k + 31 for a k (< 4) that varies by
// lane, as selects among the four words (indexing the argument array by a
// lane value would read it from memory), and sign_pair_mask of a word.
__device__ __forceinline__ unsigned sign_word(const uint32_t (&signs)[4], int k) {
  const unsigned lo = (k & 1) ? signs[1] : signs[0];
  const unsigned hi = (k & 1) ? signs[3] : signs[2];
  return (k & 2) ? hi : lo;
}
__device__ __forceinline__ unsigned sign_pair_mask_w(unsigned word, int bit0, int w) {
  const unsigned b = (word >> bit0) & 0xFFu;
  return ((b << (15 - 2 * w)) & 0x8000u) | ((b << (30 - 2 * w)) & 0x80000000u);
}
__device__ __forceinline__ bool any_sign(const uint32_t* signs) {
  return (signs[0] | signs[1] | signs[2] | signs[3]) != 0u;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  _Float16 f;
  __builtin_memcpy(&f, &h, 2);
  return (float)f;
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
  _Float16 f = (_Float16)x;  // round to nearest even
  uint16_t h;
  __builtin_memcpy(&h, &f, 2);
  return h;
}

// One metadata value (scale, offset or channel factor) at element i of an
// array starting at byte pointer p: fp32, or fp16 with M16 (read as fp32).
template <bool M16>
__device__ __forceinline__ float load_meta(const uint8_t* p, int i) {
  if constexpr (M16) return half_bits_to_float(__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p) + i));
  else return __builtin_nontemporal_load(reinterpret_cast<const float*>(p) + i);
}
template <bool M16>
__device__ __forceinline__ void store_meta(uint8_t* p, int i, float v) {
  if constexpr (M16) reinterpret_cast<uint16_t*>(p)[i] = float_to_half_bits(v);
  else reinterpret_cast<float*>(p)[i] = v;
}

// fp16 metadata keep one power of two per tile out of the scales and offsets:
// with M the largest |S|, |O| of the tile's tokens, e = floor(log2 M) - 10
// (0 for M = 0 or not normal); S and O are stored times 2^-e and the channel
// factors times 2^e (their products, all the restore uses, are unchanged).
__device__ __forceinline__ int meta_exponent(float m) {
  const int ex = (int)((__float_as_uint(m) >> 23) & 0xFFu);
  return (ex == 0 || ex == 0xFF) ? 0 : ex - 127 - 10;
}
__device__ __forceinline__ float pow2f(int e) {   // 2^e for |e| < 127
  return __uint_as_float((unsigned)(127 + e) << 23);
}

// Value of lane (lane ^ M) for M in {1, 2, 4, 8, 16} (ds_swizzle bit mode,
// within each group of 32 lanes).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16, "xor within 32 lanes");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}


}  // namespace kvq
