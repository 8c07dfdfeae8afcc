// C ABI of libkvq: host-side validation, then kernel launches on the
// caller's stream.  See include/kvq.h for the contract of every function.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kvq_status check_config(const kvq_config* cfg, bool need_paged_bits) {
  if (cfg == nullptr) return fail(KVQ_ERR_ARG, "cfg is NULL");
  if (cfg->head_dim != kvq::kHeadDim)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d unsupported (must be 128)", cfg->head_dim);
  if (cfg->page_tokens != kvq::kPage)
    return fail(KVQ_ERR_UNSUPPORTED, "page_tokens %d unsupported (must be 16)", cfg->page_tokens);
  if (cfg->tile_tokens != 32 && cfg->tile_tokens != 64 && cfg->tile_tokens != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "tile_tokens %d unsupported (32, 64 or 128)", cfg->tile_tokens);
  if (cfg->sinkhorn_iters < 0 || cfg->sinkhorn_iters > 16)
    return fail(KVQ_ERR_UNSUPPORTED, "sinkhorn_iters %d outside 0..16", cfg->sinkhorn_iters);
  if (need_paged_bits) {
    if (cfg->bits_k != 2 && cfg->bits_k != 4 && cfg->bits_k != 8)
      return fail(KVQ_ERR_UNSUPPORTED, "bits_k %d unsupported (2, 4 or 8)", cfg->bits_k);
    if (cfg->bits_v != 2 && cfg->bits_v != 4 && cfg->bits_v != 8)
      return fail(KVQ_ERR_UNSUPPORTED, "bits_v %d unsupported (2, 4 or 8)", cfg->bits_v);
    if ((cfg->bits_k == 8) != (cfg->bits_v == 8))
      return fail(KVQ_ERR_UNSUPPORTED, "8-bit codes need bits_k == bits_v == 8 (got %d, %d)", cfg->bits_k,
                  cfg->bits_v);
  }
  if (cfg->meta_fp16 != 0 && cfg->meta_fp16 != 1)
    return fail(KVQ_ERR_ARG, "meta_fp16 must be 0 or 1 (got %d)", cfg->meta_fp16);
  if (need_paged_bits && cfg->meta_fp16 && (cfg->bits_k == 8 || cfg->bits_v == 8))
    return fail(KVQ_ERR_UNSUPPORTED, "fp16 metadata slots take 2- and 4-bit codes only");
  if (cfg->k_per_channel != 0 && cfg->k_per_channel != 1)
    return fail(KVQ_ERR_ARG, "k_per_channel must be 0 or 1 (got %d)", cfg->k_per_channel);
  if (cfg->k_per_channel) {
    if (!need_paged_bits)
      return fail(KVQ_ERR_UNSUPPORTED, "per-channel K rounding is a page-pool format (paged entry points only)");
    if (cfg->meta_fp16) return fail(KVQ_ERR_UNSUPPORTED, "per-channel K slots keep fp32 metadata");
    if (cfg->bits_k == 8 || cfg->bits_v == 8)
      return fail(KVQ_ERR_UNSUPPORTED, "per-channel K slots take 2- and 4-bit codes only");
  }
  return KVQ_OK;
}

// The slot format of the paged pools for this configuration.
int slot_format(const kvq_config* cfg) {
  return cfg->k_per_channel ? kvq::kFmtKch : (cfg->meta_fp16 ? kvq::kFmtM16 : kvq::kFmtFp32);
}

kvq_status check_bits(int bits) {
  if (bits != 2 && bits != 4 && bits != 8)
    return fail(KVQ_ERR_UNSUPPORTED, "bits %d unsupported (2, 4 or 8)", bits);
  return KVQ_OK;
}

kvq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return KVQ_OK;
}

#define KVQ_TRY(x)                 \
  do {                             \
    kvq_status st_ = (x);          \
    if (st_ != KVQ_OK) return st_; \
  } while (0)

#define KVQ_NONNULL(p) \
  if ((p) == nullptr) return fail(KVQ_ERR_ARG, "%s is NULL", #p)

// Split of the context into partitions of tiles for the decode kernel (one
// workgroup of 4 waves each): about two workgroups per CU over the whole grid,
// 4..64 tiles per partition, and at most 1024 partitions per sequence.
int tiles_per_partition(int num_seqs, int kv_heads, int max_seq_len, int tile) {
  const long tiles = (long)((max_seq_len + tile - 1) / tile);
  const long total = tiles * num_seqs * kv_heads;
  long tpp = (total + 511) / 512;
  if (tpp < 4) tpp = 4;
  if (tpp > 64) tpp = 64;
  if (tpp < (tiles + 1023) / 1024) tpp = (tiles + 1023) / 1024;  // > 64 only past 65536 tiles
  if (tpp > tiles) tpp = tiles > 0 ? tiles : 1;
  return (int)tpp;
}

int max_partitions(int max_seq_len, int tile, int tpp) {
  const int tiles = (max_seq_len + tile - 1) / tile;
  return (tiles + tpp - 1) / tpp;
}

// The quantized decode splits the context into 64-token chunks; a partition
// holds whole tiles (an even number of chunks at tile 128).
int chunks_per_partition(int num_seqs, int kv_heads, int max_seq_len, int tile) {
  int cpp = tiles_per_partition(num_seqs, kv_heads, max_seq_len, 64);
  if (tile == 128 && (cpp & 1)) ++cpp;
  return cpp;
}

// The randomized rotation's sign mask travels with every launch on quantized pages.
template <class Args>
void set_signs(Args& a, const kvq_config* cfg) {
  for (int i = 0; i < 4; ++i) a.signs[i] = cfg->hadamard_signs[i];
}

// Static scratch of kvq_append_and_decode_noalloc: the decode's partition
// partials ([S][Hq][P][128] accumulators, then [S][Hq][P][2] (max, sum)),
// for callers that cannot allocate.  Every GPU the library runs on holds its
// own copy (KVQ_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code
// `scratch` is only a stand-in for the device array: its device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and only that address is passed to kernels.  Nothing in it needs to start
// at zero (the merge reads exactly the partitions the decode wrote), and
// calls that overlap on one GPU race on it.
__device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

kvq_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(KVQ_ERR_ARG, "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" {

const char* kvq_last_error(void) { return g_err; }

const char* kvq_version(void) { return "kvq 0.1 gfx950"; }

size_t kvq_slot_bytes(const kvq_config* cfg, int32_t is_v) {
  if (check_config(cfg, true) != KVQ_OK) return 0;
  return (size_t)kvq::slot_bytes(is_v ? cfg->bits_v : cfg->bits_k, cfg->tile_tokens, cfg->meta_fp16 != 0,
                                 !is_v && cfg->k_per_channel != 0);
}

kvq_status kvq_quantize_tiles(const kvq_config* cfg, const kvq_half* x, int32_t n_tokens,
                              int32_t heads, int32_t bits, uint8_t* codes, float* alpha,
                              float* tok_scale, float* tok_offset, void* stream) {
  KVQ_TRY(check_config(cfg, false));
  KVQ_TRY(check_bits(bits));
  KVQ_NONNULL(x);
  KVQ_NONNULL(codes);
  KVQ_NONNULL(alpha);
  KVQ_NONNULL(tok_scale);
  KVQ_NONNULL(tok_offset);
  if (n_tokens <= 0 || heads <= 0) return fail(KVQ_ERR_ARG, "n_tokens %d and heads %d must be > 0", n_tokens, heads);
  if ((long)((n_tokens + cfg->tile_tokens - 1) / cfg->tile_tokens) > 2147483647L || heads > 65535)
    return fail(KVQ_ERR_ARG, "too many tiles or heads for one launch");
  kvq::QuantArgs a{};
  a.x = x;
  a.codes = codes;
  a.alpha = alpha;
  a.scale = tok_scale;
  a.offset = tok_offset;
  a.n_tokens = n_tokens;
  a.heads = heads;
  a.iters = cfg->sinkhorn_iters;
  set_signs(a, cfg);
  return launched(kvq::launch_quantize_dense(a, cfg->tile_tokens, bits, (hipStream_t)stream),
                  "kvq_quantize_tiles");
}

kvq_status kvq_dequantize(const kvq_config* cfg, const uint8_t* codes, const float* alpha,
                          const float* tok_scale, const float* tok_offset, int32_t n_tokens,
                          int32_t heads, int32_t bits, kvq_half* out, void* stream) {
  KVQ_TRY(check_config(cfg, false));
  KVQ_TRY(check_bits(bits));
  KVQ_NONNULL(codes);
  KVQ_NONNULL(alpha);
  KVQ_NONNULL(tok_scale);
  KVQ_NONNULL(tok_offset);
  KVQ_NONNULL(out);
  if (n_tokens <= 0 || heads <= 0) return fail(KVQ_ERR_ARG, "n_tokens %d and heads %d must be > 0", n_tokens, heads);
  kvq::DequantArgs a{codes, alpha, tok_scale, tok_offset, n_tokens, heads, out};
  set_signs(a, cfg);
  return launched(kvq::launch_dequantize(a, cfg->tile_tokens, bits, (hipStream_t)stream), "kvq_dequantize");
}

kvq_status kvq_quantize_to_pages(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t kv_heads,
                                 const int32_t* block_table, int32_t max_blocks, void* pool_k,
                                 void* pool_v, kvq_half* staging_k, kvq_half* staging_v,
                                 void* stream) {
  KVQ_TRY(check_config(cfg, true));
  KVQ_NONNULL(k);
  KVQ_NONNULL(v);
  KVQ_NONNULL(cu_seqlens);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  if ((staging_k == nullptr) != (staging_v == nullptr))
    return fail(KVQ_ERR_ARG, "staging_k and staging_v must both be set or both be NULL");
  if (num_seqs <= 0 || kv_heads <= 0 || total_tokens <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, kv_heads, total_tokens and max_blocks must be > 0");
  if (2 * kv_heads > 65535 || num_seqs > 65535) return fail(KVQ_ERR_ARG, "too many heads or sequences");
  const int tile = cfg->tile_tokens;
  if (max_blocks < tile / kvq::kPage)
    return fail(KVQ_ERR_ARG, "max_blocks %d is smaller than one tile", max_blocks);
  kvq::QuantArgs a{};
  a.src[0] = k;
  a.src[1] = v;
  a.pool[0] = (uint8_t*)pool_k;
  a.pool[1] = (uint8_t*)pool_v;
  a.staging[0] = staging_k;
  a.staging[1] = staging_v;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.kv_heads = kv_heads;
  a.iters = cfg->sinkhorn_iters;
  set_signs(a, cfg);
  return launched(kvq::launch_quantize_paged(a, tile, cfg->bits_k, cfg->bits_v, slot_format(cfg), num_seqs, total_tokens,
                                             (hipStream_t)stream),
                  "kvq_quantize_to_pages");
}

kvq_status kvq_append_and_requant(const kvq_config* cfg, const kvq_half* k_new,
                                  const kvq_half* v_new, const int32_t* seq_lens_before,
                                  int32_t num_seqs, int32_t kv_heads, kvq_half* staging_k,
                                  kvq_half* staging_v, const int32_t* block_table,
                                  int32_t max_blocks, void* pool_k, void* pool_v, void* stream) {
  KVQ_TRY(check_config(cfg, true));
  KVQ_NONNULL(k_new);
  KVQ_NONNULL(v_new);
  KVQ_NONNULL(seq_lens_before);
  KVQ_NONNULL(staging_k);
  KVQ_NONNULL(staging_v);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  if (num_seqs <= 0 || kv_heads <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, kv_heads and max_blocks must be > 0");
  if (kv_heads > 65535 || num_seqs > 65535) return fail(KVQ_ERR_ARG, "too many heads or sequences");
  if (max_blocks < cfg->tile_tokens / kvq::kPage)
    return fail(KVQ_ERR_ARG, "max_blocks %d is smaller than one tile", max_blocks);
  kvq::QuantArgs a{};
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.pool[0] = (uint8_t*)pool_k;
  a.pool[1] = (uint8_t*)pool_v;
  a.staging[0] = staging_k;
  a.staging[1] = staging_v;
  a.lens_before = seq_lens_before;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.kv_heads = kv_heads;
  a.iters = cfg->sinkhorn_iters;
  set_signs(a, cfg);
  return launched(kvq::launch_append(a, cfg->tile_tokens, cfg->bits_k, cfg->bits_v, slot_format(cfg), num_seqs,
                                     (hipStream_t)stream),
                  "kvq_append_and_requant");
}

size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t num_seqs, int32_t q_heads,
                                  int32_t kv_heads, int32_t max_seq_len) {
  if (check_config(cfg, true) != KVQ_OK) return 0;
  if (num_seqs <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0) return 0;
  const int cpp = chunks_per_partition(num_seqs, kv_heads, max_seq_len, cfg->tile_tokens);
  const int parts = max_partitions(max_seq_len, 64, cpp);
  return (size_t)num_seqs * q_heads * parts * (kvq::kHeadDim + 2) * sizeof(float);
}

kvq_status kvq_paged_decode_attn(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                 int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                 int32_t max_blocks, const int32_t* seq_lens,
                                 int32_t max_seq_len, const void* pool_k, const void* pool_v,
                                 float sm_scale, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  KVQ_TRY(check_config(cfg, true));
  KVQ_NONNULL(q);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(seq_lens);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  KVQ_NONNULL(out);
  KVQ_NONNULL(workspace);
  if (num_seqs <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, q_heads, kv_heads, max_seq_len and max_blocks must be > 0");
  if (q_heads % kv_heads != 0)
    return fail(KVQ_ERR_ARG, "q_heads %d is not a multiple of kv_heads %d", q_heads, kv_heads);
  const int group = q_heads / kv_heads;
  if (group > 16) return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d larger than 16", group);
  if (kv_heads > 65535 || num_seqs > 65535 || (long)num_seqs * q_heads > 2147483647L)
    return fail(KVQ_ERR_ARG, "too many heads or sequences");
  const int tile = cfg->tile_tokens;
  const long need_blocks = (long)((max_seq_len + tile - 1) / tile) * (tile / kvq::kPage);
  if (need_blocks > max_blocks)
    return fail(KVQ_ERR_ARG, "max_blocks %d cannot hold %d tokens in whole tiles", max_blocks, max_seq_len);
  const size_t need = kvq_decode_workspace_bytes(cfg, num_seqs, q_heads, kv_heads, max_seq_len);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const int tpp = chunks_per_partition(num_seqs, kv_heads, max_seq_len, tile);
  const int parts = max_partitions(max_seq_len, 64, tpp);
  if (tpp > 64 || parts > 1024)
    return fail(KVQ_ERR_UNSUPPORTED, "max_seq_len %d is beyond 65536 chunks of 64 tokens", max_seq_len);
  kvq::DecodeArgs a{};
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.pool_k = (const uint8_t*)pool_k;
  a.pool_v = (const uint8_t*)pool_v;
  a.out = out;
  a.ws_acc = (float*)workspace;
  a.ws_ml = (float*)workspace + (size_t)num_seqs * q_heads * parts * kvq::kHeadDim;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.max_blocks = max_blocks;
  a.tiles_per_part = tpp;
  a.max_parts = parts;
  a.max_tiles = (max_seq_len + 63) / 64;   // in 64-token chunks
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.unit_tokens = 64;
  a.n_q = 1;
  a.out_scale = 1.0f;
  set_signs(a, cfg);
  return launched(kvq::launch_decode(a, tile, cfg->bits_k, cfg->bits_v, slot_format(cfg), (hipStream_t)stream),
                  "kvq_paged_decode_attn");
}

// Row blocks of the multi-query kernel per (sequence, kv head): 8 rows each.

size_t kvq_multi_query_workspace_bytes(const kvq_config* cfg, int32_t num_seqs, int32_t n_q, int32_t q_heads,
                                       int32_t kv_heads, int32_t max_seq_len) {
  if (check_config(cfg, true) != KVQ_OK) return 0;
  if (num_seqs <= 0 || n_q <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0) return 0;
  if (q_heads % kv_heads != 0 || n_q > max_seq_len) return 0;
  const int rb = kvq::mq_row_blocks(n_q, q_heads / kv_heads);
  const int cpp = chunks_per_partition(num_seqs * rb, kv_heads, max_seq_len, cfg->tile_tokens);
  const int parts = max_partitions(max_seq_len, 64, cpp);
  return (size_t)num_seqs * n_q * q_heads * parts * (kvq::kHeadDim + 2) * sizeof(float);
}

kvq_status kvq_paged_multi_query_attn(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs, int32_t n_q,
                                      int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                      int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                                      const void* pool_k, const void* pool_v, float sm_scale, float* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  KVQ_TRY(check_config(cfg, true));
  KVQ_NONNULL(q);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(seq_lens);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  KVQ_NONNULL(out);
  KVQ_NONNULL(workspace);
  if (num_seqs <= 0 || n_q <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, n_q, q_heads, kv_heads, max_seq_len and max_blocks must be > 0");
  if (q_heads % kv_heads != 0)
    return fail(KVQ_ERR_ARG, "q_heads %d is not a multiple of kv_heads %d", q_heads, kv_heads);
  if (n_q > max_seq_len)
    return fail(KVQ_ERR_ARG, "n_q %d exceeds max_seq_len %d (the queries are cached tokens)", n_q, max_seq_len);
  const int group = q_heads / kv_heads;
  if (group > 16) return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d larger than 16", group);
  const int rb = kvq::mq_row_blocks(n_q, group);
  if (num_seqs > 65535 || (long)kv_heads * rb * num_seqs > 2147483647L ||
      (long)num_seqs * n_q * q_heads > 2147483647L)
    return fail(KVQ_ERR_ARG, "too many heads, queries or sequences");
  const int tile = cfg->tile_tokens;
  const long need_blocks = (long)((max_seq_len + tile - 1) / tile) * (tile / kvq::kPage);
  if (need_blocks > max_blocks)
    return fail(KVQ_ERR_ARG, "max_blocks %d cannot hold %d tokens in whole tiles", max_blocks, max_seq_len);
  const size_t need = kvq_multi_query_workspace_bytes(cfg, num_seqs, n_q, q_heads, kv_heads, max_seq_len);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const int tpp = chunks_per_partition(num_seqs * rb, kv_heads, max_seq_len, tile);
  const int parts = max_partitions(max_seq_len, 64, tpp);
  if (tpp > 64 || parts > 1024)
    return fail(KVQ_ERR_UNSUPPORTED, "max_seq_len %d is beyond 65536 chunks of 64 tokens", max_seq_len);
  kvq::DecodeArgs a{};
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.pool_k = (const uint8_t*)pool_k;
  a.pool_v = (const uint8_t*)pool_v;
  a.out = out;
  a.ws_acc = (float*)workspace;
  a.ws_ml = (float*)workspace + (size_t)num_seqs * n_q * q_heads * parts * kvq::kHeadDim;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.max_blocks = max_blocks;
  a.tiles_per_part = tpp;
  a.max_parts = parts;
  a.max_tiles = (max_seq_len + 63) / 64;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.unit_tokens = 64;
  a.n_q = n_q;
  a.out_scale = 1.0f;
  set_signs(a, cfg);
  return launched(kvq::launch_multi_query(a, tile, cfg->bits_k, cfg->bits_v, slot_format(cfg), (hipStream_t)stream),
                  "kvq_paged_multi_query_attn");
}

static kvq_status append_and_decode_impl(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                 const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                 kvq_half* staging_k, kvq_half* staging_v, const int32_t* block_table,
                                 int32_t max_blocks, void* pool_k, void* pool_v, const kvq_half* q,
                                 int32_t q_heads, int32_t max_seq_len, float sm_scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  KVQ_TRY(check_config(cfg, true));
  KVQ_NONNULL(k_new);
  KVQ_NONNULL(v_new);
  KVQ_NONNULL(seq_lens_before);
  KVQ_NONNULL(staging_k);
  KVQ_NONNULL(staging_v);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  KVQ_NONNULL(q);
  KVQ_NONNULL(out);
  if (!noalloc) KVQ_NONNULL(workspace);
  if (num_seqs <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, q_heads, kv_heads, max_seq_len and max_blocks must be > 0");
  if (q_heads % kv_heads != 0)
    return fail(KVQ_ERR_ARG, "q_heads %d is not a multiple of kv_heads %d", q_heads, kv_heads);
  const int group = q_heads / kv_heads;
  if (group > 16) return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d larger than 16", group);
  if (kv_heads > 65535 || num_seqs > 65535 || (long)num_seqs * q_heads > 2147483647L)
    return fail(KVQ_ERR_ARG, "too many heads or sequences");
  const int tile = cfg->tile_tokens;
  const long need_blocks = (long)((max_seq_len + tile - 1) / tile) * (tile / kvq::kPage);
  if (need_blocks > max_blocks)
    return fail(KVQ_ERR_ARG, "max_blocks %d cannot hold %d tokens in whole tiles", max_blocks, max_seq_len);
  const size_t need = kvq_decode_workspace_bytes(cfg, num_seqs, q_heads, kv_heads, max_seq_len);
  if (noalloc && need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
    return fail(KVQ_ERR_WORKSPACE,
                "these sizes need %zu bytes of partition partials, beyond the %zu bytes of the library's "
                "static scratch (use kvq_append_and_decode with a workspace)", need,
                (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
  if (!noalloc && workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const int tpp = chunks_per_partition(num_seqs, kv_heads, max_seq_len, tile);
  const int parts = max_partitions(max_seq_len, 64, tpp);
  if (tpp > 64 || parts > 1024)
    return fail(KVQ_ERR_UNSUPPORTED, "max_seq_len %d is beyond 65536 chunks of 64 tokens", max_seq_len);
  if (noalloc) KVQ_TRY(scratch_of_current_device((hipStream_t)stream, &workspace));
  kvq::DecodeArgs a{};
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens_before;
  a.pool_k = (const uint8_t*)pool_k;
  a.pool_v = (const uint8_t*)pool_v;
  a.out = out;
  a.ws_acc = (float*)workspace;
  a.ws_ml = (float*)workspace + (size_t)num_seqs * q_heads * parts * kvq::kHeadDim;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.max_blocks = max_blocks;
  a.tiles_per_part = tpp;
  a.max_parts = parts;
  a.max_tiles = (max_seq_len + 63) / 64;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.unit_tokens = 64;
  a.n_q = 1;
  a.out_scale = 1.0f;
  kvq::QuantArgs qa{};
  qa.src[0] = k_new;
  qa.src[1] = v_new;
  qa.pool[0] = (uint8_t*)pool_k;
  qa.pool[1] = (uint8_t*)pool_v;
  qa.staging[0] = staging_k;
  qa.staging[1] = staging_v;
  qa.lens_before = seq_lens_before;
  qa.block_table = block_table;
  qa.max_blocks = max_blocks;
  qa.kv_heads = kv_heads;
  qa.iters = cfg->sinkhorn_iters;
  set_signs(a, cfg);
  set_signs(qa, cfg);
  return launched(kvq::launch_append_decode(a, qa, tile, cfg->bits_k, cfg->bits_v, slot_format(cfg),
                                           (hipStream_t)stream),
                  noalloc ? "kvq_append_and_decode_noalloc" : "kvq_append_and_decode");
}

kvq_status kvq_append_and_decode(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                 const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                 kvq_half* staging_k, kvq_half* staging_v, const int32_t* block_table,
                                 int32_t max_blocks, void* pool_k, void* pool_v, const kvq_half* q,
                                 int32_t q_heads, int32_t max_seq_len, float sm_scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return append_and_decode_impl(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, staging_k, staging_v,
                                block_table, max_blocks, pool_k, pool_v, q, q_heads, max_seq_len, sm_scale, out,
                                workspace, workspace_bytes, stream, false);
}

kvq_status kvq_append_and_decode_noalloc(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                         const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                         kvq_half* staging_k, kvq_half* staging_v, const int32_t* block_table,
                                         int32_t max_blocks, void* pool_k, void* pool_v, const kvq_half* q,
                                         int32_t q_heads, int32_t max_seq_len, float sm_scale, float* out,
                                         void* stream) {
  return append_and_decode_impl(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, staging_k, staging_v,
                                block_table, max_blocks, pool_k, pool_v, q, q_heads, max_seq_len, sm_scale, out,
                                nullptr, 0, stream, true);
}

size_t kvq_baseline_page_bytes(int32_t fp8) { return (size_t)kvq::kPage * kvq::kHeadDim * (fp8 ? 1 : 2); }

static kvq_status fill_baseline(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                                const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seq_len,
                                int32_t kv_heads, const int32_t* block_table, int32_t max_blocks,
                                void* pool_k, void* pool_v, bool fp8, float k_scale, float v_scale,
                                void* stream, const char* what) {
  KVQ_TRY(check_config(cfg, false));
  KVQ_NONNULL(k);
  KVQ_NONNULL(v);
  KVQ_NONNULL(cu_seqlens);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  if (num_seqs <= 0 || kv_heads <= 0 || max_seq_len <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, kv_heads, max_seq_len and max_blocks must be > 0");
  if (kv_heads > 65535 || num_seqs > 65535) return fail(KVQ_ERR_ARG, "too many heads or sequences");
  if ((max_seq_len + kvq::kPage - 1) / kvq::kPage > max_blocks)
    return fail(KVQ_ERR_ARG, "max_blocks %d cannot hold %d tokens", max_blocks, max_seq_len);
  if (fp8 && !(k_scale > 0.f && v_scale > 0.f)) return fail(KVQ_ERR_ARG, "fp8 scales must be > 0");
  kvq::BaseFillArgs a{k, v, cu_seqlens, block_table, max_blocks, kv_heads, (uint8_t*)pool_k, (uint8_t*)pool_v,
                      k_scale, v_scale};
  return launched(kvq::launch_fill_baseline(a, fp8, num_seqs, max_seq_len, (hipStream_t)stream), what);
}

kvq_status kvq_fill_pages_fp16(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seq_len,
                               int32_t kv_heads, const int32_t* block_table, int32_t max_blocks,
                               void* pool_k, void* pool_v, void* stream) {
  return fill_baseline(cfg, k, v, cu_seqlens, num_seqs, max_seq_len, kv_heads, block_table, max_blocks,
                       pool_k, pool_v, false, 1.f, 1.f, stream, "kvq_fill_pages_fp16");
}

kvq_status kvq_rematerialize_fp16_pages(const kvq_config* cfg, const void* pool_k, const void* pool_v,
                                        const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                        int32_t num_seqs, int32_t max_seq_len, int32_t kv_heads, kvq_half* base_k,
                                        kvq_half* base_v, void* stream) {
  KVQ_TRY(check_config(cfg, true));
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(seq_lens);
  KVQ_NONNULL(base_k);
  KVQ_NONNULL(base_v);
  if (num_seqs <= 0 || kv_heads <= 0 || max_seq_len <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, kv_heads, max_seq_len and max_blocks must be > 0");
  if (kv_heads > 32767 || num_seqs > 65535) return fail(KVQ_ERR_ARG, "too many heads or sequences");
  const int T = cfg->tile_tokens;
  if ((max_seq_len + T - 1) / T * (T / kvq::kPage) > max_blocks)
    return fail(KVQ_ERR_ARG, "max_blocks %d cannot hold whole tiles of %d tokens", max_blocks, max_seq_len);
  kvq::RematArgs a{(const uint8_t*)pool_k, (const uint8_t*)pool_v, block_table, max_blocks, seq_lens, kv_heads,
                   base_k, base_v};
  set_signs(a, cfg);
  return launched(kvq::launch_rematerialize(a, T, cfg->bits_k, cfg->bits_v, slot_format(cfg), num_seqs, max_seq_len,
                                            (hipStream_t)stream),
                  "kvq_rematerialize_fp16_pages");
}

kvq_status kvq_fill_pages_fp8(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seq_len,
                              int32_t kv_heads, const int32_t* block_table, int32_t max_blocks,
                              void* pool_k, void* pool_v, float k_scale, float v_scale, void* stream) {
  return fill_baseline(cfg, k, v, cu_seqlens, num_seqs, max_seq_len, kv_heads, block_table, max_blocks,
                       pool_k, pool_v, true, k_scale, v_scale, stream, "kvq_fill_pages_fp8");
}

static kvq_status append_baseline(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                  const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                  const int32_t* block_table, int32_t max_blocks, void* pool_k, void* pool_v,
                                  bool fp8, float k_scale, float v_scale, void* stream, const char* what) {
  KVQ_TRY(check_config(cfg, false));
  KVQ_NONNULL(k_new);
  KVQ_NONNULL(v_new);
  KVQ_NONNULL(seq_lens_before);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  if (num_seqs <= 0 || kv_heads <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, kv_heads and max_blocks must be > 0");
  if (kv_heads > 65535 || num_seqs > 65535) return fail(KVQ_ERR_ARG, "too many heads or sequences");
  if (fp8 && !(k_scale > 0.f && v_scale > 0.f)) return fail(KVQ_ERR_ARG, "fp8 scales must be > 0");
  kvq::BaseFillArgs a{k_new, v_new, nullptr, block_table, max_blocks, kv_heads, (uint8_t*)pool_k, (uint8_t*)pool_v,
                      k_scale, v_scale};
  return launched(kvq::launch_append_baseline(a, seq_lens_before, fp8, num_seqs, (hipStream_t)stream), what);
}

kvq_status kvq_append_pages_fp16(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                 const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                 const int32_t* block_table, int32_t max_blocks, void* pool_k, void* pool_v,
                                 void* stream) {
  return append_baseline(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, block_table, max_blocks, pool_k,
                         pool_v, false, 1.f, 1.f, stream, "kvq_append_pages_fp16");
}

kvq_status kvq_append_pages_fp8(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                const int32_t* block_table, int32_t max_blocks, void* pool_k, void* pool_v,
                                float k_scale, float v_scale, void* stream) {
  return append_baseline(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, block_table, max_blocks, pool_k,
                         pool_v, true, k_scale, v_scale, stream, "kvq_append_pages_fp8");
}

size_t kvq_baseline_workspace_bytes(const kvq_config* cfg, int32_t num_seqs, int32_t q_heads,
                                    int32_t kv_heads, int32_t max_seq_len) {
  if (check_config(cfg, false) != KVQ_OK) return 0;
  if (num_seqs <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0) return 0;
  const int tpp = tiles_per_partition(num_seqs, kv_heads, max_seq_len, 64);
  const int parts = max_partitions(max_seq_len, 64, tpp);
  return (size_t)num_seqs * q_heads * parts * (kvq::kHeadDim + 2) * sizeof(float);
}

static kvq_status decode_baseline(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs, int32_t q_heads,
                                  int32_t kv_heads, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t max_seq_len, const void* pool_k,
                                  const void* pool_v, float sm_scale, bool fp8, float k_scale, float v_scale,
                                  float* out, void* workspace, size_t workspace_bytes, void* stream,
                                  const char* what) {
  KVQ_TRY(check_config(cfg, false));
  KVQ_NONNULL(q);
  KVQ_NONNULL(block_table);
  KVQ_NONNULL(seq_lens);
  KVQ_NONNULL(pool_k);
  KVQ_NONNULL(pool_v);
  KVQ_NONNULL(out);
  KVQ_NONNULL(workspace);
  if (num_seqs <= 0 || q_heads <= 0 || kv_heads <= 0 || max_seq_len <= 0 || max_blocks <= 0)
    return fail(KVQ_ERR_ARG, "num_seqs, q_heads, kv_heads, max_seq_len and max_blocks must be > 0");
  if (q_heads % kv_heads != 0)
    return fail(KVQ_ERR_ARG, "q_heads %d is not a multiple of kv_heads %d", q_heads, kv_heads);
  const int group = q_heads / kv_heads;
  if (group > 16) return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d larger than 16", group);
  if (kv_heads > 65535 || num_seqs > 65535) return fail(KVQ_ERR_ARG, "too many heads or sequences");
  if ((max_seq_len + kvq::kPage - 1) / kvq::kPage > max_blocks)
    return fail(KVQ_ERR_ARG, "max_blocks %d cannot hold %d tokens", max_blocks, max_seq_len);
  if (fp8 && !(k_scale > 0.f && v_scale > 0.f)) return fail(KVQ_ERR_ARG, "fp8 scales must be > 0");
  const size_t need = kvq_baseline_workspace_bytes(cfg, num_seqs, q_heads, kv_heads, max_seq_len);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const int tpp = tiles_per_partition(num_seqs, kv_heads, max_seq_len, 64);
  const int parts = max_partitions(max_seq_len, 64, tpp);
  if (tpp > 64 || parts > 1024)
    return fail(KVQ_ERR_UNSUPPORTED, "max_seq_len %d is beyond 65536 blocks of 64 tokens", max_seq_len);
  kvq::DecodeArgs a{};
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.pool_k = (const uint8_t*)pool_k;
  a.pool_v = (const uint8_t*)pool_v;
  a.out = out;
  a.ws_acc = (float*)workspace;
  a.ws_ml = (float*)workspace + (size_t)num_seqs * q_heads * parts * kvq::kHeadDim;
  a.num_seqs = num_seqs;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.max_blocks = max_blocks;
  a.tiles_per_part = tpp;
  a.max_parts = parts;
  a.max_tiles = (max_seq_len + 63) / 64;
  a.sm_scale_log2 = sm_scale * (fp8 ? k_scale : 1.f) * 1.4426950408889634f;
  a.unit_tokens = 64;
  a.n_q = 1;
  a.out_scale = fp8 ? v_scale : 1.f;
  return launched(kvq::launch_decode_baseline(a, fp8, (hipStream_t)stream), what);
}

kvq_status kvq_paged_decode_attn_fp16(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                      int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                      int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                                      const void* pool_k, const void* pool_v, float sm_scale, float* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_baseline(cfg, q, num_seqs, q_heads, kv_heads, block_table, max_blocks, seq_lens, max_seq_len,
                         pool_k, pool_v, sm_scale, false, 1.f, 1.f, out, workspace, workspace_bytes, stream,
                         "kvq_paged_decode_attn_fp16");
}

kvq_status kvq_paged_decode_attn_fp8(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                     int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                     int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                                     const void* pool_k, const void* pool_v, float k_scale, float v_scale,
                                     float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return decode_baseline(cfg, q, num_seqs, q_heads, kv_heads, block_table, max_blocks, seq_lens, max_seq_len,
                         pool_k, pool_v, sm_scale, true, k_scale, v_scale, out, workspace, workspace_bytes,
                         stream, "kvq_paged_decode_attn_fp8");
}

kvq_status kvq_bandwidth_probe(const void* src, void* dst, size_t bytes, void* stream) {
  KVQ_NONNULL(src);
  KVQ_NONNULL(dst);
  if (bytes == 0 || bytes % 16 != 0) return fail(KVQ_ERR_ARG, "bytes must be a positive multiple of 16");
  return launched(kvq::launch_copy_probe(src, dst, bytes, (hipStream_t)stream), "kvq_bandwidth_probe");
}

}  // extern "C"
