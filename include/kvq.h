/*
 * kvq.h - C ABI of the MI355X (gfx950) variance-normalized KV-cache tile
 * quantizer and its paged decode-attention read path.
 *
 * The method: the KV cache is quantized one fixed-size token tile at a time;
 * each raw fp16 tile is rotated along the channel dimension with a Hadamard
 * transform (spreading channel-concentrated outliers), then put through a
 * Sinkhorn-like iterative variance normalization that evens out the
 * per-channel variance, then rounded to nearest, asymmetrically, to a
 * low-bit cache.  Source: page "Huawei's KVarN boosts vLLM KV-cache capacity
 * by 5x without accuracy loss" (axbrief.com), section "기존 방식과 달라진
 * 지점", restated in its section "별도의 캘리브레이션이나 모델 변경 없이
 * 플래그 하나로 적용" (nothing is calibrated: every statistic comes from the
 * tile).  K and V are compressed and restored inside the pipeline with the
 * cache kept in pages (page "화웨이가 공개한 KVarN — LLM 추론의 '메모리 먹는
 * 하마' KV 캐시를 양자화로 길들이기", ttj.kr, section "양자화로 캐시를
 * 다이어트시킨다"), and the attention backend reads the compressed pages
 * directly instead of re-materializing fp16 (aitrends.kr article 74976,
 * TL;DR and the glossary entries on KV compression and the attention
 * backend).
 *
 * What the pages leave open is fixed here as follows (every function uses it):
 *   - Hadamard: orthonormal Sylvester order, on every token row of K and of V
 *     (head_dim 128); with cfg->hadamard_signs non-zero the rotation is
 *     H * diag(s) (a seeded +-1 diagonal first, the common randomized variant;
 *     the pages do not say whether signs are used) and the restore diag(s) * H.
 *     Every call on the same pages must pass the same signs.
 *   - One normalization iteration = channel step (each channel divided by its
 *     population std over the tile's valid tokens) then token step (each token
 *     divided by its population std over the 128 channels).  A channel/token
 *     whose std is at most 1e-2 times its RMS keeps factor 1.  The channel
 *     factors alpha[128] are stored per tile; the token factors are folded
 *     into the per-token scale and offset.
 *   - Rounding: per token row of the tile, zero-point = row minimum, step =
 *     (max - min) / (2^bits - 1), round half to even; a zero-range row gets
 *     codes 0 and step 0.  Stored per token: scale S = beta*step and offset
 *     O = beta*min (fp32).  Restore: rotated row = alpha * (S * code + O),
 *     token = Hadamard(rotated row).
 *   - Tiles start at token 0 of each sequence; the last may be partial and
 *     its statistics use only its valid rows.
 *   - Code widths: 4 and 2 bits, and 8 bits (the integer widths the ttj.kr
 *     page names in its section "양자화로 캐시를 다이어트시킨다" are 8 and 4);
 *     K and V may mix 2 and 4, while 8 is used for both or neither.
 *
 * Conventions for every function:
 *   - Pointers to data are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), contiguous in the documented layouts, at least 16-byte
 *     aligned (pools and code buffers: 256-byte aligned recommended).
 *     `cfg` and scalar arguments live on the host.
 *   - The caller owns and allocates every buffer.  The library allocates
 *     nothing, keeps no state between calls except a thread-local error
 *     message (and, for kvq_append_and_decode_noalloc, its static device
 *     scratch and each device's address of it), and never synchronizes: each
 *     call enqueues its kernels on
 *     `stream` (a hipStream_t passed as void*, NULL = default stream) and
 *     returns.
 *   - Arguments are validated on the host before any launch.  On a non-OK
 *     status nothing was launched (except KVQ_ERR_HIP, reported when a
 *     launch fails) and kvq_last_error() describes the problem.  Contents of
 *     device arrays (lengths, page ids) are trusted: out-of-range values are
 *     undefined behaviour, as for any kernel argument.
 *   - Inputs must be finite.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t kvq_half; /* IEEE 754 binary16 bit pattern */

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,         /* null pointer, non-positive size, inconsistent shapes */
  KVQ_ERR_UNSUPPORTED = -2, /* head_dim != 128, page_tokens != 16, tile not 32/64/128,
                               bits not 2/4/8 (or 8 on one of K/V only),
                               iters outside 0..16, GQA group > 16 */
  KVQ_ERR_HIP = -3,         /* a kernel launch failed */
  KVQ_ERR_WORKSPACE = -4    /* workspace smaller than kvq_decode_workspace_bytes() */
} kvq_status;

typedef struct {
  int32_t head_dim;       /* must be 128 */
  int32_t page_tokens;    /* must be 16 */
  int32_t tile_tokens;    /* 32, 64 or 128 (a multiple of page_tokens) */
  int32_t bits_k;         /* code width of K: 2 or 4, or 8 with bits_v = 8 */
  int32_t bits_v;         /* code width of V: 2 or 4, or 8 with bits_k = 8 */
  int32_t sinkhorn_iters; /* normalization iterations, 0..16 */
  uint32_t hadamard_signs[4]; /* randomized rotation: bit c mod 32 of word c/32
                                 set = channel c negated before the Hadamard
                                 (and after the inverse); all 0 = plain H */
  int32_t meta_fp16;      /* 0: slot metadata (scale, offset, channel factors)
                             in fp32; 1: in fp16 (2- and 4-bit codes only), see
                             the page-pool layout */
  int32_t k_per_channel;  /* 0: K rounded per token (as V); 1: K tiles rounded
                             per channel over the tile's tokens (2- and 4-bit
                             codes, fp32 metadata, paged entry points only),
                             see the page-pool layout */
} kvq_config;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kvq_last_error(void);

/* Library version string. */
const char* kvq_version(void);

/*
 * Page-pool layout.  A page holds 16 consecutive tokens of one sequence.  A
 * pool is an array [num_pages][kv_heads][slot] of bytes; a slot is
 *   codes : 16*128*bits/8 bytes (layout below)
 *   scale : float32[16]   per token S   (0 for rows past the sequence end)
 *   offset: float32[16]   per token O   (0 for rows past the sequence end)
 *   alpha : float32[16*128/tile_tokens] the slice j*L..(j+1)*L-1 (L = 2048/T)
 *           of the tile's channel factors, j = the page's index in its tile.
 * With cfg->meta_fp16 = 1 the three metadata arrays hold IEEE fp16 (2 bytes
 *   each, same order; 72 bytes per token at 4 bits, tile 64, against 80), and
 *   one power of two per tile moves from S and O into alpha: with M the
 *   largest |S|, |O| of the tile's tokens, e = floor(log2 M) - 10 (0 if M is 0),
 *   the slots hold S*2^-e, O*2^-e and alpha*2^e rounded to nearest even (the
 *   restore alpha*(S*code + O) only sees their products).  Codes are the same
 *   as with fp32 metadata.
 * With cfg->k_per_channel = 1 a K slot is
 *   codes | beta: float32[16] per token (0 past the sequence end) |
 *   A: float32[16*128/tile_tokens] | M: float32[16*128/tile_tokens]
 *   (1344 bytes at 4 bits, tile 64): the tile is rounded per channel over
 *   its valid tokens (zero-point min, step (max - min)/(2^bits - 1)), A is
 *   the slice of the tile's channel scales alpha*step and M of its zero
 *   offsets in code units min/step (a channel of zero range: A = alpha*min,
 *   M = 1, codes 0), the same page-in-tile slicing as alpha; the restored
 *   rotated row is beta*A*(code + M).  V slots are unchanged.
 * Unit order of a token's 128 codes (dense codes and K slots): 16 units of
 *   8 fields, a unit being 8*bits bits (a little-endian 32-bit word at 4
 *   bits, a 16-bit half at 2 bits, a little-endian 64-bit pair of words at 8), unit u at bit 8*bits*u of the token's
 *   codes; field m (bits [bits*m, bits*(m+1)) of the unit) holds channel
 *   u + 16*m.
 * K-slot codes: each token's units cut into 4 blocks of 4 units (4*bits
 *   bytes); block k stores, token after token, units 4k..4k+3 of each of the
 *   16 tokens (block k of token t at byte 4*bits*(16*k + t)).
 * V-slot codes: 64 runs of 4*bits bytes; run l (at byte 4*bits*l) holds the
 *   channels l (h = 0) and 64 + l (h = 1) of the 16 tokens, read as
 *   little-endian 32-bit words of F = 32/bits fields.  Token t = 4g + r
 *   (quad g, r < 4) of channel half h forms the pair p = 2g + h, stored in word
 *   p / (F/4) of the run, field f = 2m + (r>>1) + (F/2)(r&1) with
 *   m = p mod (F/4), field f being bits [bits*f, bits*(f+1)) of the word.
 * Rows of a page past the sequence's end hold code 0, scale 0 and offset 0.
 * Contract: a sequence owns a page for every page of every tile it has
 * started (pages are allocated in whole tiles), so a partial tile's channel
 * factors always have a home.  The block table is int32 [num_seqs][max_blocks]
 * of page ids; page p of sequence s holds its tokens 16p..16p+15.
 * Returns 0 for an invalid config.
 */
size_t kvq_slot_bytes(const kvq_config* cfg, int32_t is_v);

/*
 * kvq_quantize_tiles - quantize one token run per head in the dense layout.
 *   x          fp16 [n_tokens][heads][128]; tile j of each head covers tokens
 *              j*T .. min(n_tokens, (j+1)*T)-1.
 *   bits       2, 4 or 8 (cfg->bits_k/bits_v are ignored here).
 *   codes      uint8 [n_tokens][heads][128*bits/8], each token's codes in
 *              unit order (see the page-pool layout below).
 *   alpha      float32 [ceil(n_tokens/T)][heads][128] channel factors.
 *   tok_scale  float32 [n_tokens][heads] per token S.
 *   tok_offset float32 [n_tokens][heads] per token O.
 * Errors: KVQ_ERR_ARG for null pointers or n_tokens/heads <= 0,
 * KVQ_ERR_UNSUPPORTED for an unsupported config or bits.
 */
kvq_status kvq_quantize_tiles(const kvq_config* cfg, const kvq_half* x, int32_t n_tokens,
                              int32_t heads, int32_t bits, uint8_t* codes, float* alpha,
                              float* tok_scale, float* tok_offset, void* stream);

/*
 * kvq_dequantize - restore fp16 tokens from the dense layout of
 * kvq_quantize_tiles (same shapes): out[t][h] = Hadamard(alpha * (S*code + O))
 * computed in fp32 and rounded to nearest-even fp16.
 */
kvq_status kvq_dequantize(const kvq_config* cfg, const uint8_t* codes, const float* alpha,
                          const float* tok_scale, const float* tok_offset, int32_t n_tokens,
                          int32_t heads, int32_t bits, kvq_half* out, void* stream);

/*
 * kvq_quantize_to_pages - quantize a prefill of K and V into the page pools.
 *   k, v         fp16 [total_tokens][kv_heads][128], sequences packed back to
 *                back; sequence s is rows cu_seqlens[s] .. cu_seqlens[s+1]-1.
 *   cu_seqlens   int32 [num_seqs+1], device, non-decreasing.
 *   total_tokens host: cu_seqlens[num_seqs] (or more); the launch covers
 *                total_tokens / T + num_seqs tile slots, which hold every
 *                tile of any length mix with at most one idle slot per
 *                sequence (a smaller value leaves the last tiles unwritten).
 *   block_table  int32 [num_seqs][max_blocks], device; a tile whose pages
 *                would lie past max_blocks is not written.
 *   pool_k/pool_v  K and V pools (layout above; bits from cfg).
 *   staging_k/staging_v  fp16 [num_seqs][T][kv_heads][128] or NULL: rows
 *                of a last tile that is not full are copied there (needed
 *                by kvq_append_and_requant).
 * K uses cfg->bits_k, V cfg->bits_v; both use cfg->sinkhorn_iters.
 */
kvq_status kvq_quantize_to_pages(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int32_t kv_heads,
                                 const int32_t* block_table, int32_t max_blocks, void* pool_k,
                                 void* pool_v, kvq_half* staging_k, kvq_half* staging_v,
                                 void* stream);

/*
 * kvq_append_and_requant - append one decode token per sequence and
 * re-quantize the tile it lands in.
 *   k_new, v_new     fp16 [num_seqs][kv_heads][128].
 *   seq_lens_before  int32 [num_seqs], device: tokens cached before this one.
 *   staging_k/_v     fp16 [num_seqs][T][kv_heads][128]: rows 0..r-1 of the
 *                    partial tile (r = seq_len_before mod T) must hold that
 *                    tile's fp16 rows (kvq_quantize_to_pages and earlier
 *                    appends keep them); the new row is written at r.
 * The whole tile (rows 0..r) is quantized again, as in kvq_quantize_to_pages,
 * and its pages rewritten.  The caller advances its lengths afterwards.
 */
kvq_status kvq_append_and_requant(const kvq_config* cfg, const kvq_half* k_new,
                                  const kvq_half* v_new, const int32_t* seq_lens_before,
                                  int32_t num_seqs, int32_t kv_heads, kvq_half* staging_k,
                                  kvq_half* staging_v, const int32_t* block_table,
                                  int32_t max_blocks, void* pool_k, void* pool_v, void* stream);

/* Bytes of workspace kvq_paged_decode_attn needs for these sizes. */
size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t num_seqs, int32_t q_heads,
                                  int32_t kv_heads, int32_t max_seq_len);

/*
 * kvq_paged_decode_attn - one decode step of attention straight from the
 * quantized pages (no fp16 K/V is rebuilt).
 *   q            fp16 [num_seqs][q_heads][128]; query head h reads kv head
 *                h / (q_heads / kv_heads).
 *   seq_lens     int32 [num_seqs], device: tokens to attend (newest included);
 *                a sequence of length 0 gets a zero output row.
 *   max_seq_len  host upper bound of seq_lens (sizes the grid); every
 *                seq_lens entry must be <= max_seq_len (not checked: the
 *                lengths live on the device).
 *   sm_scale     softmax scale (1/sqrt(128) for standard attention).
 *   out          float32 [num_seqs][q_heads][128]:
 *                softmax(sm_scale * q.K^T) V over the restored tokens,
 *                computed as scores (H q * alpha_K).(S code + O) and values
 *                Hadamard(sum_t p_t alpha_V (S code + O)), fp32 accumulation.
 *   workspace    device scratch of at least kvq_decode_workspace_bytes().
 * Errors: KVQ_ERR_WORKSPACE if the workspace is too small; KVQ_ERR_ARG if
 * q_heads is not a multiple of kv_heads; KVQ_ERR_UNSUPPORTED if the group is
 * larger than 16.
 */
kvq_status kvq_paged_decode_attn(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                 int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                 int32_t max_blocks, const int32_t* seq_lens,
                                 int32_t max_seq_len, const void* pool_k, const void* pool_v,
                                 float sm_scale, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * kvq_append_and_decode - one decode step in one launch (plus the partition
 * merge): the new token is compressed into the cache inside the pipeline and
 * the attention reads the compressed pages, the new token included (ttj.kr
 * page, section "양자화로 캐시를 다이어트시킨다"; aitrends.kr article 74976,
 * TL;DR).  Equivalent to kvq_append_and_requant of (k_new, v_new) at position
 * seq_lens_before[s] followed by kvq_paged_decode_attn over
 * seq_lens_before[s] + 1 tokens: arguments as those two functions
 * (max_seq_len bounds seq_lens_before + 1; the workspace is sized by
 * kvq_decode_workspace_bytes for max_seq_len), and the pages, staging rows and
 * output are bit-identical to those of the two calls made in order.  The
 * re-quantized tile is read only by the last partition of its (sequence, kv
 * head), whose workgroup writes it before attending.  Errors as those two
 * functions.
 */
kvq_status kvq_append_and_decode(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                 const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                 kvq_half* staging_k, kvq_half* staging_v, const int32_t* block_table,
                                 int32_t max_blocks, void* pool_k, void* pool_v, const kvq_half* q,
                                 int32_t q_heads, int32_t max_seq_len, float sm_scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_append_and_decode_noalloc - kvq_append_and_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as kvq_append_and_decode (bit-identical pages, staging rows and
 * output), without the workspace arguments: the partition partials go to a
 * static device array of the library, KVQ_NOALLOC_SCRATCH_BYTES per GPU,
 * which each GPU the library runs on holds until the process ends.  The call
 * allocates nothing.
 *   - The stream must belong to the current device (KVQ_ERR_ARG otherwise);
 *     the first call on a device looks up that device's copy of the array.
 *   - KVQ_ERR_WORKSPACE if kvq_decode_workspace_bytes() of these sizes
 *     exceeds KVQ_NOALLOC_SCRATCH_BYTES (checked on the host before any
 *     device call).
 *   - All calls on one GPU share its array: calls that overlap on one GPU
 *     (on different streams, or from several threads without ordering)
 *     race on it.  Calls ordered on one stream are safe; each leaves its
 *     partials behind, and none needs the array cleared.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
kvq_status kvq_append_and_decode_noalloc(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                         const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                         kvq_half* staging_k, kvq_half* staging_v, const int32_t* block_table,
                                         int32_t max_blocks, void* pool_k, void* pool_v, const kvq_half* q,
                                         int32_t q_heads, int32_t max_seq_len, float sm_scale, float* out,
                                         void* stream);

/* Bytes of workspace kvq_paged_multi_query_attn needs for these sizes (0 for
 * invalid sizes, n_q > max_seq_len included). */
size_t kvq_multi_query_workspace_bytes(const kvq_config* cfg, int32_t num_seqs, int32_t n_q,
                                       int32_t q_heads, int32_t kv_heads, int32_t max_seq_len);

/*
 * kvq_paged_multi_query_attn - several queries per sequence read straight
 * from the quantized pages (aitrends.kr article 74976, TL;DR: the attention
 * backend reads the compressed pages; no fp16 K/V is rebuilt), e.g. the
 * tokens of a chunked prefill or a speculative draft being verified.
 *   q            fp16 [num_seqs][n_q][q_heads][128]: the n_q newest tokens of
 *                each sequence, already in the cache (appended beforehand);
 *                query head h reads kv head h / (q_heads / kv_heads).
 *   seq_lens     int32 [num_seqs], device: cached tokens, the n_q queries
 *                included.  Query i of sequence s sits at position
 *                seq_lens[s] - n_q + i and attends to the tokens 0 .. that
 *                position (causal).  A query at a negative position (a
 *                sequence shorter than n_q) sees no token and gets zeros.
 *   max_seq_len  host upper bound of seq_lens (sizes the grid; not checked
 *                against the device lengths); n_q <= max_seq_len.
 *   sm_scale     softmax scale (1/sqrt(128) for standard attention).
 *   out          float32 [num_seqs][n_q][q_heads][128], computed as in
 *                kvq_paged_decode_attn (with n_q = 1 the two give the same
 *                values).
 *   workspace    device scratch of at least kvq_multi_query_workspace_bytes().
 * The (query, head) pairs of a kv head run in workgroups of up to 8; each
 * such workgroup reads the pages of its partition, so very long query runs
 * read the pages several times (from L2 where they fit).
 * Errors: KVQ_ERR_ARG for null pointers, sizes <= 0, q_heads not a multiple
 * of kv_heads, n_q > max_seq_len, too many rows; KVQ_ERR_UNSUPPORTED for a
 * GQA group above 16; KVQ_ERR_WORKSPACE for a small workspace.
 */
kvq_status kvq_paged_multi_query_attn(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                      int32_t n_q, int32_t q_heads, int32_t kv_heads,
                                      const int32_t* block_table, int32_t max_blocks,
                                      const int32_t* seq_lens, int32_t max_seq_len, const void* pool_k,
                                      const void* pool_v, float sm_scale, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Baselines (fp16 and fp8 paged KV without the quantizer), for comparing the
 * quantized read path with the two modes the aitrends.kr page (article
 * 74976, TL;DR) runs on the same workload.  Page layout per (page, kv head):
 * K [16 tokens][128 channels], V [128 channels][16 tokens] (channel-major),
 * elements fp16 or OCP E4M3 bytes (value = byte decoded times the tensor's
 * scale; the fill rounds x / scale to nearest, ties to even).  A pool is
 * [num_pages][kv_heads][16*128] elements; rows past a sequence's end are 0.
 * Block tables as for the quantized pools (one page per 16 tokens).
 */
size_t kvq_baseline_page_bytes(int32_t fp8); /* 4096 (fp16) or 2048 (fp8) */

/* Write a prefill (k, v fp16 [total][kv_heads][128], packed by cu_seqlens)
 * into fp16 pools.  Errors as kvq_quantize_to_pages. */
kvq_status kvq_fill_pages_fp16(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                               const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seq_len,
                               int32_t kv_heads, const int32_t* block_table, int32_t max_blocks,
                               void* pool_k, void* pool_v, void* stream);

/* Same into E4M3 pools with per-tensor scales k_scale, v_scale > 0
 * (KVQ_ERR_ARG otherwise). */
kvq_status kvq_fill_pages_fp8(const kvq_config* cfg, const kvq_half* k, const kvq_half* v,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seq_len,
                              int32_t kv_heads, const int32_t* block_table, int32_t max_blocks,
                              void* pool_k, void* pool_v, float k_scale, float v_scale, void* stream);

/* Append one decode token per sequence to fp16 (resp. E4M3) pools: k_new,
 * v_new fp16 [num_seqs][kv_heads][128] go to position seq_lens_before[s]
 * (device int32 [num_seqs]) of sequence s, K as row p % 16 of the page
 * holding p, V as column p % 16, encoded as the fills encode (E4M3: x / scale
 * rounded to nearest, ties to even; |x| / scale must stay within 448).  The
 * page must exist in the block table (a position past max_blocks pages is
 * skipped).  The caller advances its lengths afterwards.  Errors as the fills. */
kvq_status kvq_append_pages_fp16(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                 const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                 const int32_t* block_table, int32_t max_blocks, void* pool_k, void* pool_v,
                                 void* stream);
kvq_status kvq_append_pages_fp8(const kvq_config* cfg, const kvq_half* k_new, const kvq_half* v_new,
                                const int32_t* seq_lens_before, int32_t num_seqs, int32_t kv_heads,
                                const int32_t* block_table, int32_t max_blocks, void* pool_k, void* pool_v,
                                float k_scale, float v_scale, void* stream);

/* Workspace bytes of the two baseline decode functions. */
size_t kvq_baseline_workspace_bytes(const kvq_config* cfg, int32_t num_seqs, int32_t q_heads,
                                    int32_t kv_heads, int32_t max_seq_len);

/* One decode step of softmax(sm_scale q.K^T) V over fp16 (resp. E4M3) pages;
 * arguments, output and errors as kvq_paged_decode_attn (only head_dim and
 * page_tokens of cfg are used). */
kvq_status kvq_paged_decode_attn_fp16(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                      int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                      int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                                      const void* pool_k, const void* pool_v, float sm_scale, float* out,
                                      void* workspace, size_t workspace_bytes, void* stream);
kvq_status kvq_paged_decode_attn_fp8(const kvq_config* cfg, const kvq_half* q, int32_t num_seqs,
                                     int32_t q_heads, int32_t kv_heads, const int32_t* block_table,
                                     int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                                     const void* pool_k, const void* pool_v, float k_scale, float v_scale,
                                     float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * kvq_rematerialize_fp16_pages - the read path the direct decode avoids:
 * restore every cached token of the quantized pages to fp16 before attention
 * (aitrends.kr article 74976, TL;DR, and its glossary entry on the attention
 * backend: reading compressed pages directly instead of re-materializing).
 * Each token of sequence s (seq_lens[s] tokens, device) is rebuilt as
 * kvq_dequantize does (Hadamard(alpha * (S*code + O)), fp32, rounded to fp16)
 * and written into the fp16 pools base_k, base_v (the layout of
 * kvq_fill_pages_fp16) at the same page ids (block_table).  Rows of a
 * sequence's last page past its end are written 0; pages past that are not
 * touched.  kvq_paged_decode_attn_fp16 then reads them.
 *   max_seq_len  host bound of seq_lens; max_blocks must hold the pages of
 *                whole tiles up to it.
 * Errors: as kvq_quantize_to_pages (KVQ_ERR_ARG for null pointers, sizes <= 0,
 * too small a block table; KVQ_ERR_UNSUPPORTED for the config).
 */
kvq_status kvq_rematerialize_fp16_pages(const kvq_config* cfg, const void* pool_k, const void* pool_v,
                                        const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                        int32_t num_seqs, int32_t max_seq_len, int32_t kv_heads, kvq_half* base_k,
                                        kvq_half* base_v, void* stream);

/*
 * kvq_bandwidth_probe - measurement helper, not part of the method: copies
 * `bytes` (a positive multiple of 16) from src to dst with a plain streaming
 * kernel, so that achieved HBM bandwidth and profiler byte counters can be
 * calibrated against a kernel of known traffic (2 * bytes).
 */
kvq_status kvq_bandwidth_probe(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
