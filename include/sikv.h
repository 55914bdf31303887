/*
 * sikv.h - C ABI of the self-indexing compressed-key decode path (gfx950 / MI355X).
 *
 * The method: "Self-Indexing KVCache: Predicting Sparse Attention from
 * Compressed Keys" (web summary of arXiv 2603.14224, technical part).  Keys are
 * normalised by their channel mean, split into 4-dim sub-vectors and sign-coded
 * (one of 16 clusters per sub-vector, 1 bit per channel) plus one fp32 scale per
 * token (§2.1 item 1).  A decoding query builds a 16-entry table per sub-vector
 * and scores every cached token by table look-up and accumulation (LUT-GEMV),
 * then keeps the top-k (§2.1 item 2).  Attention runs over the top-k plus 64
 * full-precision sink tokens, with the keys dequantised inside the kernel
 * (§2.1 items 3 and 4).
 *
 * Conventions shared by every call
 *   - Pointers named in the cache descriptor and the arguments are DEVICE
 *     pointers (hipMalloc'd or torch CUDA tensors) unless stated otherwise; the
 *     descriptor itself and the workspace size query live in HOST memory.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Ownership: every buffer belongs to the caller.  The library never
 *     allocates, frees or keeps device memory; scratch comes from the caller's
 *     workspace (size from sikv_workspace_bytes, 256-byte aligned start).
 *   - Asynchrony: every call only enqueues kernels on `stream` (a hipStream_t;
 *     NULL = the null stream) and returns.  Buffers must stay valid until the
 *     stream has run the work.  No call synchronises.
 *   - Errors: arguments are validated on the host before anything is launched;
 *     an invalid call returns a negative status and launches nothing.  A failed
 *     launch returns SIKV_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.  No C++ exception crosses this ABI.
 *   - Shapes: head_dim 128 and 64 sinks only (SIKV_ERR_UNSUPPORTED otherwise);
 *     query heads per KV head (G = n_q_heads / n_kv_heads) from 1 to 8, query
 *     head h*G+g belongs to KV head h.
 *   - State: the library keeps none, apart from the one allocation-free entry
 *     point's static device scratch (sikv_append_decode_step_static).
 *     Everything any other call reads is in its arguments and the descriptor
 *     (including the optional caller-owned timer and the flags word), so those
 *     calls may run concurrently from several threads on different streams with
 *     disjoint buffers and workspaces.
 */
#ifndef SIKV_H
#define SIKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SIKV_ABI_VERSION 7
#define SIKV_HEAD_DIM 128
#define SIKV_N_SINK 64
#define SIKV_MAX_GROUP 8

typedef int32_t sikv_status;
#define SIKV_OK 0
#define SIKV_ERR_INVALID_ARG (-1) /* null/misaligned pointer, bad size or range   */
#define SIKV_ERR_UNSUPPORTED (-2) /* valid but outside v1 (head_dim, sinks, G)     */
#define SIKV_ERR_WORKSPACE (-3)   /* workspace missing, misaligned or too small    */
#define SIKV_ERR_HIP (-4)         /* a kernel launch or HIP runtime call failed    */

/* bits of sikv_cache_desc.flags (every other bit must be 0) */
#define SIKV_FLAG_EXACT_SELECT 1 /* score_topk skips its sampled threshold and
                                    always takes its exact whole-head selection
                                    path (same result, slower; for tests) */

/* Caller-owned kernel timer (sikv_timer_create); opaque. */
typedef struct sikv_timer sikv_timer;

/* op codes of sikv_workspace_bytes */
#define SIKV_OP_ENCODE 0
#define SIKV_OP_SCORE_TOPK 1
#define SIKV_OP_SPARSE_ATTN 2
#define SIKV_OP_DECODE_STEP 3
#define SIKV_OP_KMEANS 4

/*
 * The compressed cache of one layer (caller-owned device arrays), described in
 * host memory.  Index order [b][h][t][...] with b < batch, h < n_kv_heads,
 * t < capacity.  Layout (§2.1 item 3: token-wise, so any token can be fetched
 * on its own):
 *   codes  uint8 [B][Hkv][capacity][16]: bit c of a token's code (byte c/8,
 *          bit c%8, least significant first) is 1 iff its key channel c is
 *          below the channel mean; nibble j (low nibble first) is the cluster
 *          of sub-vector j (channels 4j..4j+3, bit i = channel 4j+i).  16-byte
 *          aligned.
 *   alpha  fp32 [B][Hkv][capacity]: per-token scale, mean |k_c - mu_c|.
 *   mu     fp32 [B][Hkv][128]: channel mean of the non-sink prefill keys.
 *   k_sink bf16 [B][Hkv][64][128]: the first 64 key rows, unquantised.
 *   v      bf16 value cache, element (b,h,t,c) at v[b*v_stride_b + h*v_stride_h
 *          + t*v_stride_t + c] (strides in elements, multiples of 8; rows
 *          16-byte aligned).  Only read.
 *   codebook  NULL: the 16 centres of every sub-vector are the sign vertices
 *          (+1 for bit 0, -1 for bit 1 per channel) scaled by alpha.  Else
 *          fp32 [B][Hkv][32][16][4], 16-byte aligned: data-derived centres
 *          (§2.1 item 1, one-pass clustering by sign pattern; §2.1 item 2, the
 *          query is dotted with the 16 centres): sikv_encode with
 *          recompute_mu = 1 writes them, every scoring and attention call
 *          uses them (key_t = mu + alpha_t * centre of its cluster, per
 *          sub-vector).  Appended tokens keep the prefill centres.
 *   vrec, v_sink  NULL: attention reads the bf16 V cache `v`.  Else (both set;
 *          vrec 64-byte, v_sink 16-byte aligned) the values are kept 2-bit (the
 *          pages' 2-bit setting, read as a per-token value scheme; the 64 sinks
 *          stay full precision, §2.1 item 3) in one 64-byte record per token,
 *          vrec uint8 [B][Hkv][capacity][64]: bytes 0..31 the value codes
 *          (channel c at byte c/4, bits 2*(c%4)), bytes 32..47 four uint32
 *          words, one per group of 32 channels (fp16 scale in the low half, fp16
 *          zero point in the high half), bytes 48..63 a copy of the token's
 *          16-byte key code; v_sink bf16 [B][Hkv][64][128].  sikv_encode_v (or
 *          the fused step) writes bytes 0..47 and v_sink, sikv_encode (or the
 *          fused step) also writes the key code copy; `v` is then not read and
 *          may be NULL.  Value of channel c: zero + code * scale of its group.
 *          One record holds all an attended token needs but its scale alpha.
 *   seq_lens  NULL: every sequence has n_tokens tokens.  Else (ragged batch, a
 *          device array int32 [B], 4-byte aligned, read by the kernels) sequence
 *          b has seq_lens[b] tokens and n_tokens is the longest (it sizes grids
 *          and workspaces); a length outside (64, n_tokens] is clamped into it.
 *          Scoring, top-k and attention of sequence b use its own tokens
 *          64..seq_lens[b]-1, its top-k is k_b = min(k, seq_lens[b] - 64) and row
 *          b of idx holds k_b positions followed by -1; the fused append step
 *          writes the new token of sequence b at row seq_lens[b]-1 (seq_lens
 *          already counts it).  sikv_encode / sikv_encode_v ignore it: ragged
 *          prefill is one call per sequence on a batch-1 view (pointers offset
 *          to that sequence's rows).
 *   page_table, page_size, pages_per_seq, n_pages  page_table NULL: each (b, h)
 *          owns capacity contiguous rows of the per-token arrays.  Else (paged,
 *          a device array int32 [B][pages_per_seq], 4-byte aligned) token t of
 *          sequence b lives in pool page p = page_table[b][t / page_size], which
 *          holds page_size tokens of every KV head: codes uint8
 *          [n_pages][Hkv][page_size][16], alpha fp32 [n_pages][Hkv][page_size],
 *          vrec uint8 [n_pages][Hkv][page_size][64], and a bf16 V pool `v` laid out
 *          [n_pages][Hkv][page_size][128] (v_stride_b = Hkv*page_size*128,
 *          v_stride_h = page_size*128, v_stride_t = 128).  page_size is a power of
 *          two >= 256, capacity = pages_per_seq * page_size, and n_pages * Hkv *
 *          page_size < 2^31.  mu, k_sink, codebook, v_sink stay per sequence.  Page
 *          ids are trusted (the caller keeps them in [0, n_pages)).
 *   flags  0, or SIKV_FLAG_EXACT_SELECT (above); any other bit is invalid.
 *   timer  NULL, or a timer from sikv_timer_create: every kernel the call
 *          launches is bracketed by events recorded with it (measurement
 *          only; see the timer functions at the end of this file).
 * n_tokens (N) is the number of valid tokens of every sequence (64 < N <=
 * capacity; the longest one with seq_lens); candidates for top-k are the tokens
 * 64..N-1.
 */
typedef struct sikv_cache_desc {
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t n_tokens;
  int32_t n_sink;
  uint8_t *codes;
  float *alpha;
  float *mu;
  uint16_t *k_sink;
  const uint16_t *v;
  int64_t v_stride_b;
  int64_t v_stride_h;
  int64_t v_stride_t;
  float *codebook;
  uint8_t *vrec;
  uint16_t *v_sink;
  const int32_t *seq_lens;
  const int32_t *page_table;
  int32_t page_size;
  int32_t pages_per_seq;
  int32_t n_pages;
  int32_t flags;
  sikv_timer *timer;
} sikv_cache_desc;

/*
 * sikv_encode - compress keys into the cache (§2.1 item 1: channel-mean
 * normalisation, then sign codes of 4-dim sub-vectors; §2.1 item 3: the 64
 * sink rows kept in full precision at prefill).
 *   k            bf16 keys of tokens t_begin..t_end-1: element (b,h,t,c) at
 *                k[b*k_stride_b + h*k_stride_h + (t - t_begin)*k_stride_t + c]
 *                (strides in elements, multiples of 8; k 16-byte aligned).
 *   recompute_mu 1: prefill.  Requires t_begin == 0 and t_end == n_tokens; mu
 *                is recomputed from tokens 64..N-1 (fixed adjacent-pair fp32
 *                tree over the token axis, then one rounded division), then
 *                codes and alpha are written for tokens 0..N-1 and k_sink for
 *                0..63.  Needs workspace (SIKV_OP_ENCODE).
 *                0: append.  mu is kept; codes and alpha are written for
 *                t_begin..t_end-1 (t_end <= capacity; rows below 64 also go to
 *                k_sink).  The caller then raises n_tokens.  Needs no workspace.
 *   alpha is the adjacent-pair fp32 tree of |fl(k_c - mu_c)| over the 128
 *   channels times 2^-7.  Results are bit-identical to that definition.
 *   With a codebook, prefill also writes it: centre (j, p) = mean over the
 *   tokens 64..N-1 whose sub-vector j has pattern p of x = fl(fl(k_c - mu_c) /
 *   alpha_t) (0 if alpha_t = 0), summed exactly as rint(x * 2^24) in int64,
 *   then fl32((sum * 2^-24) / count) in fp64; an empty cluster keeps its sign
 *   vertex.  Bit-identical to that definition.  Prefill workspace grows by
 *   B*Hkv*ceil(N/4096)*2560*8 bytes.
 */
sikv_status sikv_encode(const sikv_cache_desc *cache, const uint16_t *k, int64_t k_stride_b,
                        int64_t k_stride_h, int64_t k_stride_t, int32_t t_begin, int32_t t_end,
                        int32_t recompute_mu, void *ws, size_t ws_bytes, void *stream);

/*
 * sikv_encode_v - 2-bit value codes of tokens t_begin..t_end-1 (requires vrec
 * and v_sink in the descriptor), bytes 0..47 of their records.  Per token and group of 32 channels: z = min
 * (+0 when zero), s = fl32((max - z) / 3), both rounded to fp16 (nearest even);
 * code = clamp(rint(fl32(fl32(v - z16) / s16)), 0, 3), 0 when s16 = 0.  Rows
 * below 64 are also copied whole to v_sink.  Stateless per token: the same call
 * serves prefill and append.  Bit-identical to that definition.
 *   v  bf16 values of those tokens: element (b,h,t,c) at v[b*v_stride_b +
 *      h*v_stride_h + (t - t_begin)*v_stride_t + c] (strides multiples of 8,
 *      16-byte aligned).  No workspace.
 */
sikv_status sikv_encode_v(const sikv_cache_desc *cache, const uint16_t *v, int64_t v_stride_b,
                          int64_t v_stride_h, int64_t v_stride_t, int32_t t_begin, int32_t t_end,
                          void *stream);

/*
 * sikv_score_topk - compressed-domain retrieval (§2.1 item 2).  For every KV
 * head h the selection query is the sum of its G query heads; its table holds,
 * per sub-vector j and pattern p, the dot product of the query's 4 channels
 * with the sign vertex p (+1 for bit 0, -1 for bit 1).  The score of token t is
 * alpha_t * sum_j LUT[j][nibble_j(code_t)] (fp32), and the top_k tokens of
 * 64..N-1 with the largest scores (ties: smaller t) are written to idx.
 *   q          bf16 [B][n_q_heads][128], contiguous.
 *   top_k      1..N-64.
 *   idx        int32 [B][Hkv][top_k], ascending token positions.
 *   scores_opt NULL, or fp32 [B][Hkv][capacity] (logical positions, also for a
 *          paged cache): receives every candidate's
 *              score (test hook; entries t < 64 and t >= N untouched).
 */
sikv_status sikv_score_topk(const sikv_cache_desc *cache, const uint16_t *q, int32_t n_q_heads,
                            int32_t top_k, int32_t *idx, float *scores_opt, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * sikv_sparse_attn - attention over the 64 sinks plus the selected tokens,
 * dequantisation fused in (§2.1 items 3 and 4).  For query head g of KV head
 * h and S = {0..63} U idx[b][h]: key_t = k_sink row (t < 64) or
 * mu + alpha_t * v(code_t); logit = sm_scale * q_g . key_t; softmax over S;
 * out = sum_t p_t V_t.  fp32 arithmetic, fp32 output.
 *   idx  int32 [B][Hkv][top_k], distinct positions in 64..N-1 (any order;
 *        ascending is fastest).  Not checked on the device.
 *   out  fp32 [B][n_q_heads][128].
 */
sikv_status sikv_sparse_attn(const sikv_cache_desc *cache, const uint16_t *q, int32_t n_q_heads,
                             const int32_t *idx, int32_t top_k, float sm_scale, float *out,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * sikv_decode_step - sikv_score_topk followed by sikv_sparse_attn on the same
 * stream.  The current token must already be in the cache (sikv_encode with
 * recompute_mu = 0).  idx_out_opt: NULL, or int32 [B][Hkv][top_k] to receive
 * the selection.
 */
sikv_status sikv_decode_step(const sikv_cache_desc *cache, const uint16_t *q, int32_t n_q_heads,
                             int32_t top_k, float sm_scale, int32_t *idx_out_opt, float *out,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * sikv_append_decode_step - the current token's key enters the cache and the
 * step runs, in one call: exactly sikv_encode(k_new, t_begin = n_tokens-1,
 * t_end = n_tokens, recompute_mu = 0) followed by sikv_decode_step, with the
 * encode folded into the step's first kernel (one launch fewer per step).
 * Results (codes and scale of the new row, idx, out) are bit-identical to the
 * two calls.  n_tokens already counts the new token.
 *   k_new  bf16 key of token n_tokens-1: element (b,h,c) at
 *          k_new[b*k_stride_b + h*k_stride_h + c] (strides in elements,
 *          multiples of 8; 16-byte aligned).
 *   v_new  NULL, or (quantised values) that token's bf16 value row, same
 *          stride scheme, encoded as sikv_encode_v would before the step.
 * Workspace: SIKV_OP_DECODE_STEP.
 */
sikv_status sikv_append_decode_step(const sikv_cache_desc *cache, const uint16_t *k_new,
                                    int64_t k_stride_b, int64_t k_stride_h,
                                    const uint16_t *v_new, int64_t v_stride_b,
                                    int64_t v_stride_h, const uint16_t *q, int32_t n_q_heads,
                                    int32_t top_k, float sm_scale, int32_t *idx_out_opt,
                                    float *out, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the library's static device scratch (sikv_append_decode_step_static). */
#define SIKV_STATIC_SCRATCH_BYTES ((size_t)80 << 20)

/*
 * sikv_append_decode_step_static - sikv_append_decode_step for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and results.  Its scratch is a static array of
 * SIKV_STATIC_SCRATCH_BYTES in the library's device code, one per GPU, held
 * until the process ends; the call allocates and frees nothing.
 *   - Calls whose workspace need, sikv_workspace_bytes(SIKV_OP_DECODE_STEP,
 *     ...), exceeds SIKV_STATIC_SCRATCH_BYTES return SIKV_ERR_WORKSPACE and
 *     launch nothing (80 MiB covers 4 x 8 KV heads at 128K tokens).
 *   - The scratch of the stream's device is used (the current device for the
 *     null stream).  Every call on one GPU shares it and it keeps the last
 *     call's contents (no kernel reads scratch it did not write in the same
 *     call): calls that overlap on one GPU, on different streams or threads,
 *     race and give undefined results.  Serialise them.
 */
sikv_status sikv_append_decode_step_static(const sikv_cache_desc *cache, const uint16_t *k_new,
                                           int64_t k_stride_b, int64_t k_stride_h,
                                           const uint16_t *v_new, int64_t v_stride_b,
                                           int64_t v_stride_h, const uint16_t *q,
                                           int32_t n_q_heads, int32_t top_k, float sm_scale,
                                           int32_t *idx_out_opt, float *out, void *stream);

/* Workspace bytes needed by `op` (SIKV_OP_*) for this cache and call shape.
 * Host only, launches nothing.  Returns 0 for an invalid combination. */
size_t sikv_workspace_bytes(int32_t op, const sikv_cache_desc *cache, int32_t n_q_heads,
                            int32_t top_k);

/* Static description of a status code; never NULL. */
const char *sikv_status_str(sikv_status status);

int32_t sikv_abi_version(void);
size_t sikv_desc_size(void);

/*
 * Measurement helpers (not part of the method).
 *
 * sikv_dense_attn - dense bf16 decode attention over all N tokens of an
 * unquantised cache (the comparator the method is measured against): for query
 * head g of KV head h, softmax(sm_scale * q_g . K_t) over t < N, times V.
 * K and V bf16 with the stride scheme of sikv_cache_desc; q bf16
 * [B][n_q_heads][128]; out fp32 [B][n_q_heads][128].  Workspace from
 * sikv_dense_workspace_bytes.  timer: NULL or a caller-owned timer (as in the
 * descriptor).
 */
sikv_status sikv_dense_attn(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                            int32_t n_tokens, const uint16_t *q, const uint16_t *k,
                            int64_t k_stride_b, int64_t k_stride_h, int64_t k_stride_t,
                            const uint16_t *v, int64_t v_stride_b, int64_t v_stride_h,
                            int64_t v_stride_t, float sm_scale, float *out, void *ws,
                            size_t ws_bytes, void *stream, sikv_timer *timer);
size_t sikv_dense_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                  int32_t n_tokens);

/*
 * Comparators of the pages' module speed-ups (technical summary §4, efficiency:
 * the sign clustering against K-means with 20 iterations; LUT retrieval against
 * the full dot product).  Not part of the decode path.
 *
 * sikv_kmeans_codebook - the iterative clustering that the one-pass sign
 * clustering replaces (§2.1 item 1): n_iter (1..1000) Lloyd iterations over the
 * points x = fl32(fl32(k - mu) / alpha_t) of the prefill tokens [64, n_tokens),
 * 16 clusters per sub-vector position, started from the 16 sign vertices; a
 * point goes to its nearest centre, the squared distance in fp32 as
 * ((d0^2 + d1^2) + d2^2) + d3^2 with d_i = fl32(x_i - c_i), the lowest index
 * on ties; a centre is the mean of its points (sums of rint(x * 2^24) in int64,
 * exact; fl32((sum * 2^-24) / count) in fp64); an empty cluster keeps its
 * centre.  One iteration gives exactly the one-pass codebook.  Needs the
 * cache's codebook (written), mu and alpha (from sikv_encode's prefill over the
 * same keys k, laid out as in sikv_encode).  Workspace: SIKV_OP_KMEANS.
 */
sikv_status sikv_kmeans_codebook(const sikv_cache_desc *cache, const uint16_t *k,
                                 int64_t k_stride_b, int64_t k_stride_h, int64_t k_stride_t,
                                 int32_t n_iter, void *ws, size_t ws_bytes, void *stream);

/*
 * sikv_dense_scores - full dot-product retrieval scores: scores[(b*n_kv_heads +
 * h) * n_tokens + t] = qbar_h . K[b,h,t] for every t < n_tokens, with qbar_h the
 * fp32 sum (g ascending) of the G query rows h*G..h*G+G-1 (the selection query
 * of the LUT-GEMV score), K bf16 with the stride scheme of sikv_cache_desc,
 * q bf16 [B][n_q_heads][128].  No workspace.  timer: NULL or a caller-owned
 * timer.
 */
sikv_status sikv_dense_scores(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                              int32_t n_tokens, const uint16_t *q, const uint16_t *k,
                              int64_t k_stride_b, int64_t k_stride_h, int64_t k_stride_t,
                              float *scores, void *stream, sikv_timer *timer);

/* Plain device copy of `bytes` (multiple of 16, both pointers 16-byte
 * aligned): the reference kernel for bandwidth and traffic-counter scaling.
 * timer: NULL or a caller-owned timer. */
sikv_status sikv_stream_copy(void *dst, const void *src, size_t bytes, void *stream,
                             sikv_timer *timer);

/*
 * Kernel timer (measurement only, not part of the method).  A timer is a host
 * object owned by the caller: sikv_timer_create makes one, sikv_timer_destroy
 * frees it and its events.  A call whose descriptor (or timer argument) names
 * a timer brackets each kernel it launches with two HIP events recorded with
 * the launch itself, on the call's stream, created on the current device the
 * first time they are needed and reused afterwards.  sikv_timer_read
 * synchronises on the pending events and returns, per kernel id
 * (0 <= id < sikv_timer_count()), the number of launches and their summed
 * duration in milliseconds since the last reset.  A timer must be used by one
 * thread at a time and on one device; separate timers are independent.
 */
sikv_status sikv_timer_create(sikv_timer **out);
sikv_status sikv_timer_destroy(sikv_timer *timer);
sikv_status sikv_timer_reset(sikv_timer *timer);
sikv_status sikv_timer_read(sikv_timer *timer, int32_t id, int64_t *launches, double *total_ms);
int32_t sikv_timer_count(void);          /* number of kernel ids (a constant)        */
const char *sikv_timer_name(int32_t id); /* static name of kernel id; never NULL     */

#ifdef __cplusplus
}
#endif

#endif /* SIKV_H */
