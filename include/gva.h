/*
 * libgva -- Grouped Value Attention (GVA) absorbed decode attention on
 * AMD Instinct MI355X (gfx950).  Plain C ABI: no HIP or torch types appear in
 * the signatures; streams are passed as `void*` (a hipStream_t, NULL for the
 * default stream).
 *
 * The method (summaries of "Grouped Value Attention: Efficient KV Caching
 * via On-Demand Key Reconstruction"):
 *   - The cache keeps only G grouped value rows V[T,G,d_h] per sequence and
 *     one positional key k_rope[T,d_r] that all H query heads share
 *     (onedev.kr review, sections "How it works" and "How it differs").
 *   - Head h's content key is rebuilt from its group's values by a fixed map,
 *     K_h = V_g(h) M_h, M_h of size d_h x d_n; because M_h is fixed the map
 *     folds into the query once per token, q~_h = q_nope,h M_h^T, and the
 *     content score is <q~_h, v_j> exactly (onedev.kr review, "How it works";
 *     bisque.today explainer, Equation 7).
 *   - Position goes through a separate decoupled-RoPE slice of width d_r: the
 *     query slice is rotated to the query position and the shared key is
 *     stored already rotated, k_rope = (x_j W_r) R_j^T (onedev.kr review,
 *     "How it differs").
 *
 * Conventions shared by every entry point
 *   Memory    All tensor pointers are DEVICE pointers to dense row-major
 *             arrays, owned by the caller; the library allocates and frees
 *             nothing and keeps no state between calls (the one exception
 *             is the fixed device scratch of gva_decode_step_noalloc).
 *             Pointers to arrays read with vector loads (marked "16B") must
 *             be 16-byte aligned.
 *   Streams   Every call only enqueues work on `stream` and returns; results
 *             are ready when the stream reaches that point.
 *   Errors    Argument errors are detected on the host before any HIP call
 *             and return a non-zero gva_status with nothing enqueued.  A
 *             failed kernel launch returns GVA_ERR_HIP.  Device-resident
 *             values (sequence lengths, positions, block ids) cannot be
 *             checked synchronously: kernels range-check them and turn an
 *             out-of-range value into NaN outputs (decode) or a skipped
 *             write (append) rather than an out-of-bounds access.
 *   Layouts   Paged caches hold `num_blocks` blocks of `block_size` tokens:
 *               v_pool [num_blocks][block_size][G][d_h]
 *               k_pool [num_blocks][block_size][d_r]
 *             Token j of sequence b lives in block block_table[b][j/bs],
 *             slot j%bs.  A contiguous cache is the identity table.
 *   Positions 0-based.  In decode the query token is the last cached token
 *             of its sequence (position seq_lens[b]-1) and attends to itself.
 *             The *_multi entry points take q_len = L tokens per sequence:
 *             token i sits at position (last position) - (L-1) + i, and in
 *             decode query i (position seq_lens[b]-L+i) attends causally to
 *             positions 0 .. seq_lens[b]-L+i.
 *   Heads     Query head h reads value group g(h) = h / (H/G).
 */
#ifndef GVA_H
#define GVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GVA_ABI_VERSION 4

typedef enum gva_status {
  GVA_OK = 0,
  GVA_ERR_NULL = 1,        /* a required pointer is NULL                    */
  GVA_ERR_SHAPE = 2,       /* a size is non-positive or sizes disagree      */
  GVA_ERR_UNSUPPORTED = 3, /* valid sizes the library has no kernel for    */
  GVA_ERR_ALIGN = 4,       /* a 16B pointer is not 16-byte aligned          */
  GVA_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returns */
  GVA_ERR_HIP = 6,         /* the HIP runtime rejected a launch             */
  GVA_ERR_SCRATCH = 7      /* needs more than the library's fixed device
                              scratch (gva_decode_step_noalloc only)        */
} gva_status;

typedef enum gva_dtype {
  GVA_F32 = 0,  /* IEEE binary32 cache                     */
  GVA_BF16 = 1  /* bfloat16 cache (round-to-nearest-even)  */
} gva_dtype;

/* Sizes of one call.  Fields an entry point does not use are ignored.
 * Supported: 1 <= H/G, H % G == 0; d_h in {32, 64, 128} (GQA: d_h in
 * {32, 64, 128}); 0 <= d_r <= 64 and even; 1 <= d_n <= 256; block_size == 64;
 * num_blocks, max_blocks >= 1; B * G <= 65535 for the entry points that
 * read the caches (one launch row per sequence and value group; larger
 * batches are GVA_ERR_UNSUPPORTED: split them).  d_r = 0 drops the positional slice: then
 * q_rope, k_new and k_pool are not read and may be NULL, and with M_h = I,
 * d_n = d_h it is the variant whose keys are the values themselves
 * (bisque.today explainer, Figure 3: half the GQA cache). */
typedef struct gva_shape {
  int32_t B;           /* sequences in the batch                      */
  int32_t H;           /* query heads                                 */
  int32_t G;           /* value groups                                */
  int32_t d_h;         /* value row width = absorbed content width    */
  int32_t d_n;         /* unrotated content slice of each query head  */
  int32_t d_r;         /* rotated position slice / shared key width (0: none) */
  int32_t block_size;  /* tokens per cache block                      */
  int32_t max_blocks;  /* columns of block_table                      */
  int32_t num_blocks;  /* blocks in each pool                         */
  int32_t cache_dtype; /* gva_dtype of v_pool and k_pool              */
} gva_shape;

/* Library ABI version (GVA_ABI_VERSION of the build). */
int32_t gva_abi_version(void);

/* Static text for a status code (never NULL). */
const char* gva_status_string(int32_t status);

/* Persistent cache scalars per token, G*d_h + d_r: the grouped values plus
 * one positional key shared by all heads, not G*d_r (onedev.kr review, "How
 * it differs": N_GVA = T*G*d_h + T*d_r).  Returns 0 for a NULL shape. */
uint64_t gva_cache_scalars_per_token(const gva_shape* shape);

/* Calibration helper, not a step of the method: the decode is bound by the
 * rate of its cache read (onedev.kr review, "Premises and limits"), and
 * this call states the achievable read rate of the same bytes with the
 * decode's load form.  It reads `bytes` bytes at `buf` with 16-byte
 * non-temporal loads, GVA_PROBE_BLOCKS blocks each over one contiguous
 * range, and block i writes the XOR of the 32-bit words of its range to
 * xor_out[i] (0 for an empty range); the XOR of all GVA_PROBE_BLOCKS words
 * is the XOR of every 32-bit word of the buffer.
 *   buf: device, 16B (may be NULL when bytes == 0); bytes: a multiple of 16;
 *   xor_out: device, GVA_PROBE_BLOCKS uint32, 4-byte aligned, all written;
 *   stream: hipStream_t or NULL.
 * Errors (before any HIP call): GVA_ERR_NULL (xor_out NULL, or buf NULL with
 * bytes > 0), GVA_ERR_ALIGN (buf not 16-byte aligned, bytes not a multiple
 * of 16, or xor_out not 4-byte aligned); a failed launch, GVA_ERR_HIP. */
#define GVA_PROBE_BLOCKS 1024
gva_status gva_stream_read_probe(const void* buf, uint64_t bytes, uint32_t* xor_out,
                                 void* stream);

/* Absorb each head's fixed key map into its query, once per query token
 * (onedev.kr review, "How it works"; bisque.today explainer, Equation 7):
 *
 *   qa[b][h][e]       = s * sum_n q_nope[b][h][n] * M[h][e][n]   (e < d_h)
 *   qa[b][h][d_h + i] = s * (R(pos[b]) q_rope[b][h])[i]           (i < d_r)
 *
 * R(p) rotates each adjacent pair (2i, 2i+1) by angle p * rope_base^(-2i/d_r)
 * (angles, sines and cosines in float64).  s = softmax_scale, or
 * 1/sqrt(d_n + d_r) when softmax_scale <= 0.
 *   q_nope [B][H][d_n] f32, q_rope [B][H][d_r] f32, M [H][d_h][d_n] f32,
 *   pos [B] i32 (query positions), qa [B][H][d_h + d_r] f32 (written).
 * Uses B, H, d_h, d_n, d_r. */
gva_status gva_absorb_query(const gva_shape* shape, const float* q_nope,
                            const float* q_rope, const float* M,
                            const int32_t* pos, float softmax_scale,
                            float rope_base, float* qa, void* stream);

/* Write one new token per sequence into the paged caches, before attention
 * (onedev.kr review, "How it differs": the positional key is cached already
 * rotated, k_rope = (x_j W_r) R_j^T):
 *
 *   v_pool[blk][slot][g][:] = round(v_new[b][g][:])
 *   k_pool[blk][slot][:]    = round(R(pos[b]) k_new[b][:])
 *
 * with blk = block_table[b][pos[b]/block_size], slot = pos[b] % block_size,
 * R as in gva_absorb_query (rotation in float64) and round the cache dtype's
 * single round-to-nearest-even from the exact value.
 *   v_new [B][G][d_h] f32, k_new [B][d_r] f32 (unrotated x_j W_r),
 *   pos [B] i32, block_table [B][max_blocks] i32, v_pool/k_pool as above.
 * A sequence whose pos or block id is out of range is skipped.
 * Uses B, G, d_h, d_r, block_size, max_blocks, num_blocks, cache_dtype. */
gva_status gva_append_cache(const gva_shape* shape, const float* v_new,
                            const float* k_new, const int32_t* pos,
                            const int32_t* block_table, float rope_base,
                            void* v_pool, void* k_pool, void* stream);

/* Bytes of workspace gva_decode_attention needs for these sizes and this
 * upper bound on sequence length: per-sequence completion counters followed
 * by the split-context partial results.  A workspace must be zero-filled
 * once, when it is allocated; every call leaves its counters zero again, so
 * it can be reused (and captured in graphs) without clearing by calls with
 * the same sizes and max_seq_len (the counters' place depends on them: a
 * workspace that served other sizes must be zero-filled again).  Calls that
 * run concurrently need separate workspaces. */
gva_status gva_decode_workspace_size(const gva_shape* shape,
                                     int32_t max_seq_len, size_t* bytes);

/* Decode attention of the absorbed query over the value cache (onedev.kr
 * review, "How it works": content attention reads only the value cache and
 * builds no key tensor):
 *
 *   score[b][h][j] = <qa[b][h][0:d_h], V[b][j][g(h)]>
 *                  + <qa[b][h][d_h:], k_rope[b][j]>          (j < seq_lens[b])
 *   p = softmax_j(score);   out[b][h] = sum_j p_j V[b][j][g(h)]
 *   lse[b][h] = log sum_j exp(score[b][h][j])
 *
 * The scale is already folded into qa (gva_absorb_query).  The context is
 * split into chunks whose partial softmax states are merged by log-sum-exp;
 * the split depends only on the sizes, so results are bitwise reproducible.
 *   qa [B][H][d_h + d_r] f32 (16B), v_pool/k_pool (16B), block_table
 *   [B][max_blocks] i32, seq_lens [B] i32 on the device, each
 *   <= min(max_seq_len, max_blocks*block_size); max_seq_len (host) >= 0;
 *   workspace of at least gva_decode_workspace_size bytes (16B, zero-filled
 *   at allocation, see above); out [B][H][d_h] f32 (16B); lse [B][H] f32 or
 *   NULL.
 * seq_lens[b] == 0 gives out = 0 and lse = -inf.  Uses every shape field
 * except d_n. */
gva_status gva_decode_attention(const gva_shape* shape, const float* qa,
                                const void* v_pool, const void* k_pool,
                                const int32_t* block_table,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                void* workspace, size_t workspace_bytes,
                                float* out, float* lse, void* stream);

/* One decode step in two launches: append each sequence's new token (when
 * v_new and k_new are given; both or neither), absorb the maps into the
 * queries, and run gva_decode_attention -- the calls above, fused.  The new
 * token and the query sit at position seq_lens[b] - 1 (seq_lens already
 * counts the new token).  The absorbed query lives in the workspace.
 *   q_nope, q_rope, M, softmax_scale, rope_base as gva_absorb_query;
 *   v_new, k_new as gva_append_cache, or both NULL; v_pool, k_pool,
 *   block_table, seq_lens, max_seq_len, out, lse as gva_decode_attention;
 *   workspace of at least gva_decode_step_workspace_size bytes (16B,
 *   zero-filled at allocation like the decode workspace).
 * Uses every shape field. */
gva_status gva_decode_step_workspace_size(const gva_shape* shape,
                                          int32_t max_seq_len, size_t* bytes);
gva_status gva_decode_step(const gva_shape* shape, const float* q_nope,
                           const float* q_rope, const float* M,
                           float softmax_scale, float rope_base,
                           const float* v_new, const float* k_new,
                           void* v_pool, void* k_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t max_seq_len, void* workspace,
                           size_t workspace_bytes, float* out, float* lse,
                           void* stream);

/* The decode and the step with the context split planned from the host copy
 * of the sequence lengths, for ragged batches.  The decode reads the whole
 * cache every step and is bound by that read (onedev.kr review, "Premises
 * and limits"); the pages leave longer and uneven contexts unmeasured
 * (agihunt.info summary, the "three gaps" paragraph).  gva_decode_attention
 * sizes its chunks from max_seq_len alone, so on a ragged batch the blocks
 * of the longest sequences hold most of the work while others sit idle.
 * Here the chunk is the smallest multiple of block_size for which the
 * batch's (sequence, chunk) items, at least one per sequence, number at most
 * 256 (one block per compute unit); every item then holds about the same
 * number of tokens.  The results equal gva_decode_attention's up to the
 * fp32 summation order (a different split), and are bitwise reproducible
 * for the same lengths.
 *   seq_lens_host [B] i32 in host memory, read during the call only: each
 *   in [0, max_seq_len] (else GVA_ERR_SHAPE, before any HIP call), and
 *   equal to seq_lens on the device.  A sequence whose device length gives
 *   another chunk count than its host length gets NaN outputs, like any
 *   other invalid length.
 *   workspace: at least gva_decode_workspace_size_lens (decode) or
 *   gva_decode_step_workspace_size_lens (step) bytes, zero-filled at
 *   allocation; these sizes depend on the shape only (not on the lengths).
 * Supported: one query token, bf16 cache, H = 4 G, the shapes the
 * matrix-core decode covers, B <= 256; other shapes give
 * GVA_ERR_UNSUPPORTED.  Other arguments, layouts and errors as
 * gva_decode_attention and gva_decode_step. */
gva_status gva_decode_workspace_size_lens(const gva_shape* shape, size_t* bytes);
gva_status gva_decode_attention_lens(const gva_shape* shape, const float* qa,
                                     const void* v_pool, const void* k_pool,
                                     const int32_t* block_table,
                                     const int32_t* seq_lens,
                                     const int32_t* seq_lens_host,
                                     int32_t max_seq_len, void* workspace,
                                     size_t workspace_bytes, float* out,
                                     float* lse, void* stream);
gva_status gva_decode_step_workspace_size_lens(const gva_shape* shape,
                                               size_t* bytes);
gva_status gva_decode_step_lens(const gva_shape* shape, const float* q_nope,
                                const float* q_rope, const float* M,
                                float softmax_scale, float rope_base,
                                const float* v_new, const float* k_new,
                                void* v_pool, void* k_pool,
                                const int32_t* block_table,
                                const int32_t* seq_lens,
                                const int32_t* seq_lens_host,
                                int32_t max_seq_len, void* workspace,
                                size_t workspace_bytes, float* out, float* lse,
                                void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * step as gva_decode_step (same kernels, bit-identical results), with the
 * workspace taken from a fixed device array inside the library instead of
 * a caller's buffer: GVA_NOALLOC_SCRATCH_BYTES per GPU, reserved when the
 * library's code is loaded on that GPU and held until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress), so make the first call outside graph
 * capture.  Every call clears the split counters it uses (in its first
 * launch), so no earlier call's contents matter.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, threads) race and must be serialised by the
 * caller.  A call whose workspace (gva_decode_step_workspace_size) exceeds
 * GVA_NOALLOC_SCRATCH_BYTES returns GVA_ERR_SCRATCH before any HIP call.
 * Other arguments, layouts and errors as gva_decode_step. */
#define GVA_NOALLOC_SCRATCH_BYTES (16u << 20)
gva_status gva_decode_step_noalloc(const gva_shape* shape, const float* q_nope,
                                   const float* q_rope, const float* M,
                                   float softmax_scale, float rope_base,
                                   const float* v_new, const float* k_new,
                                   void* v_pool, void* k_pool,
                                   const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   float* out, float* lse, void* stream);

/* Several tokens per sequence (q_len = L, 1 <= L <= 65536): the entry points
 * above with one more size.  Each query token is absorbed on its own, once
 * per head and token (onedev.kr review, "How it works"), and attends
 * causally; L = 1 is exactly the single-token call.  Layouts:
 *   q_nope [B][H][L][d_n], q_rope [B][H][L][d_r], qa [B][H][L][d_h + d_r],
 *   out [B][H][L][d_h], lse [B][H][L]      (query token i of head h);
 *   v_new [B][L][G][d_h], k_new [B][L][d_r] (new token i of sequence b).
 * gva_absorb_query_multi: pos[b] is the position of the LAST query token;
 *   token i is rotated to pos[b] - (L-1) + i.
 * gva_append_cache_multi: pos[b] is the position of the LAST new token;
 *   token i is written at pos[b] - (L-1) + i.
 * gva_decode_attention_multi: query i of sequence b sits at position
 *   seq_lens[b] - L + i and scores positions j <= seq_lens[b] - L + i only.
 *   0 < seq_lens[b] < L is invalid (NaN outputs, like other bad lengths).
 * gva_decode_step_multi: append the L new tokens (when v_new/k_new are
 *   given), absorb the L queries, decode; seq_lens already counts the new
 *   tokens.
 * Kernels: with L >= 16, or where the split kernels have no instance for
 *   the column count H*L, a bf16 cache with H/G in {1, 2, 4, 8}, d_h in
 *   {64, 128} and d_r in {0, 16, 24, 32} goes to the blocked (prefill)
 *   kernel: queries are matrix columns and each 64-token key block is
 *   staged once per block of queries (the pages note that prefill is
 *   dominated by large matrix products).  It needs no workspace
 *   (gva_decode_workspace_bytes_multi may report 0).  Other L go to the
 *   split decode kernels with H*L columns, or fail GVA_ERR_UNSUPPORTED.
 * Other arguments, errors and workspace rules as the single-token calls;
 * q_len < 1 is GVA_ERR_SHAPE, q_len > 65536 GVA_ERR_UNSUPPORTED. */
gva_status gva_absorb_query_multi(const gva_shape* shape, int32_t q_len,
                                  const float* q_nope, const float* q_rope,
                                  const float* M, const int32_t* pos,
                                  float softmax_scale, float rope_base,
                                  float* qa, void* stream);
gva_status gva_append_cache_multi(const gva_shape* shape, int32_t q_len,
                                  const float* v_new, const float* k_new,
                                  const int32_t* pos,
                                  const int32_t* block_table, float rope_base,
                                  void* v_pool, void* k_pool, void* stream);
gva_status gva_decode_workspace_size_multi(const gva_shape* shape,
                                           int32_t q_len, int32_t max_seq_len,
                                           size_t* bytes);
gva_status gva_decode_attention_multi(const gva_shape* shape, int32_t q_len,
                                      const float* qa, const void* v_pool,
                                      const void* k_pool,
                                      const int32_t* block_table,
                                      const int32_t* seq_lens,
                                      int32_t max_seq_len, void* workspace,
                                      size_t workspace_bytes, float* out,
                                      float* lse, void* stream);
gva_status gva_decode_step_workspace_size_multi(const gva_shape* shape,
                                                int32_t q_len,
                                                int32_t max_seq_len,
                                                size_t* bytes);
gva_status gva_decode_step_multi(const gva_shape* shape, int32_t q_len,
                                 const float* q_nope, const float* q_rope,
                                 const float* M, float softmax_scale,
                                 float rope_base, const float* v_new,
                                 const float* k_new, void* v_pool,
                                 void* k_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t max_seq_len,
                                 void* workspace, size_t workspace_bytes,
                                 float* out, float* lse, void* stream);

/* Decode of the GVA variant that keeps ordinary RoPE on the whole
 * reconstructed key (agihunt.info summary and cctest.ai article: the
 * best-scoring GVA row, which cannot use absorbed decode):
 *
 *   k_j  = R(j) (V[b][j][g(h)] M_h)        (rebuilt and rotated per token)
 *   score[b][h][j] = s * <R(t) q[b][h], k_j>,  t = seq_lens[b] - 1
 *   p = softmax_j(score);   out[b][h] = sum_j p_j V[b][j][g(h)]
 *
 * R as in gva_absorb_query over all d_k = shape->d_n dims; the cache holds
 * values only (d_r must be 0).  Because R(j) sits between the map and the
 * query, M_h cannot be folded into the query once per step: every key is
 * rebuilt at every step (d_h * d_k multiply-adds per token and head), which
 * is the cost the decoupled slice avoids.
 *   q [B][H][d_k] f32 (unrotated), M [H][d_h][d_k] f32, s = softmax_scale
 *   or 1/sqrt(d_k) when <= 0; v_pool, block_table, seq_lens, max_seq_len,
 *   out, lse as gva_decode_attention; workspace of at least
 *   gva_decode_rope_keys_workspace_size bytes (16B; no zero-fill needed).
 * Kernels exist for bf16 caches, d_h in {64, 128}, d_k in {16, 32, 48, 64},
 * H/G <= 8; other sizes give GVA_ERR_UNSUPPORTED.  Two launches (partial
 * records, then the log-sum-exp merge). */
gva_status gva_decode_rope_keys_workspace_size(const gva_shape* shape,
                                               int32_t max_seq_len,
                                               size_t* bytes);
gva_status gva_decode_rope_keys(const gva_shape* shape, const float* q,
                                const float* M, float softmax_scale,
                                float rope_base, const void* v_pool,
                                const int32_t* block_table,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                void* workspace, size_t workspace_bytes,
                                float* out, float* lse, void* stream);

/* Same-shape grouped-query attention decode, the baseline GVA is compared
 * with: each group stores both a key and a value row per token
 * (onedev.kr review, "What it is"; N_GQA = 2*T*G*d_h):
 *
 *   score[b][h][j] = s * <q[b][h], K[b][j][g(h)]>;  softmax;  out = sum p V
 *
 *   q [B][H][d_h] f32 (16B, position encoding already applied),
 *   k_pool/v_pool [num_blocks][block_size][G][d_h] (16B), s = softmax_scale
 *   or 1/sqrt(d_h) when <= 0; other arguments as gva_decode_attention.
 * Uses B, H, G, d_h, block_size, max_blocks, num_blocks, cache_dtype. */
gva_status gqa_decode_workspace_size(const gva_shape* shape,
                                     int32_t max_seq_len, size_t* bytes);

/* The same GQA context with q_len = L query tokens per sequence (query i at
 * position seq_lens[b] - L + i, attending causally), the comparison the
 * pages draw for prefill (onedev.kr review, "Premises and limits": prefill is
 * dominated by matrix products, so GVA need not be faster there):
 *   q [B][H][L][d_h] f32 (rotated), out [B][H][L][d_h], lse [B][H][L];
 *   other arguments, errors and workspace rules as gqa_decode_attention and
 *   the *_multi calls (L >= 16 on a bf16 cache with H/G in {1, 2, 4, 8},
 *   d_h in {64, 128} takes the blocked kernel, no workspace). */
gva_status gqa_decode_workspace_size_multi(const gva_shape* shape, int32_t q_len,
                                           int32_t max_seq_len, size_t* bytes);
gva_status gqa_decode_attention_multi(const gva_shape* shape, int32_t q_len,
                                      const float* q, float softmax_scale,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t max_seq_len,
                                      void* workspace, size_t workspace_bytes,
                                      float* out, float* lse, void* stream);
gva_status gqa_decode_attention(const gva_shape* shape, const float* q,
                                float softmax_scale, const void* k_pool,
                                const void* v_pool,
                                const int32_t* block_table,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                void* workspace, size_t workspace_bytes,
                                float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GVA_H */
