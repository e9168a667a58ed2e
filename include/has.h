/* has.h -- head-aware sparse decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libhas.so.  The operations follow three method descriptions:
 *
 *   [AoH]  "Resumen Técnico: Autonomía de Cabezales (Autonomy-of-Heads, AoH)"
 *          (gist.science, paper 2608.06849), Metodología §1-§4.
 *   [FASA] "FASA: Frequency-aware Sparse Attention" (gist.science, paper
 *          2602.03152), §2.A-§2.C.
 *   [CLSA] "El enrutamiento compartido entre capas acelera la atención
 *          dispersa 7 veces ..." (seventnews.com, on "CLSA: You Only Index
 *          Once"), section "Cómo funciona CLSA".
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer to contiguous row-major data
 *     (one exception, stated at the split cache), aligned to 16 bytes, owned
 *     by the caller.  The library never allocates
 *     or frees memory and never synchronises the stream.
 *   - `stream` is a hipStream_t (NULL = the default stream); all device work
 *     is enqueued on it, in order, and is asynchronous to the host.
 *   - `ws`/`ws_bytes` is caller-owned scratch memory of at least the size the
 *     matching *_workspace() query returns; its contents on entry do not
 *     matter and are undefined on exit.  Two calls that run concurrently
 *     must not share a workspace.
 *   - Arguments are validated on the host before anything is enqueued: an
 *     error status means nothing was launched and no output was written.
 *     HAS_ERR_HIP means a HIP call failed while enqueueing; outputs are then
 *     undefined.  has_last_error() gives a message (thread-local).
 *   - Array contents are not checked (finite values; i_dom entries distinct
 *     and in [0, d_head/2); labels in {0, 1}), except when the environment
 *     variable HAS_DEBUG is "1": then i_dom and labels are copied to the host
 *     (synchronising `stream`) and checked before anything is launched, and
 *     a violation returns HAS_ERR_INVALID_ARG.
 *   - The first decode call on each device creates a side stream and two
 *     events (kept until the process ends).  When a call's streaming groups
 *     attend to at least 2^20 cache rows in total, their attention runs on
 *     that side stream, ordered after the caller's stream and joined back
 *     into it before the call's last kernel, so the caller sees one ordered
 *     sequence on `stream`.  Smaller calls enqueue everything on `stream`.
 *   - Threads may call the library concurrently on distinct streams (their
 *     side-stream work is serialised).
 */
#ifndef HAS_H_
#define HAS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int has_status;
#define HAS_OK 0
#define HAS_ERR_INVALID_ARG 1 /* a size, pointer or alignment is invalid */
#define HAS_ERR_UNSUPPORTED 2 /* valid, but outside what the kernels implement */
#define HAS_ERR_WORKSPACE 3   /* ws is NULL or smaller than the query says */
#define HAS_ERR_HIP 4         /* a HIP runtime call failed */

typedef enum { HAS_F32 = 0, HAS_BF16 = 1 } has_dtype;

/* Rotary pairing of the d/2 frequency chunks ([FASA] §2.A: RoPE splits a
 * d-vector into d/2 two-dimensional subspaces).  Chunk f holds channels
 * (f, f + d/2) in the rotate-half layout and (2f, 2f + 1) in the interleaved
 * layout. */
#define HAS_ROPE_ROTATE_HALF 0
#define HAS_ROPE_INTERLEAVED 1

const char* has_status_string(has_status s);
const char* has_last_error(void);

/* ------------------------------------------------------------------ AoH --
 * aoh_label: data-free head labelling from frozen weights ([AoH] §1-§4).
 *
 * For query head h of layer l, with KV group g = h / (n_q_heads/n_kv_heads):
 *   W_Q^h = w_q[l, h*d_head : (h+1)*d_head, :]    (d_head x d_model)
 *   W_K^g = w_k[l, g*d_head : (g+1)*d_head, :]
 *   C_h = (W_Q^h W_Q^hT)(W_K^g W_K^gT)           ([AoH] §3, d_head x d_head)
 * whose eigenvalues are the squared nonzero singular values sigma^2 of the
 * operator M_h = W_K^T W_Q ([AoH] §1).  Then, with s = sigma / sum(sigma),
 *   er_head[l, h]  = exp(-sum_k s_k ln s_k)       ([AoH] §2; 0 ln 0 = 0)
 *   er_group[l, g] = mean of er_head over the group's query heads ([AoH] §4)
 *   labels[l, g]   = 1 (retrieval) for the n_retrieval lowest er_group over
 *                    all (l, g), ties to the lower l*n_kv_heads + g; when
 *                    n_retrieval < 0, labels = (er_group < er_threshold).
 *                    0 = streaming.
 *
 * w_q: [n_layers, n_q_heads*d_head, d_model], w_k: [n_layers,
 * n_kv_heads*d_head, d_model], both of dtype `wdt` (the layout of a
 * PyTorch nn.Linear weight).  er_head [n_layers, n_q_heads] f32 and
 * er_group [n_layers, n_kv_heads] f32 may be NULL; labels
 * [n_layers, n_kv_heads] uint8 is required.
 * Supported: d_head in {64, 128}, d_model a multiple of 64, d_model >= d_head,
 * 0 <= n_retrieval <= n_layers*n_kv_heads (or < 0 for the threshold).
 * Precision: the Gram products W W^T accumulate in fp32 on the matrix
 * cores; the Cholesky factor, the congruence L^T G_Q L (fp64 matrix cores)
 * and the tridiagonalisation run in fp64; eigenvalue bisection in fp32. */
size_t aoh_label_workspace(int n_layers, int n_q_heads, int n_kv_heads, int d_model, int d_head);
has_status aoh_label(int n_layers, int n_q_heads, int n_kv_heads, int d_model, int d_head,
                     has_dtype wdt, const void* w_q, const void* w_k, int n_retrieval,
                     float er_threshold, float* er_head, float* er_group, uint8_t* labels,
                     void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------- decode --
 * Shape of one decode call.  n_layers layers, `batch` sequences, each with a
 * cache of ctx_len tokens at positions 0..ctx_len-1 (the current token
 * included); queries are for position ctx_len-1.
 *   n_q_heads % n_kv_heads == 0, G = n_q_heads / n_kv_heads in {1,2,4,8}
 *   d_head in {64, 128}; 1 <= n_dom <= d_head/2, and n_dom <= 32 for fp32
 *   caches (the dominant-key row holds at most 256 bytes; else
 *   HAS_ERR_UNSUPPORTED)
 *   1 <= n_fac <= ctx_len; n_sink >= 0, window >= 0, n_sink + window >= 1
 *   ctx_len <= 4194304; n_layers * n_kv_heads <= 8192
 */
typedef struct has_decode_dims {
  int n_layers;
  int batch;
  int n_q_heads;
  int n_kv_heads;
  int d_head;
  int ctx_len;
  int n_fac;      /* tokens kept per retrieval (layer, sequence, KV group) */
  int n_sink;     /* streaming heads: first n_sink tokens ... */
  int window;     /* ... plus the last `window` tokens */
  int n_dom;      /* |I_dom|, dominant frequency chunks per KV group */
  int kv_dtype;   /* has_dtype of q, k_cache, v_cache, k_dom */
  int rope_layout;/* HAS_ROPE_ROTATE_HALF or HAS_ROPE_INTERLEAVED */
} has_decode_dims;

/* Elements per row of the dominant-key copy: 2*n_dom rounded up to a power
 * of two count of 16-byte vectors (zero padded). */
int kdom_row_elems(const has_decode_dims* dims);

/* kdom_pack: builds the dominant-chunk key copy that TIP scoring reads
 * ([FASA] §2.C: only the dominant key components need to be touched for
 * scoring).  For every cache row t of slice (l, b, g) and i < n_dom, c in {0,1}:
 *   k_dom[l,b,g,t, 2i+c] = k_cache[l,b,g,t, chan(i_dom[l,g,i], c)]
 * with chan() from rope_layout; the padding elements are 0.
 * k_cache [n_layers,batch,n_kv_heads,ctx_len,d_head] (kv_dtype), i_dom
 * [n_layers,n_kv_heads,n_dom] int32, k_dom
 * [n_layers,batch,n_kv_heads,ctx_len,kdom_row_elems] (kv_dtype).
 * Meant for cache-write time; not part of a decode step. */
has_status kdom_pack(const has_decode_dims* dims, const void* k_cache, const int32_t* i_dom,
                     void* k_dom, void* stream);

/* sparse_decode_step: one decode step of head-heterogeneous token-sparse
 * attention over all n_layers layers.  For every (l, b, g):
 *   labels[l,g] = 1 (retrieval, [FASA] §2.B):
 *     qbar = mean of q[l,b,h] over the group's heads h;
 *     s_t  = sum over f in i_dom[l,g] of the chunk-f part of qbar . k_t
 *            (TIP, [FASA] §2.B.1), for t < ctx_len, fp32;
 *     S    = the n_fac tokens with the largest s_t, ties to the lower t;
 *   labels[l,g] = 0 (streaming, [AoH] §4):
 *     S    = [0, n_sink) united with [ctx_len - window, ctx_len).
 *   For each head h of the group (FAC, [FASA] §2.B.2, full d_head):
 *     out[l,b,h] = sum_{t in S} softmax_t(q[l,b,h].k_t / sqrt(d_head)) v_t.
 * q [n_layers,batch,n_q_heads,d_head] and the caches
 * [n_layers,batch,n_kv_heads,ctx_len,d_head] hold post-RoPE values of
 * kv_dtype; k_dom is kdom_pack's output for the same i_dom; labels
 * [n_layers,n_kv_heads] uint8; out [n_layers,batch,n_q_heads,d_head] f32.
 * idx_out [n_layers,batch,n_kv_heads,n_fac] int32 receives S ascending for
 * retrieval groups and -1 for streaming groups; it may be NULL.
 * Accumulation is fp32; scores and selection are deterministic. */
size_t sparse_decode_workspace(const has_decode_dims* dims);

/* Which of the two exact selection paths ([FASA] §2.B.1 top-N_fac, the same
 * set either way) sparse_decode_step takes for these dims; host only, no HIP
 * call.  1: prefiltered (a sampled key threshold; TIP writes only the tokens
 * at or above it, and the final kernel ranks them, or on steps of at most 512
 * attention units without the side stream the attention units themselves).
 * 0: general (TIP writes every
 * score, an exact radix threshold follows).  -1: invalid dims, the reason in
 * has_last_error().  The prefiltered path needs 8192 <= ctx_len <= 524288
 * and its 16384 candidate slots to hold the expected candidates with room to
 * spare (their expected count within 80% of the slots), and beyond ctx_len
 * 131072 also n_fac <= 8192. */
int sparse_selection_path(const has_decode_dims* dims);
has_status sparse_decode_step(const has_decode_dims* dims, const void* q, const void* k_cache,
                              const void* v_cache, const void* k_dom, const int32_t* i_dom,
                              const uint8_t* labels, float* out, int32_t* idx_out, void* ws,
                              size_t ws_bytes, void* stream);

/* sparse_decode_step_noalloc: sparse_decode_step for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and errors as sparse_decode_step, without ws/ws_bytes: the
 * scratch is a fixed array of HAS_NOALLOC_SCRATCH_BYTES in device memory,
 * one per GPU, set up by the first call on that GPU and held until the
 * process ends.  The call itself allocates nothing.  Dims whose
 * sparse_decode_workspace() exceeds HAS_NOALLOC_SCRATCH_BYTES are rejected
 * with HAS_ERR_WORKSPACE before anything is launched (64 MiB covers one
 * Llama-3-8B-shaped layer at batch 16 and 32768 tokens, or batch 4 at
 * 131072).  Every call on one GPU shares that GPU's array, and each call
 * leaves its contents behind: two calls that can overlap on one GPU (on
 * different streams, or from different threads without ordering) race on
 * it and their results are undefined. */
#define HAS_NOALLOC_SCRATCH_BYTES (64u << 20)
has_status sparse_decode_step_noalloc(const has_decode_dims* dims, const void* q, const void* k_cache,
                                      const void* v_cache, const void* k_dom, const int32_t* i_dom,
                                      const uint8_t* labels, float* out, int32_t* idx_out, void* stream);

/* sparse_decode_step_per_head: the per-query-head selection variant, to
 * ablate the group-mean TIP above ([FASA] §2.B.1 scores with one head's
 * query; with G heads per KV group, sparse_decode_step scores with their mean
 * and the group shares one index).  Here every query head h of a retrieval
 * group selects its own n_fac tokens from its own scores
 *   s_t = sum over f in i_dom[l,g] of the chunk-f part of q[l,b,h] . k_t
 * (ties to the lower t) and attends over them; streaming groups as in
 * sparse_decode_step.  Arguments as in sparse_decode_step except idx_out
 * [n_layers,batch,n_q_heads,n_fac] (-1 rows for heads of streaming groups),
 * and n_layers * n_q_heads <= 8192.  It gathers G times the selected rows
 * of sparse_decode_step; a group's dominant key rows and streaming rows are
 * still read once for its G heads (bf16 caches on steps large enough for a
 * separate threshold launch; otherwise each head reads them). */
size_t sparse_decode_per_head_workspace(const has_decode_dims* dims);
has_status sparse_decode_step_per_head(const has_decode_dims* dims, const void* q, const void* k_cache,
                                       const void* v_cache, const void* k_dom, const int32_t* i_dom,
                                       const uint8_t* labels, float* out, int32_t* idx_out, void* ws,
                                       size_t ws_bytes, void* stream);

/* Split cache ([AoH] §4: a streaming head only ever attends to the sink and
 * the recent window, so it need not keep the rest of its cache).  With
 * n_ret pairs (l, g) labelled retrieval and n_str = n_layers*n_kv_heads -
 * n_ret labelled streaming, each kind numbered in increasing l*n_kv_heads+g:
 *   k_ret, v_ret  [n_ret, batch, capacity, d_head]   full rows, row = position
 *   k_dom_ret     [n_ret, batch, capacity, kdom_row_elems]
 *   k_str, v_str  [n_str, batch, n_sink + window, d_head]
 * A streaming group's row for position p sits in slot p when p < n_sink,
 * else in slot n_sink + (p - n_sink) mod window (the window is a ring).
 * The caller sizes the arrays from the labels; the library cannot check
 * their extents.  k_ret and v_ret may instead live in pinned host memory
 * (hipHostMalloc): the memory-saving variant of [FASA] §2.C (FASA-M), where
 * only the dominant-key copy k_dom_ret stays in HBM and the selected rows
 * are read over the host link.  The library maps them to their
 * device-visible address; memory that is neither device memory nor pinned
 * host memory is rejected (HAS_ERR_INVALID_ARG).  Every other array is
 * device memory.
 *
 * kv_append: writes positions [pos, pos + n_new) of new post-RoPE rows
 * k_new, v_new [n_layers, batch, n_kv_heads, n_new, d_head] into a split
 * cache: a retrieval group gets its rows and their dominant-chunk copy
 * (as kdom_pack) at those positions; a streaming group keeps the positions
 * below n_sink and the last `window` positions of the call.  One call per
 * decoded token (n_new = 1) keeps the cache current; one call with pos = 0
 * fills it from a prefill.  Calls must come in increasing position order
 * for the rings to hold the latest window.  dims->ctx_len and n_fac are not
 * used; 0 <= pos, 1 <= n_new, pos + n_new <= capacity <= 4194304. */
has_status kv_append(const has_decode_dims* dims, int capacity, int pos, int n_new, const void* k_new,
                     const void* v_new, const int32_t* i_dom, const uint8_t* labels, void* k_ret, void* v_ret,
                     void* k_dom_ret, void* k_str, void* v_str, void* stream);

/* sparse_decode_step_split: sparse_decode_step over a split cache holding
 * positions 0..ctx_len-1 (ctx_len <= capacity): the same results, reading
 * retrieval groups' rows and k_dom from their slabs and streaming groups'
 * sink and window from their rings.  q, i_dom, labels, out and idx_out as
 * in sparse_decode_step; the workspace is sparse_decode_workspace(dims). */
has_status sparse_decode_step_split(const has_decode_dims* dims, int capacity, const void* q, const void* k_ret,
                                    const void* v_ret, const void* k_dom_ret, const void* k_str, const void* v_str,
                                    const int32_t* i_dom, const uint8_t* labels, float* out, int32_t* idx_out,
                                    void* ws, size_t ws_bytes, void* stream);

/* shared_index_decode: CLSA mode ([CLSA] "Cómo funciona CLSA").  The
 * dims->n_layers = N layers share ONE cache.  The index is computed once per
 * (b, g) by TIP + top-n_fac (as in sparse_decode_step) from the indexer
 * query q_index [batch,n_q_heads,d_head] (NULL: q[0]) and then reused by all
 * N layers: for layer n with labels[n,g] = 1 (or labels == NULL),
 *   out[n,b,h] = FAC over the shared index with the layer's own q[n,b,h];
 * with labels[n,g] = 0 the layer attends to sink + window of the cache.
 * q [N,batch,n_q_heads,d_head]; k_cache, v_cache [batch,n_kv_heads,ctx_len,
 * d_head]; k_dom [batch,n_kv_heads,ctx_len,kdom_row_elems] (kdom_pack with
 * n_layers = 1); i_dom [n_kv_heads,n_dom]; labels [N,n_kv_heads] or NULL;
 * out [N,batch,n_q_heads,d_head] f32; idx_out [batch,n_kv_heads,n_fac] or
 * NULL. */
size_t shared_index_workspace(const has_decode_dims* dims);
has_status shared_index_decode(const has_decode_dims* dims, const void* q, const void* q_index,
                               const void* k_cache, const void* v_cache, const void* k_dom,
                               const int32_t* i_dom, const uint8_t* labels, float* out,
                               int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* sparse_select: the index alone -- the TIP scores and exact top-n_fac of
 * sparse_decode_step's retrieval branch ([FASA] §2.B.1) -- for one layer
 * over one cache, so that it can serve several fac_attend calls ([CLSA]
 * "Cómo funciona CLSA": the index is computed once and later layers attend
 * over it).  dims->n_layers must be 1; n_sink and window are not used.
 * q_index [batch,n_q_heads,d_head]; k_dom [batch,n_kv_heads,ctx_len,
 * kdom_row_elems] (kdom_pack with n_layers = 1); i_dom [n_kv_heads,n_dom];
 * idx_out [batch,n_kv_heads,n_fac] int32 (required) receives each group's
 * selection, ascending, ties to the lower token. */
size_t sparse_select_workspace(const has_decode_dims* dims);
has_status sparse_select(const has_decode_dims* dims, const void* q_index, const void* k_dom,
                         const int32_t* i_dom, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* fac_attend: FAC attention of one layer over a given index ([FASA] §2.B.2):
 *   out[b,h] = sum over the n_fac entries t of idx[b,g] of
 *              softmax_t(q[b,h].k_t / sqrt(d_head)) v_t,     g = h / G,
 * with full d_head rows of one cache; an entry repeated r times contributes
 * its row r times.  One sparse_select followed by one fac_attend per layer,
 * each with that layer's q, is the layer-by-layer form of the shared index
 * ([CLSA]).  dims->n_layers must be 1; n_sink, window, n_dom and
 * rope_layout are not used.  q [batch,n_q_heads,d_head] (kv_dtype); k_cache,
 * v_cache [batch,n_kv_heads,ctx_len,d_head]; idx [batch,n_kv_heads,n_fac]
 * int32 with entries in [0, ctx_len): an entry outside is clamped into that
 * range, so no read leaves the cache (with HAS_DEBUG=1 it is rejected
 * instead); out [batch,n_q_heads,d_head] f32. */
size_t fac_attend_workspace(const has_decode_dims* dims);
has_status fac_attend(const has_decode_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* idx, float* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------- diagnostics --
 * Per-kernel device time.  While enabled (process-wide), every kernel the
 * library launches is bracketed by HIP events recorded on the caller's
 * stream.  has_timing_collect waits for the recorded events, writes up to
 * `max` entries (kernel name -- a static string --, summed milliseconds,
 * launch count), clears the records and returns the number of entries, or
 * -1 if a HIP event call failed. */
has_status has_timing_enable(int on);
int has_timing_collect(const char** names, double* total_ms, int* launches, int max);

#ifdef __cplusplus
}
#endif
#endif /* HAS_H_ */
