/*
 * qat.h -- C ABI of the query-aware selective sparse attention library
 * (ESA token selection and MoBA block selection) for AMD MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are caller-owned, contiguous, row-major DEVICE pointers in the
 *   token-major layout [batch, tokens, heads, head_dim] ("BTHD") unless a
 *   stride argument says otherwise. Nothing is retained after a call returns;
 *   no ownership moves across the boundary.
 * - Element types: QAT_BF16 (bfloat16) or QAT_F32 (float32) as stated per
 *   argument; selections are int32; log-sum-exp outputs are float32 in the
 *   natural-log domain.
 * - Scratch memory comes only from the caller's workspace (`ws`, `ws_bytes`),
 *   sized by the matching *_workspace_size() query; the library itself never
 *   allocates device memory. `ws` must be 256-byte aligned.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Work is enqueued asynchronously on it; no call synchronises the host.
 * - Every call returns a qat_status. Arguments are validated on the host
 *   before anything is enqueued; on QAT_EINVAL / QAT_EUNSUPPORTED /
 *   QAT_EWORKSPACE nothing has been launched and outputs are untouched.
 *   QAT_EHIP reports a failed kernel launch. qat_last_error() returns a
 *   thread-local description of the last non-OK status.
 * - Calls that share a workspace must not overlap in time.
 *
 * Sources (the pages this library implements):
 *   [ESA]  Efficient Selective Attention write-up (hlszyjy.com/post/6872.html)
 *   [MoBA] Mixture of Block Attention write-up (dtcms.com/wzjs/567377.html)
 *   [CCA]  CCA-Attention ICML 2025 write-up (m.jxzklqfsx.com/article/817694.html)
 */
#ifndef QAT_H_
#define QAT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qat_status {
  QAT_OK = 0,
  QAT_EINVAL = -1,        /* bad argument (null pointer, size, range) */
  QAT_EUNSUPPORTED = -2,  /* valid request this library does not implement */
  QAT_EWORKSPACE = -3,    /* workspace null, misaligned or too small */
  QAT_EHIP = -4           /* a HIP launch failed */
};

enum qat_dtype { QAT_F32 = 0, QAT_BF16 = 1 };

#define QAT_ABI_VERSION 3

/* Thread-local text for the last non-OK status of this thread ("" if none). */
const char* qat_last_error(void);
/* Returns QAT_ABI_VERSION of the loaded library. */
int qat_abi_version(void);

/*
 * Kernel timing for benchmarks: while enabled, the library records a pair of
 * HIP events on the launch stream around each of its main kernels
 * (names: "moba_meanpool", "moba_select", "moba_dispatch", "moba_past_attn",
 * "moba_current_attn", "moba_generic_attn", "moba_decode_select",
 * "moba_decode_attn", "moba_decode_combine", "moba_bwd_delta", "moba_bwd_dq_past",
 * "moba_bwd_dq", "moba_bwd_own", "moba_bwd_gated", "esa_bwd_dq", "esa_bwd_kv", "cca_pool", "cca_attn",
 * "esa_compress", "esa_scores" (its two passes' kernels: "esa_rowmax", "esa_colsum"),
 * "esa_decode_scan", "esa_topk", "esa_prefill_attn", "esa_decode_attn",
 * "esa_generic_attn"). The events are timing-only (created without the
 * system-scope fence on completion, so recording them does not slow the
 * kernels they bracket); qat_timing_query waits on them and returns the
 * summed milliseconds and the launch count for one name, and is meant to be
 * called after the caller has synchronised with the timed work;
 * qat_timing_reset drops the records. qat_timing_select(name) restricts the
 * records to that one stage (NULL: every stage), so that a timed region
 * carries only the events it needs. Host memory only; no device memory is
 * allocated.
 */
int qat_timing_enable(int on);
int qat_timing_select(const char* name);
int qat_timing_reset(void);
int qat_timing_query(const char* name, double* total_ms, int* count);

/* ======================================================================
 * ESA -- token-level selection by compressed q/k   [ESA]
 * ====================================================================== */

/*
 * One sequence chunk of queries at positions [chunk_start, chunk_start +
 * chunk_len) against a KV cache of ctx_len rows per sequence
 * (chunk_start + chunk_len <= ctx_len). Decode is chunk_len == 1.
 * The keys before the chunk are split into four parts ([ESA], paragraph on
 * the four-part token split): initial I = [0, min(n_init, c0)), local
 * L = [max(n_init, c0 - window), c0), middle M = [n_init, max(n_init,
 * c0 - window)) (the candidates), and the chunk itself (causal).
 */
typedef struct {
  int64_t batch;        /* sequences */
  int64_t n_heads;      /* H */
  int64_t head_dim;     /* d: 64 or 128 */
  int64_t d_c;          /* compressed dimension: multiple of 32, <= 256 */
  int64_t ctx_len;      /* rows of the KV and compressed-key caches per sequence */
  int64_t chunk_start;  /* c0 */
  int64_t chunk_len;    /* m >= 1 */
  int32_t n_init;       /* initial tokens always attended, >= 0 */
  int32_t window;       /* local tokens before the chunk, >= 0 */
  int32_t topk;         /* middle tokens selected, >= 1 */
  int32_t radius;       /* neighbour-influence radius r >= 0 */
  float clip;           /* score-correction floor C > 0 (may be +inf) */
  float scale;          /* softmax scale > 0, e.g. 1/sqrt(d) */
  int32_t dtype;        /* qat_dtype of q, K, V and outputs */
  int32_t correction;   /* qat_esa_correction: reading of the score correction */
  float vote_tau;       /* QAT_CORR_VOTES temperature; <= 0: 1/sqrt(d_c) (per head: 1/sqrt(d)) */
  int32_t per_head;     /* 0: one selection per sequence, all heads merged (esa_select);
                           1: one selection per (sequence, head) (esa_select_heads);
                           sel / n_sel then hold [batch, H, topk] / [batch, H] */
} qat_esa_params;

/*
 * The score correction of [ESA] (paragraph on score correction: keep the
 * relative size of scores, stop one token from dominating; the formula
 * itself is not in the text), in one of two readings:
 *   QAT_CORR_CLAMP  s^_ij = max(s_ij - max_j' s_ij', -clip)        (default)
 *   QAT_CORR_VOTES  s^_ij = softmax over the middle part of vote_tau * s_i.
 *                   (each query casts a total vote of 1); `clip` is unused.
 */
enum qat_esa_correction { QAT_CORR_CLAMP = 0, QAT_CORR_VOTES = 1 };

/* Workspace bytes for esa_select (or esa_select_heads) + esa_sparse_attn with
 * these parameters. */
int esa_workspace_size(const qat_esa_params* p, size_t* bytes);

/*
 * Compression by the one-layer map of [ESA] (paragraph on compressing q and
 * k to about 3.2% with a one-layer MLP; read as one affine map):
 *   out[i, :] = round(W x[i, :] + bias)
 * x: n rows of d_model elements (in_dtype), row i at x + i*x_stride elements;
 * x and W 16-byte aligned, x_stride a multiple of 8 (QAT_EINVAL otherwise).
 * W: [d_c, d_model] (in_dtype), bias: [d_c] float32 or NULL.
 * out: row i at out + i*out_stride elements, out_dtype QAT_F32 or QAT_BF16.
 * Accumulation is float64, rounded once (nearest even) to out_dtype, so the
 * bf16 compressed-key cache holds the correctly rounded exact products.
 * ws may be NULL when ws_bytes from esa_compress_workspace_size() is 0.
 */
int esa_compress_workspace_size(int64_t n, int64_t d_model, int64_t d_c, size_t* bytes);
int esa_compress(const void* x, int64_t n, int64_t x_stride, int64_t d_model, int32_t in_dtype,
                 const void* W, const float* bias, int64_t d_c,
                 void* out, int64_t out_stride, int32_t out_dtype,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Token selection ([ESA], paragraphs on query-aware importance, head merging,
 * score correction, neighbour influence and top-k):
 *   q~_i   = Wq concat_h(q_i^h) + bq                 (float64 -> float32)
 *   s_ij   = <q~_i, k~_j>,  j in M                     (k~ = compressed cache)
 *   u_j    = sum_i max(s_ij - max_j' s_ij', -clip)     (correction; READING)
 *   u'_j   = max{u_t : t in M, |t - j| <= radius}       (neighbour; READING)
 *   sel    = positions of the min(topk, |M|) largest u'_j, ties to the
 *            smaller position, ascending, -1 padded.
 * q: [batch, chunk_len, H, d] (dtype), Wq: [d_c, H*d] (dtype), bq: [d_c]
 * float32 or NULL, kc_cache: [batch, ctx_len, d_c] bfloat16 (as written by
 * esa_compress). Outputs: sel [batch, topk] int32, n_sel [batch] int32,
 * scores [batch, |M|] float32 (u'_j, may be NULL). Requires p->per_head == 0.
 */
int esa_select(const qat_esa_params* p, const void* q, const void* Wq, const float* bq,
               const void* kc_cache, int32_t* sel, int32_t* n_sel, float* scores,
               void* ws, size_t ws_bytes, void* stream);

/*
 * Per-head token selection, the comparison arm of [ESA]'s ablation on head
 * merging (the write-up scores with all heads merged and reports that doing
 * so changes little against selecting per head). READING: with no per-head
 * compression map given, head h scores the middle part with its own
 * uncompressed rows, s^h_ij = <q_i^h, k_j^h> (bf16 products, float32 sums),
 * then the correction (vote_tau <= 0 means 1/sqrt(d)), the sum over the
 * chunk's queries, the neighbour step and the top-k run per head, exactly as
 * in esa_select.
 * Requires p->per_head == 1, bfloat16 (QAT_EUNSUPPORTED otherwise) and one
 * sequence's cache below 2^31 elements; d_c is ignored.
 * q: [batch, chunk_len, H, d], k_cache: [batch, ctx_len, H, d]. Outputs:
 * sel [batch, H, topk] int32 (ascending, -1 padded), n_sel [batch, H]
 * int32, scores [batch, H, |M|] float32 (u'_j per head, may be NULL).
 * esa_sparse_attn / esa_sparse_attn_bwd with the same params (per_head = 1)
 * let head h attend its own selection.
 */
int esa_select_heads(const qat_esa_params* p, const void* q, const void* k_cache, int32_t* sel, int32_t* n_sel,
                     float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Attention over the fused parts ([ESA], global attention over initial plus
 * selected tokens fused with window attention over local tokens; [CCA],
 * global-local fusion into one unified K/V): query t = c0 + i attends
 * I u S u L u [c0, t] with one joint softmax per head, S = sel[0:n_sel]
 * shared by all heads (p->per_head == 1: head h uses its own selection,
 * bfloat16 and caches below 2^31 elements per sequence only).
 * q: [batch, chunk_len, H, d]; k_cache, v_cache: [batch, ctx_len, H, d];
 * sel/n_sel: as produced by esa_select (positions must lie in M).
 * out: [batch, chunk_len, H, d] (dtype); lse: [batch, chunk_len, H] float32
 * or NULL.
 */
int esa_sparse_attn(const qat_esa_params* p, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* sel, const int32_t* n_sel,
                    void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Gradients of esa_sparse_attn with the selection held fixed (the top-k is
 * a discrete choice; [ESA] learns the compression map offline, so no
 * gradient reaches it): for each chunk query i and head h with key list
 * I u S u L u [c0, c0 + i] ([ESA] four-part split),
 *   p_j = exp(scale q.k_j - lse),  dp_j = dO.v_j,  D = sum_j p_j dp_j,
 *   dq = scale sum_j p_j (dp_j - D) k_j,
 *   dk_j += scale p_j (dp_j - D) q,  dv_j += p_j dO.
 * q, k_cache, v_cache, sel, n_sel as given to esa_sparse_attn; lse: its
 * output for the same queries (required); dout: [batch, chunk_len, H, d].
 * bfloat16 inputs only (QAT_EUNSUPPORTED otherwise), and one sequence's
 * cache must hold fewer than 2^31 elements.
 * dq: [batch, chunk_len, H, d] float32, written. dk, dv: [batch, ctx_len, H,
 * d] float32, ADDED to at the attended positions (gradient accumulation
 * over chunks; zero them before the first chunk); other rows untouched.
 * Deterministic. Workspace: esa_bwd_workspace_size(p).
 */
int esa_bwd_workspace_size(const qat_esa_params* p, size_t* bytes);
int esa_sparse_attn_bwd(const qat_esa_params* p, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* sel, const int32_t* n_sel, const void* dout, const float* lse, float* dq,
                        float* dk, float* dv, void* ws, size_t ws_bytes, void* stream);

/* ======================================================================
 * MoBA -- block-level selection by mean-pooled keys   [MoBA]
 * ====================================================================== */

/*
 * Sequences of seq_len tokens split into blocks of `block` keys (block b =
 * keys [b*block, (b+1)*block), [MoBA] section 3 partition). Queries
 * [q_start, q_start + q_len) are processed. Query head h reads KV head
 * h / (n_q_heads / n_kv_heads).
 */
typedef struct {
  int64_t batch;
  int64_t seq_len;      /* N */
  int64_t n_q_heads;    /* Hq */
  int64_t n_kv_heads;   /* Hkv, divides Hq */
  int64_t head_dim;     /* 64 or 128 */
  int64_t q_start;      /* first query position processed */
  int64_t q_len;        /* number of query positions processed */
  int32_t block;        /* B >= 1 */
  int32_t topk;         /* blocks per query INCLUDING the forced current one, 1..16 */
  int32_t window;       /* extra local keys [t - window + 1, t], >= 0 */
  float scale;          /* softmax scale > 0 */
  int32_t dtype;        /* qat_dtype of q, k, v and out */
} qat_moba_params;

int moba_workspace_size(const qat_moba_params* p, size_t* bytes);

/*
 * Block gating ([MoBA] section 3: affinity s_b = <q, mean_pool(K[block b])>,
 * top-k gate, causality, forced current block):
 *   for b < cur(t) = floor(t / block): s_b = <q_{t,h}, mean(K[block b, g(h)])>
 *   blk[t, h] = ascending( top-(topk-1) blocks by s_b, ties to the smaller
 *               block  U  {cur(t)} ), -1 padded to topk.
 * Block means are accumulated in float64 and held in float32; scores are
 * float32.
 * q: [batch, seq_len, Hq, d], k: [batch, seq_len, Hkv, d].
 * blk: [batch, q_len, Hq, topk] int32 for the rows q_start .. q_start+q_len-1.
 */
int moba_block_select(const qat_moba_params* p, const void* q, const void* k, int32_t* blk,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse attention ([MoBA] section 2, Softmax(q K[I]^T) V[I]): query t
 * attends the union of its gated earlier blocks (whole), the causal part
 * [cur(t)*block, t] of its own block and, if window > 0, the keys
 * [max(0, t - window + 1), t]; one softmax per (t, h), each key once.
 * blk: as written by moba_block_select for the same q_start/q_len (earlier
 * blocks distinct and ahead of the current block; the last of the topk slots
 * is taken for the current block and never attended as an earlier one).
 * out: [batch, q_len, Hq, d] (dtype); lse: [batch, q_len, Hq] float32 or NULL.
 */
int moba_sparse_attn(const qat_moba_params* p, const void* q, const void* k, const void* v,
                     const int32_t* blk, void* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * Gradients of moba_sparse_attn with the gating held fixed ([MoBA] sections
 * 2-3: the attention is softmax attention over the gated set; the gate is a
 * parameter-free top-k, a discrete choice). For each processed row (t, h)
 * with key set I(t, h) (gated earlier blocks whole + [cur(t)*block, t]):
 *   p_j = exp(scale q.k_j - lse),  dp_j = dO.v_j,  D = sum_j p_j dp_j,
 *   dq = scale sum_j p_j (dp_j - D) k_j,
 *   dk_j += scale p_j (dp_j - D) q,  dv_j += p_j dO  (GQA: the query heads of
 *   a KV head add into it).
 * q, k, v, blk as given to moba_sparse_attn (q the whole sequence); lse: its
 * output for the same rows (required; D is formed from the probabilities in
 * float32, not from a rounded forward output); dout: [batch, q_len, Hq, d]
 * (dtype).
 * dq: [batch, q_len, Hq, d] float32; dk, dv: [batch, seq_len, Hkv, d]
 * float32, overwritten in full (zero for keys no processed row attends).
 * window must be 0 (QAT_EUNSUPPORTED otherwise). For bfloat16 inputs the
 * results are deterministic (every sum in a fixed order); the float32 path
 * adds dk, dv across row tiles with float atomics, so its last bits may vary
 * from run to run. Workspace: moba_bwd_workspace_size(p) (it holds float32
 * partials: rows x (topk - 1) x (2 d + 4) for dq, and per run of 8 dispatch
 * tiles and 128-key chunk the dk, dv sums).
 */
int moba_bwd_workspace_size(const qat_moba_params* p, size_t* bytes);
int moba_sparse_attn_bwd(const qat_moba_params* p, const void* q, const void* k, const void* v,
                         const int32_t* blk, const void* dout, const float* lse, float* dq, float* dk, float* dv,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Decode steps ([MoBA] section 3: gating and attention are defined per query
 * token, so generation applies them to each new token; complete blocks never
 * change once written, so their means are computed once and kept).
 *
 * moba_block_means: the means of complete blocks [first_block, first_block +
 * n_blocks) into the caller's cache
 *   kbar: [batch, seq_len / block, Hkv, d] float32, block b at row b,
 * accumulated in float64 as in moba_block_select. Only those rows are
 * written. k as in moba_block_select. Requires first_block >= 0, n_blocks >=
 * 0 and first_block + n_blocks <= seq_len / block (complete blocks only).
 * Workspace: moba_workspace_size(p).
 */
int moba_block_means(const qat_moba_params* p, const void* k, int64_t first_block, int64_t n_blocks,
                     float* kbar, void* ws, size_t ws_bytes, void* stream);

/*
 * moba_decode_select: the gating of moba_block_select (same scores, order,
 * ties and output) for the rows q_start .. q_start+q_len-1, scored against a
 * kbar cache filled by moba_block_means for every block below the rows' own
 * blocks (blocks 0 .. (q_start+q_len-1)/block - 1).
 * q: [batch, q_len, Hq, d] -- only the processed rows. kbar may be NULL
 * when no row has an earlier block (topk == 1 or every row in block 0).
 * No workspace.
 */
int moba_decode_select(const qat_moba_params* p, const void* q, const float* kbar, int32_t* blk,
                       void* stream);

/*
 * moba_decode_attn: moba_sparse_attn (same key sets and outputs) with
 * q: [batch, q_len, Hq, d] holding only the processed rows; k, v hold the
 * whole sequence (the KV cache, positions 0 .. seq_len-1; keys past a row's
 * position are never read). With q_len <= 8 and no window each row's keys
 * are cut into pieces of up to 256 keys attended in parallel and merged by
 * log-sum-exp. Workspace: moba_workspace_size(p).
 */
int moba_decode_attn(const qat_moba_params* p, const void* q, const void* k, const void* v,
                     const int32_t* blk, void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * moba_decode_attn_noalloc: moba_decode_attn for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, serving
 * loops and harnesses that forbid allocation). Same arguments, key sets and
 * outputs as moba_decode_attn without ws / ws_bytes; it calls no allocator.
 * Its partial results go to a fixed 16 MiB device array inside the library
 * (one per GPU, held until the process ends), so it takes only the
 * split-key case: q_len <= 8, window 0, at most 64 pieces of 256 keys per
 * row, and rows * pieces * (head_dim + 1) * 4 bytes (pieces = topk *
 * ceil(block / 256)) within the 16 MiB; anything else returns
 * QAT_EUNSUPPORTED before any device work. Every call on one GPU shares that
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and give wrong results; serialise them. The array needs no clearing (each
 * call writes every piece it reads).
 */
int moba_decode_attn_noalloc(const qat_moba_params* p, const void* q, const void* k, const void* v,
                             const int32_t* blk, void* out, float* lse, void* stream);

/* ======================================================================
 * CCA-style core-token attention   [CCA]
 * ====================================================================== */

/*
 * [CCA] sections on global-aware pooling, the locality-preserving module and
 * the global-local fusion (the page drops the formulas; readings):
 *   groups of `group` tokens, group i = [i*group, (i+1)*group);
 *   core key / value of group i and query head h: the group's keys / values
 *     weighted by a_j = softmax_j(scale <q_{last of group i, h}, k_j>);
 *   query t attends, in one softmax, the core tokens of groups
 *     i < ls(t) / group and the raw tokens [ls(t), t], where
 *     ls(t) = max(0, floor(t/group)*group - ceil(window/group)*group)
 *     (a group-aligned window of at least `window` earlier tokens).
 * q: [batch, seq_len, Hq, d], k, v: [batch, seq_len, Hkv, d], bfloat16.
 */
typedef struct {
  int64_t batch;
  int64_t seq_len;
  int64_t n_q_heads;
  int64_t n_kv_heads;   /* divides n_q_heads */
  int64_t head_dim;     /* 64 or 128 */
  int64_t q_start;      /* first query position processed */
  int64_t q_len;
  int32_t group;        /* g >= 1 */
  int32_t window;       /* w >= 0 */
  float scale;          /* softmax scale > 0 (pooling and attention) */
  int32_t dtype;        /* QAT_BF16 only */
} qat_cca_params;

/*
 * Core keys / values of the groups the processed rows read (groups
 * 0 .. ls(q_start+q_len-1)/group - 1) into kc, vc: [batch, seq_len/group,
 * Hq, d] bfloat16 (rows of other groups untouched). No workspace.
 */
int cca_pool(const qat_cca_params* p, const void* q, const void* k, const void* v, void* kc, void* vc,
             void* stream);
/*
 * Attention of the rows q_start .. q_start+q_len-1 over their core tokens
 * (from cca_pool) and their window. out: [batch, q_len, Hq, d] bfloat16;
 * lse: [batch, q_len, Hq] float32 natural log, or NULL. No workspace.
 */
int cca_attn(const qat_cca_params* p, const void* q, const void* k, const void* v, const void* kc,
             const void* vc, void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QAT_H_ */
