// Host-side launchers of the HIP kernels, called by the C ABI layer after it
// has validated the arguments. Each enqueues on stream `s` and returns
// hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace qat {

// ---- compression (compress.hip) -------------------------------------------
int compress_splits(int64_t n, int64_t d_model, int64_t d_c);
hipError_t launch_compress_partial(const void* x, int64_t n, int64_t x_stride, int64_t d_model, bool x_bf16,
                                   const void* W, bool w_bf16, int64_t d_c, int nsplit, double* partial,
                                   hipStream_t s);
// kind 0: float32 out, 1: bf16 out, 2: float32 out plus bf16 hi/lo rows.
bool compress_bf16_rows_ok(int64_t n, int64_t d_model, int64_t d_c);
hipError_t launch_compress_bf16_rows(const void* x, int64_t n, int64_t x_stride, int64_t d_model, const void* W,
                                     int64_t d_c, const float* bias, float* out, bf16* hi, bf16* lo, hipStream_t s);
hipError_t launch_compress_finalize(const double* partial, int nsplit, int64_t n, int64_t d_c, const float* bias,
                                    void* out, int64_t out_stride, int kind, bf16* hi, bf16* lo, hipStream_t s);

// ---- MoBA gating (moba_select.hip) ----------------------------------------
int meanpool_splits(int block);
// Means of blocks [first, first + count) (count < 0: through nbc) into kbar
// [batch, nbc, hkv*d]; planes: NULL, or 3 * batch*nbc*hkv*d bfloat16 (hi/mid/lo
// split of the means), written only for the whole range.
hipError_t launch_moba_meanpool(const void* k, bool bf, int64_t batch, int64_t seq_len, int64_t hkv, int64_t d,
                                int block, int64_t nbc, double* partial, float* kbar, bf16* planes,
                                hipStream_t s, int64_t first = 0, int64_t count = -1);
// Scoring from float32 means kbar [batch, nbc, hkv, d] (a cache of complete
// blocks); q laid out as for launch_moba_decode.
hipError_t launch_moba_select_means(const void* q, bool bf, const float* kbar, int32_t* blk, int64_t batch,
                                    int64_t seq_len, int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv,
                                    int64_t d, int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk,
                                    hipStream_t s);
// bfloat16 queries score on the matrix cores from `planes`; float32 ones use `kbar`
hipError_t launch_moba_select(const void* q, bool bf, const float* kbar, const bf16* planes, int32_t* blk,
                              int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t nbc,
                              int64_t q_start, int64_t q_len, int block, int topk, hipStream_t s);

// ---- MoBA attention (moba_attn.hip) ---------------------------------------
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
int64_t moba_max_tiles(int64_t nrows, int topk, int64_t nbuckets);
int moba_rows_per_tile();   // query rows per dispatch tile
// tiles: {element offset of the block's K/V rows (low, high word), first
// entry, row count}; entries: {row * 16 + slot, row index of the query in q}
// stable (wg_counts, wg_base non-NULL, each moba_dispatch_stable_ints
// int32): the entries of a bucket are placed in an order fixed by the rows
// (no atomics decide it), which the gradient pass needs for reproducible
// dK/dV sums; NULL: the faster atomic placement, order arbitrary.
hipError_t launch_moba_dispatch(const int32_t* blk, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
                                int64_t d, int64_t q_start, int64_t q_len, int block, int topk, int64_t nbc,
                                int32_t* counts, int32_t* offsets, int32_t* cursor, int2* entries, int4* tiles,
                                int32_t* ntiles, hipStream_t s, int32_t* wg_counts = nullptr,
                                int32_t* wg_base = nullptr, int32_t* wg_loc = nullptr,
                                float* part_lse = nullptr);
// int32 elements of the per-workgroup bucket counts that the atomic placement
// records in its count pass (wg_loc), 0 when the buckets do not fit in LDS
int64_t moba_dispatch_wg_ints(int64_t nrows, int64_t nbuckets);
// int32 elements of each stable-placement array, 0 when the bucket count is
// too large for it (the atomic placement is then used)
int64_t moba_dispatch_stable_ints(int64_t nrows, int64_t nbuckets, int topk);
hipError_t launch_moba_attn_mfma(const void* q, const void* k, const void* v, const int32_t* blk,
                                 const int4* tiles, const int32_t* ntiles, const int2* entries, void* part_o,
                                 float* part_lse, void* out, float* lse, int64_t batch, int64_t seq_len, int64_t hq,
                                 int64_t hkv, int64_t d, int64_t nbc, int64_t q_start, int64_t q_len, int block,
                                 int topk, float scale, int64_t max_tiles, hipStream_t s);

// ---- MoBA gradients (moba_bwd.hip) -----------------------------------------
// dq [rows, d] and delta [rows] written; dk, dv [batch, seq_len, hkv, d]
// written in full (own-block kernel) and then added to (gated rows over the
// dispatch tiles). dq_part: moba_bwd_part_floats floats (bfloat16 path).
// tile_off: the dispatch's per-bucket tile prefix (nbuckets + 1 entries);
// run_off: nbuckets + 1 int32 scratch; kv_part: moba_bwd_kv_part_floats.
int moba_bwd_chunks(int block);
int64_t moba_bwd_part_floats(int64_t rows, int topk, int64_t d);
int64_t moba_bwd_kv_part_floats(int64_t max_tiles, int64_t nbuckets, int block, int64_t d);
hipError_t launch_moba_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                           const void* dout, const float* lse, const int4* tiles, const int32_t* ntiles,
                           const int2* entries, int64_t max_tiles, const int32_t* tile_off, int64_t nbuckets,
                           int32_t* run_off, float* kv_part, float* dq_part, float* dq, float* delta, float* dk,
                           float* dv, bool bf, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d,
                           int64_t q_start, int64_t q_len, int block, int topk, float scale, hipStream_t s);

// ---- generic per-row attention (attn_generic.hip) -------------------------
// q holds q_seq positions per sequence from position q_off on (the whole
// sequence: q_seq = seq_len, q_off = 0; only the processed rows: q_seq =
// q_len, q_off = q_start).
// MoBA with few query rows (no window): pieces of up to 256 keys, one wave
// each; po: rows * moba_decode_pieces * d floats, plse: rows * pieces floats.
int moba_decode_pieces(int block, int topk);
hipError_t launch_moba_decode(const void* q, const void* k, const void* v, const int32_t* blk, float* po,
                              float* plse, void* out, float* lse, bool bf, int64_t batch, int64_t seq_len,
                              int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv, int64_t d, int64_t q_start,
                              int64_t q_len, int block, int topk, float scale, hipStream_t s);
hipError_t launch_moba_generic(const void* q, const void* k, const void* v, const int32_t* blk, void* out,
                               float* lse, bool bf, int64_t batch, int64_t seq_len, int64_t q_seq, int64_t q_off,
                               int64_t hq, int64_t hkv, int64_t d, int64_t q_start, int64_t q_len, int block,
                               int topk, int window, float scale, hipStream_t s);
hipError_t launch_esa_generic(const void* q, const void* k, const void* v, const int32_t* sel, const int32_t* n_sel,
                              void* out, float* lse, bool bf, int64_t batch, int64_t H, int64_t d, int64_t ctx_len,
                              int64_t c0, int64_t m, int64_t n_init, int64_t window, int topk, float scale,
                              hipStream_t s);

// ---- ESA selection (esa_select.hip) ---------------------------------------
int esa_key_splits(int64_t n_mid, int64_t m);
int esa_prefill_qsplits_eff(int64_t n_mid, int64_t m);
int esa_scan_wgs(int64_t n_mid);
// Where selection v's scoring operands live: q rows at
// q + (v / vh) q_outer + (v % vh) q_inner + i q_row, key rows likewise.
// Merged heads: one selection per sequence, vh = 1, rows of d_c elements
// (q~ [B, m, d_c], compressed cache [B, T, d_c]). Per head: one selection per
// (sequence, head), vh = H, q [B, m, H, d] and K [B, T, H, d], rows of H d.
struct ScGeom {
  int64_t q_outer, q_inner, q_row;
  int64_t k_outer, k_inner, k_row;
  int64_t vh;
  __device__ __forceinline__ int64_t qoff(int64_t v) const { return (v / vh) * q_outer + (v % vh) * q_inner; }
  __device__ __forceinline__ int64_t koff(int64_t v) const { return (v / vh) * k_outer + (v % vh) * k_inner; }
};
// nsel selections; dc: the scored width (d_c, or d per head). q_lo NULL:
// q is exactly bf16 (one term). tau2 > 0: the softmax-vote reading of the
// correction at temperature tau2 / log2(e) (rowsum_part / ssum_part hold the
// per-split exp sums); tau2 = 0: the clamp reading.
hipError_t launch_esa_prefill_scores(const bf16* q_hi, const bf16* q_lo, const bf16* kc, const ScGeom& g,
                                     int64_t nsel, int64_t m, int64_t mid0, int64_t n_mid, int64_t dc, float clip,
                                     float tau2, float* rowmax_part, float* rowsum_part, float* rowmax,
                                     float* upart, int32_t* hist0, int64_t nhist, hipStream_t s);
// q: float32 (q_bf16 false) or bfloat16 rows
hipError_t launch_esa_decode_scan(const void* q, bool q_bf16, const bf16* kc, const ScGeom& g, int64_t nsel,
                                  int64_t mid0, int64_t n_mid, int64_t dc, float tau2, float* s_out,
                                  float* smax_part, float* ssum_part, int32_t* hist0, int64_t nhist,
                                  hipStream_t s);
int esa_topk_slices(int64_t n_mid);
int esa_topk_max_radius();
// hist: batch*3*2048 int32, wgcnt: batch*esa_topk_slices(n_mid) int2 (scratch);
// hist_clear: the scoring kernels have already zeroed hist (hist0/nhist of
// the scoring launchers), else a fill runs first
// mode 0: prefill importance sums; 1: decode, clamp; 2: decode, votes
hipError_t launch_esa_topk(int mode, const float* upart, int nqsplit, const float* s_in, const float* smax_part,
                           const float* ssum_part, int nsmax, float clip, float tau2, int64_t batch, int64_t n_mid,
                           int radius, int topk, int64_t mid0,
                           int32_t* hist, int2* wgcnt, uint32_t* keys, float* scores_out, int32_t* sel,
                           int32_t* n_sel, bool hist_clear, hipStream_t s);

// ---- ESA attention (esa_attn.hip) -----------------------------------------
int esa_decode_splits(int64_t batch, int64_t n_init, int64_t topk, int64_t window);
bool esa_decode_supported(int64_t H, int64_t D, bool per_head);
int64_t esa_keylist_len(int64_t n_init, int64_t topk, int64_t window, int64_t m);
hipError_t launch_esa_prefill_attn(const void* q, const void* k, const void* v, const int32_t* sel,
                                   const int32_t* n_sel, int32_t* keylist, void* out, float* lse, int64_t batch,
                                   int64_t H, int64_t D, int64_t ctx_len, int64_t c0, int64_t m, int64_t n_init,
                                   int64_t window, int topk, float scale, bool per_head, hipStream_t s);
// keylist [nsel, esa_keylist_len]: per selection the gathered key positions
// (initial, selected, local) then the chunk's positions
hipError_t launch_esa_keylist(const int32_t* sel, const int32_t* n_sel, int32_t* keylist, int64_t nsel, int64_t c0,
                              int64_t m, int64_t n_init, int64_t window, int topk, hipStream_t s);

// ---- CCA-style core-token attention (cca.hip), bfloat16 -------------------
// groups [0, cca_groups_needed) pooled for the processed positions
int64_t cca_groups_needed(int64_t seq_len, int64_t q_start, int64_t q_len, int group, int window);
hipError_t launch_cca_pool(const void* q, const void* k, const void* v, void* kc, void* vc, int64_t batch,
                           int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t ngroups, int64_t npool,
                           int group, float scale, hipStream_t s);
hipError_t launch_cca_attn(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out,
                           float* lse, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d,
                           int64_t q_start, int64_t q_len, int64_t ngroups, int group, int window, float scale,
                           hipStream_t s);

// ---- ESA gradients (esa_bwd.hip), bfloat16 --------------------------------
// dq [batch, m, H, D] and delta [batch, m, H] written; dk, dv [batch,
// ctx_len, H, D] added to at the key lists' positions.
hipError_t launch_esa_bwd(const void* q, const void* k, const void* v, const int32_t* sel, const int32_t* n_sel,
                          const void* dout, const float* lse, int32_t* keylist, float* dq, float* delta, float* dk,
                          float* dv, int64_t batch, int64_t H, int64_t D, int64_t ctx_len, int64_t c0, int64_t m,
                          int64_t n_init, int64_t window, int topk, float scale, bool per_head,
                          hipStream_t s);

hipError_t launch_esa_decode_attn(const void* q, const void* k, const void* v, const int32_t* sel,
                                  const int32_t* n_sel, float* po, float* pm, float* pl, void* out, float* lse,
                                  int64_t batch, int64_t H, int64_t D, int64_t ctx_len, int64_t c0, int64_t n_init,
                                  int64_t window, int topk, float scale, bool per_head,
                                  hipStream_t s);

}  // namespace qat
