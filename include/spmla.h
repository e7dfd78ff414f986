/*
 * spmla.h - C ABI of the MI355X (gfx950) sparse-MLA prefill library.
 *
 * One DeepSeek-style MLA attention layer, prefill only. The four steps are the
 * ones described on the page "perf(ds4): extend sparse prefill scheduling to
 * 10K", section Summary:
 *   1. an integer indexer scores every query token against the ratio-4
 *      compressed latent rows it can see;
 *   2. which compressed rows a query can see follows from its position alone
 *      (no stored quadratic mask; same page, Memory and execution shape);
 *   3. per-token top-k of those rows is handed directly to attention;
 *   4. streaming online-softmax attention reads each selected F16 latent row
 *      (plus a sliding window of raw rows) once and shares it between the 16
 *      query heads, over independent 2,048-token query bands.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a caller-owned DEVICE pointer to a dense,
 *    row-major array, 16-byte aligned. The library never frees or keeps it.
 *  - The library allocates no device memory. Scratch space comes from a
 *    caller workspace whose size spmla_prefill_workspace_bytes() returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns without
 *    synchronizing: the caller must synchronize the stream before reading
 *    outputs or freeing any argument.
 *  - All argument checks run on the host before anything is enqueued; on a
 *    negative return nothing was enqueued. spmla_last_error() then returns a
 *    message (thread-local, valid until the next call on the same thread).
 *  - n_q == 0 is a valid empty call: it checks the descriptor and returns 0.
 *  - fp16 arrays hold IEEE binary16 bit patterns (uint16_t).
 *  - Results are deterministic: no floating-point atomics; every reduction
 *    runs in a fixed order, so repeated calls give bit-identical outputs.
 */
#ifndef SPMLA_H
#define SPMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SPMLA_OK 0
#define SPMLA_EINVAL (-1)       /* null pointer, inconsistent sizes        */
#define SPMLA_EUNSUPPORTED (-2) /* valid but not a shape the kernels cover */
#define SPMLA_EWORKSPACE (-3)   /* workspace too small                     */
#define SPMLA_EHIP (-4)         /* a HIP launch reported an error          */

/*
 * Sizes of one prefill call. Queries are the absolute token positions
 * q_pos0 .. q_pos0 + n_q - 1 of a sequence whose raw latent rows 0 .. n_raw-1
 * are all present (n_raw >= q_pos0 + n_q).
 *
 *   n_comp    compressed rows = floor(n_raw / ratio): row j stands for raw
 *             rows ratio*j .. ratio*j+ratio-1; a trailing partial group is
 *             not compressed yet. Row j is visible to query t iff
 *             ratio*(j+1) <= t+1.
 *   window    W: the raw rows max(0, t-W+1) .. t (own row included) are
 *             always attended, in addition to the selected compressed rows.
 *   top_k     k: compressed rows selected per query (fewer when fewer are
 *             visible).
 *   band      queries per scheduling band of spmla_prefill (2048 on the
 *             pages); results do not depend on it.
 *   n_heads   query heads sharing each latent row (16).
 *   d_qk      latent width used by the logits (576 = 512 value + 64 rope).
 *   d_v       value width: the first d_v dims of a latent row (512).
 *   idx_heads, idx_dim   indexer heads and their width (4, 64).
 *   scale     softmax scale applied to the full d_qk-wide dot (1/sqrt(576));
 *             finite and > 0.
 *
 * Kernels cover n_heads == 16, d_qk == 576, d_v == 512, idx_heads == 4,
 * idx_dim == 64, 1 <= top_k <= 4096 and n_comp <= 32768; other valid values
 * return SPMLA_EUNSUPPORTED.
 */
typedef struct spmla_desc {
  int32_t n_q;
  int32_t q_pos0;
  int32_t n_raw;
  int32_t n_comp;
  int32_t ratio;
  int32_t window;
  int32_t top_k;
  int32_t band;
  int32_t n_heads;
  int32_t d_qk;
  int32_t d_v;
  int32_t idx_heads;
  int32_t idx_dim;
  float scale;
} spmla_desc;

/* Message for the last failed call on this thread ("" if none). */
const char* spmla_last_error(void);

/* Library ABI version (increments on any signature or layout change). */
int spmla_abi_version(void);

/*
 * Host-only check of a descriptor (same rules as every entry point).
 * Returns SPMLA_OK, SPMLA_EINVAL or SPMLA_EUNSUPPORTED.
 */
int spmla_check_desc(const spmla_desc* desc);

/*
 * Number of scheduling bands of spmla_prefill: ceil(n_q / band). The last
 * band holds n_q - (bands-1)*band queries (page "perf(ds4): extend sparse
 * prefill scheduling to 10K", Summary and Production workflow: five 2,048
 * bands admit 10,240 tokens; 9,133 tokens = 4 full bands + 941).
 * Returns the count (>= 0) or a negative error code.
 */
int spmla_num_bands(const spmla_desc* desc);

/*
 * Step 1+2 - indexer scores (page "perf(ds4): extend sparse prefill
 * scheduling to 10K", Summary: indexer over ratio-4 compressed rows with
 * analytically derived causal visibility).
 *
 *   scores[t][j] = sum_h iw[t][h] * max(0, sum_d iq[t][h][d] * ik[j][d])
 *                  if compressed row j is visible to query t, else INT32_MIN.
 *
 *   iq      int8  [n_q][idx_heads][idx_dim]
 *   iw      int8  [n_q][idx_heads]
 *   ik      int8  [n_comp][idx_dim]             (may be NULL if n_comp == 0)
 *   scores  int32 [n_q][n_comp]  (output; exact integers)
 *
 * Exact for every int8 input: a head dot product is at most 64*128*128 =
 * 2^20 in magnitude and a score at most 4*128*2^20 = 2^29, so no real
 * score equals INT32_MIN.
 *
 * Writes the full n_q x n_comp matrix: meant for tests and short calls;
 * spmla_prefill holds at most 128 MiB of it (one selection group) at once.
 */
int spmla_indexer_scores(const spmla_desc* desc, const int8_t* iq, const int8_t* iw,
                         const int8_t* ik, int32_t* scores, void* stream);

/*
 * Step 3 - top-k handoff (same page, Summary: authoritative long-prefill
 * top-k rows passed directly to attention, selected-row order preserved).
 *
 * For each query t, with n_vis(t) = min(n_comp, (q_pos0+t+1)/ratio):
 *   sel[t][0 .. n_sel-1] = the n_sel = min(top_k, n_vis(t)) visible rows
 *     ordered by score descending, then by lower row index;
 *   sel[t][n_sel .. top_k-1] = -1.
 *
 *   scores  int32 [n_q][n_comp] as written by spmla_indexer_scores (only
 *           entries j < n_vis(t) are read)
 *   sel     int32 [n_q][top_k]  (output)
 *   n_sel   int32 [n_q]         (output; may be NULL)
 */
int spmla_topk(const spmla_desc* desc, const int32_t* scores, int32_t* sel, int32_t* n_sel,
               void* stream);

/*
 * Step 4 - streaming sparse attention (page "perf(ds4): extend sparse
 * prefill scheduling to 10K", Summary; page "perf(ds4): unify gfx1151
 * sparse-prefill stack", Validation completed: FP32-staged streaming MLA).
 *
 * For query t and head h the key set is the selected compressed rows
 * kv_comp[sel[t][i]] (i < n_sel) followed by the window rows kv_raw[s],
 * s = max(0, q_pos0+t-window+1) .. q_pos0+t; both kinds are entries of ONE
 * softmax:
 *   z      = scale * <q[t][h][:], key[:]>           (all d_qk dims)
 *   out    = sum softmax(z) * key[0:d_v]            (fp32 accumulate)
 *   lse    = log(sum exp(z))                        (natural log)
 * Entries i < min(top_k, n_vis(t)) of a sel row are read; -1 entries
 * (padding) are skipped.
 *
 *   q        fp16  [n_q][n_heads][d_qk]
 *   kv_comp  fp16  [n_comp][d_qk]          (may be NULL if n_comp == 0)
 *   kv_raw   fp16  [n_raw][d_qk]
 *   sel      int32 [n_q][top_k]            (as written by spmla_topk)
 *   out      fp32  [n_q][n_heads][d_v]     (output)
 *   lse      fp32  [n_q][n_heads]          (output; may be NULL)
 * Every sel entry should be -1 or in [0, n_vis(t)); any other entry is
 * skipped like -1 (the gather reads a valid row in its place and the key is
 * masked out of the softmax), never dereferenced. A call over more than
 * `band` queries is dealt to the GPU band by band in one launch.
 */
int spmla_sparse_attn(const spmla_desc* desc, const uint16_t* q, const uint16_t* kv_comp,
                      const uint16_t* kv_raw, const int32_t* sel, float* out, float* lse,
                      void* stream);

/*
 * Query-tiled ("grouped") variant of spmla_sparse_attn (page "perf(ds4):
 * unify gfx1151 sparse-prefill stack", Validation completed: the streaming
 * kernel replaced a grouped one, measured side by side). Same arguments,
 * same results up to fp32 summation order. Each pair of adjacent queries
 * (t, t+1) shares one gather of the union of their keys: t's selected rows,
 * t+1's selected rows that t did not select, and the union of the two
 * windows; every gathered row is read once for both. Selected rows of one
 * query must be distinct.
 */
int spmla_sparse_attn_grouped(const spmla_desc* desc, const uint16_t* q, const uint16_t* kv_comp,
                              const uint16_t* kv_raw, const int32_t* sel, float* out, float* lse,
                              void* stream);

/*
 * Ratio-4 compression of raw latent rows: the step before the path (page
 * "perf(ds4): extend sparse prefill scheduling to 10K", Summary: ratio-4
 * compressed rows kept in F16, state committed in chronological order).
 *
 *   kv_comp[j][d] = fp16( (kv_raw[4j][d] + kv_raw[4j+1][d] + kv_raw[4j+2][d]
 *                          + kv_raw[4j+3][d]) / 4 )
 * for comp_begin <= j < n_comp, with n_comp = floor(n_raw / 4): only complete
 * groups, so the n_raw mod 4 newest raw rows stay uncompressed until their
 * group completes. The sum is exact and rounded once (nearest, ties to
 * even); -0 results only from four -0 inputs; inf / NaN as in IEEE addition.
 * Rows before comp_begin (already committed) are not touched, so a prefill
 * that appends raw rows compresses only the groups it completed.
 *
 *   kv_raw   fp16  [n_raw][d_qk]   (reads rows 4*comp_begin .. 4*n_comp-1)
 *   kv_comp  fp16  [n_comp][d_qk]  (writes rows comp_begin .. n_comp-1)
 *   comp_begin  0 <= comp_begin <= n_comp
 * Only desc->n_raw, n_comp, ratio (must be 4) and d_qk are used.
 */
int spmla_compress(const spmla_desc* desc, const uint16_t* kv_raw, uint16_t* kv_comp, int32_t comp_begin,
                   void* stream);

/*
 * Workspace bytes spmla_prefill needs for this descriptor: the largest
 * selection scratch of its selection groups (a group's indexer scores, or
 * its fused handoff's thresholds, slot counts and candidate slots), or the
 * key-split partials of a small call when larger, plus the selected rows of
 * its largest group twice (score order, and ascending row order for the
 * attention's gathers). A selection group is a run of consecutive whole
 * bands that select the same way, as many as fit 128 MiB of scores or
 * 512 MiB of fused-handoff scratch (at least one band).
 * Returns SPMLA_OK and writes *bytes, or an error code.
 */
int spmla_prefill_workspace_bytes(const spmla_desc* desc, size_t* bytes);

/*
 * Steps 1-4 for all n_q queries in bands of `band` queries (page "perf(ds4):
 * extend sparse prefill scheduling to 10K": Summary, five independent 2,048-
 * token bands admit one 10,240-token frontier; Production workflow, the
 * 9,133-token prompt runs as one step of 4 full bands + a ragged 941-query
 * band; Memory and execution shape, visibility derived, no mask stored),
 * all enqueued on `stream` with no host round trip.
 *
 *   q, kv_comp, kv_raw, iq, iw, ik   as in spmla_indexer_scores and
 *                                    spmla_sparse_attn (read only)
 *   out      fp32  [n_q][n_heads][d_v]      (output)
 *   lse      fp32  [n_q][n_heads]           (output, may be NULL)
 *   sel_out  int32 [n_q][top_k]             (output, may be NULL; as
 *                                            spmla_topk writes it)
 *   workspace, workspace_bytes   caller-owned device scratch of at least
 *            spmla_prefill_workspace_bytes(desc) bytes, 16-byte aligned;
 *            its contents on entry do not matter and are garbage on return
 *            (SPMLA_EWORKSPACE, nothing enqueued, when too small).
 * The workspace must not be used by other work on any stream until this
 * call's work on `stream` completes. Errors as for every entry point.
 *
 * Attention runs band by band. Selection
 * runs once per selection group, before the group's first attention launch:
 * through the score matrix (one indexer and one top-k launch for all of the
 * group's queries), or, for bands of at least 256 queries that each see
 * more than 4,096 (and at least 8 * top_k) compressed rows, through the
 * fused handoff, which never writes the score matrix. Same inputs and
 * outputs as the three calls above;
 * sel_out (int32 [n_q][top_k]) and lse may be NULL. When the compressed
 * rows exceed 4 MiB the attention takes each selection in ascending row
 * order, so out and lse can differ from spmla_sparse_attn on sel_out in
 * fp32 summation order (not beyond the parity tolerance).
 */
int spmla_prefill(const spmla_desc* desc, const uint16_t* q, const uint16_t* kv_comp,
                  const uint16_t* kv_raw, const int8_t* iq, const int8_t* iw, const int8_t* ik,
                  float* out, float* lse, int32_t* sel_out, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * spmla_prefill without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP stream capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same inputs, outputs and results
 * as spmla_prefill (bit for bit: the schedule below only changes how
 * queries are grouped into launches, and results do not depend on it).
 *
 * Scratch: a 64 MiB array in the library's device image (one per GPU that
 * loads the library, held until the process ends); its device address is
 * looked up on the first call on each device. The call allocates nothing
 * and calls no allocating routine. Selection groups hold at most 32 MiB of
 * scratch each, and when a call's scratch would still exceed 64 MiB its
 * bands are halved until it fits (e.g. the 8,192 queries after 114,687
 * tokens run in bands of 512). Returns SPMLA_EWORKSPACE, with nothing
 * enqueued, if even one-query bands do not fit.
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (several streams, or several host threads) race and corrupt each
 * other; the caller orders them, e.g. on one stream. The array keeps the
 * last call's contents; no part of it needs to start at zero. `stream`
 * must belong to the current device (else SPMLA_EINVAL).
 */
int spmla_prefill_noalloc(const spmla_desc* desc, const uint16_t* q, const uint16_t* kv_comp,
                          const uint16_t* kv_raw, const int8_t* iq, const int8_t* iw, const int8_t* ik,
                          float* out, float* lse, int32_t* sel_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPMLA_H */
