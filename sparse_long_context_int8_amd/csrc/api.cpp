// C ABI of the sparse-MLA prefill library: argument checks, workspace
// sizing and the band schedule. Every check runs on the host before any HIP
// call, so a rejected call enqueues nothing (and needs no GPU).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/spmla.h"
#include "spmla_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SPMLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks every rule that does not involve a pointer.
int check_desc(const spmla_desc* d) {
  if (!d) return fail(SPMLA_EINVAL, "desc is NULL");
  if (d->n_q < 0) return fail(SPMLA_EINVAL, "n_q=%d < 0", d->n_q);
  if (d->q_pos0 < 0) return fail(SPMLA_EINVAL, "q_pos0=%d < 0", d->q_pos0);
  if (d->ratio < 1) return fail(SPMLA_EINVAL, "ratio=%d < 1", d->ratio);
  if (d->window < 1) return fail(SPMLA_EINVAL, "window=%d < 1", d->window);
  if (d->top_k < 1) return fail(SPMLA_EINVAL, "top_k=%d < 1", d->top_k);
  if (d->band < 1) return fail(SPMLA_EINVAL, "band=%d < 1", d->band);
  if (d->n_heads < 1 || d->d_qk < 1 || d->d_v < 1 || d->idx_heads < 1 || d->idx_dim < 1)
    return fail(SPMLA_EINVAL, "head counts and widths must be >= 1");
  if (d->d_v > d->d_qk) return fail(SPMLA_EINVAL, "d_v=%d > d_qk=%d", d->d_v, d->d_qk);
  if ((int64_t)d->n_raw < (int64_t)d->q_pos0 + d->n_q)
    return fail(SPMLA_EINVAL, "n_raw=%d < q_pos0+n_q=%lld", d->n_raw,
                (long long)d->q_pos0 + d->n_q);
  if (d->n_comp != d->n_raw / d->ratio)
    return fail(SPMLA_EINVAL, "n_comp=%d != floor(n_raw/ratio)=%d", d->n_comp, d->n_raw / d->ratio);
  if (!std::isfinite(d->scale) || !(d->scale > 0.f))
    return fail(SPMLA_EINVAL, "scale must be finite and > 0");
  if (d->n_heads != spmla::kHeads || d->d_qk != spmla::kDqk || d->d_v != spmla::kDv)
    return fail(SPMLA_EUNSUPPORTED, "kernels cover n_heads=16, d_qk=576, d_v=512 (got %d, %d, %d)",
                d->n_heads, d->d_qk, d->d_v);
  if (d->idx_heads != spmla::kIdxHeads || d->idx_dim != spmla::kIdxDim)
    return fail(SPMLA_EUNSUPPORTED, "kernels cover idx_heads=4, idx_dim=64 (got %d, %d)",
                d->idx_heads, d->idx_dim);
  if (d->top_k > spmla::kMaxTopK)
    return fail(SPMLA_EUNSUPPORTED, "top_k=%d > %d", d->top_k, spmla::kMaxTopK);
  if (d->n_comp > spmla::kMaxComp)
    return fail(SPMLA_EUNSUPPORTED, "n_comp=%d > %d", d->n_comp, spmla::kMaxComp);
  return SPMLA_OK;
}

#define REQUIRE_PTR(p)                                                              \
  do {                                                                              \
    if (!(p)) return fail(SPMLA_EINVAL, "%s is NULL", #p);                          \
    if (!aligned16(p)) return fail(SPMLA_EINVAL, "%s is not 16-byte aligned", #p);  \
  } while (0)
#define OPTIONAL_PTR(p)                                                             \
  do {                                                                              \
    if ((p) && !aligned16(p)) return fail(SPMLA_EINVAL, "%s is not 16-byte aligned", #p); \
  } while (0)

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPMLA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Row stride of the band score matrix in the prefill workspace: a multiple
// of 4 so that the indexer writes 16-byte groups.
int64_t band_ld(const spmla_desc* d) { return ((int64_t)d->n_comp + 3) / 4 * 4; }
size_t scores_bytes_per_band(const spmla_desc* d) {
  const int64_t rows = d->band < d->n_q ? d->band : d->n_q;
  return (size_t)rows * (size_t)band_ld(d) * sizeof(int32_t);
}
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }


// Selection groups: consecutive bands that select the same way get one set
// of selection launches for all their queries, while the group's scratch
// fits a budget: the score matrix (dense selection, 128 MiB) or the fused
// handoff's thresholds, slot counts and candidate slots (512 MiB). The
// attention still runs band by band. One launch per step instead of one per
// band removes the ramp and tail of short, latency-bound launches.
struct GroupBudget {
  size_t dense;  // score-matrix bytes of one group
  size_t fused;  // fused-handoff scratch bytes of one group
  size_t sel;    // bytes of a group's two selection copies (score and row order)
};
constexpr GroupBudget kGroupBudget{(size_t)128 << 20, (size_t)512 << 20, SIZE_MAX};
int64_t group_rows_within(const spmla_desc* d, size_t per_band, size_t budget, size_t sel_budget) {
  const int64_t band_rows = d->band < d->n_q ? d->band : d->n_q;
  const size_t sel_per_band = 2 * (size_t)band_rows * (size_t)d->top_k * sizeof(int32_t);
  int64_t bands = per_band ? (int64_t)(budget / per_band) : INT64_MAX / 2 / (band_rows > 0 ? band_rows : 1);
  if (sel_budget != SIZE_MAX && sel_per_band > 0 && (int64_t)(sel_budget / sel_per_band) < bands)
    bands = (int64_t)(sel_budget / sel_per_band);
  if (bands < 1) bands = 1;
  const int64_t rows = bands * band_rows;
  return rows < d->n_q ? rows : d->n_q;
}
int64_t dense_group_rows(const spmla_desc* d, const GroupBudget& gb) {
  return group_rows_within(d, scores_bytes_per_band(d), gb.dense, gb.sel);
}
int64_t fused_group_rows(const spmla_desc* d, const GroupBudget& gb) {
  const int band_rows = d->band < d->n_q ? d->band : d->n_q;
  const spmla::FusedPlan plan = spmla::fused_plan(d->n_comp, d->top_k);
  return group_rows_within(d, spmla::fused_workspace_bytes(band_rows, plan), gb.fused, gb.sel);
}
int band_len(const spmla_desc* d, int64_t b0) { return (int)((d->n_q - b0) < d->band ? (d->n_q - b0) : d->band); }
bool fused_band(const spmla_desc* d, int64_t b0) {
  return d->n_comp > 0 && spmla::fused_applies(band_len(d, b0), d->q_pos0 + (int)b0, d->n_comp, d->ratio, d->top_k);
}

// Calls f(g0, g1, fused) for the selection groups of a call in order: each
// is a run of whole bands [g0, g1) that select the same way, as many as fit
// that way's budget. spmla_prefill runs exactly these groups, and the
// workspace is sized from them.
template <typename F>
void for_each_group(const spmla_desc* d, const GroupBudget& gb, F&& f) {
  const int64_t dense_cap = dense_group_rows(d, gb), fused_cap = fused_group_rows(d, gb);
  for (int64_t g0 = 0; g0 < d->n_q;) {
    const bool fused = fused_band(d, g0);
    const int64_t cap = fused ? fused_cap : dense_cap;  // a multiple of the band unless it covers every query
    int64_t g1 = g0 + band_len(d, g0);
    while (g1 < d->n_q && g1 - g0 < cap && fused_band(d, g1) == fused) g1 += band_len(d, g1);
    f(g0, g1, fused);
    g0 = g1;
  }
}

// Workspace layout: scratch reused by the steps in stream order (a group's
// score matrix or fused-handoff slots, then the attention's key-split
// partials of a small call; a group's selection scratch is dead once its
// top-k has run, before its first attention launch), then the selections of
// the largest group in score order and in ascending row order.
struct WsLayout {
  size_t scratch = 0;
  size_t sel = 0;  // bytes of one selection copy
  size_t total() const { return scratch + 2 * sel; }
};
WsLayout ws_layout(const spmla_desc* d, const GroupBudget& gb) {
  WsLayout w;
  const int band_rows = d->band < d->n_q ? d->band : d->n_q;
  w.scratch = round_up(spmla::attn_partial_bytes(band_rows, spmla::attn_splits(d->n_q)), 256);
  int64_t max_rows = 0;
  for_each_group(d, gb, [&](int64_t g0, int64_t g1, bool fused) {
    const int64_t rows = g1 - g0;
    const size_t need = fused ? spmla::fused_workspace_bytes((int)rows, spmla::fused_plan(d->n_comp, d->top_k))
                              : round_up((size_t)rows * (size_t)band_ld(d) * sizeof(int32_t), 256);
    if (need > w.scratch) w.scratch = need;
    if (rows > max_rows) max_rows = rows;
  });
  w.sel = round_up((size_t)max_rows * (size_t)d->top_k * sizeof(int32_t), 256);
  return w;
}

spmla::AttnArgs attn_args(const spmla_desc* d, const uint16_t* q, const uint16_t* kv_comp,
                          const uint16_t* kv_raw, const int32_t* sel, float* out, float* lse) {
  spmla::AttnArgs a;
  a.q = reinterpret_cast<const _Float16*>(q);
  a.kv_comp = reinterpret_cast<const _Float16*>(kv_comp);
  a.kv_raw = reinterpret_cast<const _Float16*>(kv_raw);
  a.sel = sel;
  a.out = out;
  a.lse = lse;
  a.n_q = d->n_q;
  a.q_pos0 = d->q_pos0;
  a.n_comp = d->n_comp;
  a.n_raw = d->n_raw;
  a.ratio = d->ratio;
  a.window = d->window;
  a.top_k = d->top_k;
  a.scale_log2e = (float)((double)d->scale * 1.4426950408889634);
  a.splits = 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.band_items = 0;
  return a;
}

// Steps 1-4 of a checked call: selection per group, attention per band, all
// enqueued on `st`. `ws` holds at least ws_layout(d, gb).total() bytes.
int run_prefill(const spmla_desc* d, const uint16_t* q, const uint16_t* kv_comp, const uint16_t* kv_raw,
                const int8_t* iq, const int8_t* iw, const int8_t* ik, float* out, float* lse, int32_t* sel_out,
                char* ws, const GroupBudget& gb, hipStream_t st) {
  int rc = SPMLA_OK;
  const WsLayout lay = ws_layout(d, gb);
  int32_t* scores = reinterpret_cast<int32_t*>(ws);
  int32_t* ws_sel = reinterpret_cast<int32_t*>(ws + lay.scratch);
  int32_t* ws_sel_asc = reinterpret_cast<int32_t*>(ws + lay.scratch + lay.sel);
  // Attention takes each selection in ascending row order when the
  // compressed rows outgrow one die's L2: the queries in flight on a die then
  // sweep the rows together and share what they gather (the softmax does not
  // depend on the order of its keys).
  const bool ascending = spmla::rows_beyond_l2(d->n_comp);

  for_each_group(d, gb, [&](int64_t g0, int64_t g1, bool fused) {
    if (rc) return;
    const int gn = (int)(g1 - g0);
    const int gpos0 = d->q_pos0 + (int)g0;
    // The group's selections: rows g0 .. g1-1 of sel_out, or the workspace.
    int32_t* gsel = sel_out ? sel_out + g0 * d->top_k : ws_sel;
    if (fused) {
      // Long history: indexer -> top-k handoff without the score matrix.
      spmla::FusedArgs fa{};
      fa.iq = iq + g0 * spmla::kIdxHeads * spmla::kIdxDim;
      fa.iw = iw + g0 * spmla::kIdxHeads;
      fa.ik = ik;
      fa.sel = gsel;
      fa.n_sel = nullptr;
      fa.sel_asc = ascending ? ws_sel_asc : nullptr;
      fa.n_q = gn;
      fa.q_pos0 = gpos0;
      fa.n_comp = d->n_comp;
      fa.ratio = d->ratio;
      fa.top_k = d->top_k;
      fa.plan = spmla::fused_plan(d->n_comp, d->top_k);
      spmla::fused_bind_workspace(fa, ws);
      rc = hip_status(spmla::launch_fused_topk(fa, st), "fused selection launch");
      if (rc) return;
    } else {
      if (d->n_comp > 0) {
        spmla::IndexerArgs ia;
        ia.iq = iq + g0 * spmla::kIdxHeads * spmla::kIdxDim;
        ia.iw = iw + g0 * spmla::kIdxHeads;
        ia.ik = ik;
        ia.scores = scores;
        ia.ld_scores = band_ld(d);
        ia.n_q = gn;
        ia.q_pos0 = gpos0;
        ia.n_comp = d->n_comp;
        ia.ratio = d->ratio;
        ia.fill_invisible = 0;  // top-k reads only the rows each token can see
        ia.span = 0;
        rc = hip_status(spmla::launch_indexer(ia, st), "indexer launch");
        if (rc) return;
      }
      spmla::TopkArgs ta;
      ta.scores = scores;
      ta.ld_scores = band_ld(d);
      ta.sel = gsel;
      ta.n_sel = nullptr;
      ta.sel_asc = ascending ? ws_sel_asc : nullptr;
      ta.n_q = gn;
      ta.q_pos0 = gpos0;
      ta.n_comp = d->n_comp;
      ta.ratio = d->ratio;
      ta.top_k = d->top_k;
      rc = hip_status(spmla::launch_topk(ta, st), "top-k launch");
      if (rc) return;
    }

    // Attention band by band: whole queries in one launch over the group's
    // bands (each band dealt to the dies as its own launch would be, the next
    // band starting as the previous one drains); key splits in a launch per
    // band, whose partials share the scratch.
    if (spmla::attn_splits(d->n_q) == 1) {
      const int32_t* sel = ascending ? ws_sel_asc : gsel;
      spmla::AttnArgs aa = attn_args(d, q + g0 * spmla::kHeads * spmla::kDqk, kv_comp, kv_raw, sel,
                                     out + g0 * spmla::kHeads * spmla::kDv, lse ? lse + g0 * spmla::kHeads : nullptr);
      aa.n_q = gn;
      aa.q_pos0 = gpos0;
      aa.band_items = d->band;
      rc = hip_status(spmla::launch_attn(aa, st), "attention launch");
      return;
    }
    for (int64_t b0 = g0; b0 < g1; b0 += d->band) {
      const int bn = band_len(d, b0);
      const int64_t row = b0 - g0;  // first row of this band's selections within the group
      const int32_t* sel = ascending ? ws_sel_asc + row * d->top_k : gsel + row * d->top_k;
      spmla::AttnArgs aa = attn_args(d, q + b0 * spmla::kHeads * spmla::kDqk, kv_comp, kv_raw, sel,
                                     out + b0 * spmla::kHeads * spmla::kDv,
                                     lse ? lse + b0 * spmla::kHeads : nullptr);
      aa.n_q = bn;
      aa.q_pos0 = d->q_pos0 + (int)b0;
      aa.splits = spmla::attn_splits(d->n_q);
      if (aa.splits > 1) {  // a small call: split each key list, partials in the scratch
        const size_t items = (size_t)bn * aa.splits;
        aa.part_o = reinterpret_cast<float*>(ws);
        aa.part_ml = aa.part_o + items * spmla::kHeads * spmla::kDv;
      }
      rc = hip_status(spmla::launch_attn(aa, st), "attention launch");
      if (rc) return;
    }
  });
  if (rc) return rc;
  return ok();
}

}  // namespace

extern "C" {

const char* spmla_last_error(void) { return g_last_error.c_str(); }

int spmla_abi_version(void) { return 1; }

int spmla_check_desc(const spmla_desc* desc) {
  const int rc = check_desc(desc);
  return rc ? rc : ok();
}

int spmla_num_bands(const spmla_desc* desc) {
  const int rc = check_desc(desc);
  if (rc) return rc;
  ok();
  return (int)(((int64_t)desc->n_q + desc->band - 1) / desc->band);
}

int spmla_indexer_scores(const spmla_desc* d, const int8_t* iq, const int8_t* iw, const int8_t* ik,
                         int32_t* scores, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->n_q == 0) return ok();
  REQUIRE_PTR(iq);
  REQUIRE_PTR(iw);
  if (d->n_comp > 0) {
    REQUIRE_PTR(ik);
    REQUIRE_PTR(scores);
  }
  spmla::IndexerArgs a;
  a.iq = iq;
  a.iw = iw;
  a.ik = ik;
  a.scores = scores;
  a.ld_scores = d->n_comp;
  a.n_q = d->n_q;
  a.q_pos0 = d->q_pos0;
  a.n_comp = d->n_comp;
  a.ratio = d->ratio;
  a.fill_invisible = 1;  // the full matrix is the documented output
  a.span = 0;
  return hip_status(spmla::launch_indexer(a, (hipStream_t)stream), "indexer launch");
}

int spmla_topk(const spmla_desc* d, const int32_t* scores, int32_t* sel, int32_t* n_sel,
               void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->n_q == 0) return ok();
  if (d->n_comp > 0) REQUIRE_PTR(scores);
  REQUIRE_PTR(sel);
  OPTIONAL_PTR(n_sel);
  spmla::TopkArgs a;
  a.scores = scores;
  a.ld_scores = d->n_comp;
  a.sel = sel;
  a.n_sel = n_sel;
  a.sel_asc = nullptr;
  a.n_q = d->n_q;
  a.q_pos0 = d->q_pos0;
  a.n_comp = d->n_comp;
  a.ratio = d->ratio;
  a.top_k = d->top_k;
  return hip_status(spmla::launch_topk(a, (hipStream_t)stream), "top-k launch");
}

int spmla_sparse_attn(const spmla_desc* d, const uint16_t* q, const uint16_t* kv_comp,
                      const uint16_t* kv_raw, const int32_t* sel, float* out, float* lse,
                      void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->n_q == 0) return ok();
  REQUIRE_PTR(q);
  if (d->n_comp > 0) REQUIRE_PTR(kv_comp);
  REQUIRE_PTR(kv_raw);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(lse);
  spmla::AttnArgs a = attn_args(d, q, kv_comp, kv_raw, sel, out, lse);
  a.band_items = d->band;  // a call over several bands is dealt to the dies band by band
  return hip_status(spmla::launch_attn(a, (hipStream_t)stream), "attention launch");
}

int spmla_sparse_attn_grouped(const spmla_desc* d, const uint16_t* q, const uint16_t* kv_comp,
                              const uint16_t* kv_raw, const int32_t* sel, float* out, float* lse,
                              void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->n_q == 0) return ok();
  REQUIRE_PTR(q);
  if (d->n_comp > 0) REQUIRE_PTR(kv_comp);
  REQUIRE_PTR(kv_raw);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(lse);
  const spmla::AttnArgs a = attn_args(d, q, kv_comp, kv_raw, sel, out, lse);
  return hip_status(spmla::launch_attn_grouped(a, (hipStream_t)stream), "grouped attention launch");
}

int spmla_compress(const spmla_desc* d, const uint16_t* kv_raw, uint16_t* kv_comp, int32_t comp_begin,
                   void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->ratio != 4) return fail(SPMLA_EUNSUPPORTED, "compression is built for ratio 4 (got %d)", d->ratio);
  if (comp_begin < 0 || comp_begin > d->n_comp)
    return fail(SPMLA_EINVAL, "comp_begin %d outside [0, n_comp=%d]", comp_begin, d->n_comp);
  if (comp_begin == d->n_comp) return ok();
  REQUIRE_PTR(kv_raw);
  REQUIRE_PTR(kv_comp);
  return hip_status(spmla::launch_compress(kv_raw, kv_comp, comp_begin, d->n_comp, (hipStream_t)stream),
                    "compress launch");
}

int spmla_prefill_workspace_bytes(const spmla_desc* d, size_t* bytes) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!bytes) return fail(SPMLA_EINVAL, "bytes is NULL");
  *bytes = ws_layout(d, kGroupBudget).total();
  return ok();
}

int spmla_prefill(const spmla_desc* d, const uint16_t* q, const uint16_t* kv_comp,
                  const uint16_t* kv_raw, const int8_t* iq, const int8_t* iw, const int8_t* ik,
                  float* out, float* lse, int32_t* sel_out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->n_q == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv_raw);
  REQUIRE_PTR(iq);
  REQUIRE_PTR(iw);
  if (d->n_comp > 0) {
    REQUIRE_PTR(kv_comp);
    REQUIRE_PTR(ik);
  }
  REQUIRE_PTR(out);
  OPTIONAL_PTR(lse);
  OPTIONAL_PTR(sel_out);
  size_t need = 0;
  spmla_prefill_workspace_bytes(d, &need);
  if (workspace_bytes < need)
    return fail(SPMLA_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  REQUIRE_PTR(workspace);

  return run_prefill(d, q, kv_comp, kv_raw, iq, iw, ik, out, lse, sel_out, static_cast<char*>(workspace),
                     kGroupBudget, (hipStream_t)stream);
}

int spmla_prefill_noalloc(const spmla_desc* d, const uint16_t* q, const uint16_t* kv_comp,
                          const uint16_t* kv_raw, const int8_t* iq, const int8_t* iw, const int8_t* ik,
                          float* out, float* lse, int32_t* sel_out, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->n_q == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv_raw);
  REQUIRE_PTR(iq);
  REQUIRE_PTR(iw);
  if (d->n_comp > 0) {
    REQUIRE_PTR(kv_comp);
    REQUIRE_PTR(ik);
  }
  REQUIRE_PTR(out);
  OPTIONAL_PTR(lse);
  OPTIONAL_PTR(sel_out);
  // Selection groups whose selection scratch and selection copies each take
  // at most half the array; bands halve until the call's scratch fits
  // (results do not depend on the band).
  const size_t cap = spmla::kNoAllocScratchBytes;
  const GroupBudget gb{cap / 2, cap / 2, cap / 2};
  spmla_desc dd = *d;
  size_t need = ws_layout(&dd, gb).total();
  while (need > cap && dd.band > 1) {
    dd.band = (dd.band + 1) / 2;
    need = ws_layout(&dd, gb).total();
  }
  if (need > cap)
    return fail(SPMLA_EWORKSPACE, "needs %zu bytes of scratch even at band %d; the no-alloc scratch holds %zu",
                need, dd.band, cap);
  // The scratch is per device: the stream must run on the current device.
  int cur = -1, sdev = -1;
  rc = hip_status(hipGetDevice(&cur), "current device");
  if (rc) return rc;
  rc = hip_status(hipStreamGetDevice((hipStream_t)stream, &sdev), "device of the stream");
  if (rc) return rc;
  if (sdev != cur) return fail(SPMLA_EINVAL, "stream is on device %d, the current device is %d", sdev, cur);
  void* scratch = nullptr;
  rc = hip_status(spmla::noalloc_scratch(&scratch), "no-alloc scratch address");
  if (rc) return rc;
  return run_prefill(&dd, q, kv_comp, kv_raw, iq, iw, ik, out, lse, sel_out, static_cast<char*>(scratch), gb,
                     (hipStream_t)stream);
}

}  // extern "C"
