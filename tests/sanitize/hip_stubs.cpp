// Host-only stand-ins for the HIP runtime and the kernel launchers, used to
// build the library's host code (argument checks, workspace sizing, band and
// selection-group schedule) with AddressSanitizer and UndefinedBehavior-
// Sanitizer on a machine without a GPU.
//
// Every launcher checks that each array it would read or write lies inside
// one of the regions the fuzz driver registered for the call (fake device
// addresses that are never dereferenced), with the extent the kernel's
// indexing implies. A violation prints the launch and aborts.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "spmla_internal.h"
#include "stub_regions.h"

namespace stub {

Region g_regions[kMaxRegions];
int g_n_regions = 0;
long g_launches = 0;

void clear() { g_n_regions = 0; }

void add(const char* name, const void* base, size_t bytes) {
  if (g_n_regions >= kMaxRegions) {
    std::fprintf(stderr, "too many regions\n");
    std::abort();
  }
  g_regions[g_n_regions++] = Region{name, reinterpret_cast<uintptr_t>(base), bytes};
}

void require(const char* what, const void* p, double bytes) {
  if (bytes <= 0) return;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  for (int i = 0; i < g_n_regions; ++i) {
    const Region& r = g_regions[i];
    if (lo >= r.base && lo - r.base <= r.bytes && bytes <= (double)(r.bytes - (lo - r.base))) return;
  }
  std::fprintf(stderr, "OUT OF BOUNDS: %s at %#lx, %.0f bytes, in no registered region\n", what,
               (unsigned long)lo, bytes);
  for (int i = 0; i < g_n_regions; ++i)
    std::fprintf(stderr, "  region %s [%#lx, +%zu)\n", g_regions[i].name, (unsigned long)g_regions[i].base,
                 g_regions[i].bytes);
  std::abort();
}

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "BROKEN LAUNCH INVARIANT: %s\n", what);
    std::abort();
  }
}

}  // namespace stub

using stub::expect;
using stub::require;

// ------------------------------------------------------------ HIP runtime
extern "C" {
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) {
  *d = 0;
  return hipSuccess;
}
}

namespace spmla {

namespace {
int n_vis_max(int q_pos0, int n_q, int n_comp, int ratio) {
  const long long t_last = (long long)q_pos0 + n_q - 1;
  const long long v = (t_last + 1) / ratio;
  return (int)(v < n_comp ? v : n_comp);
}
}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t) {
  ++stub::g_launches;
  if (a.n_q <= 0 || a.n_comp <= 0) return hipSuccess;  // the launcher enqueues nothing
  expect(a.ld_scores >= a.n_comp, "indexer: row stride below n_comp");
  require("indexer iq", a.iq, (double)a.n_q * kIdxHeads * kIdxDim);
  require("indexer iw", a.iw, (double)a.n_q * kIdxHeads);
  require("indexer ik", a.ik, (double)a.n_comp * kIdxDim);
  // 16-byte groups may run up to the next multiple of 4 columns when the
  // stride is a multiple of 4 (the stride then covers them).
  const long long cols = a.ld_scores % 4 == 0 ? ((long long)a.n_comp + 3) / 4 * 4 : a.n_comp;
  expect(cols <= a.ld_scores, "indexer: 16-byte groups past the row stride");
  require("indexer scores", a.scores, 4.0 * ((double)(a.n_q - 1) * a.ld_scores + cols));
  return hipSuccess;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t) {
  ++stub::g_launches;
  if (a.n_q <= 0) return hipSuccess;
  expect(a.top_k >= 1 && a.top_k <= kMaxTopK && a.n_comp <= kMaxComp, "topk: sizes");
  const int nv = n_vis_max(a.q_pos0, a.n_q, a.n_comp, a.ratio);
  if (nv > 0) require("topk scores", a.scores, 4.0 * ((double)(a.n_q - 1) * a.ld_scores + nv));
  require("topk sel", a.sel, 4.0 * a.n_q * a.top_k);
  if (a.sel_asc) require("topk sel_asc", a.sel_asc, 4.0 * a.n_q * a.top_k);
  if (a.n_sel) require("topk n_sel", a.n_sel, 4.0 * a.n_q);
  return hipSuccess;
}

hipError_t launch_fused_topk(const FusedArgs& f, hipStream_t) {
  ++stub::g_launches;
  if (f.n_q <= 0) return hipSuccess;
  expect(f.n_q >= 256, "fused: fewer than 256 tokens");
  expect(fused_applies(f.n_q, f.q_pos0, f.n_comp, f.ratio, f.top_k), "fused: launched where it does not apply");
  expect(f.plan.n_spans * f.plan.span >= f.n_comp && f.plan.n_spans <= 512, "fused: span plan");
  require("fused iq", f.iq, (double)f.n_q * kIdxHeads * kIdxDim);
  require("fused iw", f.iw, (double)f.n_q * kIdxHeads);
  require("fused ik", f.ik, (double)f.n_comp * kIdxDim);
  require("fused sel", f.sel, 4.0 * f.n_q * f.top_k);
  if (f.sel_asc) require("fused sel_asc", f.sel_asc, 4.0 * f.n_q * f.top_k);
  if (f.n_sel) require("fused n_sel", f.n_sel, 4.0 * f.n_q);
  require("fused thresh", f.thresh, 4.0 * f.n_q);
  require("fused n_redo", f.n_redo, 4.0);
  require("fused redo_list", f.redo_list, 4.0 * f.n_q);
  require("fused counts", f.counts, 4.0 * f.n_q * f.plan.n_spans);
  require("fused cand", f.cand, 8.0 * f.n_q * f.plan.n_spans * f.plan.cap);
  return hipSuccess;
}

namespace {
void check_attn(const AttnArgs& a, const char* kind) {
  char what[64];
  auto req = [&](const char* field, const void* p, double bytes) {
    std::snprintf(what, sizeof what, "%s %s", kind, field);
    require(what, p, bytes);
  };
  expect((long long)a.q_pos0 + a.n_q <= a.n_raw, "attention: query rows beyond n_raw");
  expect(a.n_comp == a.n_raw / a.ratio, "attention: n_comp");
  req("q", a.q, 2.0 * a.n_q * kHeads * kDqk);
  if (n_vis_max(a.q_pos0, a.n_q, a.n_comp, a.ratio) > 0) req("kv_comp", a.kv_comp, 2.0 * a.n_comp * kDqk);
  req("kv_raw", a.kv_raw, 2.0 * ((double)a.q_pos0 + a.n_q) * kDqk);
  req("sel", a.sel, 4.0 * a.n_q * a.top_k);
  req("out", a.out, 4.0 * a.n_q * kHeads * kDv);
  if (a.lse) req("lse", a.lse, 4.0 * a.n_q * kHeads);
  expect(a.splits >= 1 && a.splits <= kMaxSplits, "attention: splits");
  if (a.splits > 1) {
    req("part_o", a.part_o, 4.0 * a.n_q * a.splits * kHeads * kDv);
    req("part_ml", a.part_ml, 8.0 * a.n_q * a.splits * kHeads);
    const uintptr_t o_end = reinterpret_cast<uintptr_t>(a.part_o) + (size_t)a.n_q * a.splits * kHeads * kDv * 4;
    expect(reinterpret_cast<uintptr_t>(a.part_ml) >= o_end, "attention: partial O and (m, l) overlap");
  }
}
}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t) {
  ++stub::g_launches;
  if (a.n_q <= 0) return hipSuccess;
  check_attn(a, "attention");
  return hipSuccess;
}

hipError_t launch_attn_grouped(const AttnArgs& a, hipStream_t) {
  ++stub::g_launches;
  if (a.n_q <= 0) return hipSuccess;
  check_attn(a, "grouped attention");
  expect(a.splits == 1, "grouped attention: splits");
  return hipSuccess;
}

hipError_t launch_compress(const uint16_t* kv_raw, uint16_t* kv_comp, int comp_begin, int n_comp, hipStream_t) {
  ++stub::g_launches;
  expect(comp_begin >= 0 && comp_begin < n_comp, "compress: range");
  require("compress kv_raw", kv_raw, 2.0 * 4 * n_comp * kDqk);
  require("compress kv_comp", kv_comp, 2.0 * n_comp * kDqk);
  return hipSuccess;
}

hipError_t noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(stub::kScratchBase);
  return hipSuccess;
}

}  // namespace spmla
