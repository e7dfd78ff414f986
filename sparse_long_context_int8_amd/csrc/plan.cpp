// Host-side planning shared by the C ABI and the launchers: which selection
// path a launch takes, the fused handoff's span plan and workspace layout,
// and the key splits of small calls. Plain host C++ (no device code), so the
// C ABI's schedule can also be built and checked without a GPU.
#include <algorithm>

#include "spmla_internal.h"

namespace spmla {

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

// The fused selection serves a launch of at least 256 tokens (fewer leave
// its passes latency-bound, and their score band is small) when every token
// keeps at most 2048 of more than 4096 visible rows and sees at least 8 rows
// per kept row, so that the 1-in-8 sample (16-row blocks) holds enough rows
// above the threshold.
bool fused_applies(int n_q, int q_pos0, int n_comp, int ratio, int top_k) {
  if (n_q < 256 || top_k > 2048) return false;
  const int nv_min = std::min(n_comp, (q_pos0 + 1) / ratio);
  return nv_min > 4096 && nv_min >= 8 * top_k;
}

FusedPlan fused_plan(int n_comp, int top_k) {
  FusedPlan p;
  p.span = 512;
  p.n_spans = (n_comp + p.span - 1) / p.span;  // <= 64 <= finish block
  p.cap = p.span / 4;                         // about 2.5x the expected count
  p.stride = 8;
  // The sample holds about k/8 rows above the k-th score; asking for four
  // standard deviations more makes a threshold below it very likely.
  const int base = (top_k + p.stride - 1) / p.stride;
  int sd = 1;
  while (sd * sd < base) ++sd;
  p.rank = base + 4 * sd + 16;
  return p;
}

size_t fused_workspace_bytes(int n_q, const FusedPlan& p) {
  const size_t nq = (size_t)n_q;
  return align256(nq * 4) + align256(4) + align256(nq * 4) + align256(nq * p.n_spans * 4) +
         align256(nq * p.n_spans * p.cap * 8);
}

void fused_bind_workspace(FusedArgs& a, void* ws) {
  char* w = static_cast<char*>(ws);
  const size_t nq = (size_t)a.n_q;
  a.thresh = reinterpret_cast<int32_t*>(w);
  w += align256(nq * 4);
  a.n_redo = reinterpret_cast<int32_t*>(w);
  w += align256(4);
  a.redo_list = reinterpret_cast<int32_t*>(w);
  w += align256(nq * 4);
  a.counts = reinterpret_cast<int32_t*>(w);
  w += align256(nq * a.plan.n_spans * 4);
  a.cand = reinterpret_cast<int32_t*>(w);
}

int attn_splits(int n_q_call) {
  if (n_q_call >= 512 || n_q_call <= 0) return 1;  // an empty call has nothing to split
  const int s = (1024 + n_q_call - 1) / n_q_call;
  return s < kMaxSplits ? s : kMaxSplits;
}

size_t attn_partial_bytes(int rows, int splits) {
  if (splits <= 1) return 0;
  const size_t items = (size_t)rows * splits;
  return items * kHeads * kDv * sizeof(float) + items * kHeads * 2 * sizeof(float);
}

}  // namespace spmla
