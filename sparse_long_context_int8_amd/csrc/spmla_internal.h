// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Every launcher assumes the host has validated its arguments: sizes are in
// range, pointers are non-null where the step reads or writes them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace spmla {

// Shapes the kernels are compiled for (MLA layer: 16 heads sharing a
// 576-wide latent of which the first 512 dims are the value; int8 indexer of
// 4 heads x 64 dims).
constexpr int kHeads = 16;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kMaxTopK = 4096;
constexpr int kMaxComp = 32768;
constexpr int kMaxSplits = 32;  // key splits per query of a small call
constexpr size_t kDieL2Bytes = (size_t)4 << 20;  // L2 of one accelerator die
// Compressed rows beyond one die's L2: the attention then gathers them from
// MALL or HBM, in ascending row order (spmla_prefill hands it the selection
// sorted so) with its loads spread over each chunk's softmax.
inline bool rows_beyond_l2(int n_comp) { return (size_t)n_comp * kDqk * 2 > kDieL2Bytes; }

struct IndexerArgs {
  const int8_t* iq;   // [n_q][4][64]
  const int8_t* iw;   // [n_q][4]
  const int8_t* ik;   // [n_comp][64]
  int32_t* scores;    // [n_q][ld_scores]
  int64_t ld_scores;  // row stride of scores (elements) >= n_comp
  int32_t n_q;
  int32_t q_pos0;     // absolute position of query 0 of this launch
  int32_t n_comp;
  int32_t ratio;
  int32_t fill_invisible;  // also write INT32_MIN where no token can see the row
  int32_t span;            // compressed rows per workgroup (set by the launcher)
  int32_t xcd_tiles;       // token tiles dealt to dies by tile mod 8 (set by the launcher)
};

struct TopkArgs {
  const int32_t* scores;  // [n_q][ld_scores]
  int64_t ld_scores;
  int32_t* sel;           // [n_q][top_k]
  int32_t* n_sel;         // [n_q] or null
  int32_t* sel_asc;       // [n_q][top_k] or null: the same rows in ascending order, -1 padded
  int32_t n_q;
  int32_t q_pos0;
  int32_t n_comp;
  int32_t ratio;
  int32_t top_k;
};

// Selection for long histories without a materialized score band
// (indexer -> top-k handoff): a sampled pass sets a per-token score
// threshold, a collect pass recomputes exact scores and keeps the candidates
// at or above it in fixed per-(token, span) slots, a finish pass selects and
// sorts them exactly, and tokens whose candidates do not provably contain the
// top-k (too few, or a slot overflowed) are redone from recomputed scores.
struct FusedPlan {
  int32_t span;     // compressed rows per collect workgroup (multiple of 64)
  int32_t n_spans;  // ceil(n_comp / span)
  int32_t cap;      // candidate slots per (token, span)
  int32_t stride;   // sampling stride of the threshold pass
  int32_t rank;     // sample rank whose bin sets the threshold
};

struct FusedArgs {
  const int8_t* iq;  // [n_q][4][64]
  const int8_t* iw;  // [n_q][4]
  const int8_t* ik;  // [n_comp][64]
  int32_t* sel;      // [n_q][top_k]
  int32_t* n_sel;    // [n_q] or null
  int32_t* sel_asc;  // [n_q][top_k] or null (see TopkArgs)
  int32_t n_q;
  int32_t q_pos0;
  int32_t n_comp;
  int32_t ratio;
  int32_t top_k;
  FusedPlan plan;
  // Workspace (fused_workspace_bytes): thresh [n_q], the recompute list
  // (n_redo, redo_list [n_q]), counts [n_q][n_spans] and
  // cand [n_q][n_spans][cap] x (score, row).
  int32_t* thresh;
  int32_t* n_redo;
  int32_t* redo_list;
  int32_t* counts;
  int32_t* cand;
};

// Whether the fused selection serves this launch (every token sees many
// more rows than it keeps), its plan, and its workspace.
bool fused_applies(int n_q, int q_pos0, int n_comp, int ratio, int top_k);
FusedPlan fused_plan(int n_comp, int top_k);
size_t fused_workspace_bytes(int n_q, const FusedPlan& p);
void fused_bind_workspace(FusedArgs& a, void* ws);

struct AttnArgs {
  const _Float16* q;        // [n_q][16][576]
  const _Float16* kv_comp;  // [n_comp][576]
  const _Float16* kv_raw;   // [n_raw][576]
  const int32_t* sel;       // [n_q][top_k]
  float* out;               // [n_q][16][512]
  float* lse;               // [n_q][16] or null
  int32_t n_q;
  int32_t q_pos0;
  int32_t n_comp;
  int32_t n_raw;
  int32_t ratio;
  int32_t window;
  int32_t top_k;
  float scale_log2e;        // softmax scale * log2(e)
  // Key splits per query (1: each workgroup does a whole query). With more,
  // each (query, split) writes a partial O [16][512] and (m, l) [16] to
  // part_o / part_ml, and a merge pass writes out and lse.
  int32_t splits;
  float* part_o;            // [n_q * splits][16][512]
  float* part_ml;           // [n_q * splits][16][2]
  // Whole queries only (splits == 1): if > 0, the launch covers its queries
  // as consecutive bands of band_items queries (the last one ragged), each
  // dealt to the dies as a launch of its own would be, band after band, so
  // that a band's first queries start as the previous band's last finish.
  int32_t band_items;
};

// Key splits per query for a call of n_q_call queries (enough work items to
// fill the chip when the call is small; a function of the whole call, so
// results do not depend on how it is cut into bands) and the partial-result
// bytes of `rows` queries.
int attn_splits(int n_q_call);
size_t attn_partial_bytes(int rows, int splits);

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
hipError_t launch_fused_topk(const FusedArgs& a, hipStream_t stream);
// Parts of the fused selection that compute indexer scores (indexer.hip).
hipError_t launch_sample_threshold(const FusedArgs& a, hipStream_t stream);
hipError_t launch_collect(const FusedArgs& a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);
// Query-tiled variant: pairs of adjacent queries share one gather of their
// key union (same results as launch_attn up to fp32 summation order).
hipError_t launch_attn_grouped(const AttnArgs& a, hipStream_t stream);
// kv_comp rows comp_begin .. n_comp-1 from kv_raw (ratio 4, d_qk wide).
hipError_t launch_compress(const uint16_t* kv_raw, uint16_t* kv_comp, int comp_begin, int n_comp,
                           hipStream_t stream);

// Bytes of the device-resident scratch array of spmla_prefill_noalloc, and
// its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace spmla
