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
};

struct TopkArgs {
  const int32_t* scores;  // [n_q][ld_scores]
  int64_t ld_scores;
  int32_t* sel;           // [n_q][top_k]
  int32_t* n_sel;         // [n_q] or null
  int32_t n_q;
  int32_t q_pos0;
  int32_t n_comp;
  int32_t ratio;
  int32_t top_k;
};

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
};

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace spmla
