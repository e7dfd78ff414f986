// Integer indexer scores on CDNA4 matrix cores.
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): every query token is scored against the ratio-4 compressed
// rows it can see, and visibility comes from positions alone. Score form:
//   S[t][j] = sum_h w[t][h] * max(0, <iq[t][h][:], ik[j][:]>)
// with int8 inputs, so every value is an exact int32.
//
// The head dot products form a dense int8 contraction
//   [n_q*4 rows (t,h)] x [64] . [64] x [n_comp]
// which runs on v_mfma_i32_16x16x64_i8. A 16-row A tile holds 4 query tokens
// x 4 heads (row r = 4*t_local + h); in the 16x16 result a lane owns rows
// 4*(lane/16) .. +3 of one column, i.e. all 4 heads of one (token, row) pair,
// so ReLU and the weighted head sum finish inside the lane with integer ops.
#include "spmla_internal.h"

namespace spmla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kQTile = 64;   // query tokens per workgroup (16 per wave)
constexpr int kJTile = 64;   // compressed rows per workgroup (4 MFMA columns)

__global__ __launch_bounds__(256) void indexer_kernel(IndexerArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t_base = blockIdx.y * kQTile + wave * 16;  // first token of this wave
  const int j_base = blockIdx.x * kJTile;
  if (t_base >= a.n_q) return;

  // Visible rows of the last token of this wave bound the useful columns.
  const int t_last = min(t_base + 15, a.n_q - 1);
  const int nv_last = min(a.n_comp, (a.q_pos0 + t_last + 1) / a.ratio);

  const int col = lane & 15;  // MFMA column within a 16-wide tile
  const int grp = lane >> 4;  // which 16-byte slice of the 64-wide k dim

  // A fragments: 4 tiles of 4 tokens x 4 heads. Row r of tile m is the
  // 64-byte vector iq[t_base + 4m + r/4][r%4][:], i.e. flat row 4*t + r.
  v4i afrag[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = 4 * (t_base + 4 * m) + col;  // flat (token, head) row
    const int tok = t_base + 4 * m + (col >> 2);
    if (tok < a.n_q) {
      afrag[m] = *reinterpret_cast<const v4i*>(a.iq + (int64_t)row * kIdxDim + grp * 16);
    } else {
      afrag[m] = v4i{0, 0, 0, 0};
    }
  }
  // Weights of the token this lane owns in each tile: 4 int8 packed in 32 bits.
  int wpack[4];
  int tok_of[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tok = t_base + 4 * m + grp;
    tok_of[m] = tok;
    wpack[m] = tok < a.n_q ? *reinterpret_cast<const int*>(a.iw + (int64_t)tok * kIdxHeads) : 0;
  }

#pragma unroll
  for (int jt = 0; jt < kJTile / 16; ++jt) {
    const int j0 = j_base + jt * 16;
    if (j0 >= a.n_comp) break;
    const int j = j0 + col;
    v4i acc[4];
    if (j0 < nv_last) {
      // B fragment: 16 compressed keys (columns) x 64.
      v4i bfrag = v4i{0, 0, 0, 0};
      if (j < a.n_comp) bfrag = *reinterpret_cast<const v4i*>(a.ik + (int64_t)j * kIdxDim + grp * 16);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag[m], bfrag, v4i{0, 0, 0, 0}, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = v4i{0, 0, 0, 0};
    }
    if (j >= a.n_comp) continue;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tok = tok_of[m];
      if (tok >= a.n_q) continue;
      const int nv = min(a.n_comp, (a.q_pos0 + tok + 1) / a.ratio);
      int s = INT32_MIN;
      if (j < nv) {
        const int w = wpack[m];
        s = 0;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int wh = (int)(int8_t)((w >> (8 * h)) & 0xff);
          s += wh * max(acc[m][h], 0);
        }
      }
      a.scores[(int64_t)tok * a.ld_scores + j] = s;
    }
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream) {
  if (a.n_q <= 0 || a.n_comp <= 0) return hipSuccess;
  dim3 grid((a.n_comp + kJTile - 1) / kJTile, (a.n_q + kQTile - 1) / kQTile);
  hipLaunchKernelGGL(indexer_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spmla
