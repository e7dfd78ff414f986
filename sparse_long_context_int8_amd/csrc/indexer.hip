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
//
// A workgroup holds 64 tokens (16 per wave, their A tiles in registers) and
// sweeps a span of compressed rows 64 at a time. Of the four B tiles of a
// step, tile u takes rows j0 + 4c + u in column c, so each lane ends up with
// 4 adjacent scores of one token and writes them as one 16-byte store: a
// store instruction covers 4 token rows x 256 contiguous bytes.
#include "spmla_internal.h"

namespace spmla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kQTile = 64;  // query tokens per workgroup (16 per wave)
constexpr int kJStep = 64;  // compressed rows per step (4 MFMA column tiles)

// VEC: 16-byte stores; the row stride is a multiple of 4 and at least n_comp
// rounded up to 4, so a group that straddles n_comp stays inside the row
// (its entries past n_comp are INT32_MIN).
template <bool VEC>
__global__ __launch_bounds__(256) void indexer_kernel(IndexerArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t_base = blockIdx.y * kQTile + wave * 16;  // first token of this wave
  if (t_base >= a.n_q) return;
  const int j_begin = blockIdx.x * a.span;
  const int j_end = min(a.n_comp, j_begin + a.span);

  // Rows visible to the last token of this wave bound the columns to score.
  const int t_last = min(t_base + 15, a.n_q - 1);
  const int nv_wave = min(a.n_comp, (a.q_pos0 + t_last + 1) / a.ratio);

  const int col = lane & 15;  // MFMA column within a 16-wide tile
  const int grp = lane >> 4;  // which 16-byte slice of the 64-wide k dim

  // A fragments: 4 tiles of 4 tokens x 4 heads. Row r of tile m is the
  // 64-byte vector iq[t_base + 4m + r/4][r%4][:], i.e. flat row 4*t + r.
  v4i afrag[4];
  int wpack[4];  // weights of the token this lane owns in tile m (4 x int8)
  int tok_of[4];
  int nv_of[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = 4 * (t_base + 4 * m) + col;
    const int tok_a = t_base + 4 * m + (col >> 2);
    afrag[m] = tok_a < a.n_q ? *reinterpret_cast<const v4i*>(a.iq + (int64_t)row * kIdxDim + grp * 16)
                             : v4i{0, 0, 0, 0};
    const int tok = t_base + 4 * m + grp;
    tok_of[m] = tok;
    wpack[m] = tok < a.n_q ? *reinterpret_cast<const int*>(a.iw + (int64_t)tok * kIdxHeads) : 0;
    nv_of[m] = min(a.n_comp, (a.q_pos0 + tok + 1) / a.ratio);
  }

  auto store4 = [&](int tok, int j, v4i s) {
    int32_t* dst = a.scores + (int64_t)tok * a.ld_scores + j;
    if constexpr (VEC) {
      if (j < a.n_comp) *reinterpret_cast<v4i*>(dst) = s;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j + u < a.n_comp) dst[u] = s[u];
    }
  };

  const int j_score_end = min(j_end, nv_wave);
  int j0 = j_begin;
  for (; j0 < j_score_end; j0 += kJStep) {
    v4i bfrag[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jr = j0 + 4 * col + u;
      bfrag[u] = jr < a.n_comp ? *reinterpret_cast<const v4i*>(a.ik + (int64_t)jr * kIdxDim + grp * 16)
                               : v4i{0, 0, 0, 0};
    }
    const int jl = j0 + 4 * col;  // first of this lane's 4 rows
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4i acc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag[m], bfrag[u], v4i{0, 0, 0, 0}, 0, 0, 0);
      if (tok_of[m] >= a.n_q) continue;
      v4i s;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int v = 0;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int wh = (int)(int8_t)((wpack[m] >> (8 * h)) & 0xff);
          v += wh * max(acc[u][h], 0);
        }
        s[u] = jl + u < nv_of[m] ? v : INT32_MIN;
      }
      if (jl < j_end) store4(tok_of[m], jl, s);
    }
  }
  // Rows no token of this wave can see.
  if (a.fill_invisible) {
    const v4i inv = v4i{INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
    for (; j0 < j_end; j0 += kJStep) {
      const int jl = j0 + 4 * col;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (tok_of[m] < a.n_q && jl < j_end) store4(tok_of[m], jl, inv);
    }
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a_in, hipStream_t stream) {
  if (a_in.n_q <= 0 || a_in.n_comp <= 0) return hipSuccess;
  IndexerArgs a = a_in;
  // Column span per workgroup: whole 64-row steps, enough workgroups to
  // cover the chip several times over.
  const int col_steps = (a.n_comp + kJStep - 1) / kJStep;
  const int q_tiles = (a.n_q + kQTile - 1) / kQTile;
  int steps_per_wg = (int)(((int64_t)col_steps * q_tiles) / 2048);
  if (steps_per_wg < 1) steps_per_wg = 1;
  a.span = steps_per_wg * kJStep;
  dim3 grid((a.n_comp + a.span - 1) / a.span, q_tiles);
  // 16-byte groups may run past n_comp into the row padding, never past
  // the row stride.
  const int64_t n_comp4 = ((int64_t)a.n_comp + 3) / 4 * 4;
  const bool vec = (a.ld_scores % 4 == 0) && (a.ld_scores >= n_comp4) && ((uintptr_t)a.scores % 16 == 0);
  if (vec) {
    hipLaunchKernelGGL(indexer_kernel<true>, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(indexer_kernel<false>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace spmla
