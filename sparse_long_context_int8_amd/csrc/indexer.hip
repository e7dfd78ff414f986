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

// The weights of one token, sign-extended.
struct HeadWeights {
  int w[4];
};
__device__ __forceinline__ HeadWeights head_weights(int wpack) {
  HeadWeights w;
#pragma unroll
  for (int h = 0; h < 4; ++h) w.w[h] = (int)(int8_t)((wpack >> (8 * h)) & 0xff);
  return w;
}
constexpr int kQTile = 64;  // query tokens per workgroup (16 per wave)
constexpr int kJStep = 64;  // compressed rows per step (4 MFMA column tiles)

// The 64 tokens of a workgroup seen from one lane: A tiles (tile m holds
// tokens t_base + 4m .. +3 of the wave), and the token whose scores this lane
// receives in each tile, with its weights and visible-row count.
struct TokenTiles {
  v4i afrag[4];
  HeadWeights w[4];  // weights of the lane's token in tile m
  int tok[4];
  int nv[4];

  __device__ __forceinline__ void load(const int8_t* iq, const int8_t* iw, int n_q, int q_pos0, int n_comp,
                                       int ratio, int t_base, int col, int grp) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // Row r of tile m is the 64-byte vector iq[t_base + 4m + r/4][r%4][:].
      const int row = 4 * (t_base + 4 * m) + col;
      const int tok_a = t_base + 4 * m + (col >> 2);
      afrag[m] = tok_a < n_q ? *reinterpret_cast<const v4i*>(iq + (int64_t)row * kIdxDim + grp * 16)
                             : v4i{0, 0, 0, 0};
      tok[m] = t_base + 4 * m + grp;
      w[m] = head_weights(tok[m] < n_q ? *reinterpret_cast<const int*>(iw + (int64_t)tok[m] * kIdxHeads) : 0);
      nv[m] = min(n_comp, (q_pos0 + tok[m] + 1) / ratio);
    }
  }
};

// B tiles of one 64-row step: tile u, column c holds compressed row j0+4c+u.
__device__ __forceinline__ void load_b(const int8_t* ik, int n_comp, int j0, int col, int grp, v4i (&b)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int jr = j0 + 4 * col + u;
    b[u] = jr < n_comp ? *reinterpret_cast<const v4i*>(ik + (int64_t)jr * kIdxDim + grp * 16) : v4i{0, 0, 0, 0};
  }
}

// Weighted head sum of one 16x16 result: the 4 heads of the lane's token.
// A head dot product of 64 int8 pairs is at most 64 * 128 * 128 = 2^20 in
// magnitude and a weight at most 128, so ReLU'd products and weights both
// fit the signed 24-bit operands of the full-rate integer multiply-add, and
// every product (<= 2^27) and the sum (<= 2^29) are exact in int32.
__device__ __forceinline__ int head_sum(v4i acc, const HeadWeights& w) {
  int s = __mul24(max(acc[0], 0), w.w[0]);
#pragma unroll
  for (int h = 1; h < 4; ++h) s += __mul24(max(acc[h], 0), w.w[h]);
  return s;
}
// Scores of the lane's token in tile m for rows j0+4c .. j0+4c+3.
__device__ __forceinline__ v4i tile_scores(const TokenTiles& tt, int m, const v4i (&b)[4]) {
  v4i s;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(tt.afrag[m], b[u], v4i{0, 0, 0, 0}, 0, 0, 0);
    s[u] = head_sum(acc, tt.w[m]);
  }
  return s;
}

// VEC: 16-byte stores; the row stride is a multiple of 4 and at least n_comp
// rounded up to 4, so a group that straddles n_comp stays inside the row
// (its entries past n_comp are INT32_MIN).
// Dies: workgroups are dealt to the 8 dies round-robin by their linear index.
constexpr int kDies = 8;

template <bool VEC>
__global__ __launch_bounds__(256) void indexer_kernel(IndexerArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // With xcd_tiles, every span of token tile T runs on die T mod 8 (the grid
  // has a multiple of 8 tiles): the tile's query rows are then read by the
  // workgroups of one die, whose L2 serves all but the first.
  int span_idx = blockIdx.x, tile = blockIdx.y;
  if (a.xcd_tiles) {
    const unsigned lin = blockIdx.y * gridDim.x + blockIdx.x;
    const unsigned q = lin / kDies;
    tile = (int)(kDies * (q / gridDim.x) + lin % kDies);
    span_idx = (int)(q % gridDim.x);
  }
  const int t_base = tile * kQTile + wave * 16;  // first token of this wave
  if (t_base >= a.n_q) return;
  const int j_begin = span_idx * a.span;
  const int j_end = min(a.n_comp, j_begin + a.span);

  // Rows visible to the last token of this wave bound the columns to score.
  const int t_last = min(t_base + 15, a.n_q - 1);
  const int nv_wave = min(a.n_comp, (a.q_pos0 + t_last + 1) / a.ratio);

  const int col = lane & 15;  // MFMA column within a 16-wide tile
  const int grp = lane >> 4;  // which 16-byte slice of the 64-wide k dim
  TokenTiles tt;
  tt.load(a.iq, a.iw, a.n_q, a.q_pos0, a.n_comp, a.ratio, t_base, col, grp);

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
    load_b(a.ik, a.n_comp, j0, col, grp, bfrag);
    const int jl = j0 + 4 * col;  // first of this lane's 4 rows
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4i s = tile_scores(tt, m, bfrag);
      if (tt.tok[m] >= a.n_q) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (jl + u >= tt.nv[m]) s[u] = INT32_MIN;
      if (jl < j_end) store4(tt.tok[m], jl, s);
    }
  }
  // Rows no token of this wave can see.
  if (a.fill_invisible) {
    const v4i inv = v4i{INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
    for (; j0 < j_end; j0 += kJStep) {
      const int jl = j0 + 4 * col;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (tt.tok[m] < a.n_q && jl < j_end) store4(tt.tok[m], jl, inv);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused selection, score-side passes.

// Monotone 11-bit code of an int32 score: 32 exact small magnitudes, then
// 32 steps per power of two (a float with 5 mantissa bits), negatives
// mirrored below 1024. code(x) <= code(y) whenever x <= y.
__device__ __forceinline__ int mag_code(unsigned y) {  // 0 .. 863
  if (y < 32) return (int)y;
  const int e = 31 - __clz((int)y);
  return 32 + 32 * (e - 5) + (int)((y >> (e - 5)) & 31);
}
__device__ __forceinline__ int score_code(int x) {
  return x >= 0 ? 1024 + mag_code((unsigned)x) : 1023 - mag_code((unsigned)(-(x + 1)));
}
// Smallest magnitude with a given code (0 .. 864; 864 gives 2^31).
__device__ __forceinline__ int64_t mag_lo(int f) {
  if (f < 32) return f;
  const int e = (f - 32) / 32 + 5;
  return (int64_t)(32 + (f - 32) % 32) << (e - 5);
}
// Smallest score whose code is c: every score >= it has code >= c.
__device__ __forceinline__ int code_lo(int c) {
  return c >= 1024 ? (int)mag_lo(c - 1024) : (int)(-mag_lo(1023 - c + 1));
}

constexpr int kCodes = 2048;

// Threshold pass (also clears the recompute list of the finish pass): one
// workgroup per 4 tokens (one A tile); its 4 waves take turns over the
// sampled rows, one block of 16 consecutive rows in every 16 * stride (whole
// 128-byte lines of the int8 keys, where single rows every stride apart would
// use half of each line). Each workgroup starts its walk over the sampled
// blocks at its own offset, so that the workgroups in flight read different
// key lines at any moment instead of all queueing on the same L2 channel.
// Each sampled visible score lands in a per-token LDS histogram of score
// codes (16-bit counts, two per word: a token has at most 4,096 samples); the
// threshold is the lowest score of the code bin in which the count from the
// top reaches `rank` (INT32_MIN if fewer samples than that).
__global__ __launch_bounds__(256) void sample_threshold_kernel(FusedArgs a) {
  __shared__ unsigned hist[4][kCodes / 2];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * 4;
  for (int i = threadIdx.x; i < 2 * kCodes; i += 256) (&hist[0][0])[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.n_redo = 0;  // the finish pass fills the list

  const int tok_a = t0 + (col >> 2);
  const v4i afrag = tok_a < a.n_q
                        ? *reinterpret_cast<const v4i*>(a.iq + ((int64_t)4 * t0 + col) * kIdxDim + grp * 16)
                        : v4i{0, 0, 0, 0};
  const int tok = t0 + grp;
  const HeadWeights hw = head_weights(tok < a.n_q ? *reinterpret_cast<const int*>(a.iw + (int64_t)tok * kIdxHeads) : 0);
  const int nv = tok < a.n_q ? min(a.n_comp, (a.q_pos0 + tok + 1) / a.ratio) : 0;
  const int t_last = min(t0 + 3, a.n_q - 1);
  const int nv_max = min(a.n_comp, (a.q_pos0 + t_last + 1) / a.ratio);
  const int stride = a.plan.stride;
  const int n_steps = (nv_max + 16 * stride - 1) / (16 * stride);
  const int rot = n_steps > 0 ? (int)(((unsigned)blockIdx.x * 97u) % (unsigned)n_steps) : 0;
  __syncthreads();

  constexpr int kUnroll = 4;
  for (int s0 = wave * kUnroll; s0 < n_steps; s0 += 4 * kUnroll) {
    v4i b[kUnroll];
    int j[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      int step = s0 + q + rot;
      if (step >= n_steps) step -= n_steps;
      j[q] = 16 * stride * step + col;
      b[q] = (s0 + q < n_steps && j[q] < a.n_comp)
                 ? *reinterpret_cast<const v4i*>(a.ik + (int64_t)j[q] * kIdxDim + grp * 16)
                 : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag, b[q], v4i{0, 0, 0, 0}, 0, 0, 0);
      if (s0 + q < n_steps && j[q] < nv) {
        const int c = score_code(head_sum(acc, hw));
        atomicAdd(&hist[grp][c >> 1], 1u << (16 * (c & 1)));
      }
    }
  }
  __syncthreads();

  // Wave w sets the threshold of token t0 + w; lane l owns codes
  // kCodes-1 - kPer*l down to kCodes - kPer*(l+1) (scanned from the top),
  // kPer / 2 words, which it sums in a rotated order so that the lanes of a
  // read hit different LDS banks.
  constexpr int kPer = kCodes / 64;
  constexpr int kWords = kPer / 2;
  const int tw = t0 + wave;
  if (tw >= a.n_q) return;
  const unsigned* const hw_row = hist[wave];
  const int w_lo = (kCodes - kPer * (lane + 1)) / 2;  // the lane's lowest word
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    const unsigned v = hw_row[w_lo + ((i + lane) & (kWords - 1))];
    tot += (int)(v & 0xffffu) + (int)(v >> 16);
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  const int need = a.plan.rank;
  int code = -1;
  int above = incl - tot;
  if (above < need && need <= incl) {
    for (int i = 0; i < kPer; ++i) {
      const int c = kCodes - 1 - kPer * lane - i;
      above += (int)((hw_row[c >> 1] >> (16 * (c & 1))) & 0xffffu);
      if (above >= need) {
        code = c;
        break;
      }
    }
  }
  // One lane found it (or none, when the sample is smaller than the rank).
  const unsigned long long found = __ballot(code >= 0);
  if (found == 0) {
    if (lane == 0) a.thresh[tw] = INT32_MIN;
  } else if (code >= 0) {
    a.thresh[tw] = code_lo(code);
  }
}

// Collect pass: the indexer's 64-token x span tiling with exact scores; every
// visible score >= the token's threshold is written as (score, row) into the
// token's slots for this span. In a 16x16 result the 16 lanes of a row hold
// one token (4 adjacent key rows each), and only this wave sees that token,
// so its slot counter lives in registers: per step, one inclusive scan of the
// lanes' counts inside each 16-lane row (the four tiles' counts packed one
// byte each: at most 64 per row) gives every lane its place, and a swizzle
// broadcasts the row total. The step's candidates of a row are first packed
// in the wave's LDS area, then written with one store instruction per tile
// and 16 of them (16 consecutive slots per row): scattered single stores,
// one instruction per tile and key row, were a quarter of the pass. Slots
// follow (step, lane, key row) order. The count written at the end is the
// true count, so the finish pass can detect a full span.
__global__ __launch_bounds__(256) void collect_kernel(FusedArgs a) {
  __shared__ int2 stage_[4][4][4][64];  // [wave][tile m][row grp][entry]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t_base = blockIdx.y * kQTile + wave * 16;
  if (t_base >= a.n_q) return;
  const int span_idx = blockIdx.x;
  const int j_begin = span_idx * a.plan.span;
  const int j_end = min(a.n_comp, j_begin + a.plan.span);
  const int t_last = min(t_base + 15, a.n_q - 1);
  const int nv_wave = min(a.n_comp, (a.q_pos0 + t_last + 1) / a.ratio);
  const int col = lane & 15, grp = lane >> 4;
  const int cap = a.plan.cap;
  int2(*const stage)[4][64] = stage_[wave];

  TokenTiles tt;
  tt.load(a.iq, a.iw, a.n_q, a.q_pos0, a.n_comp, a.ratio, t_base, col, grp);
  int thr[4], lim[4];
  int32_t* slots[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bool ok = tt.tok[m] < a.n_q;
    thr[m] = ok ? a.thresh[tt.tok[m]] : INT32_MAX;
    lim[m] = ok ? min(tt.nv[m], j_end) : 0;  // rows below lim are visible and in the span
    slots[m] = a.cand + 2 * (((int64_t)(ok ? tt.tok[m] : 0) * a.plan.n_spans + span_idx) * cap);
  }

  int run[4] = {0, 0, 0, 0};  // slots claimed so far by the row's token in tile m
  const int j_score_end = min(j_end, nv_wave);
  for (int j0 = j_begin; j0 < j_score_end; j0 += kJStep) {
    v4i bfrag[4];
    load_b(a.ik, a.n_comp, j0, col, grp, bfrag);
    const int jl = j0 + 4 * col;
    v4i sc[4];
    int packed = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      sc[m] = tile_scores(tt, m, bfrag);
      int c = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) c += (jl + u < lim[m] && sc[m][u] >= thr[m]) ? 1 : 0;
      packed |= c << (8 * m);
    }
    // Inclusive scan inside each 16-lane row (row_shr 1, 2, 4, 8), then the
    // row total from the row's lane 15 (swizzle: lane (l & 16) | 15 of each
    // 32-lane half).
    int incl = packed;
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, false);
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, false);
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, false);
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, false);
    const int tot = __builtin_amdgcn_ds_swizzle(incl, 0x1f0);
    const int excl = incl - packed;
    // Pack the row's candidates (LDS operations of one wave complete in
    // order, so the reads below see these writes).
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      int e = (excl >> (8 * m)) & 0xff;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (jl + u < lim[m] && sc[m][u] >= thr[m]) {
          stage[m][grp][e] = int2{sc[m][u], jl + u};
          ++e;
        }
      }
    }
    // Entries col, col + 16, ... of each row go to consecutive slots.
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int n = (tot >> (8 * m)) & 0xff;
      for (int e = col; e < n; e += 16) {
        const int pos = run[m] + e;
        if (pos < cap) *reinterpret_cast<int2*>(slots[m] + 2 * pos) = stage[m][grp][e];
      }
      run[m] += n;
    }
  }
  if (col == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (tt.tok[m] < a.n_q) a.counts[(int64_t)tt.tok[m] * a.plan.n_spans + span_idx] = run[m];
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
  // Die-aligned tiles for launches of at least 16 tiles (fewer would leave
  // padding workgroups idle for a sizeable share of the grid).
  a.xcd_tiles = q_tiles >= 16 ? 1 : 0;
  const int grid_tiles = a.xcd_tiles ? (q_tiles + kDies - 1) / kDies * kDies : q_tiles;
  dim3 grid((a.n_comp + a.span - 1) / a.span, grid_tiles);
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

hipError_t launch_sample_threshold(const FusedArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_threshold_kernel, dim3((a.n_q + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_collect(const FusedArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  dim3 grid(a.plan.n_spans, (a.n_q + kQTile - 1) / kQTile);
  hipLaunchKernelGGL(collect_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spmla
