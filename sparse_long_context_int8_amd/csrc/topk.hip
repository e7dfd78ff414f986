// Per-token top-k of the visible compressed rows.
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): the long-prefill top-k rows go straight to attention and
// the selected-row order is preserved. Order: score descending, then lower
// row index; fewer than k visible rows are all taken and the rest is -1.
//
// One workgroup per query token. The token's visible scores stay in
// registers (PER per thread). Each row gets a unique integer key that
// encodes both ordering rules,
//     key = ((score - min_score) << ebits) | (n_vis - 1 - row),
// so the k-th largest key is found by an MSD radix select over 8-bit digits
// (LDS histogram per digit, only the bits that differ between rows are
// visited), then the k winners are sorted in LDS by a bitonic network.
// Integer only: the result is exact and does not depend on thread timing.
#include "spmla_internal.h"

namespace spmla {
namespace {

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

template <int BLOCK, int PER>
__global__ __launch_bounds__(BLOCK) void topk_kernel(TopkArgs a) {
  constexpr int NW = BLOCK / 64;
  __shared__ int hist[256];
  __shared__ int red_max[NW], red_min[NW];
  __shared__ int s_bin, s_above, s_count, s_cnt;
  extern __shared__ unsigned long long keys[];  // next_pow2(top_k) entries

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int t = a.q_pos0 + r;
  const int nv = min(a.n_comp, (t + 1) / a.ratio);
  const int k = a.top_k;
  const int nsel = min(k, nv);
  int32_t* sel_row = a.sel + (int64_t)r * k;

  if (nsel == 0) {
    for (int i = tid; i < k; i += BLOCK) sel_row[i] = -1;
    if (a.n_sel && tid == 0) a.n_sel[r] = 0;
    return;
  }

  // Scores of this token in registers; element e = i*BLOCK + tid.
  const int32_t* row = a.scores + (int64_t)r * a.ld_scores;
  int sc[PER];
  int vmax = INT32_MIN, vmin = INT32_MAX;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * BLOCK + tid;
    sc[i] = e < nv ? row[e] : INT32_MIN;
    if (e < nv) {
      vmax = max(vmax, sc[i]);
      vmin = min(vmin, sc[i]);
    }
  }
  vmax = wave_max_i(vmax);
  vmin = wave_min_i(vmin);
  if (lane == 0) {
    red_max[wave] = vmax;
    red_min[wave] = vmin;
  }
  __syncthreads();
  vmax = red_max[0];
  vmin = red_min[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    vmax = max(vmax, red_max[w]);
    vmin = min(vmin, red_min[w]);
  }
  // Bits of the row part and of the score part of the key.
  const int ebits = nv > 1 ? 32 - __clz(nv - 1) : 0;
  const unsigned span = (unsigned)vmax - (unsigned)vmin;  // exact: vmax >= vmin
  const int sbits = span ? 32 - __clz(span) : 0;
  const int total_bits = sbits + ebits;

  auto key_of = [&](int i) -> unsigned long long {
    const int e = i * BLOCK + tid;
    const unsigned long long s = (unsigned)sc[i] - (unsigned)vmin;
    return (s << ebits) | (unsigned long long)(nv - 1 - e);
  };

  // Radix select of the nsel-th largest key (all keys when nv <= k).
  unsigned long long thresh = 0;
  if (nv > k) {
    int need = k;
    unsigned long long prefix = 0;
    int shift = ((total_bits + 7) / 8) * 8 - 8;
    while (true) {
      for (int b = tid; b < 256; b += BLOCK) hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = i * BLOCK + tid;
        if (e < nv) {
          const unsigned long long key = key_of(i);
          if ((key >> (shift + 8)) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
        }
      }
      __syncthreads();
      if (wave == 0) {
        // Lane L holds bins 255-4L .. 252-4L (descending order).
        int c[4];
        int tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = hist[255 - 4 * lane - q];
          tot += c[q];
        }
        int incl = tot;  // inclusive scan over lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(incl, o);
          if (lane >= o) incl += v;
        }
        int above = incl - tot;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above < need && need <= above + c[q]) {
            s_bin = 255 - 4 * lane - q;
            s_above = above;
            s_count = c[q];
          }
          above += c[q];
        }
      }
      __syncthreads();
      const int bin = s_bin, above = s_above, count = s_count;
      need -= above;
      prefix = (prefix << 8) | (unsigned)bin;
      if (count == need || shift == 0) {
        thresh = prefix << shift;
        break;
      }
      shift -= 8;
      __syncthreads();  // hist is cleared again at the top of the loop
    }
  }

  // Collect the nsel winners (keys >= thresh), stored as key + 1 so that the
  // zero padding sorts after every real entry.
  int p2 = 1;
  while (p2 < nsel) p2 <<= 1;
  if (tid == 0) s_cnt = 0;
  for (int i = tid; i < p2; i += BLOCK) keys[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * BLOCK + tid;
    if (e < nv) {
      const unsigned long long key = key_of(i);
      if (key >= thresh) {
        const int pos = atomicAdd(&s_cnt, 1);
        if (pos < p2) keys[pos] = key + 1;  // pos < nsel <= p2 by construction
      }
    }
  }
  __syncthreads();

  // Bitonic sort, descending.
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (p2 >> 1); i += BLOCK) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const unsigned long long x = keys[lo], y = keys[hi];
        if (desc ? (x < y) : (x > y)) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  const unsigned long long emask = ebits ? ((1ull << ebits) - 1) : 0ull;
  for (int i = tid; i < k; i += BLOCK) {
    int v = -1;
    if (i < nsel) v = (nv - 1) - (int)((keys[i] - 1) & emask);
    sel_row[i] = v;
  }
  if (a.n_sel && tid == 0) a.n_sel[r] = nsel;
}

template <int BLOCK, int PER>
hipError_t launch_cfg(const TopkArgs& a, hipStream_t stream) {
  int p2 = 1;
  while (p2 < a.top_k) p2 <<= 1;
  const size_t lds = sizeof(unsigned long long) * (size_t)p2;
  hipLaunchKernelGGL((topk_kernel<BLOCK, PER>), dim3(a.n_q), dim3(BLOCK), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  const int nc = a.n_comp;
  if (nc <= 256 * 4) return launch_cfg<256, 4>(a, stream);
  if (nc <= 256 * 8) return launch_cfg<256, 8>(a, stream);
  if (nc <= 1024 * 8) return launch_cfg<1024, 8>(a, stream);
  if (nc <= 1024 * 16) return launch_cfg<1024, 16>(a, stream);
  return launch_cfg<1024, 32>(a, stream);  // n_comp <= 32768 (host-checked)
}

}  // namespace spmla
