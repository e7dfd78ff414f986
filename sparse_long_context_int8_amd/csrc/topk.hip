// Per-token top-k of the visible compressed rows.
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): the long-prefill top-k rows go straight to attention and
// the selected-row order is preserved. Order: score descending, then lower
// row index; fewer than k visible rows are all taken and the rest is -1.
//
// One workgroup per query token; its visible scores stay in registers (PER
// per thread). Every row gets a unique integer key encoding both rules,
//     key = ((score - min_score) << ebits) | (n_vis - 1 - row),
// so "the k largest keys" is exactly the selection and "keys descending" is
// exactly the output order.
//   1. coarse pass: an LDS histogram of the top 11 bits of (score - min)
//      locates the bin holding the k-th largest key (2048 bins keep LDS
//      atomic contention low for bell-shaped score distributions);
//   2. refinement: MSD radix select over the remaining key bits, only for
//      the rows in that bin (usually a handful);
//   3. the winners (padded with zeros to a power of two S >= BLOCK) are
//      sorted by a compile-time bitonic network: pairs inside a thread in
//      registers, across lanes with swizzles, across waves through LDS.
// Integer only: exact, and independent of thread timing.
#include "spmla_internal.h"

namespace spmla {
namespace {

typedef unsigned long long u64;

constexpr int kBins1 = 2048;  // coarse-pass bins (11 bits)
constexpr int kBits1 = 11;

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
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}
// 64-bit value of lane (lane ^ M) of the same wave.
template <int M>
__device__ __forceinline__ u64 lane_xor(u64 v) {
  unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
  if constexpr (M < 32) {
    // ds_swizzle bit-mask mode: source lane = lane ^ M inside each 32 lanes
    constexpr int kPat = (M << 10) | 0x1f;
    lo = (unsigned)__builtin_amdgcn_ds_swizzle((int)lo, kPat);
    hi = (unsigned)__builtin_amdgcn_ds_swizzle((int)hi, kPat);
  } else {
    lo = __shfl_xor(lo, 32);
    hi = __shfl_xor(hi, 32);
  }
  return ((u64)hi << 32) | lo;
}

// Bitonic network sorting S = BLOCK*E keys descending, fully unrolled.
// Thread t holds positions t*E .. t*E+E-1. A compare-exchange whose partner
// is in the same thread runs in registers, one in another lane of the wave
// runs through a lane swizzle, and one in another wave goes through LDS
// (two alternating buffers of S keys, one barrier per step).
template <int BLOCK, int E>
struct BitonicDesc {
  static constexpr int S = BLOCK * E;

  template <int SIZE, int STRIDE>
  __device__ static __forceinline__ void step(u64 (&v)[E], u64* buf, int tid, int& flip) {
    if constexpr (STRIDE < E) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (i & STRIDE) continue;
        const bool desc = ((tid * E + i) & SIZE) == 0;
        const u64 x = v[i], y = v[i + STRIDE];
        const bool sw = desc ? (x < y) : (x > y);
        v[i] = sw ? y : x;
        v[i + STRIDE] = sw ? x : y;
      }
    } else {
      u64 p[E];
      if constexpr (STRIDE < 64 * E) {
#pragma unroll
        for (int i = 0; i < E; ++i) p[i] = lane_xor<STRIDE / E>(v[i]);
      } else {
        u64* b = buf + flip * S;
#pragma unroll
        for (int i = 0; i < E; ++i) b[tid * E + i] = v[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < E; ++i) p[i] = b[(tid * E + i) ^ STRIDE];
        flip ^= 1;
      }
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int e = tid * E + i;
        const bool keep_max = ((e & SIZE) == 0) == ((e & STRIDE) == 0);
        const u64 hi = v[i] > p[i] ? v[i] : p[i];
        const u64 lo = v[i] > p[i] ? p[i] : v[i];
        v[i] = keep_max ? hi : lo;
      }
    }
  }

  template <int SIZE, int STRIDE>
  __device__ static __forceinline__ void merge(u64 (&v)[E], u64* buf, int tid, int& flip) {
    step<SIZE, STRIDE>(v, buf, tid, flip);
    if constexpr (STRIDE > 1) merge<SIZE, STRIDE / 2>(v, buf, tid, flip);
  }

  template <int SIZE>
  __device__ static __forceinline__ void sort_from(u64 (&v)[E], u64* buf, int tid, int& flip) {
    merge<SIZE, SIZE / 2>(v, buf, tid, flip);
    if constexpr (SIZE < S) sort_from<SIZE * 2>(v, buf, tid, flip);
  }

  // buf: 2*S keys of LDS. Every thread of the block must call this.
  __device__ static __forceinline__ void sort(u64 (&v)[E], u64* buf, int tid) {
    int flip = 0;
    if constexpr (S > 1) sort_from<2>(v, buf, tid, flip);
  }
};

// Bins are scanned from the top. Finds the bin b in which the running count
// of elements above first reaches `need`; returns it through shared slots.
// `hist` holds nbins counters; all threads of the block must call this.
template <int BLOCK>
__device__ __forceinline__ void find_bin(const int* hist, int nbins, int need, int* s_bin, int* s_above,
                                         int* s_count, int* red) {
  constexpr int NW = BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (nbins + BLOCK - 1) / BLOCK;
  // Thread t owns bins [nbins-1 - t*per, ...) going down.
  int tot = 0;
  for (int i = 0; i < per; ++i) {
    const int b = nbins - 1 - (tid * per + i);
    if (b >= 0) tot += hist[b];
  }
  const int incl = wave_incl_scan(tot, lane);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  int above = before + incl - tot;
  if (above < need && need <= above + tot) {
    for (int i = 0; i < per; ++i) {
      const int b = nbins - 1 - (tid * per + i);
      if (b < 0) break;
      const int c = hist[b];
      if (above < need && need <= above + c) {
        *s_bin = b;
        *s_above = above;
        *s_count = c;
        break;
      }
      above += c;
    }
  }
  (void)NW;
  __syncthreads();
}

template <int BLOCK, int PER, int E>
__global__ __launch_bounds__(BLOCK) void topk_kernel(TopkArgs a) {
  constexpr int NW = BLOCK / 64;
  constexpr int S = BLOCK * E;  // sort size
  __shared__ int hist[kBins1];
  __shared__ int red_a[NW], red_b[NW], red_c[NW];
  __shared__ int s_bin, s_above, s_count, s_cnt;
  extern __shared__ u64 keys[];  // 2*S entries

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
    sc[i] = e < nv ? __builtin_nontemporal_load(row + e) : INT32_MIN;
    if (e < nv) {
      vmax = max(vmax, sc[i]);
      vmin = min(vmin, sc[i]);
    }
  }
  vmax = wave_max_i(vmax);
  vmin = wave_min_i(vmin);
  if (lane == 0) {
    red_a[wave] = vmax;
    red_b[wave] = vmin;
  }
  __syncthreads();
  vmax = red_a[0];
  vmin = red_b[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    vmax = max(vmax, red_a[w]);
    vmin = min(vmin, red_b[w]);
  }
  const int ebits = nv > 1 ? 32 - __clz(nv - 1) : 0;
  const unsigned span = (unsigned)vmax - (unsigned)vmin;  // exact: vmax >= vmin
  const int sbits = span ? 32 - __clz(span) : 0;
  auto key_of = [&](int i) -> u64 {
    const int e = i * BLOCK + tid;
    const u64 s = (unsigned)sc[i] - (unsigned)vmin;
    return (s << ebits) | (u64)(nv - 1 - e);
  };

  u64 thresh = 0;  // selected iff key >= thresh
  if (nv > k) {
    // 1. coarse pass on the top kBits1 bits of (score - min).
    const int sh1 = sbits > kBits1 ? sbits - kBits1 : 0;
    for (int b = tid; b < kBins1; b += BLOCK) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = i * BLOCK + tid;
      if (e < nv) atomicAdd(&hist[((unsigned)sc[i] - (unsigned)vmin) >> sh1], 1);
    }
    __syncthreads();
    find_bin<BLOCK>(hist, kBins1, k, &s_bin, &s_above, &s_count, red_c);
    const int bin1 = s_bin;
    int need = k - s_above;
    const int low_bits = sh1 + ebits;  // key bits below the coarse digit
    u64 prefix = (u64)bin1;            // key >> shift must equal this
    if (s_count == need || low_bits == 0) {
      thresh = prefix << low_bits;
    } else {
      // 2. refine inside the bin with 8-bit digits of the remaining bits.
      int shift = ((low_bits + 7) / 8) * 8 - 8;
      // The first refinement digit may straddle the coarse digit: candidates
      // are matched on key >> low_bits, digits taken below that.
      int top = low_bits;  // bits of the key above `top` are fixed to prefix
      while (true) {
        __syncthreads();
        for (int b = tid; b < 256; b += BLOCK) hist[b] = 0;
        __syncthreads();
        const int dbits = top - shift;  // digit width this pass (<= 8)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int e = i * BLOCK + tid;
          if (e < nv) {
            const u64 key = key_of(i);
            if ((key >> top) == prefix) atomicAdd(&hist[(key >> shift) & ((1u << dbits) - 1)], 1);
          }
        }
        __syncthreads();
        find_bin<BLOCK>(hist, 1 << dbits, need, &s_bin, &s_above, &s_count, red_c);
        need -= s_above;
        prefix = (prefix << dbits) | (u64)s_bin;
        top = shift;
        if (s_count == need || shift == 0) {
          thresh = prefix << shift;
          break;
        }
        shift = shift >= 8 ? shift - 8 : 0;
      }
    }
  }

  // Collect the nsel winners into keys[0 .. nsel); stored as key + 1 so that
  // the zero padding up to S sorts after every real entry.
  if (tid == 0) s_cnt = 0;
  for (int i = tid; i < S; i += BLOCK) keys[i] = 0;
  __syncthreads();
  // One LDS atomic per wave and register: lanes take consecutive slots.
  const u64 below = (1ull << lane) - 1;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * BLOCK + tid;
    const bool take = e < nv && key_of(i) >= thresh;
    const u64 m = __ballot(take);
    if (m == 0) continue;  // wave-uniform
    int base = 0;
    if (lane == 0) base = atomicAdd(&s_cnt, __popcll(m));
    base = __shfl(base, 0);
    const int pos = base + __popcll(m & below);
    if (take && pos < S) keys[pos] = key_of(i) + 1;  // pos < nsel <= S by construction
  }
  __syncthreads();

  // 3. sort descending; thread t ends up holding ranks t*E .. t*E+E-1.
  u64 v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = keys[tid * E + i];
  BitonicDesc<BLOCK, E>::sort(v, keys, tid);

  const u64 emask = ebits ? ((1ull << ebits) - 1) : 0ull;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int rank = tid * E + i;
    if (rank < k) sel_row[rank] = rank < nsel ? (nv - 1) - (int)((v[i] - 1) & emask) : -1;
  }
  for (int i = S + tid; i < k; i += BLOCK) sel_row[i] = -1;  // only when k > S
  if (a.n_sel && tid == 0) a.n_sel[r] = nsel;
}

// Sort size for a launch: at least one element per thread, and at least the
// most winners any query of the launch can have.
inline int sort_size(int block, int top_k, int n_comp) {
  const int m = min(top_k, n_comp);
  int s = block;
  while (s < m) s <<= 1;
  return s;
}

template <int BLOCK, int PER, int E>
hipError_t launch_e(const TopkArgs& a, hipStream_t stream) {
  // keys[S] plus the second buffer of the cross-wave exchange.
  const size_t lds = 2 * sizeof(u64) * (size_t)(BLOCK * E);
  hipLaunchKernelGGL((topk_kernel<BLOCK, PER, E>), dim3(a.n_q), dim3(BLOCK), lds, stream, a);
  return hipGetLastError();
}

template <int BLOCK, int PER>
hipError_t launch_cfg(const TopkArgs& a, hipStream_t stream) {
  const int e = sort_size(BLOCK, a.top_k, a.n_comp) / BLOCK;
  switch (e) {
    case 1: return launch_e<BLOCK, PER, 1>(a, stream);
    case 2: return launch_e<BLOCK, PER, 2>(a, stream);
    case 4: return launch_e<BLOCK, PER, 4>(a, stream);
    // S <= BLOCK*PER since n_comp <= BLOCK*PER for this configuration
    case 8: if constexpr (8 <= PER && BLOCK * 8 <= 4096) return launch_e<BLOCK, PER, 8>(a, stream); break;
    case 16: if constexpr (16 <= PER && BLOCK * 16 <= 4096) return launch_e<BLOCK, PER, 16>(a, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;  // unreachable: top_k <= 4096 is host-checked
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  const int nc = a.n_comp;
  if (nc <= 256 * 4) return launch_cfg<256, 4>(a, stream);
  if (nc <= 256 * 8) return launch_cfg<256, 8>(a, stream);
  if (nc <= 512 * 8) return launch_cfg<512, 8>(a, stream);
  if (nc <= 1024 * 8) return launch_cfg<1024, 8>(a, stream);
  if (nc <= 1024 * 16) return launch_cfg<1024, 16>(a, stream);
  return launch_cfg<1024, 32>(a, stream);  // n_comp <= 32768 (host-checked)
}

}  // namespace spmla
