// Per-token top-k of the visible compressed rows.
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): the long-prefill top-k rows go straight to attention and
// the selected-row order is preserved. Order: score descending, then lower
// row index; fewer than k visible rows are all taken and the rest is -1.
//
// One workgroup per query token; its elements (visible scores, or the
// candidates of the fused selection) stay in registers, PER per thread.
// Every row gets a unique integer key encoding both rules,
//     key = ((score - min_score) << ebits) | (n_vis - 1 - row),
// so "the k largest keys" is exactly the selection and "keys descending" is
// exactly the output order.
//   1. coarse pass: an LDS histogram of the top 11 bits of (score - min)
//      locates the bin holding the k-th largest key (2048 bins keep LDS
//      atomic contention low for bell-shaped score distributions);
//   2. refinement: MSD radix select over the remaining key bits, only for
//      the rows in that bin (usually a handful);
//   3. ordering: the keys at or above the threshold are counted per bucket
//      (the top 11 bits of their offset), bucket offsets come from one
//      prefix scan, every key is scattered from registers into its bucket,
//      and each key's place inside its bucket is the number of larger keys
//      in the bucket
//      (buckets hold a few keys for spread-out scores); the first k places
//      are the output.
// The refinement (2) runs only while the keys at or above the threshold
// would exceed k + kSlack; usually the coarse bin already gets there, and its
// extra keys simply fall beyond place k.
// Integer only: exact, and independent of thread timing.
#include "spmla_internal.h"

namespace spmla {
namespace {

typedef unsigned long long u64;

constexpr int kBins1 = 2048;  // coarse-pass and ordering bins (11 bits)
constexpr int kBits1 = 11;
// Elements beyond k a workgroup may collect and order. With top_k 512 over
// at most 2,048 rows a workgroup then holds 8,256 B of static and 6,016 B of
// dynamic LDS, so eight share a CU and a 2,048-token band runs in one round.
constexpr int kSlack = 240;
// Registers per thread up to which kept keys are scattered into their buckets
// straight from registers (above it they are collected first).
constexpr int kDirectPer = 16;

// Wave-wide scans and reductions with DPP (no LDS round trips): row_shr:n
// shifts within each 16-lane row (lanes without a source take the identity),
// then row_bcast:15 / row_bcast:31 (GCN/CDNA only) carry row totals into the
// rows above. The inclusive result of lane 63 is the wave total.
template <typename Op>
__device__ __forceinline__ int wave_incl(int v, int id, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xa, 0xf, false));  // row_bcast:15 -> rows 1, 3
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xc, 0xf, false));  // row_bcast:31 -> rows 2, 3
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
  return __builtin_amdgcn_readlane(wave_incl(v, INT32_MIN, [](int x, int y) { return max(x, y); }), 63);
}
__device__ __forceinline__ int wave_min_i(int v) {
  return __builtin_amdgcn_readlane(wave_incl(v, INT32_MAX, [](int x, int y) { return min(x, y); }), 63);
}
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
  return wave_incl(v, 0, [](int x, int y) { return x + y; });
}

// Bins are scanned from the top. Finds the bin b in which the running count
// of elements above first reaches `need`; returns it through shared slots.
// `hist` holds nbins <= MAXBINS counters; all threads of the block must call
// this. Thread t owns bins nbins-1 - (t*PER + i), i < PER, going down, and
// keeps their counts in registers for the search.
template <int BLOCK, int MAXBINS>
__device__ __forceinline__ void find_bin(const int* hist, int nbins, int need, int* s_bin, int* s_above,
                                         int* s_count, int* red) {
  constexpr int PER = (MAXBINS + BLOCK - 1) / BLOCK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c[PER];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = nbins - 1 - (tid * PER + i);
    c[i] = b >= 0 ? hist[b] : 0;
    tot += c[i];
  }
  const int incl = wave_incl_scan(tot, lane);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  int above = before + incl - tot;
  if (above < need && need <= above + tot) {
    // This thread's bins hold the need-th element: the first bin, going
    // down, at which the running count reaches it (no more LDS reads).
    int bin = -1, at = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (bin < 0 && need <= above + c[i]) {
        bin = nbins - 1 - (tid * PER + i);
        at = above;
        cnt = c[i];
      }
      above += c[i];
    }
    *s_bin = bin;
    *s_above = at;
    *s_count = cnt;
  }
  __syncthreads();
}

// Bucket offsets, largest bucket first: hist[b] (the count of bucket b)
// becomes the number of elements in buckets above b, i.e. the fill cursor of
// bucket b. Ends with a barrier.
template <int BLOCK>
__device__ __forceinline__ void bucket_offsets(int* hist, int* red) {
  constexpr int kPer = kBins1 / BLOCK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c[kPer];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = hist[kBins1 - 1 - (tid * kPer + i)];
    tot += c[i];
  }
  const int incl = wave_incl_scan(tot, lane);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int base = incl - tot;
  for (int w = 0; w < wave; ++w) base += red[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    hist[kBins1 - 1 - (tid * kPer + i)] = base;
    base += c[i];
  }
  __syncthreads();
}

// Where a workgroup's elements come from.
enum Src : int {
  kDense = 0,      // row r of the score matrix: element e is row e
  kCandidate = 1,  // (score, row) candidates of the fused selection
  kRecompute = 2,  // scores recomputed from the indexer inputs (listed tokens)
};

// Selection and ordering for token r of the launch. LDS: `keys` holds
// min(top_k + kSlack, BLOCK * PER) bucketed keys (and as many collected ones
// when PER > kDirectPer), then (for the ascending copy) a bitmap of the
// visible rows.
template <int BLOCK, int PER, int SRC>
__device__ __forceinline__ void topk_token(const TopkArgs& a, const FusedArgs& f, int r) {
  constexpr int NW = BLOCK / 64;
  __shared__ int hist[kBins1];
  __shared__ int red_a[NW], red_b[NW], red_c[NW];
  __shared__ int s_bin, s_above, s_count;
  __shared__ int aux[BLOCK + 1];  // span offsets (candidates) or the query row (recompute)
  // Candidates: the span of each collected slot (spans < 256).
  __shared__ unsigned char span_of[SRC == kCandidate ? BLOCK * PER : 1];
  static_assert(SRC != kCandidate || (kMaxComp + 511) / 512 <= 255, "span indices fit a byte");
  extern __shared__ u64 keys[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t = a.q_pos0 + r;
  const int nv = min(a.n_comp, (t + 1) / a.ratio);
  const int k = a.top_k;
  const int nsel = min(k, nv);
  int32_t* sel_row = a.sel + (int64_t)r * k;

  if (nsel == 0) {
    for (int i = tid; i < k; i += BLOCK) sel_row[i] = -1;
    if (a.sel_asc)
      for (int i = tid; i < k; i += BLOCK) a.sel_asc[(int64_t)r * k + i] = -1;
    if (a.n_sel && tid == 0) a.n_sel[r] = 0;
    return;
  }

  // Elements of this token in registers, n_el of them. Dense and recomputed
  // elements are rows 0 .. nv-1 in order (element i*BLOCK + tid: register i
  // holds one when tid < nv - i*BLOCK, a compare with a scalar); candidates
  // carry their row, and bit i of `vm` says whether register i holds one.
  int sc[PER];
  int jx[SRC == kCandidate ? PER : 1];
  int n_el = nv;
  unsigned vm = 0u;
  static_assert(PER <= 32, "validity bits");
  auto valid = [&](int i) -> bool {
    if constexpr (SRC == kCandidate) return (vm >> i) & 1u;
    else return tid < nv - i * BLOCK;
  };
  // Score range of the elements (dense rows: taken as they load).
  int vmax = INT32_MIN, vmin = INT32_MAX;
  if constexpr (SRC == kDense) {
    // The visible scores as a buffer resource (one scalar base, one offset
    // register per load). Every lane loads, past the visible rows the last
    // visible score (nv >= 1 here), so no branch stands between the loads,
    // all are in flight at once, and that copy changes neither the minimum
    // nor the maximum; the element is then marked invisible (INT32_MIN).
    const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.scores + (int64_t)r * a.ld_scores), (short)0, nv * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = i * BLOCK + tid;
      const int v = __builtin_amdgcn_raw_buffer_load_b32(row, min(e, nv - 1) * 4, 0, 2);  // aux 2: non-temporal
      vmax = max(vmax, v);
      vmin = min(vmin, v);
      sc[i] = valid(i) ? v : INT32_MIN;
    }
  } else if constexpr (SRC == kRecompute) {
    // S[t][j] = sum_h w[t][h] * max(0, <iq[t][h][:], ik[j][:]>), exact.
    const int* qrow = reinterpret_cast<const int*>(f.iq + (int64_t)r * kIdxHeads * kIdxDim);
    if (tid < kIdxHeads * kIdxDim / 4) aux[tid] = qrow[tid];
    if (tid == 0) aux[kIdxHeads * kIdxDim / 4] = *reinterpret_cast<const int*>(f.iw + (int64_t)r * kIdxHeads);
    __syncthreads();
    const int wpack = aux[kIdxHeads * kIdxDim / 4];
#pragma unroll 1
    for (int i = 0; i < PER; ++i) {
      const int e = i * BLOCK + tid;
      sc[i] = INT32_MIN;
      if (e < nv) {
        const int4* krow = reinterpret_cast<const int4*>(f.ik + (int64_t)e * kIdxDim);
        int kv[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int4 v = krow[c];
          kv[4 * c] = v.x;
          kv[4 * c + 1] = v.y;
          kv[4 * c + 2] = v.z;
          kv[4 * c + 3] = v.w;
        }
        int tot = 0;
#pragma unroll
        for (int h = 0; h < kIdxHeads; ++h) {
          int d = 0;
#pragma unroll
          for (int c = 0; c < 16; ++c) d = __builtin_amdgcn_sdot4(aux[16 * h + c], kv[c], d, false);
          tot += (int)(int8_t)((wpack >> (8 * h)) & 0xff) * max(d, 0);
        }
        sc[i] = tot;
      }
    }
  } else {
    // Candidates. The token goes on the recompute list if a span overflowed
    // its slots, if fewer than nsel candidates exist (the threshold was too
    // high), or if they do not fit this workgroup: then they are not provably
    // a superset of the top-k. Register i of wave w holds slot `lane` of span
    // w + NW*i: those loads go out together with the span counts (one
    // round trip), and a slot is an element while it is below its span's
    // count. A span with more than 64 candidates does not fit that layout;
    // then the slots are packed by a prefix scan over the spans (a second
    // round trip).
    const int ns = f.plan.n_spans;  // <= BLOCK (host-checked)
    const int cap = f.plan.cap;
    static_assert(NW * PER >= (kMaxComp + 511) / 512, "one register per span and lane");
    const int32_t* cand_row = f.cand + 2 * ((int64_t)r * ns * cap);
    int cnt_i[PER];
    int wtot = 0, wflags = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sp = wave + NW * i;  // wave-uniform
      cnt_i[i] = sp < ns ? f.counts[(int64_t)r * ns + sp] : 0;
      sc[i] = INT32_MIN;
      jx[i] = 0;
      if (sp < ns && lane < cap) {
        const int2 c = *reinterpret_cast<const int2*>(cand_row + 2 * ((int64_t)sp * cap + lane));
        sc[i] = c.x;
        jx[i] = c.y;
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      wtot += min(cnt_i[i], cap);
      wflags |= (cnt_i[i] > cap ? 1 : 0) | (cnt_i[i] > 64 ? 2 : 0);
    }
    if (lane == 0) {
      red_a[wave] = wtot;
      red_b[wave] = wflags;
    }
    __syncthreads();
    int total = 0, flags = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      total += red_a[w];
      flags |= red_b[w];
    }
    __syncthreads();  // every wave has read red_a and red_b before they are written again
    const bool fail = (flags & 1) || total < nsel || total > BLOCK * PER;
    if (fail) {
      if (tid == 0) f.redo_list[atomicAdd(f.n_redo, 1)] = r;
      return;
    }
    n_el = total;
    if (!(flags & 2)) {
#pragma unroll
      for (int i = 0; i < PER; ++i) vm |= lane < min(cnt_i[i], cap) ? 1u << i : 0u;
    } else {
      // Packed: element e = i*BLOCK + tid; slots [aux[s], aux[s] + held)
      // are span s's, each labelled with its span so that an element finds
      // its span with one LDS read.
      const int cnt = tid < ns ? f.counts[(int64_t)r * ns + tid] : 0;
      const int held = min(cnt, cap);
      const int incl = wave_incl_scan(held, lane);
      if (lane == 63) red_a[wave] = incl;
      __syncthreads();
      int before = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) before += w < wave ? red_a[w] : 0;
      if (tid < ns) aux[tid] = before + incl - held;
      __syncthreads();
      if (tid < ns)
        for (int e = aux[tid], e1 = aux[tid] + held; e < e1; ++e) span_of[e] = (unsigned char)tid;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = i * BLOCK + tid;
        sc[i] = INT32_MIN;
        jx[i] = 0;
        if (e < n_el) {
          const int lo = span_of[e];
          const int2 c = *reinterpret_cast<const int2*>(cand_row + 2 * ((int64_t)lo * cap + (e - aux[lo])));
          sc[i] = c.x;
          jx[i] = c.y;
          vm |= 1u << i;
        }
      }
    }
  }
  if constexpr (SRC != kDense) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (valid(i)) {
        vmax = max(vmax, sc[i]);
        vmin = min(vmin, sc[i]);
      }
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
  const u64 emask = ebits ? ((1ull << ebits) - 1) : 0ull;
  const unsigned span = (unsigned)vmax - (unsigned)vmin;  // exact: vmax >= vmin
  const int sbits = span ? 32 - __clz(span) : 0;
  auto key_of = [&](int i) -> u64 {
    const int j = SRC == kCandidate ? jx[i] : i * BLOCK + tid;
    const u64 s = (unsigned)sc[i] - (unsigned)vmin;
    return (s << ebits) | (u64)(nv - 1 - j);
  };

  // Elements with key >= thresh are collected and ordered, the first nsel
  // places kept. The threshold only has to leave at most `cap` of them and
  // keep every winner: the coarse bin holding the k-th key usually does, so
  // the refinement below only runs when that bin is crowded (heavy ties).
  const int cap = min(k + kSlack, BLOCK * PER);  // n_el <= BLOCK * PER
  u64 thresh = 0;
  const int sh1 = sbits > kBits1 ? sbits - kBits1 : 0;
  // With few registers per thread and a threshold on a coarse bin boundary,
  // the coarse bins at or above it serve as the ordering buckets: hist
  // already holds their counts, exactly the n_coarse kept elements.
  bool coarse_buckets = false;
  int n_coarse = 0;
  if (n_el > cap) {
    // 1. coarse pass on the top kBits1 bits of (score - min).
    for (int b = tid; b < kBins1; b += BLOCK) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (valid(i)) atomicAdd(&hist[((unsigned)sc[i] - (unsigned)vmin) >> sh1], 1);
    __syncthreads();
    find_bin<BLOCK, kBins1>(hist, kBins1, k, &s_bin, &s_above, &s_count, red_c);
    const int bin1 = s_bin;
    int need = k - s_above;
    const int low_bits = sh1 + ebits;  // key bits below the coarse digit
    u64 prefix = (u64)bin1;            // key >> shift must equal this
    if (s_above + s_count <= cap || low_bits == 0) {
      thresh = prefix << low_bits;
      coarse_buckets = PER <= kDirectPer && s_above + s_count <= cap;
      n_coarse = s_above + s_count;
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
          if (valid(i)) {
            const u64 key = key_of(i);
            if ((key >> top) == prefix) atomicAdd(&hist[(key >> shift) & ((1u << dbits) - 1)], 1);
          }
        }
        __syncthreads();
        find_bin<BLOCK, 256>(hist, 1 << dbits, need, &s_bin, &s_above, &s_count, red_c);
        need -= s_above;
        prefix = (prefix << dbits) | (u64)s_bin;
        top = shift;
        if ((k - need) + s_count <= cap || shift == 0) {
          thresh = prefix << shift;
          break;
        }
        shift = shift >= 8 ? shift - 8 : 0;
      }
    }
  }

  // 3. Bucket the elements >= thresh (at most cap, at least nsel) for
  // ordering by the top 11 bits of key - thresh (no key exceeds key_hi):
  // counts per bucket, bucket offsets by one prefix scan, then a scatter into
  // the buckets (in any order inside one: the placement below ranks a
  // bucket's keys by value). With few registers per thread the kept keys are
  // scattered straight from registers; with many (long rows, few kept) they
  // are first collected in place order by a block-wide scan, so that the
  // scatter loops over the few kept keys instead of every register.
  const u64 key_hi = ((u64)span << ebits) | emask;
  const u64 kspan = key_hi - thresh;
  const int kbits = kspan ? 64 - __clzll(kspan) : 0;
  const int shb = kbits > kBits1 ? kbits - kBits1 : 0;
  // key >> (ebits + sh1) is the coarse bin (score - min) >> sh1.
  auto bucket_of = [&](u64 key) -> int {
    return coarse_buckets ? (int)(key >> (ebits + sh1)) : (int)((key - thresh) >> shb);
  };
  u64* const bucketed = keys;
  if (!coarse_buckets) {
    __syncthreads();
    for (int b = tid; b < kBins1; b += BLOCK) hist[b] = 0;
  }
  if constexpr (PER <= kDirectPer) {
    if (!coarse_buckets) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (valid(i)) {
          const u64 key = key_of(i);
          if (key >= thresh) atomicAdd(&hist[bucket_of(key)], 1);
        }
      }
    }
    __syncthreads();
    bucket_offsets<BLOCK>(hist, red_c);
    // Slots of up to 8 elements are claimed before any is written, so their
    // LDS atomics are in flight together.
    constexpr int G = PER < 8 ? PER : 8;
#pragma unroll
    for (int i0 = 0; i0 < PER; i0 += G) {
      int slot[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int i = i0 + u;
        slot[u] = -1;
        if (valid(i)) {
          const u64 key = key_of(i);
          if (key >= thresh) slot[u] = atomicAdd(&hist[bucket_of(key)], 1);
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u)
        if (slot[u] >= 0 && slot[u] < cap) bucketed[slot[u]] = key_of(i0 + u);  // < cap by construction
    }
  } else {
    u64* const collected = keys + cap;
    // key_of(i) >= thresh from 32-bit parts, without forming the key (most
    // elements of a long row fail it): a score above ts, or equal to it at a
    // row of at most jm (thresh >> ebits <= span, so ts <= vmax). Dense and
    // recomputed elements past the visible rows hold INT32_MIN at a row >= nv
    // > jm and so never pass; candidate slots past their count carry no row
    // and are masked by vm. ts and jm are block-uniform (scalar registers).
    const int ts = __builtin_amdgcn_readfirstlane((int)((unsigned)vmin + (unsigned)(thresh >> ebits)));
    const int jm = __builtin_amdgcn_readfirstlane(nv - 1 - (int)(thresh & emask));
    auto kept_of = [&](int i) -> bool {
      const bool pass = sc[i] > ts || (sc[i] == ts && (SRC == kCandidate ? jx[i] <= jm : tid <= jm - i * BLOCK));
      return SRC == kCandidate ? (valid(i) && pass) : pass;
    };
    int mine = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) mine += kept_of(i) ? 1 : 0;
    const int mine_incl = wave_incl_scan(mine, lane);
    if (lane == 63) red_a[wave] = mine_incl;
    __syncthreads();
    int pos = mine_incl - mine;
#pragma unroll
    for (int w = 0; w < NW; ++w) pos += w < wave ? red_a[w] : 0;
    // The kept elements go out as scores and rows (two arrays over the
    // collected space): the branch around the write is taken in nearly every
    // register of every wave, so it holds as little as possible; keys and
    // bucket counts are formed in passes over the collected elements, where
    // every thread has work.
    int* const kept_sc = reinterpret_cast<int*>(collected);
    int* const kept_row = kept_sc + cap;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (kept_of(i)) {
        if (pos < cap) {  // by construction
          kept_sc[pos] = sc[i];
          kept_row[pos] = SRC == kCandidate ? jx[i] : i * BLOCK + tid;
        }
        ++pos;
      }
    }
    int total_kept = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) total_kept += red_a[w];
    total_kept = min(total_kept, cap);
    auto kept_key = [&](int e) -> u64 {
      return ((u64)((unsigned)kept_sc[e] - (unsigned)vmin) << ebits) | (u64)(unsigned)(nv - 1 - kept_row[e]);
    };
    __syncthreads();
    for (int e = tid; e < total_kept; e += BLOCK) atomicAdd(&hist[(int)((kept_key(e) - thresh) >> shb)], 1);
    __syncthreads();
    bucket_offsets<BLOCK>(hist, red_c);
    for (int e = tid; e < total_kept; e += BLOCK) {
      const u64 key = kept_key(e);
      bucketed[atomicAdd(&hist[(int)((key - thresh) >> shb)], 1)] = key;
    }
  }
  __syncthreads();
  // After the scatter hist[b] is the end of bucket b; bucket 0 comes last, so
  // hist[0] is the number of keys collected (with coarse buckets the bins
  // below the threshold stay unfilled: their count is known).
  const int n_coll = coarse_buckets ? n_coarse : min(hist[0], cap);
  // Ascending order (optional): the winners' rows are marked in a bitmap of
  // the visible rows (nv <= kMaxComp bits), which follows the bucketed keys
  // and their collected copy (the launcher reserves asc_bitmap_words(n_comp)
  // words), and read back in
  // row order after a block-wide scan of the words' popcounts.
  const int nwords = (nv + 31) >> 5;
  unsigned* const bits = reinterpret_cast<unsigned*>(keys + (PER <= kDirectPer ? 1 : 2) * cap);
  if (a.sel_asc) {
    for (int i = tid; i < nwords; i += BLOCK) bits[i] = 0u;
    __syncthreads();
  }
  // Place of an element = its bucket's start + larger keys in the bucket; the
  // first nsel places are the selection, in order. After the scatter hist[b]
  // is the end of bucket b, and the end of the bucket above (placed before
  // it) is its start.
  for (int p = tid; p < n_coll; p += BLOCK) {
    const u64 key = bucketed[p];
    const int b = bucket_of(key);
    const int st = b + 1 < kBins1 ? hist[b + 1] : 0, en = hist[b];
    int place = st;
    // Four bucket entries per step (independent reads; most buckets hold
    // only a few keys).
    for (int q = st; q < en; q += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = q + j < en;
        const u64 o = in ? bucketed[q + j] : 0ull;
        place += (in && o > key) ? 1 : 0;
      }
    }
    if (place < nsel) {
      const int row = (nv - 1) - (int)(key & emask);
      sel_row[place] = row;
      if (a.sel_asc) atomicOr(&bits[row >> 5], 1u << (row & 31));
    }
  }
  for (int i = nsel + tid; i < k; i += BLOCK) sel_row[i] = -1;
  if (a.sel_asc) {
    __syncthreads();
    const int wpt = (nwords + BLOCK - 1) / BLOCK;  // words per thread, consecutive
    int cnt = 0;
    for (int i = 0; i < wpt; ++i) {
      const int w = tid * wpt + i;
      if (w < nwords) cnt += __popc(bits[w]);
    }
    const int incl = wave_incl_scan(cnt, lane);
    if (lane == 63) red_a[wave] = incl;
    __syncthreads();
    int pos = incl - cnt;
#pragma unroll
    for (int w = 0; w < NW; ++w) pos += w < wave ? red_a[w] : 0;
    int32_t* asc_row = a.sel_asc + (int64_t)r * k;
    for (int i = 0; i < wpt; ++i) {
      const int w = tid * wpt + i;
      if (w < nwords) {
        unsigned m = bits[w];
        while (m) {
          asc_row[pos++] = 32 * w + (__ffs(m) - 1);
          m &= m - 1;
        }
      }
    }
    for (int i = nsel + tid; i < k; i += BLOCK) asc_row[i] = -1;
  }
  if (a.n_sel && tid == 0) a.n_sel[r] = nsel;
}

// One workgroup per token; the recompute pass instead walks the list of
// tokens the candidate pass could not settle.
template <int BLOCK, int PER, int SRC>
__global__ __launch_bounds__(BLOCK) void topk_kernel(TopkArgs a, FusedArgs f) {
  if constexpr (SRC == kRecompute) {
    const int n = *f.n_redo;
    for (int i = blockIdx.x; i < n; i += gridDim.x) {
      topk_token<BLOCK, PER, SRC>(a, f, f.redo_list[i]);
      __syncthreads();  // LDS is reused by the next token
    }
  } else {
    topk_token<BLOCK, PER, SRC>(a, f, blockIdx.x);
  }
}

// Words of LDS reserved after the bucketed keys for the ascending-order
// bitmap: one bit per compressed row a token can see.
size_t asc_bitmap_words(int n_comp) { return ((size_t)n_comp + 31) / 32; }

template <int BLOCK, int PER, int SRC>
hipError_t launch_cfg(const TopkArgs& a, const FusedArgs& f, int grid, hipStream_t stream) {
  // keys: the bucketed elements (at most top_k + kSlack), their collected
  // copy when PER > kDirectPer, then the ascending-order bitmap.
  const int cap = std::min(a.top_k + kSlack, BLOCK * PER);
  size_t lds = sizeof(u64) * (size_t)cap * (PER <= kDirectPer ? 1 : 2);
  if (a.sel_asc) lds += sizeof(unsigned) * asc_bitmap_words(a.n_comp);
  hipLaunchKernelGGL((topk_kernel<BLOCK, PER, SRC>), dim3(grid), dim3(BLOCK), lds, stream, a, f);
  return hipGetLastError();
}

// Block and elements per thread for `n` elements per token.
template <int SRC>
hipError_t launch_by_size(int n, const TopkArgs& a, const FusedArgs& f, int grid, hipStream_t stream) {
  if (n <= 256 * 4) return launch_cfg<256, 4, SRC>(a, f, grid, stream);
  if (n <= 256 * 8) return launch_cfg<256, 8, SRC>(a, f, grid, stream);
  if (n <= 256 * 16) return launch_cfg<256, 16, SRC>(a, f, grid, stream);
  if (n <= 1024 * 8) return launch_cfg<1024, 8, SRC>(a, f, grid, stream);
  if (n <= 1024 * 16) return launch_cfg<1024, 16, SRC>(a, f, grid, stream);
  return launch_cfg<1024, 32, SRC>(a, f, grid, stream);  // n <= 32768 (host-checked)
}

constexpr int kFinishBlock = 512;
constexpr int kFinishPer = 8;  // candidates a finish workgroup holds: 4096
constexpr int kRedoGrid = 128;  // workgroups that share the recompute list

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  return launch_by_size<kDense>(a.n_comp, a, FusedArgs{}, a.n_q, stream);
}

hipError_t launch_fused_topk(const FusedArgs& f, hipStream_t stream) {
  if (f.n_q <= 0) return hipSuccess;
  TopkArgs a{};
  a.sel = f.sel;
  a.n_sel = f.n_sel;
  a.sel_asc = f.sel_asc;
  a.n_q = f.n_q;
  a.q_pos0 = f.q_pos0;
  a.n_comp = f.n_comp;
  a.ratio = f.ratio;
  a.top_k = f.top_k;
  hipError_t e = launch_sample_threshold(f, stream);  // also clears the recompute list
  if (e != hipSuccess) return e;
  e = launch_collect(f, stream);
  if (e != hipSuccess) return e;
  e = launch_cfg<kFinishBlock, kFinishPer, kCandidate>(a, f, f.n_q, stream);
  if (e != hipSuccess) return e;
  return launch_by_size<kRecompute>(f.n_comp, a, f, f.n_q < kRedoGrid ? f.n_q : kRedoGrid, stream);
}

}  // namespace spmla
