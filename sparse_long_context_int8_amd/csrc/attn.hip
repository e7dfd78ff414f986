// Streaming sparse MLA attention on CDNA4 (gfx950).
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): each selected F16 latent row is read once and shared by
// the sixteen query heads, with an online softmax; the page "perf(ds4): unify
// gfx1151 sparse-prefill stack" (Validation completed) stages in FP32 and
// uses a fast exponential. Here: fp16 operands on matrix cores, fp32
// accumulation and softmax, exp2 with log2(e) folded into the scale.
//
// One workgroup per query token (or per key split of one). Its key list is
// the selected compressed rows followed by the sliding-window raw rows; keys
// stream through a ring of LDS buffers in chunks of CHUNK rows gathered with
// direct global->LDS loads, so each row crosses the memory system once per
// query.
//
// LDS image of a chunk (per buffer):
//   region A: CHUNK rows x 1024 B = latent dims 0..511 (the value part),
//             one wave-wide 16-byte-per-lane load per row;
//   region B: CHUNK rows x 128 B  = latent dims 512..575 (the rope part),
//             one load per wave covering its rows.
// 16-byte units are XOR-swizzled per row so that the K reads (16 rows x 16 B
// per pass) and the transposed V reads (8 rows x 32 B per pass) hit distinct
// banks.
//
// Per chunk (W waves):
//   QK: S^T[16 keys x 16 heads] = K . Q^T on v_mfma_f32_16x16x32_f16; the
//       CHUNK/16 key tiles x (W / tiles) slices of the 576-dim contraction
//       are spread over the waves, Q^T slices stay in registers;
//   exchange S^T partials through LDS; every wave runs the same online
//       softmax update, so each lane owns one head and rescaling is
//       lane-local;
//   PV: O^T[512/W dims x 16 heads] += V^T . P^T per wave, V^T fragments read
//       with ds_read_b64_tr_b16 (the gfx950 transpose load) from the
//       row-major region A before the exchange, P^T built in registers.
// A chunk's buffer is refilled right after the exchange (the gather of the
// chunk NBUF places later), so NBUF gathers are in flight while softmax and
// PV run.
#include "spmla_internal.h"

#include <type_traits>

namespace spmla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(1))) const char gbl_char;

constexpr int kRowBytes = kDqk * 2;  // 1152: one latent row
constexpr int kXcds = 8;             // accelerator complex dies, round-robin dispatch

// Work items are cut into 2 * kXcds contiguous slices of slice_len items; die
// x takes slice 2*kXcds-1-x, then slice x (workgroup index x + kXcds * l). Each
// die keeps runs of neighbouring queries (their window rows stay in its L2),
// and when the cost of a query grows with its position (the first band of a
// prefill: more visible rows) every die gets one later and one earlier slice,
// the later one first.
__host__ __device__ inline int attn_slice_len(int n_items) { return (n_items + 2 * kXcds - 1) / (2 * kXcds); }
__device__ inline int attn_item_at(int idx, int n_items) {
  const int slice_len = attn_slice_len(n_items);
  const int x = idx % kXcds, l = idx / kXcds;
  return l < slice_len ? (2 * kXcds - 1 - x) * slice_len + l : x * slice_len + (l - slice_len);
}
// Banded launch (AttnArgs::band_items): band b takes workgroups
// [b * G, (b + 1) * G) with G = 2 * kXcds * slice_len(band_items), a multiple
// of kXcds, so each band is dealt to the dies exactly as its own launch would
// be. Returns the item, or n_items for a workgroup without one.
__device__ inline int attn_item_banded(int n_items, int band_items) {
  const int g = 2 * kXcds * attn_slice_len(band_items);
  const int b = blockIdx.x / g;
  const int first = b * band_items;
  if (first >= n_items) return n_items;
  const int n_band = min(band_items, n_items - first);
  const int it = attn_item_at(blockIdx.x - b * g, n_band);
  return it < n_band ? first + it : n_items;
}

// XOR swizzles of the 16-byte units of the LDS images, as linear maps of
// the row index bits. They were chosen by measuring the LDS bank-conflict
// counter on gfx950 for every access pattern of this kernel (K-fragment
// reads of both key tiles at all 18 k-steps, transposed V reads for every
// output tile, S^T exchange writes and reads): all of them run without
// conflicts.
// Region A (value dims, 64 units per row): bits (n1, n1^n3, n0, n0^n2^n3).
__device__ __forceinline__ int swz_a(int n) {
  return ((n >> 1) & 1) | ((((n >> 1) ^ (n >> 3)) & 1) << 1) | ((n & 1) << 2) |
         (((n ^ (n >> 2) ^ (n >> 3)) & 1) << 3);
}
// Region B (rope dims, 8 units per row): bits (n0, n1, n0^n2^n4).
__device__ __forceinline__ int swz_b(int n) { return (n & 3) | (((n ^ (n >> 2) ^ (n >> 4)) & 1) << 2); }
// S^T exchange rows (one per head): float4 slot XOR (h1, h0, h2).
__device__ __forceinline__ int swz_s(int h) { return ((h >> 1) & 1) | ((h & 1) << 1) | (h & 4); }

// Workgroup barrier for LDS traffic. __syncthreads() would also wait for
// every outstanding global->LDS load (its release fence covers them), i.e.
// for the gather of the next chunk; those loads are waited for explicitly
// with vmcnt instead, so this barrier only drains this wave's LDS ops.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]). Emitted as the
// builtin so the compiler's own wait insertion knows the loads completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// LDS reads of the streamed rows are issued as inline assembly. The
// compiler's wait insertion would otherwise treat every read of one buffer
// as possibly depending on the global->LDS loads still landing in the other
// buffer and wait for all of them (vmcnt(0)), which serializes the gather
// pipeline. Each group of reads is followed by an lgkmcnt wait (lds_wait,
// lds_wait_n or the barrier's) and fence_reg() on the results, so no value
// is used before it has arrived.
__device__ __forceinline__ half8 lds_read_b128(unsigned addr) {
  half8 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ float4v lds_read_f4(unsigned addr) {
  float4v v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ short4v lds_read_tr16(unsigned addr) {
  short4v v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ int lds_read_i32(unsigned addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ unsigned long long lds_read_u64(unsigned addr) {
  unsigned long long v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
// The same reads at base + OFF with OFF in the instruction's 16-bit offset
// field when it fits (a chunk buffer's offset and a read's fixed part then
// cost no address arithmetic per read).
template <int OFF>
__device__ __forceinline__ half8 lds_read_b128_at(unsigned base) {
  static_assert(OFF >= 0, "offset");
  half8 v;
  if constexpr (OFF <= 65535) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF));
  else asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(base + OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ short4v lds_read_tr16_at(unsigned base) {
  static_assert(OFF >= 0, "offset");
  short4v v;
  if constexpr (OFF <= 65535) asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF));
  else asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(base + OFF));
  return v;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Waits until at most N LDS operations are outstanding (they complete in
// issue order); N fits the 4-bit counter.
template <int N>
__device__ __forceinline__ void lds_wait_n() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
template <typename T>
__device__ __forceinline__ void fence_reg(T& v) {
  asm volatile("" : "+v"(v));
}

template <int WAVES, int CHUNK, int NBUF, int WPE, int GROUP>
struct Cfg {
  static constexpr int kHw = WAVES * GROUP;       // waves in the workgroup
  static constexpr int kRowsPerHw = CHUNK / kHw;  // rows of a chunk each wave gathers
  static constexpr int kTiles = CHUNK / 16;
  static constexpr int kHalves = WAVES / kTiles;  // slices of the 576 contraction
  // Slice h covers k-steps [start(h), start(h) + len(h)) of the 18 steps of
  // 32 latent dims; slices differ in length by at most one step.
  static constexpr int kAllSteps = kDqk / 32;
  static constexpr int kSteps = (kAllSteps + kHalves - 1) / kHalves;  // longest slice
  static constexpr int len(int h) { return kAllSteps / kHalves + (h < kAllSteps % kHalves ? 1 : 0); }
  static constexpr int start(int h) {
    return h * (kAllSteps / kHalves) + (h < kAllSteps % kHalves ? h : kAllSteps % kHalves);
  }
  static constexpr int kNt = (kDv / WAVES) / 16;  // 16-dim output tiles per wave
  // PV steps: 32 keys (16x16x32 MFMA) or, for 16-key chunks, 16 keys
  // (16x16x16 MFMA); each lane holds kKpl keys of one head per step.
  static constexpr int kPvKeys = CHUNK >= 32 ? 32 : 16;
  static constexpr int kPvSteps = CHUNK / kPvKeys;
  static constexpr int kKpl = kPvKeys / 4;
  static constexpr int kUnits = kKpl / 4;  // 16-byte S^T units (and V^T reads) per lane and PV step
  static constexpr int kBufA = CHUNK * 1024;
  static constexpr int kBufB = CHUNK * 128;
  static constexpr int kBuf = kBufA + kBufB;
  static constexpr int kSStride = CHUNK;  // floats per head row of S^T partials
  static constexpr int kSBytes = kHalves * kHeads * kSStride * 4;
  static constexpr int kSBufs = GROUP == 1 ? 1 : 2;  // S^T exchange areas per query
  // Streaming (GROUP == 1): selected indices and validity masks of the
  // chunks in flight (at most 2 * NBUF + 2), slot = chunk mod kSlots, a power
  // of two.
  static constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }
  static constexpr int kSlots = GROUP == 1 ? pow2_at_least(2 * NBUF + 2) : 1;
  static constexpr int kLds = NBUF * kBuf + GROUP * kSBufs * kSBytes + kSlots * (4 * CHUNK + 8);
  // Global->LDS loads a wave issues per chunk: its rows, one rope load, and
  // (streaming) the selected indices of a later chunk.
  static constexpr int kOpsPerChunk = kRowsPerHw + 2;
  static constexpr int kWaitAhead = 1 + (NBUF - 1) * kOpsPerChunk;
  static_assert(kTiles * kHalves == WAVES, "QK work must split evenly");
  static_assert(CHUNK % kHw == 0 && kRowsPerHw <= 8, "gather rows split evenly, one rope load per wave");
  static_assert(start(kHalves - 1) <= 16, "rope steps live in the last slice");
  static_assert(CHUNK == 16 || CHUNK % 32 == 0, "PV steps are 16 or 32 keys");
  static_assert(CHUNK <= 64, "validity is one 64-bit mask per chunk");
  static_assert(GROUP == 1 || NBUF == 2, "the pair variant double-buffers");
  static_assert(NBUF >= 2 && kWaitAhead < 64, "vmcnt range");
  static_assert(kLds * ((WPE * 4) / kHw) <= 160 * 1024, "LDS for the requested occupancy");
};

// S^T exchange slot (16-byte unit of a head row) of key unit u (keys
// 4u .. 4u+3) for head h: rows of 32 keys XOR (h1, h0, h2), rows of 16 keys
// XOR (h1, h2), so that the 8 lanes of one 16-byte access phase hit
// distinct banks.
template <int CHUNK>
__device__ __forceinline__ int s_slot(int u, int h) {
  if constexpr (CHUNK == 16) return u ^ ((h >> 1) & 3);
  return u ^ swz_s(h);
}

// Calls f(integral_constant<int, h>) for the runtime slice index h < N
// (wave-uniform), so that each slice's LDS addresses are compile-time.
template <int N, typename F>
__device__ __forceinline__ void with_slice(int h, F&& f) {
  if constexpr (N == 1) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (h == N - 1) f(std::integral_constant<int, N - 1>{});
    else with_slice<N - 1>(h, f);
  }
}
// Calls f(integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Max and sum over the four lanes l, l^16, l^32, l^48 (one head's keys)
// with the gfx950 row swaps: a swap of a value with itself leaves, in its
// two results, the value of lane l and of its partner lane.
__device__ __forceinline__ unsigned fbits(float v) { return __builtin_bit_cast(unsigned, v); }
__device__ __forceinline__ float ffrom(unsigned v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ float max4_heads(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  const float m = fmaxf(ffrom(a[0]), ffrom(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(m), fbits(m), false, false);
  return fmaxf(ffrom(b[0]), ffrom(b[1]));
}
__device__ __forceinline__ float sum4_heads(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  const float m = ffrom(a[0]) + ffrom(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(m), fbits(m), false, false);
  return ffrom(b[0]) + ffrom(b[1]);
}

// Softmax reference is moved only when a chunk's max exceeds it by more than
// this (log2 units); probabilities are then at most 2^8, which fp16 P and
// fp32 sums hold exactly enough, and the O rescale is skipped for most chunks.
constexpr float kRescaleThreshold = 8.0f;

// GROUP == 1: streaming, one (query, key split) per workgroup of WAVES
// waves, keys through a ring of NBUF chunk buffers. A chunk's buffer is read
// (K and V^T fragments into registers) before its S^T exchange barrier; after
// that barrier the gather of the chunk NBUF places later is issued into it,
// in stages between the softmax steps, so NBUF gathers are in flight while
// softmax and PV run. The selected
// indices arrive by the same global->LDS path ahead of their gather, so the
// loop issues no other global load and each wave's only memory wait is a
// vmcnt that lets the later chunks' loads stay outstanding (loads complete
// in issue order).
// GROUP == 2: query-tiled ("grouped") variant. A workgroup of 2*WAVES waves
// takes two adjacent queries t0, t1 = t0 + 1 and streams the union of their
// keys through two chunk buffers: t0's selected rows, then t1's selected
// rows that t0 did not select, then the union of the two windows (raw rows
// ws0 .. t1). Wave group g (waves g*WAVES ..) runs the streaming per-chunk
// work for query t_g with its own mask; every gathered row is read once for
// both queries.
// FAR: the gathered rows come from beyond the dies' L2 (compressed rows
// larger than one die's L2; the selection then arrives in ascending row
// order). The loads of a chunk's gather are then spread over the whole
// softmax, a chunk's head maxima are formed before the test for a new
// reference (their exchange across lanes also spaces two gather stages), and
// the softmax sums come from the matrix cores.
// Otherwise (L2-resident rows) the head maxima are formed only when some
// lane's own maximum calls for a new reference, and the last two gather
// stages follow the exponentials and half of the PV products: the shorter
// per-chunk chain matters more there than the spacing of the loads.
template <int WAVES, int CHUNK, int NBUF, int WPE, int GROUP, bool FAR>
__global__ __launch_bounds__(64 * WAVES * GROUP) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_kernel(AttnArgs a) {
  using C = Cfg<WAVES, CHUNK, NBUF, WPE, GROUP>;
  static_assert(GROUP == 1 || GROUP == 2, "one or two queries per workgroup");
  constexpr int kHw = C::kHw;
  constexpr int kRowsPerHw = C::kRowsPerHw;
  constexpr int kKpl = C::kKpl;
  constexpr int kUnits = C::kUnits;
  __shared__ __attribute__((aligned(1024))) char bufs_[NBUF * C::kBuf];
  __shared__ __attribute__((aligned(16))) float sbuf[GROUP * C::kSBufs * C::kSBytes / 4];
  __shared__ __attribute__((aligned(16))) int sel_ring[C::kSlots * CHUNK];
  __shared__ unsigned long long valid_ring[C::kSlots];
  // Lambdas below use these pointers, never the __shared__ arrays by name.
  lds_char* const bufs = (lds_char*)bufs_;
  lds_char* const sel_lds = (lds_char*)sel_ring;
  unsigned long long* const valid_slots = valid_ring;
  const unsigned sel_ring_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)sel_ring;
  const unsigned valid_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned long long*)valid_ring;

  // Work items: (query r, key split s), or a query pair; see attn_item.
  const int n_items = GROUP == 1 ? a.n_q * a.splits : (a.n_q + 1) / 2;
  const int item = GROUP == 1 && a.band_items > 0 ? attn_item_banded(n_items, a.band_items)
                                                 : attn_item_at(blockIdx.x, n_items);
  if (item >= n_items) return;

  const int lane = threadIdx.x & 63;
  const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = hw % WAVES;  // wave within its group
  const int grp = hw / WAVES;   // which query of the pair
  const int g = lane >> 4;
  const int c16 = lane & 15;
  float* sbuf_g = sbuf + grp * C::kSBufs * (C::kSBytes / 4);
  const unsigned sbuf_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float*)sbuf_g;

  const int r = GROUP == 1 ? item / a.splits : 2 * item + grp;  // this group's query
  const int split = GROUP == 1 ? item - r * a.splits : 0;
  const bool q_valid = r < a.n_q;
  const int t = a.q_pos0 + (q_valid ? r : r - 1);

  const int nv = min(a.n_comp, (t + 1) / a.ratio);
  const int nsel = min(a.top_k, nv);
  const int ws = max(0, t - a.window + 1);
  // Key list of the workgroup (GROUP == 2: the pair's union, see below).
  int nk = nsel + (t - ws + 1);
  int n_a = 0, n_ab = 0, ws0 = 0, t0 = 0, t1 = 0;
  unsigned list_lds = 0;  // LDS address: t0's selection, then t1's extra rows
  unsigned bm1_lds = 0;   // LDS address: bitmap of the rows t1 selected
  bool has1 = false;
  if constexpr (GROUP == 2) {
    extern __shared__ int dyn[];  // bitmaps of t0's and t1's rows, then the list
    const int r0 = 2 * item;
    has1 = r0 + 1 < a.n_q;
    t0 = a.q_pos0 + r0;
    t1 = t0 + 1;
    const int nv0 = min(a.n_comp, (t0 + 1) / a.ratio);
    const int nv1 = has1 ? min(a.n_comp, (t1 + 1) / a.ratio) : 0;
    n_a = min(a.top_k, nv0);
    const int n_s1 = has1 ? min(a.top_k, nv1) : 0;
    ws0 = max(0, t0 - a.window + 1);
    const int words = (a.n_comp + 31) / 32;
    unsigned* b0 = reinterpret_cast<unsigned*>(dyn);
    unsigned* b1 = b0 + words;
    int* lst = reinterpret_cast<int*>(b1 + words);
    const int tid = threadIdx.x;
    for (int i = tid; i < 2 * words; i += 64 * kHw) b0[i] = 0u;
    __syncthreads();
    const int32_t* s0 = a.sel + (int64_t)r0 * a.top_k;
    const int32_t* s1 = a.sel + (int64_t)(r0 + 1) * a.top_k;
    for (int i = tid; i < n_a; i += 64 * kHw) {
      const int idx = s0[i];
      lst[i] = idx;
      if (idx >= 0 && idx < nv0) atomicOr(&b0[idx >> 5], 1u << (idx & 31));
    }
    for (int i = tid; i < n_s1; i += 64 * kHw) {
      const int idx = s1[i];
      if (idx >= 0 && idx < nv1) atomicOr(&b1[idx >> 5], 1u << (idx & 31));
    }
    __syncthreads();
    // t1's valid rows that t0 did not select, in t1's order: a block-wide
    // exclusive scan over consecutive runs of its list (deterministic).
    __shared__ int wsum[kHw];
    const int per = (n_s1 + 64 * kHw - 1) / (64 * kHw);
    int take = 0;
    for (int u = 0; u < per; ++u) {
      const int i = tid * per + u;
      if (i < n_s1) {
        const int idx = s1[i];
        take += (idx >= 0 && idx < nv1 && !((b0[idx >> 5] >> (idx & 31)) & 1u)) ? 1 : 0;
      }
    }
    int incl = take;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[hw] = incl;
    __syncthreads();
    int pos = n_a + incl - take, n_b = 0;
    for (int w = 0; w < kHw; ++w) {
      pos += w < hw ? wsum[w] : 0;
      n_b += wsum[w];
    }
    for (int u = 0; u < per; ++u) {
      const int i = tid * per + u;
      if (i < n_s1) {
        const int idx = s1[i];
        if (idx >= 0 && idx < nv1 && !((b0[idx >> 5] >> (idx & 31)) & 1u)) lst[pos++] = idx;
      }
    }
    __syncthreads();
    n_ab = n_a + n_b;
    nk = n_ab + ((has1 ? t1 : t0) - ws0 + 1);
    const unsigned dyn_lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)dyn;
    bm1_lds = dyn_lds + 4u * words;
    list_lds = dyn_lds + 8u * words;
  }
  const int nchunks = (nk + CHUNK - 1) / CHUNK;
  // This work item's chunks [c_begin, c_end) of the query's key list.
  const int per_split = (nchunks + a.splits - 1) / a.splits;
  const int c_begin = split * per_split;
  const int c_end = min(nchunks, c_begin + per_split);
  const int32_t* sel_row = a.sel + (int64_t)(q_valid ? r : r - 1) * a.top_k;
  const char* comp_base = reinterpret_cast<const char*>(a.kv_comp);
  const char* raw_base = reinterpret_cast<const char*>(a.kv_raw);
  const char* self_row = raw_base + (int64_t)t * kRowBytes;

  (void)has1;
  // QK work item of this wave: key tile and contraction slice.
  const int tile = wave % C::kTiles;
  const int half = wave / C::kTiles;

  half8 qf[C::kSteps];
  float4v acc_o[C::kNt];
#pragma unroll
  for (int nt = 0; nt < C::kNt; ++nt) acc_o[nt] = float4v{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();  // softmax reference (log2 domain) of head c16
  float l_run = 0.f;                // this lane's share of the softmax sum
  // FAR: the softmax sum of head c16 (all four entries) instead, as the PV
  // product of a tile of ones with the same fp16 probabilities (one more
  // product per chunk in place of the adds, which measured faster there).
  float4v acc_l = float4v{0.f, 0.f, 0.f, 0.f};

  // Streaming: the selected indices of chunk ch land in sel_ring slot
  // ch mod kSlots (lanes < CHUNK, each a 4-byte global->LDS load; every wave
  // issues the same load so that all waves count the same loads).
  auto load_sel = [&](int ch) {
    if (lane < CHUNK) {
      const int key = min(ch * CHUNK + lane, a.top_k - 1);
      lds_char* const dst = sel_lds + ((unsigned)ch % C::kSlots) * (4 * CHUNK);
      __builtin_amdgcn_global_load_lds((gbl_char*)(sel_row + key), dst, 4, 0, 0);
    }
  };
  // Streaming: row of key `key` of the query's list given its selected index
  // (used when key < nsel), and whether the query uses it.
  // Branch-free (selects only); a key the query does not use points at the
  // query's own raw row, a valid address whose contribution is masked. Row
  // offsets fit 32 bits and both factors 24 (the full-rate 24-bit multiply):
  // rows < 4 * kMaxComp + 4 (host-checked), and 131,076 * 1,152 < 2^32.
  static_assert((4ull * kMaxComp + 4) * kRowBytes < (1ull << 32), "32-bit row offsets");
  // The two bases held in vector registers (the selects below take them
  // from there instead of copying them from scalar registers per call).
  const char* comp_base_v = comp_base;
  const char* raw_base_v = raw_base;
  fence_reg(comp_base_v);
  fence_reg(raw_base_v);
  auto row_ptr = [&](int key, int selv, bool& ok) -> const char* {
    const bool is_sel = key < nsel;
    const bool sel_ok = (unsigned)selv < (unsigned)nv;
    ok = is_sel ? sel_ok : key < nk;
    const bool comp = is_sel && sel_ok;
    const int raw = (is_sel || key >= nk) ? t : ws + key - nsel;
    const unsigned off = __umul24((unsigned)(comp ? selv : raw), (unsigned)kRowBytes);
    return (comp ? comp_base_v : raw_base_v) + off;
  };
  // Pair variant: row pointer of key ch*CHUNK + lane of the pair's list, and
  // whether this group's query uses it.
  auto row_of_pair = [&](int ch, bool& ok) -> const char* {
    const int key = ch * CHUNK + lane;
    ok = false;
    const char* p = self_row;
    if (key < n_ab) {
      int idx = lds_read_i32(list_lds + 4u * key);
      lds_wait();
      fence_reg(idx);
      const bool in_range = idx >= 0 && idx < a.n_comp;
      if (in_range) p = comp_base + (int64_t)idx * kRowBytes;
      if (key < n_a) {  // t0's own selection
        const bool ok0 = idx >= 0 && idx < nv;  // grp 0: nv is t0's
        if (grp == 0) {
          ok = ok0;
        } else if (in_range && has1) {
          int word = lds_read_i32(bm1_lds + 4u * (idx >> 5));
          lds_wait();
          fence_reg(word);
          ok = ((unsigned)word >> (idx & 31)) & 1u;
        }
      } else {  // rows only t1 selected
        ok = grp == 1;
      }
    } else if (key < nk) {
      const int srow = ws0 + (key - n_ab);
      p = raw_base + (int64_t)srow * kRowBytes;
      ok = srow >= ws && srow <= t && q_valid;
    }
    return p;
  };
  // This wave's share of the gather of one chunk: kRowsPerHw value loads
  // (one row each, row n's pointer in lane n of kp = (kp_hi, kp_lo)), here
  // rows [i0, i1) of them, and one rope load covering the same rows (lane l
  // loads part of row row0 + l/8, whose pointer it holds in kr).
  const int row0 = hw * kRowsPerHw;
  const int rope_row = row0 + min(lane >> 3, kRowsPerHw - 1);
  auto gather_rows = [&](unsigned kp_lo, unsigned kp_hi, lds_char* buf, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < kRowsPerHw; ++i) {
      if (i < i0 || i >= i1) continue;
      const int n = row0 + i;
      const unsigned lo = __builtin_amdgcn_readlane(kp_lo, n);
      const unsigned hi = __builtin_amdgcn_readlane(kp_hi, n);
      const char* rowp = reinterpret_cast<const char*>(((uintptr_t)hi << 32) | lo);
      const unsigned off = (unsigned)(lane ^ swz_a(n)) << 4;  // zero-extended: SGPR base + VGPR offset form
      __builtin_amdgcn_global_load_lds((gbl_char*)(rowp + off), buf + n * 1024, 16, 0, 0);
    }
  };
  auto gather_rope = [&](const char* kr, lds_char* buf) {
    lds_char* const rope_dst = buf + C::kBufA + row0 * 128;
    if (lane < 8 * kRowsPerHw) {
      const int off = (64 + ((lane & 7) ^ swz_b(rope_row))) << 4;
      __builtin_amdgcn_global_load_lds((gbl_char*)(kr + off), rope_dst, 16, 0, 0);
    }
  };

  // Per-lane LDS addresses of this wave's K and V^T fragment reads in buffer
  // 0 (the buffer's offset and the fixed part of each read go in the read's
  // offset field). K: key row n = 16*tile + c16, k-step ks < 16 at
  // k_base[ks & 3] + 256*(ks >> 2) (the row swizzle only permutes the low four
  // 16-byte units, i.e. ks & 3 and g), k-steps 16 and 17 (rope dims) at
  // r_base[ks - 16]. V^T: output tile nt, unit u of PV step kb at
  // v_base[nt][u] + 1024*kPvKeys*kb (the swizzle depends only on the low
  // four row bits, which kPvKeys*kb leaves alone).
  const unsigned bufs_addr = (unsigned)(uintptr_t)bufs;
  unsigned k_base[4], r_base[2], v_base[C::kNt][kUnits];
  {
    const int n = 16 * tile + c16;
#pragma unroll
    for (int j = 0; j < 4; ++j) k_base[j] = bufs_addr + n * 1024 + (((4 * j + g) ^ swz_a(n)) << 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) r_base[j] = bufs_addr + C::kBufA + n * 128 + (((4 * j + g) ^ swz_b(n)) << 4);
    const int tri = (lane >> 2) & 3;
    const int trc = lane & 3;
#pragma unroll
    for (int nt = 0; nt < C::kNt; ++nt) {
      const int dv0 = (kDv / WAVES) * wave + 16 * nt;
      const int unit = (dv0 >> 3) + (trc >> 1);
      const int sub = (trc & 1) << 3;
#pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        const int nr = kKpl * g + 4 * u + tri;
        v_base[nt][u] = bufs_addr + nr * 1024 + ((unit ^ swz_a(nr)) << 4) + sub;
      }
    }
  }

  // One chunk in buffer buf_c. After the S^T exchange barrier the buffer is
  // no longer read, and stage(0) .. stage(4) may refill it: stage 0 is called right
  // after the S^T reads are issued (before their wait), stages 1-4 between
  // the steps of the softmax (FAR) or of the softmax and the PV products, so
  // that the loads of the next gather reach the memory pipeline spread out
  // rather than in one burst. No barrier is
  // needed at the end of a chunk: the S^T area is written again only after a
  // later chunk's barrier, which every wave reaches after its last read of it.
  auto compute = [&](auto buf_c, unsigned long long valid_in, unsigned valid_lds, int sb, auto&& stage) {
    constexpr int BOFF = decltype(buf_c)::value * C::kBuf;  // the chunk buffer's offset from bufs
    float* sbuf_c = sbuf_g + sb * (C::kSBytes / 4);
    const unsigned sbuf_c_addr = sbuf_addr + sb * C::kSBytes;

    // V^T fragments: O^T[dims (512/W) wave + 16nt + 4g + i][head c16] needs,
    // per PV step, keys kPvKeys*kb + kKpl*g + 4u + tri of dims dv0 + 4*trc ..
    // Streaming reads them before the S^T exchange (its buffer is refilled
    // right after it), in two halves issued behind the K fragments so that
    // the first QK products need not wait for them; the pair variant, which
    // refills only after the next chunk's barrier, reads them after the
    // exchange (fewer live registers).
    constexpr bool kEarlyV = GROUP == 1;
    constexpr int kNtHalf = C::kNt / 2;
    constexpr int kVReadsHalf = kNtHalf * C::kPvSteps * kUnits;
    short4v vt[C::kNt][C::kPvSteps][kUnits];
    auto read_v = [&](int nt_begin, int nt_end) {
#pragma unroll
      for (int nt = 0; nt < C::kNt; ++nt) {
        if (nt < nt_begin || nt >= nt_end) continue;
        static_for<C::kPvSteps>([&](auto kb_c) {
          constexpr int KB = decltype(kb_c)::value;
#pragma unroll
          for (int u = 0; u < kUnits; ++u)
            vt[nt][KB][u] = lds_read_tr16_at<BOFF + C::kPvKeys * KB * 1024>(v_base[nt][u]);
        });
      }
    };
    auto fence_v = [&]() {
#pragma unroll
      for (int nt = 0; nt < C::kNt; ++nt)
#pragma unroll
        for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
          for (int u = 0; u < kUnits; ++u) fence_reg(vt[nt][kb][u]);
    };
    unsigned long long valid = valid_in;

    // The contraction slice is a compile-time constant inside qk(), so each
    // K read address is fixed at compile time (no per-read branches).
    auto qk = [&](auto half_c) {
      constexpr int HALF = decltype(half_c)::value;
      constexpr int kLen = C::len(HALF);
      constexpr int kStart = C::start(HALF);
      // K fragments in two batches (fewer live registers). Streaming issues
      // the first half of its V^T reads behind the second batch and waits
      // only for that batch; the rest of V^T and the chunk's validity mask
      // follow the products, and the exchange barrier's wait covers them.
      constexpr int kBatch = (kLen + 1) / 2;
      static_assert(kLen > kBatch, "two K batches");
      auto read_k = [&](half8(&kf)[kBatch], auto s0_c, auto cnt_c) {
        static_for<decltype(cnt_c)::value>([&](auto s_c) {
          constexpr int S = decltype(s_c)::value;
          constexpr int KS = kStart + decltype(s0_c)::value + S;  // k-step of 32 latent dims
          if constexpr (KS < 16) {
            kf[S] = lds_read_b128_at<BOFF + 256 * (KS >> 2)>(k_base[KS & 3]);
          } else {
            kf[S] = lds_read_b128_at<BOFF>(r_base[KS - 16]);
          }
        });
      };
      // One accumulation chain: a product that takes the previous one's
      // result as its accumulator issues right behind it, and splitting the
      // chain (then adding the partial sums) measured slower.
      float4v sacc = float4v{0.f, 0.f, 0.f, 0.f};
      {
        half8 kf[kBatch];
        read_k(kf, std::integral_constant<int, 0>{}, std::integral_constant<int, kBatch>{});
        lds_wait();
#pragma unroll
        for (int s = 0; s < kBatch; ++s) fence_reg(kf[s]);
#pragma unroll
        for (int s = 0; s < kBatch; ++s)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], qf[s], sacc, 0, 0, 0);
      }
      {
        half8 kf[kBatch];
        read_k(kf, std::integral_constant<int, kBatch>{}, std::integral_constant<int, kLen - kBatch>{});
        if constexpr (kEarlyV) {
          read_v(0, kNtHalf);
          lds_wait_n<kVReadsHalf>();
        } else {
          lds_wait();
        }
#pragma unroll
        for (int s = 0; s < kLen - kBatch; ++s) fence_reg(kf[s]);
#pragma unroll
        for (int s = kBatch; s < kLen; ++s)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s - kBatch], qf[s], sacc, 0, 0, 0);
      }
      if constexpr (kEarlyV) {
        read_v(kNtHalf, C::kNt);
        valid = lds_read_u64(valid_lds);
      }
      const float4v ssum = sacc;
      const int slot = s_slot<CHUNK>(4 * tile + g, c16);
      *reinterpret_cast<float4v*>(&sbuf_c[(HALF * kHeads + c16) * C::kSStride + 4 * slot]) = ssum;
    };
    // L2-resident rows: the wave's QK products and their K reads go first on
    // its SIMD (a raised wave priority), which measured 0.3% faster per
    // prefill step; for rows beyond the L2 it measured slower.
    if constexpr (!FAR) __builtin_amdgcn_s_setprio(1);
    with_slice<C::kHalves>(half, qk);
    if constexpr (!FAR) __builtin_amdgcn_s_setprio(0);
    lds_barrier();  // also completes this wave's V^T and mask reads
    if constexpr (kEarlyV) {
      fence_v();
      fence_reg(valid);
    }

    // Online softmax for head c16 over keys kPvKeys*kb + kKpl*g + i. The S^T
    // reads are issued before after_exchange(), whose own LDS wait covers them.
    float4v sp[C::kPvSteps][C::kHalves][kUnits];
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
      for (int hh = 0; hh < C::kHalves; ++hh) {
        const unsigned srow = sbuf_c_addr + 4u * ((hh * kHeads + c16) * C::kSStride);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
          const int su = s_slot<CHUNK>((C::kPvKeys / 4) * kb + kUnits * g + u, c16);
          sp[kb][hh][u] = lds_read_f4(srow + 16u * su);
        }
      }
    if constexpr (!kEarlyV) read_v(0, C::kNt);
    stage(std::integral_constant<int, 0>{});
    lds_wait();
    if constexpr (!kEarlyV) fence_v();
    float zz[C::kPvSteps][kKpl];
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
      for (int hh = 0; hh < C::kHalves; ++hh)
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
          fence_reg(sp[kb][hh][u]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            zz[kb][4 * u + i] = hh == 0 ? sp[kb][hh][u][i] : zz[kb][4 * u + i] + sp[kb][hh][u][i];
        }
    stage(std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    // Keys past the end of the list (or rejected indices) only occur in
    // chunks that are not entirely valid.
    const unsigned vlo = __builtin_amdgcn_readfirstlane((unsigned)valid);
    const unsigned vhi = __builtin_amdgcn_readfirstlane((unsigned)(valid >> 32));
    const unsigned long long vmask = ((unsigned long long)vhi << 32) | vlo;
    constexpr unsigned long long kChunkMask = CHUNK == 64 ? ~0ull : ((1ull << CHUNK) - 1);
    if ((vmask & kChunkMask) != kChunkMask) {
#pragma unroll
      for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
        for (int i = 0; i < kKpl; ++i) {
          const int kk = C::kPvKeys * kb + kKpl * g + i;
          if (!((vmask >> kk) & 1ull)) zz[kb][i] = -__builtin_inff();
        }
    }
    float cmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
      for (int i = 0; i < kKpl; ++i) cmax = fmaxf(cmax, zz[kb][i]);
    // The fences pin each step's results ahead of the next stage's loads
    // (the compiler would otherwise sink the arithmetic to its uses).
    fence_reg(cmax);
    __builtin_amdgcn_sched_barrier(0);
    stage(std::integral_constant<int, 2>{});
    __builtin_amdgcn_sched_barrier(0);
    // Move the reference (and rescale O and l) only when needed; the test is
    // made per head on the head's maximum hmax (scale > 0, so the maximum
    // commutes with it). A lane holds a quarter of its head's keys, and no
    // head needs a new reference unless some lane's own maximum does.
    auto move_ref = [&](float hmax) {
      const bool move = hmax > m_ref + kRescaleThreshold;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - hmax) : 1.f;
      if (move) m_ref = hmax;
      if constexpr (FAR) acc_l *= alpha;
      else l_run *= alpha;
#pragma unroll
      for (int nt = 0; nt < C::kNt; ++nt) acc_o[nt] *= alpha;
    };
    if constexpr (FAR) {
      const float hmax = max4_heads(cmax) * a.scale_log2e;
      if (__ballot(hmax > m_ref + kRescaleThreshold)) move_ref(hmax);
    } else {
      const float lmax = cmax * a.scale_log2e;
      if (__ballot(lmax > m_ref + kRescaleThreshold)) move_ref(max4_heads(lmax));
    }
    float m_use = (m_ref == -__builtin_inff()) ? 0.f : m_ref;
    fence_reg(m_use);
    if constexpr (FAR) {
      __builtin_amdgcn_sched_barrier(0);
      stage(std::integral_constant<int, 3>{});
    }
    __builtin_amdgcn_sched_barrier(0);
    using pvec = std::conditional_t<kKpl == 8, half8, half4>;
    pvec pf[C::kPvSteps];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
      for (int i = 0; i < kKpl; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(zz[kb][i], a.scale_log2e, -m_use));
        if constexpr (!FAR) psum += p;
        pf[kb][i] = (_Float16)p;
      }
    if constexpr (!FAR) l_run += psum;
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb) fence_reg(pf[kb]);
    fence_reg(l_run);
    __builtin_amdgcn_sched_barrier(0);
    stage(std::integral_constant<int, FAR ? 4 : 3>{});
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T . P^T
#pragma unroll
    for (int nt = 0; nt < C::kNt; ++nt)
#pragma unroll
      for (int kb = 0; kb < C::kPvSteps; ++kb) {
        if (!FAR && nt == C::kNt / 2 && kb == 0) {
          __builtin_amdgcn_sched_barrier(0);
          stage(std::integral_constant<int, 4>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kKpl == 8) {
          const half4 hlo = __builtin_bit_cast(half4, vt[nt][kb][0]);
          const half4 hhi = __builtin_bit_cast(half4, vt[nt][kb][1]);
          const half8 vf = half8{hlo[0], hlo[1], hlo[2], hlo[3], hhi[0], hhi[1], hhi[2], hhi[3]};
          acc_o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[kb], acc_o[nt], 0, 0, 0);
        } else {
          const half4 vf = __builtin_bit_cast(half4, vt[nt][kb][0]);
          acc_o[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf[kb], acc_o[nt], 0, 0, 0);
        }
      }
    if constexpr (FAR) {
#pragma unroll
      for (int kb = 0; kb < C::kPvSteps; ++kb) {
        if constexpr (kKpl == 8) {
          const half8 ones = half8{1, 1, 1, 1, 1, 1, 1, 1};
          acc_l = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[kb], acc_l, 0, 0, 0);
        } else {
          const half4 ones = half4{1, 1, 1, 1};
          acc_l = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pf[kb], acc_l, 0, 0, 0);
        }
      }
    }
  };

  if (c_begin >= c_end) {  // an empty split: a neutral partial
    float* prow = a.part_o + ((int64_t)item * kHeads + c16) * kDv + (kDv / WAVES) * wave + 4 * g;
#pragma unroll
    for (int nt = 0; nt < C::kNt; ++nt) *reinterpret_cast<float4v*>(prow + 16 * nt) = float4v{0.f, 0.f, 0.f, 0.f};
    if (wave == 0 && g == 0) {
      a.part_ml[((int64_t)item * kHeads + c16) * 2] = -__builtin_inff();
      a.part_ml[((int64_t)item * kHeads + c16) * 2 + 1] = 0.f;
    }
    return;
  }

  // Q^T fragments of this wave's contraction slice (registers, whole query).
  auto load_q = [&]() {
    const _Float16* qrow = a.q + ((int64_t)(q_valid ? r : r - 1) * kHeads + c16) * kDqk + 8 * g;
    const int q_start = C::start(half), q_len = C::len(half);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
      if (s < q_len) qf[s] = *reinterpret_cast<const half8*>(qrow + 32 * (q_start + s));
  };

  if constexpr (GROUP == 1) {
    // Chunk ch of this work item lives in ring buffer (ch - c_begin) mod NBUF:
    // the loop below, unrolled by NBUF, then computes from a buffer known at
    // compile time.
    auto buf_of = [&](int ch) { return bufs + ((unsigned)(ch - c_begin) % NBUF) * C::kBuf; };
    // Gather of chunk ch into its ring buffer and its validity mask into its
    // slot; its selected indices are already in LDS. Split into the stages
    // of compute(): 0 reads the indices, 1 forms the row pointers, the mask
    // and the first rows' loads, 2-4 the remaining loads (4 also the rope
    // load and the index load of chunk ch + NBUF + 1).
    constexpr int kRowsPerStage = (kRowsPerHw + 3) / 4;
    int s_main = 0, s_rope = 0;
    unsigned kp_lo = 0, kp_hi = 0;
    const char* kr = self_row;
    auto issue_stage = [&](int ch, auto st_c) {
      constexpr int ST = decltype(st_c)::value;
      const int slot = (int)((unsigned)ch % C::kSlots);
      if constexpr (ST == 0) {
        s_main = lds_read_i32(sel_ring_addr + 4u * (slot * CHUNK + min(lane, CHUNK - 1)));
        s_rope = lds_read_i32(sel_ring_addr + 4u * (slot * CHUNK + rope_row));
      } else {
        if constexpr (ST == 1) {
          fence_reg(s_main);
          fence_reg(s_rope);
          bool ok, ok_rope;
          const char* kp = row_ptr(ch * CHUNK + lane, s_main, ok);
          kr = row_ptr(ch * CHUNK + rope_row, s_rope, ok_rope);
          kp_lo = (unsigned)(uintptr_t)kp;
          kp_hi = (unsigned)((uintptr_t)kp >> 32);
          const unsigned long long vm = __ballot(ok && lane < CHUNK);
          if (hw == 0 && lane == 0) valid_slots[slot] = vm;
        }
        gather_rows(kp_lo, kp_hi, buf_of(ch), (ST - 1) * kRowsPerStage, ST * kRowsPerStage);
        if constexpr (ST == 4) {
          gather_rope(kr, buf_of(ch));
          load_sel(ch + NBUF + 1);
        }
      }
    };
    // The whole gather at once (prologue).
    auto issue = [&](int ch) {
      issue_stage(ch, std::integral_constant<int, 0>{});
      lds_wait();
      issue_stage(ch, std::integral_constant<int, 1>{});
      issue_stage(ch, std::integral_constant<int, 2>{});
      issue_stage(ch, std::integral_constant<int, 3>{});
      issue_stage(ch, std::integral_constant<int, 4>{});
    };
    // Prologue: Q fragments and the indices of the first NBUF+1 chunks, all
    // waited for; then the gathers of the first NBUF chunks, each followed by
    // the index load for the chunk NBUF+1 places later (the order of loads
    // of the loop, where iteration ch issues chunk ch+NBUF and the indices of
    // chunk ch+2*NBUF+1).
#pragma unroll
    for (int k = 0; k <= NBUF; ++k) load_sel(c_begin + k);
    load_q();
    static_assert(C::len(0) == C::kSteps && C::len(1) == C::kSteps, "every wave issues kSteps Q loads");
    wait_vmcnt<C::kSteps>();  // the indices (issued before the Q loads)
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NBUF; ++k) {
      if (c_begin + k < c_end) issue(c_begin + k);  // includes the index load NBUF + 1 chunks ahead
    }
    for (int ch0 = c_begin; ch0 < c_end; ch0 += NBUF) {
      static_for<NBUF>([&](auto b_c) {
        const int ch = ch0 + decltype(b_c)::value;
        if (ch >= c_end) return;  // uniform
        // Chunk ch's loads (and all before them) are complete once at most
        // kWaitAhead later ones are outstanding, provided the chunks up to
        // ch+NBUF-1 were all issued; near the end, wait for everything.
        if (ch + NBUF - 1 < c_end) wait_vmcnt<C::kWaitAhead>();
        else wait_vmcnt<0>();
        lds_barrier();
        const bool refill = ch + NBUF < c_end;  // uniform
        compute(b_c, 0ull, valid_addr + 8u * ((unsigned)ch % C::kSlots), 0, [&](auto st_c) {
          if (refill) issue_stage(ch + NBUF, st_c);
        });
      });
    }
    wait_vmcnt<0>();  // index loads for chunks past the end
  } else {
    // Pair variant: two buffers, chunk ch computes from `cur` while the
    // gather of chunk ch+1 lands in `nxt`.
    lds_char* const buf0 = bufs;
    lds_char* const buf1 = bufs + C::kBuf;
    auto gather_pair = [&](int ch, lds_char* buf) -> unsigned long long {
      bool ok;
      const char* kp = row_of_pair(ch, ok);
      const uintptr_t kpi = (uintptr_t)kp;
      const unsigned lo = __shfl((unsigned)kpi, rope_row);
      const unsigned hi = __shfl((unsigned)(kpi >> 32), rope_row);
      const unsigned long long vm = __ballot(ok);
      gather_rows((unsigned)kpi, (unsigned)(kpi >> 32), buf, 0, kRowsPerHw);
      gather_rope(reinterpret_cast<const char*>(((uintptr_t)hi << 32) | lo), buf);
      return vm;
    };
    unsigned long long valid_cur = gather_pair(c_begin, buf0);
    load_q();
    auto step = [&](int ch, auto cur_c, lds_char* nxt) {
      wait_vmcnt<0>();
      lds_barrier();
      unsigned long long valid_next = 0;
      if (ch + 1 < c_end) valid_next = gather_pair(ch + 1, nxt);
      compute(cur_c, valid_cur, 0u, ch & 1, [](auto) {});
      valid_cur = valid_next;
    };
    for (int ch = c_begin;;) {
      step(ch, std::integral_constant<int, 0>{}, buf1);
      if (++ch >= c_end) break;
      step(ch, std::integral_constant<int, 1>{}, buf0);
      if (++ch >= c_end) break;
    }
  }

  const float l_tot = FAR ? acc_l[0] : sum4_heads(l_run);
  if (a.splits > 1) {
    // Partial result of this split: O and l relative to the reference m
    // (log2 units); attn_merge_kernel combines the splits of a query.
    float* prow = a.part_o + ((int64_t)item * kHeads + c16) * kDv + (kDv / WAVES) * wave + 4 * g;
#pragma unroll
    for (int nt = 0; nt < C::kNt; ++nt) *reinterpret_cast<float4v*>(prow + 16 * nt) = acc_o[nt];
    if (wave == 0 && g == 0) {
      a.part_ml[((int64_t)item * kHeads + c16) * 2] = m_ref;
      a.part_ml[((int64_t)item * kHeads + c16) * 2 + 1] = l_tot;
    }
    return;
  }
  if (!q_valid) return;  // the pair's missing second query
  const float inv = 1.0f / l_tot;
  if constexpr (GROUP == 1) {
    // The query's output (16 heads x 512 fp32, 32 KB contiguous) goes out as
    // whole 1 KB pieces: each wave first puts its O^T slice into LDS as
    // [head][512] rows (16-byte unit u of head h at u ^ (h & 15), so that
    // both the writes and the row reads below are conflict-free), then
    // writes 8 KB (4 heads) with one contiguous 1 KB store per instruction.
    // The chunk buffers are free here: every wave has passed the last
    // chunk's exchange barrier, after which no wave reads them.
    static_assert(NBUF * C::kBuf >= kHeads * kDv * 4, "output staging fits the chunk buffers");
    static_assert((kHeads * kDv * 4) % (WAVES * 1024) == 0, "whole 1 KB pieces per wave");
#pragma unroll
    for (int nt = 0; nt < C::kNt; ++nt) {
      const int u = (kDv / WAVES / 4) * wave + 4 * nt + g;
      *reinterpret_cast<__attribute__((address_space(3))) float4v*>(bufs + c16 * (kDv * 4) + ((u ^ c16) << 4)) =
          acc_o[nt] * inv;
    }
    lds_barrier();
    float4v* const orow = reinterpret_cast<float4v*>(a.out + (int64_t)r * kHeads * kDv);
    constexpr int kPieces = (kHeads * kDv * 4) / (WAVES * 1024);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int piece = kPieces * wave + j;  // 1 KB piece of the query's output
      const int h = piece / (kDv * 4 / 1024);
      const int u = (piece % (kDv * 4 / 1024)) * 64 + lane;
      const float4v v = *reinterpret_cast<const __attribute__((address_space(3))) float4v*>(
          bufs + h * (kDv * 4) + ((u ^ h) << 4));
      __builtin_nontemporal_store(v, orow + 64 * piece + lane);
    }
  } else {
    float* orow = a.out + ((int64_t)r * kHeads + c16) * kDv + (kDv / WAVES) * wave + 4 * g;
#pragma unroll
    for (int nt = 0; nt < C::kNt; ++nt) {
      const float4v v = acc_o[nt] * inv;
      __builtin_nontemporal_store(v, reinterpret_cast<float4v*>(orow + 16 * nt));
    }
  }
  if (a.lse && wave == 0 && g == 0) {
    a.lse[(int64_t)r * kHeads + c16] = (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

#ifndef SPMLA_ATTN_WAVES
#define SPMLA_ATTN_WAVES 4
#endif
#ifndef SPMLA_ATTN_CHUNK
#define SPMLA_ATTN_CHUNK 32
#endif
#ifndef SPMLA_ATTN_NBUF
#define SPMLA_ATTN_NBUF 2
#endif
#ifndef SPMLA_ATTN_WPE
#define SPMLA_ATTN_WPE 2
#endif

// Combines the key splits of one (query, head): with M the largest split
// reference, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s and
// lse = (M + log2 of that sum) * ln 2. A workgroup takes one quarter of the
// value dims of one (query, head); its four split groups each sum every
// fourth split (8 loads in flight per thread) and meet in LDS in a fixed
// order, and the l sum is a fixed shuffle tree, so results do not depend on
// timing.
constexpr int kMergeParts = 4;   // value-dim quarters per (query, head)
constexpr int kMergeGroups = 4;  // split groups per workgroup
constexpr int kMergeCols = kDv / kMergeParts / 4;  // float4 columns per quarter
__global__ __launch_bounds__(kMergeCols * kMergeGroups) void attn_merge_kernel(AttnArgs a) {
  __shared__ float w_s[kMaxSplits];
  __shared__ float s_lsum, s_mmax;
  __shared__ float4v part[kMergeGroups - 1][kMergeCols];
  const int qd = blockIdx.x % kMergeParts;
  const int h = (blockIdx.x / kMergeParts) % kHeads;
  const int r = blockIdx.x / (kMergeParts * kHeads);
  const int tid = threadIdx.x;
  const int ns = a.splits;  // <= kMaxSplits
  if (tid < 64) {
    const bool has = tid < ns;
    const float* ml = a.part_ml + (((int64_t)r * ns + (has ? tid : 0)) * kHeads + h) * 2;
    const float m = has ? ml[0] : -__builtin_inff();
    const float l = has ? ml[1] : 0.f;
    float m_max = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m_max = fmaxf(m_max, __shfl_xor(m_max, o));
    const float w = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - m_max);
    if (has) w_s[tid] = w;
    float wl = w * l;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wl += __shfl_xor(wl, o);
    if (tid == 0) {
      s_lsum = wl;
      s_mmax = m_max;
    }
  }
  __syncthreads();
  const int col = tid % kMergeCols;
  const int sg = tid / kMergeCols;
  const int d = qd * (kDv / kMergeParts) + 4 * col;
  const float* po = a.part_o + ((int64_t)r * ns * kHeads + h) * kDv + d;
  const int64_t stride = (int64_t)kHeads * kDv;
  float4v o = float4v{0.f, 0.f, 0.f, 0.f};
  int s = sg;
  for (; s + 7 * kMergeGroups < ns; s += 8 * kMergeGroups) {
    float4v p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = *reinterpret_cast<const float4v*>(po + (s + u * kMergeGroups) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) o += w_s[s + u * kMergeGroups] * p[u];
  }
  for (; s < ns; s += kMergeGroups) o += w_s[s] * *reinterpret_cast<const float4v*>(po + s * stride);
  if (sg > 0) part[sg - 1][col] = o;
  __syncthreads();
  if (sg != 0) return;
#pragma unroll
  for (int g = 0; g < kMergeGroups - 1; ++g) o += part[g][col];
  const float l_sum = s_lsum;
  *reinterpret_cast<float4v*>(a.out + ((int64_t)r * kHeads + h) * kDv + d) = o * (1.0f / l_sum);
  if (a.lse && qd == 0 && tid == 0)
    a.lse[(int64_t)r * kHeads + h] = (s_mmax + __builtin_amdgcn_logf(l_sum)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a_in, hipStream_t stream) {
  if (a_in.n_q <= 0) return hipSuccess;
  AttnArgs a = a_in;
  if (a.splits < 1) a.splits = 1;
  if (a.splits > 1 || a.band_items >= a.n_q) a.band_items = 0;
  int grid = 2 * kXcds * attn_slice_len(a.n_q * a.splits);
  if (a.band_items > 0) {
    const int full = a.n_q / a.band_items, rest = a.n_q - full * a.band_items;
    grid = full * 2 * kXcds * attn_slice_len(a.band_items) + (rest ? 2 * kXcds * attn_slice_len(rest) : 0);
  }
  constexpr int W = SPMLA_ATTN_WAVES;
  if (rows_beyond_l2(a.n_comp))
    hipLaunchKernelGGL((attn_kernel<W, SPMLA_ATTN_CHUNK, SPMLA_ATTN_NBUF, SPMLA_ATTN_WPE, 1, true>),
                       dim3(grid), dim3(64 * W), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<W, SPMLA_ATTN_CHUNK, SPMLA_ATTN_NBUF, SPMLA_ATTN_WPE, 1, false>),
                       dim3(grid), dim3(64 * W), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(a.n_q * kHeads * kMergeParts), dim3(kMergeCols * kMergeGroups), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_grouped(const AttnArgs& a_in, hipStream_t stream) {
  if (a_in.n_q <= 0) return hipSuccess;
  AttnArgs a = a_in;
  a.splits = 1;
  a.band_items = 0;
  const int pairs = (a.n_q + 1) / 2;
  const int grid = 2 * kXcds * attn_slice_len(pairs);
  // Bitmaps of the two queries' rows and the pair's row list.
  const size_t words = ((size_t)a.n_comp + 31) / 32;
  const size_t lds = 4 * (2 * words + 2 * (size_t)a.top_k);
  hipLaunchKernelGGL((attn_kernel<SPMLA_ATTN_WAVES, SPMLA_ATTN_CHUNK, 2, SPMLA_ATTN_WPE, 2, false>),
                     dim3(grid), dim3(128 * SPMLA_ATTN_WAVES), lds, stream, a);
  return hipGetLastError();
}

}  // namespace spmla
