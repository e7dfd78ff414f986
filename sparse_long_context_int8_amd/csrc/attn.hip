// Streaming sparse MLA attention on CDNA4 (gfx950).
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): each selected F16 latent row is read once and shared by
// the sixteen query heads, with an online softmax; the page "perf(ds4): unify
// gfx1151 sparse-prefill stack" (Validation completed) stages in FP32 and
// uses a fast exponential. Here: fp16 operands on matrix cores, fp32
// accumulation and softmax, exp2 with log2(e) folded into the scale.
//
// One workgroup per query token. Its key list is the selected compressed
// rows followed by the sliding-window raw rows; keys stream through LDS in
// chunks of CHUNK rows gathered with direct global->LDS loads, so each row
// crosses the memory system once per query.
//
// LDS image of a chunk (per buffer):
//   region A: CHUNK rows x 1024 B = latent dims 0..511 (the value part),
//             one wave-wide 16-byte-per-lane load per row;
//   region B: CHUNK rows x 128 B  = latent dims 512..575 (the rope part),
//             one load per 8 rows.
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
//       row-major region A, P^T built in registers.
// With NBUF == 2 the gather of chunk i+1 is in flight while chunk i computes.
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
// pipeline. Each group of reads ends with lds_wait() and fence_reg() on the
// results, so no value is used before it has arrived.
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
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ void fence_reg(T& v) {
  asm volatile("" : "+v"(v));
}

template <int WAVES, int CHUNK, int NBUF, int WPE, bool ROPE_REG>
struct Cfg {
  static constexpr int kRowsPerWave = CHUNK / WAVES;
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
  static constexpr int kPvSteps = CHUNK / 32;
  static constexpr int kBufA = CHUNK * 1024;
  static constexpr int kBufB = ROPE_REG ? 0 : CHUNK * 128;
  static constexpr int kBuf = kBufA + kBufB;
  static constexpr int kSStride = CHUNK;  // floats per head row of S^T partials
  static constexpr int kSBytes = kHalves * kHeads * kSStride * 4;
  static constexpr int kLds = NBUF * (kBuf + kSBytes);
  // k-steps 16 and 17 (the rope dims) belong to the last contraction slice.
  static_assert(kTiles * kHalves == WAVES, "QK work must split evenly");
  static_assert(ROPE_REG || kRowsPerWave % 8 == 0, "rope loads cover 8 rows");
  static_assert(start(kHalves - 1) <= 16, "rope steps live in the last slice");
  static_assert(CHUNK % 32 == 0, "PV steps are 32 keys");
  static_assert(kLds * ((WPE * 4) / WAVES) <= 160 * 1024, "LDS for the requested occupancy");
};

// Softmax reference is moved only when a chunk's max exceeds it by more than
// this (log2 units); probabilities are then at most 2^8, which fp16 P and
// fp32 sums hold exactly enough, and the O rescale is skipped for most chunks.
constexpr float kRescaleThreshold = 8.0f;

// GROUP == 1: streaming, one query per workgroup of WAVES waves.
// GROUP == 2: query-tiled ("grouped") variant. A workgroup of 2*WAVES waves
// takes two adjacent queries t0, t1 = t0 + 1 and streams the union of their
// keys through one set of chunk buffers: t0's selected rows, then t1's
// selected rows that t0 did not select, then the union of the two windows
// (raw rows ws0 .. t1). Wave group g (waves g*WAVES ..) runs the streaming
// per-chunk work for query t_g with its own mask; every gathered row is read
// once for both queries.
template <int WAVES, int CHUNK, int NBUF, int WPE, bool ROPE_REG, int GROUP>
__global__ __launch_bounds__(64 * WAVES * GROUP) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_kernel(AttnArgs a) {
  using C = Cfg<WAVES, CHUNK, NBUF, WPE, ROPE_REG>;
  static_assert(GROUP == 1 || GROUP == 2, "one or two queries per workgroup");
  constexpr int kHw = WAVES * GROUP;             // waves in the workgroup
  constexpr int kRowsPerHw = CHUNK / kHw;        // rows of a chunk each wave gathers
  constexpr int kRopeLoadsPerHw = (CHUNK / 8 + kHw - 1) / kHw;
  static_assert(CHUNK % kHw == 0, "gather rows split evenly");
  __shared__ __attribute__((aligned(1024))) char buf0_[C::kBuf];
  __shared__ __attribute__((aligned(1024))) char buf1_[NBUF == 2 ? C::kBuf : 16];
  __shared__ __attribute__((aligned(16))) float sbuf[GROUP * NBUF * C::kSBytes / 4];
  lds_char* buf0 = (lds_char*)buf0_;
  lds_char* buf1 = (lds_char*)buf1_;

  // Work items (query r, key split s; or a query pair) are dealt to the dies
  // in contiguous blocks so that the window rows shared by neighbouring
  // queries stay in one die's L2.
  const int n_items = GROUP == 1 ? a.n_q * a.splits : (a.n_q + 1) / 2;
  const int per_xcd = (n_items + kXcds - 1) / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= n_items) return;

  const int lane = threadIdx.x & 63;
  const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = hw % WAVES;  // wave within its group
  const int grp = hw / WAVES;   // which query of the pair
  const int g = lane >> 4;
  const int c16 = lane & 15;
  float* sbuf_g = sbuf + grp * NBUF * (C::kSBytes / 4);
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
  const bool has_rope = ROPE_REG && half == C::kHalves - 1;

  half8 qf[C::kSteps];
  float4v acc_o[C::kNt];
#pragma unroll
  for (int nt = 0; nt < C::kNt; ++nt) acc_o[nt] = float4v{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();  // softmax reference (log2 domain) of head c16
  float l_run = 0.f;                // this lane's share of the softmax sum

  // Selected index of key k0 + lane: one in-bounds load per call (the pair
  // variant reads its list from LDS in row_of instead).
  auto load_sel = [&](int ch) -> int {
    if constexpr (GROUP == 2) return 0;
    const int key = min(ch * CHUNK + lane, a.top_k - 1);
    return __builtin_nontemporal_load(sel_row + key);
  };
  // Row pointer of key k0 + lane, and whether this group's query uses it.
  auto row_of = [&](int ch, int selv, bool& ok) -> const char* {
    const int key = ch * CHUNK + lane;
    ok = false;
    const char* p = self_row;
    if constexpr (GROUP == 1) {
      if (key < nsel) {
        ok = (selv >= 0) && (selv < nv);
        if (ok) p = comp_base + (int64_t)selv * kRowBytes;
      } else if (key < nk) {
        ok = true;
        p = raw_base + (int64_t)(ws + key - nsel) * kRowBytes;
      }
    } else {
      if (key < n_ab) {
        const int idx = lds_read_i32(list_lds + 4u * key);
        lds_wait();
        const bool in_range = idx >= 0 && idx < a.n_comp;
        if (in_range) p = comp_base + (int64_t)idx * kRowBytes;
        if (key < n_a) {  // t0's own selection
          const bool ok0 = idx >= 0 && idx < nv;  // grp 0: nv is t0's
          if (grp == 0) {
            ok = ok0;
          } else if (in_range && has1) {
            const unsigned word = (unsigned)lds_read_i32(bm1_lds + 4u * (idx >> 5));
            lds_wait();
            ok = (word >> (idx & 31)) & 1u;
          }
        } else {  // rows only t1 selected
          ok = grp == 1;
        }
      } else if (key < nk) {
        const int srow = ws0 + (key - n_ab);
        p = raw_base + (int64_t)srow * kRowBytes;
        ok = srow >= ws && srow <= t && q_valid;
      }
    }
    return p;
  };
  // This wave's share of the gather of one chunk, plus (rope in registers)
  // the rope fragments of the rows this wave scores.
  const int row0 = hw * kRowsPerHw;
  auto gather = [&](const char* kp, lds_char* buf, half8 (&rope)[2]) {
    lds_char* bufA = buf;
    const uintptr_t kpi = (uintptr_t)kp;
    const unsigned kp_lo = (unsigned)kpi;
    const unsigned kp_hi = (unsigned)(kpi >> 32);
#pragma unroll
    for (int i = 0; i < kRowsPerHw; ++i) {
      const int n = row0 + i;
      const unsigned lo = __builtin_amdgcn_readlane(kp_lo, n);
      const unsigned hi = __builtin_amdgcn_readlane(kp_hi, n);
      const char* rowp = reinterpret_cast<const char*>(((uintptr_t)hi << 32) | lo);
      const int off = (lane ^ swz_a(n)) << 4;
      __builtin_amdgcn_global_load_lds((gbl_char*)(rowp + off), bufA + n * 1024, 16, 0, 0);
    }
    if constexpr (!ROPE_REG) {
      lds_char* bufB = bufA + C::kBufA;
      // Rope load j covers rows 8j .. 8j+7; they are dealt to the waves.
#pragma unroll
      for (int jj = 0; jj < kRopeLoadsPerHw; ++jj) {
        const int j = hw + jj * kHw;
        if (j < CHUNK / 8) {
          const int nb = 8 * j + (lane >> 3);
          const unsigned lo = __shfl(kp_lo, nb);
          const unsigned hi = __shfl(kp_hi, nb);
          const char* rowp = reinterpret_cast<const char*>(((uintptr_t)hi << 32) | lo);
          const int off = (64 + ((lane & 7) ^ swz_b(nb))) << 4;
          __builtin_amdgcn_global_load_lds((gbl_char*)(rowp + off), bufB + 8 * j * 128, 16, 0, 0);
        }
      }
    } else {
      if (has_rope) {
        const int nr = 16 * tile + c16;
        const unsigned lo = __shfl(kp_lo, nr);
        const unsigned hi = __shfl(kp_hi, nr);
        const char* rowp = reinterpret_cast<const char*>(((uintptr_t)hi << 32) | lo);
        rope[0] = *reinterpret_cast<const half8*>(rowp + 1024 + 16 * g);
        rope[1] = *reinterpret_cast<const half8*>(rowp + 1024 + 64 + 16 * g);
      }
    }
  };

  // Scores, softmax update and PV of one chunk already in `cur`.
  // With two buffers the S^T exchange area alternates with the chunk buffer,
  // and no barrier is needed at the end of a chunk: the buffer is refilled
  // only after the next chunk's barrier, which every wave reaches after its
  // last read of it.
  auto compute = [&](lds_char* cur, unsigned long long valid, const half8 (&rope)[2], int sb) {
    const unsigned bA = (unsigned)(uintptr_t)cur;  // LDS byte address
    float* sbuf_c = sbuf_g + sb * (C::kSBytes / 4);
    const unsigned sbuf_c_addr = sbuf_addr + sb * C::kSBytes;
    // The contraction slice is a compile-time constant inside qk(), so each
    // K read address is fixed at compile time (no per-read branches).
    auto qk = [&](auto half_c) {
      constexpr int HALF = decltype(half_c)::value;
      const int n = 16 * tile + c16;
      constexpr int kLen = C::len(HALF);
      constexpr int kStart = C::start(HALF);
      half8 kf[C::kSteps];
#pragma unroll
      for (int s = 0; s < kLen; ++s) {
        const int ks = kStart + s;  // k-step of 32 latent dims
        if (ks < 16) {
          kf[s] = lds_read_b128(bA + n * 1024 + (((4 * ks + g) ^ swz_a(n)) << 4));
        } else if constexpr (!ROPE_REG) {
          kf[s] = lds_read_b128(bA + C::kBufA + n * 128 + (((4 * (ks - 16) + g) ^ swz_b(n)) << 4));
        }
      }
      lds_wait();
#pragma unroll
      for (int s = 0; s < kLen; ++s) {
        const int ks = kStart + s;
        if (ROPE_REG && ks >= 16) kf[s] = rope[ks - 16];
        fence_reg(kf[s]);
      }
      // Three independent accumulation chains, summed in a fixed order.
      float4v sacc[3] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < kLen; ++s)
        sacc[s % 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], qf[s], sacc[s % 3], 0, 0, 0);
      const float4v ssum = (sacc[0] + sacc[1]) + sacc[2];
      const int slot = (4 * tile + g) ^ swz_s(c16);
      *reinterpret_cast<float4v*>(&sbuf_c[(HALF * kHeads + c16) * C::kSStride + 4 * slot]) = ssum;
    };
    if (half == 0) {
      qk(std::integral_constant<int, 0>{});
    } else if constexpr (C::kHalves == 2) {
      qk(std::integral_constant<int, 1>{});
    } else if constexpr (C::kHalves == 4) {
      if (half == 1) qk(std::integral_constant<int, 1>{});
      else if (half == 2) qk(std::integral_constant<int, 2>{});
      else qk(std::integral_constant<int, 3>{});
    }
    static_assert(C::kHalves == 1 || C::kHalves == 2 || C::kHalves == 4, "slice dispatch");
    lds_barrier();

    // Online softmax for head c16 over keys {32kb + 8g + i}.
    float zz[C::kPvSteps][8];
    {
      float4v sp[C::kPvSteps][C::kHalves][2];
#pragma unroll
      for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
        for (int hh = 0; hh < C::kHalves; ++hh) {
          const unsigned srow = sbuf_c_addr + 4u * ((hh * kHeads + c16) * C::kSStride);
          const int s0 = (8 * kb + 2 * g) ^ swz_s(c16);
          const int s1 = (8 * kb + 2 * g + 1) ^ swz_s(c16);
          sp[kb][hh][0] = lds_read_f4(srow + 16u * s0);
          sp[kb][hh][1] = lds_read_f4(srow + 16u * s1);
        }
      lds_wait();
#pragma unroll
      for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
        for (int hh = 0; hh < C::kHalves; ++hh) {
          fence_reg(sp[kb][hh][0]);
          fence_reg(sp[kb][hh][1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            zz[kb][i] = hh == 0 ? sp[kb][hh][0][i] : zz[kb][i] + sp[kb][hh][0][i];
            zz[kb][4 + i] = hh == 0 ? sp[kb][hh][1][i] : zz[kb][4 + i] + sp[kb][hh][1][i];
          }
        }
    }
    // Keys past the end of the list (or rejected indices) only occur in
    // chunks that are not entirely valid.
    constexpr unsigned long long kChunkMask = CHUNK == 64 ? ~0ull : ((1ull << CHUNK) - 1);
    if ((valid & kChunkMask) != kChunkMask) {
#pragma unroll
      for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kk = 32 * kb + 8 * g + i;
          if (!((valid >> kk) & 1ull)) zz[kb][i] = -__builtin_inff();
        }
    }
    float cmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) cmax = fmaxf(cmax, zz[kb][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    cmax *= a.scale_log2e;  // scale > 0, so the max commutes with it
    // Move the reference (and rescale O and l) only when needed; the test is
    // made per head and the branch is taken if any head needs it.
    const bool move = cmax > m_ref + kRescaleThreshold;
    if (__ballot(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - cmax) : 1.f;
      if (move) m_ref = cmax;
      l_run *= alpha;
#pragma unroll
      for (int nt = 0; nt < C::kNt; ++nt) acc_o[nt] *= alpha;
    }
    const float m_use = (m_ref == -__builtin_inff()) ? 0.f : m_ref;
    half8 pf[C::kPvSteps];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::kPvSteps; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(zz[kb][i], a.scale_log2e, -m_use));
        psum += p;
        pf[kb][i] = (_Float16)p;
      }
    l_run += psum;

    // O^T[dims (512/W) wave + 16nt + 4g + i][head c16] += V^T . P^T
    const int tri = (lane >> 2) & 3;
    const int trc = lane & 3;
    constexpr int kPvGroup = C::kNt * C::kPvSteps > 4 ? (4 / C::kPvSteps > 0 ? 4 / C::kPvSteps : 1) : C::kNt;
#pragma unroll
    for (int nt0 = 0; nt0 < C::kNt; nt0 += kPvGroup) {
      short4v vt[kPvGroup][C::kPvSteps][2];
#pragma unroll
      for (int j = 0; j < kPvGroup; ++j) {
        const int dv0 = (kDv / WAVES) * wave + 16 * (nt0 + j);
        const int unit = (dv0 >> 3) + (trc >> 1);
        const int sub = (trc & 1) << 3;
#pragma unroll
        for (int kb = 0; kb < C::kPvSteps; ++kb) {
          const int n_lo = 32 * kb + 8 * g + tri;
          const int n_hi = n_lo + 4;
          vt[j][kb][0] = lds_read_tr16(bA + n_lo * 1024 + ((unit ^ swz_a(n_lo)) << 4) + sub);
          vt[j][kb][1] = lds_read_tr16(bA + n_hi * 1024 + ((unit ^ swz_a(n_hi)) << 4) + sub);
        }
      }
      lds_wait();
#pragma unroll
      for (int j = 0; j < kPvGroup; ++j)
#pragma unroll
        for (int kb = 0; kb < C::kPvSteps; ++kb) {
          fence_reg(vt[j][kb][0]);
          fence_reg(vt[j][kb][1]);
          const half4 hlo = __builtin_bit_cast(half4, vt[j][kb][0]);
          const half4 hhi = __builtin_bit_cast(half4, vt[j][kb][1]);
          const half8 vf = half8{hlo[0], hlo[1], hlo[2], hlo[3], hhi[0], hhi[1], hhi[2], hhi[3]};
          acc_o[nt0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[kb], acc_o[nt0 + j], 0, 0, 0);
        }
    }
    if constexpr (NBUF == 1) lds_barrier();  // `cur` and sbuf are refilled next
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

  // Prologue: start the gather of the first chunk, then load Q^T while it
  // flies.
  unsigned long long valid_cur;
  half8 rope_cur[2], rope_nxt[2];
  {
    const int sel0 = load_sel(c_begin);
    bool ok0;
    const char* kp0 = row_of(c_begin, sel0, ok0);
    valid_cur = __ballot(ok0);
    gather(kp0, buf0, rope_cur);
  }
  {
    const _Float16* qrow = a.q + ((int64_t)(q_valid ? r : r - 1) * kHeads + c16) * kDqk + 8 * g;
    const int q_start = C::start(half), q_len = C::len(half);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
      if (s < q_len) qf[s] = *reinterpret_cast<const half8*>(qrow + 32 * (q_start + s));
  }
  int sel_next = load_sel(min(c_begin + 1, c_end - 1));

  if constexpr (NBUF == 2) {
    // Chunk ch computes from `cur` while the gather of chunk ch+1 lands in
    // `nxt`. The only wait is for this chunk's gather (and everything issued
    // before it), right before the barrier that publishes it.
    auto step = [&](int ch, lds_char* cur, lds_char* nxt) {
      wait_vmcnt<0>();
      lds_barrier();
      unsigned long long valid_next = 0;
      if (ch + 1 < c_end) {
        bool okn;
        const char* kpn = row_of(ch + 1, sel_next, okn);
        valid_next = __ballot(okn);
        sel_next = load_sel(min(ch + 2, c_end - 1));
        gather(kpn, nxt, rope_nxt);
      }
      compute(cur, valid_cur, rope_cur, ch & 1);
      valid_cur = valid_next;
      rope_cur[0] = rope_nxt[0];
      rope_cur[1] = rope_nxt[1];
    };
    for (int ch = c_begin;;) {
      step(ch, buf0, buf1);
      if (++ch >= c_end) break;
      step(ch, buf1, buf0);
      if (++ch >= c_end) break;
    }
  } else {
    for (int ch = c_begin; ch < c_end; ++ch) {
      wait_vmcnt<0>();
      lds_barrier();
      compute(buf0, valid_cur, rope_cur, 0);
      if (ch + 1 < c_end) {
        bool okn;
        const char* kpn = row_of(ch + 1, sel_next, okn);
        valid_cur = __ballot(okn);
        sel_next = load_sel(min(ch + 2, c_end - 1));
        gather(kpn, buf0, rope_cur);
      }
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = l_tot + __shfl_xor(l_tot, 32);
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
  float* orow = a.out + ((int64_t)r * kHeads + c16) * kDv + (kDv / WAVES) * wave + 4 * g;
#pragma unroll
  for (int nt = 0; nt < C::kNt; ++nt) {
    const float4v v = acc_o[nt] * inv;
    __builtin_nontemporal_store(v, reinterpret_cast<float4v*>(orow + 16 * nt));
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
#ifndef SPMLA_ATTN_ROPE_REG
#define SPMLA_ATTN_ROPE_REG 0
#endif

// Combines the key splits of one (query, head): with M the largest split
// reference, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s and
// lse = (M + log2 of that sum) * ln 2, splits summed in order. The split
// weights are formed once in LDS; the partial rows are read with independent
// loads (8 splits in flight per thread).
constexpr int kMaxSplits = 64;
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
  __shared__ float w_s[kMaxSplits];
  __shared__ float s_lsum, s_mmax;
  const int r = blockIdx.x / kHeads;
  const int h = blockIdx.x % kHeads;
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
    // l sum in split order (a fixed order for every launch)
    float wl = w * l;
    float total = 0.f;
    for (int s = 0; s < ns; ++s) total += __shfl(wl, s);
    if (tid == 0) {
      s_lsum = total;
      s_mmax = m_max;
    }
  }
  __syncthreads();
  const int d = 4 * tid;
  const float* po = a.part_o + ((int64_t)r * ns * kHeads + h) * kDv + d;
  const int64_t stride = (int64_t)kHeads * kDv;
  float4v o = float4v{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 8 <= ns; s += 8) {
    float4v p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = *reinterpret_cast<const float4v*>(po + (s + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) o += w_s[s + u] * p[u];
  }
  for (; s < ns; ++s) o += w_s[s] * *reinterpret_cast<const float4v*>(po + s * stride);
  const float l_sum = s_lsum;
  *reinterpret_cast<float4v*>(a.out + ((int64_t)r * kHeads + h) * kDv + d) = o * (1.0f / l_sum);
  if (a.lse && tid == 0) a.lse[(int64_t)r * kHeads + h] = (s_mmax + __builtin_amdgcn_logf(l_sum)) * 0.69314718055994531f;
}

}  // namespace

int attn_splits(int n_q_call) {
  if (n_q_call >= 512) return 1;
  const int s = (1024 + n_q_call - 1) / n_q_call;
  return s < kMaxSplits ? s : kMaxSplits;
}

size_t attn_partial_bytes(int rows, int splits) {
  if (splits <= 1) return 0;
  const size_t items = (size_t)rows * splits;
  return items * kHeads * kDv * sizeof(float) + items * kHeads * 2 * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a_in, hipStream_t stream) {
  if (a_in.n_q <= 0) return hipSuccess;
  AttnArgs a = a_in;
  if (a.splits < 1) a.splits = 1;
  const int per_xcd = (a.n_q * a.splits + kXcds - 1) / kXcds;
  constexpr int W = SPMLA_ATTN_WAVES;
  hipLaunchKernelGGL((attn_kernel<W, SPMLA_ATTN_CHUNK, SPMLA_ATTN_NBUF, SPMLA_ATTN_WPE,
                                  (bool)SPMLA_ATTN_ROPE_REG, 1>),
                     dim3(per_xcd * kXcds), dim3(64 * W), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(a.n_q * kHeads), dim3(kDv / 4), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_grouped(const AttnArgs& a_in, hipStream_t stream) {
  if (a_in.n_q <= 0) return hipSuccess;
  AttnArgs a = a_in;
  a.splits = 1;
  const int pairs = (a.n_q + 1) / 2;
  const int per_xcd = (pairs + kXcds - 1) / kXcds;
  // Bitmaps of the two queries' rows and the pair's row list.
  const size_t words = ((size_t)a.n_comp + 31) / 32;
  const size_t lds = 4 * (2 * words + 2 * (size_t)a.top_k);
  hipLaunchKernelGGL((attn_kernel<SPMLA_ATTN_WAVES, SPMLA_ATTN_CHUNK, SPMLA_ATTN_NBUF, SPMLA_ATTN_WPE,
                                  (bool)SPMLA_ATTN_ROPE_REG, 2>),
                     dim3(per_xcd * kXcds), dim3(128 * SPMLA_ATTN_WAVES), lds, stream, a);
  return hipGetLastError();
}

}  // namespace spmla
