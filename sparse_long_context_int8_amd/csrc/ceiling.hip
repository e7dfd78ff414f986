// Measured gather ceiling of the attention step (a measurement kernel, not
// part of the layer; built into its own library, libspmla_ceiling.so).
//
// The streaming attention reads a query's 16 x 576 fp16 query rows and its
// selected indices, moves every selected compressed row and every window row
// (1,152 B each) from the memory system into LDS with direct global->LDS
// loads, and writes 16 x 512 fp32 outputs and 16 log-sum-exps. Its rows are
// mostly L2- or MALL-resident, so the HBM roofline does not bound it. This
// kernel moves exactly the same bytes for the same queries, in the same
// order, with the same load instructions and LDS images (value part 1 KB per
// row, rope part 128 B) and whole-line output stores, and does nothing else:
// no products, no softmax, no barriers. Its rate is the ceiling of the
// attention's data movement on this chip.
//
// One workgroup of four waves per query, dealt to the eight dies as the
// attention kernel deals them; wave w loads rows 8w .. 8w+7 of every 32-row
// chunk into its own ring of NBUF chunk slots, keeping up to NBUF chunks of
// loads in flight. Row indices come from scalar loads, so the vector memory
// counter only tracks the row loads.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(1))) const char gbl_char;
typedef __attribute__((address_space(4))) const int cst_int;

constexpr int kRowBytes = 1152;
constexpr int kChunk = 32;
constexpr int kRowsPerWave = 8;
constexpr int kXcds = 8;

struct GatherArgs {
  const char* q;       // [n_q][16][576] fp16
  const char* kv_comp;
  const char* kv_raw;
  const int32_t* sel;  // [n_q][top_k], -1 padded
  float* out;          // [n_q][16][512], written with zeros
  float* lse;          // [n_q][16], written with zeros
  int32_t n_q, q_pos0, n_comp, ratio, window, top_k;
  int32_t band;        // > 0: queries dealt to the dies band by band (as the attention's banded launch)
};

__host__ __device__ inline int slice_len_of(int n_items) { return (n_items + 2 * kXcds - 1) / (2 * kXcds); }
__device__ inline int item_at(int idx, int n_items) {
  const int slice_len = slice_len_of(n_items);
  const int x = idx % kXcds, l = idx / kXcds;
  return l < slice_len ? (2 * kXcds - 1 - x) * slice_len + l : x * slice_len + (l - slice_len);
}
// Band b takes workgroups [b * G, (b + 1) * G), G = 2 * kXcds * slice_len(band),
// dealt inside its range as a launch of that band alone.
__device__ inline int item_of(int n_items, int band) {
  if (band <= 0 || band >= n_items) return item_at(blockIdx.x, n_items);
  const int g = 2 * kXcds * slice_len_of(band);
  const int b = blockIdx.x / g, first = b * band;
  if (first >= n_items) return n_items;
  const int n_band = min(band, n_items - first);
  const int it = item_at(blockIdx.x - b * g, n_band);
  return it < n_band ? first + it : n_items;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

template <int NBUF>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int kSlot = kRowsPerWave * kRowBytes;  // one wave's rows of a chunk
  __shared__ __attribute__((aligned(1024))) char ring_[4 * NBUF * kSlot];
  const int r = item_of(a.n_q, a.band);
  if (r >= a.n_q) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lds_char* const ring = (lds_char*)ring_ + wave * NBUF * kSlot;

  const int t = a.q_pos0 + r;
  const int nv = min(a.n_comp, (t + 1) / a.ratio);
  const int nsel = min(a.top_k, nv);
  const int ws = max(0, t - a.window + 1);
  const int nk = nsel + (t - ws + 1);
  const int nchunks = (nk + kChunk - 1) / kChunk;
  cst_int* const sel_row = (cst_int*)(a.sel + (int64_t)r * a.top_k);
  const char* const self_row = a.kv_raw + (int64_t)t * kRowBytes;

  auto row_ptr = [&](int key) -> const char* {
    if (key < nsel) {
      const int idx = sel_row[key];  // wave-uniform: a scalar load
      return (idx >= 0 && idx < nv) ? a.kv_comp + (int64_t)idx * kRowBytes : self_row;
    }
    if (key < nk) return a.kv_raw + (int64_t)(ws + key - nsel) * kRowBytes;
    return self_row;
  };
  auto issue = [&](int ch) {
    lds_char* const slot = ring + (ch % NBUF) * kSlot;
    const int n0 = ch * kChunk + wave * kRowsPerWave;
    const char* pr = self_row;  // rope parts: lane l loads 16 B of row l / 8
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const char* p = row_ptr(n0 + i);
      __builtin_amdgcn_global_load_lds((gbl_char*)(p + 16 * lane), slot + i * 1024, 16, 0, 0);
      if ((lane >> 3) == i) pr = p;
    }
    __builtin_amdgcn_global_load_lds((gbl_char*)(pr + 1024 + 16 * (lane & 7)), slot + kRowsPerWave * 1024, 16, 0,
                                     0);
  };
  // The query rows (18 KB: 18 loads of 1 KB over the four waves) into the
  // first slot, ahead of the gathers that later overwrite it.
  const char* const qrow = a.q + (int64_t)r * 16 * 576 * 2;
  for (int j = wave; j < 18; j += 4)
    __builtin_amdgcn_global_load_lds((gbl_char*)(qrow + 1024 * j + 16 * lane), ring + 1024 * (j / 4), 16, 0, 0);
  constexpr int kOps = kRowsPerWave + 1;  // loads per wave per chunk
#pragma unroll
  for (int k = 0; k < NBUF - 1; ++k)
    if (k < nchunks) issue(k);
  for (int ch = 0; ch < nchunks; ++ch) {
    if (ch + NBUF - 1 < nchunks) {
      wait_vmcnt<(NBUF - 1) * kOps>();  // chunk ch-1's loads are done: its slot is free
      issue(ch + NBUF - 1);
    }
  }
  wait_vmcnt<0>();
  // The output (32 KB: 8 contiguous 1 KB stores per wave) and the lse.
  typedef float float4v __attribute__((ext_vector_type(4)));
  float4v* const orow = reinterpret_cast<float4v*>(a.out + (int64_t)r * 16 * 512);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_nontemporal_store(float4v{0.f, 0.f, 0.f, 0.f}, orow + 64 * (8 * wave + j) + lane);
  if (a.lse && wave == 0 && lane < 16) a.lse[(int64_t)r * 16 + lane] = 0.f;
}

template <int NBUF>
int launch(const GatherArgs& a, hipStream_t s) {
  int grid = 2 * kXcds * slice_len_of(a.n_q);
  if (a.band > 0 && a.band < a.n_q) {
    const int full = a.n_q / a.band, rest = a.n_q - full * a.band;
    grid = full * 2 * kXcds * slice_len_of(a.band) + (rest ? 2 * kXcds * slice_len_of(rest) : 0);
  }
  hipLaunchKernelGGL(gather_kernel<NBUF>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

extern "C" {

// The data movement of spmla_sparse_attn for queries q_pos0 .. q_pos0+n_q-1:
// reads the query rows and the selected indices, gathers the key rows
// (selected compressed rows, then the window's raw rows) into LDS and
// discards them, and writes zeros to out and lse (may be NULL). nbuf: chunks
// of row loads in flight per wave, 2, 3 or 4 (LDS of 74, 111 or 147 KB per
// workgroup). Returns 0, -1 (bad argument) or -4 (launch error). Arrays as
// in spmla_sparse_attn (16-byte aligned device pointers; q [n_q][16][576]
// and kv_comp [n_comp][576], kv_raw [q_pos0+n_q][576] fp16; sel
// [n_q][top_k]; out [n_q][16][512] and lse [n_q][16] fp32). band > 0: the
// queries are dealt to the dies band by band, as spmla_prefill's attention
// launch deals them.
int spmla_ceiling_gather(const void* q, const void* kv_comp, const void* kv_raw, const int32_t* sel, float* out,
                         float* lse, int32_t n_q, int32_t q_pos0, int32_t n_comp, int32_t ratio, int32_t window,
                         int32_t top_k, int32_t nbuf, int32_t band, void* stream) {
  if (!q || !kv_raw || !sel || !out || n_q < 0 || q_pos0 < 0 || n_comp < 0 || ratio < 1 || window < 1 || top_k < 1)
    return -1;
  if (n_comp > 0 && !kv_comp) return -1;
  if (n_q == 0) return 0;
  GatherArgs a{static_cast<const char*>(q), static_cast<const char*>(kv_comp), static_cast<const char*>(kv_raw),
               sel, out, lse, n_q, q_pos0, n_comp, ratio, window, top_k, band};
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (nbuf) {
    case 2: return launch<2>(a, s);
    case 3: return launch<3>(a, s);
    case 4: return launch<4>(a, s);
    default: return -1;
  }
}

}  // extern "C"
