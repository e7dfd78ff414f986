// Streaming sparse MLA attention on CDNA4 (gfx950).
//
// Step described on the page "perf(ds4): extend sparse prefill scheduling to
// 10K" (Summary): each selected F16 latent row is read once and shared by
// the sixteen query heads, with an online softmax; the page "perf(ds4): unify
// gfx1151 sparse-prefill stack" (Validation completed) stages in FP32 and
// uses a fast exponential. Here: fp16 operands on matrix cores, fp32
// accumulation and softmax, exp2 with log2(e) folded into the scale.
//
// One workgroup (4 waves) per query token. Its key list is the selected
// compressed rows followed by the sliding-window raw rows. Keys are streamed
// in chunks of 64 rows (64 x 1152 B) that are gathered with direct
// global->LDS loads, so each row crosses the memory system once per query.
//
// Per chunk:
//   wave w: S^T[16 keys x 16 heads] = K[16w..16w+15] . Q^T  (18 MFMA 16x16x32;
//           K from LDS, Q^T held in registers for the whole query)
//   all   : exchange S^T through LDS; every wave runs the same online-softmax
//           update, so each lane owns one head and all of its rescaling is
//           lane-local
//   wave w: O^T[128 dims x 16 heads] += V^T . P^T  (16 MFMA; V^T read from
//           the row-major LDS tile with ds_read_b64_tr_b16 transpose loads,
//           P^T built in registers from the softmax)
// LDS rows are stored with a 16-byte-granular XOR swizzle that keeps both the
// K reads (16 rows x 16 B per pass) and the transposed V reads (8 rows x 32 B
// per pass) free of bank conflicts.
#include "spmla_internal.h"

namespace spmla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;                  // keys per chunk
constexpr int kRowBytes = kDqk * 2;         // 1152
constexpr int kRowUnits = kRowBytes / 16;   // 72 units of 16 B per row
constexpr int kKvBytes = kChunk * kRowBytes;
constexpr int kLoadsPerChunk = kKvBytes / 1024;  // 1 KB per wave-wide load
constexpr int kLoadsPerWave = kLoadsPerChunk / 4;
constexpr int kSStride = kChunk + 4;        // floats per head row of the S^T exchange
static_assert(kLoadsPerChunk % 4 == 0, "chunk must split evenly over 4 waves");

// XOR applied to the low 3 bits of a row's 16-byte unit index.
__device__ __forceinline__ int swz(int n) {
  return ((n >> 1) & 1) | ((((n >> 1) ^ (n >> 2)) & 1) << 1) | (((n ^ (n >> 3)) & 1) << 2);
}
// Byte offset of 16-byte unit u of LDS row n.
__device__ __forceinline__ int kv_off(int n, int u) { return n * kRowBytes + ((u ^ swz(n)) << 4); }

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(1))) const char gbl_char;

__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char kv[kKvBytes];
  __shared__ __attribute__((aligned(16))) float sbuf[kHeads * kSStride];

  const int r = blockIdx.x;
  const int t = a.q_pos0 + r;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // lane group: k-slice of MFMA operands
  const int c16 = lane & 15;  // MFMA row/column within a 16-wide tile

  const int nv = min(a.n_comp, (t + 1) / a.ratio);
  const int nsel = min(a.top_k, nv);
  const int ws = max(0, t - a.window + 1);
  const int nk = nsel + (t - ws + 1);
  const int nchunks = (nk + kChunk - 1) / kChunk;
  const int32_t* sel_row = a.sel + (int64_t)r * a.top_k;
  const char* comp_base = reinterpret_cast<const char*>(a.kv_comp);
  const char* raw_base = reinterpret_cast<const char*>(a.kv_raw);
  const char* self_row = raw_base + (int64_t)t * kRowBytes;  // always valid

  // Q^T fragments (B operand of S^T = K Q^T): head c16, dims 32s+8g .. +7.
  half8 qf[kDqk / 32];
  {
    const _Float16* qrow = a.q + ((int64_t)r * kHeads + c16) * kDqk + 8 * g;
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s) qf[s] = *reinterpret_cast<const half8*>(qrow + 32 * s);
  }

  float4v acc_o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc_o[nt] = float4v{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();  // running max (log2 domain) of head c16
  float l_run = 0.f;                // this lane's share of the softmax sum

  for (int ch = 0; ch < nchunks; ++ch) {
    const int k0 = ch * kChunk;
    // Row of key k0 + lane (lane-indexed; every wave computes the same).
    const int key = k0 + lane;
    const char* kp = self_row;
    bool ok = false;
    if (key < nsel) {
      const int s = sel_row[key];
      ok = (s >= 0) && (s < nv);
      if (ok) kp = comp_base + (int64_t)s * kRowBytes;
    } else if (key < nk) {
      ok = true;
      kp = raw_base + (int64_t)(ws + key - nsel) * kRowBytes;
    }
    const unsigned long long valid = __ballot(ok);
    const unsigned kp_lo = (unsigned)(uintptr_t)kp;
    const unsigned kp_hi = (unsigned)((uintptr_t)kp >> 32);

    // Gather: load q of this wave covers LDS bytes [q*1024, q*1024+1024),
    // i.e. 16-byte units P = q*64 + lane of the unswizzled row-major image.
#pragma unroll
    for (int m = 0; m < kLoadsPerWave; ++m) {
      const int q = wave * kLoadsPerWave + m;
      const int n0 = (q * 64) / kRowUnits;  // first row touched by this load
      const int P = q * 64 + lane;
      const int n = P / kRowUnits;
      const int p = P - n * kRowUnits;      // physical unit within row n
      const int u = p ^ swz(n);             // logical unit stored there
      const unsigned lo0 = __builtin_amdgcn_readlane(kp_lo, n0);
      const unsigned hi0 = __builtin_amdgcn_readlane(kp_hi, n0);
      const unsigned lo1 = __builtin_amdgcn_readlane(kp_lo, min(n0 + 1, kChunk - 1));
      const unsigned hi1 = __builtin_amdgcn_readlane(kp_hi, min(n0 + 1, kChunk - 1));
      const bool first = (n == n0);
      const uintptr_t rowp = ((uintptr_t)(first ? hi0 : hi1) << 32) | (first ? lo0 : lo1);
      const char* src = reinterpret_cast<const char*>(rowp) + (u << 4);
      __builtin_amdgcn_global_load_lds((gbl_char*)src, (lds_char*)(kv + q * 1024), 16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // S^T for keys 16*wave .. +15 of this chunk.
    float4v sacc = float4v{0.f, 0.f, 0.f, 0.f};
    {
      const int n = 16 * wave + c16;
#pragma unroll
      for (int s = 0; s < kDqk / 32; ++s) {
        const half8 kf = *reinterpret_cast<const half8*>(kv + kv_off(n, 4 * s + g));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[s], sacc, 0, 0, 0);
      }
    }
    // Lane holds S^T[key 16w + 4g + i][head c16]; scale and mask, then share.
    {
      float4v z;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 16 * wave + 4 * g + i;
        z[i] = ((valid >> kk) & 1ull) ? sacc[i] * a.scale_log2e : -__builtin_inff();
      }
      *reinterpret_cast<float4v*>(&sbuf[c16 * kSStride + 16 * wave + 4 * g]) = z;
    }
    __syncthreads();

    // Online softmax for head c16 over keys {32kb + 8g + i}.
    float zz[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4v lo = *reinterpret_cast<const float4v*>(&sbuf[c16 * kSStride + 32 * kb + 8 * g]);
      const float4v hi = *reinterpret_cast<const float4v*>(&sbuf[c16 * kSStride + 32 * kb + 8 * g + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zz[kb][i] = lo[i];
        zz[kb][4 + i] = hi[i];
      }
    }
    float cmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) cmax = fmaxf(cmax, zz[kb][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    half8 pf[2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(zz[kb][i] - m_use);
        psum += p;
        pf[kb][i] = (_Float16)p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc_o[nt] *= alpha;

    // O^T[dims 128w + 16nt + 4g + i][head c16] += V^T . P^T
    {
      const int tri = (lane >> 2) & 3;  // row within the 4-row transpose block
      const int trc = lane & 3;         // 4-column slice within 16 columns
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int dv0 = 128 * wave + 16 * nt;
        const int unit = (dv0 >> 3) + (trc >> 1);
        const int sub = (trc & 1) << 3;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int n_lo = 32 * kb + 8 * g + tri;
          const int n_hi = n_lo + 4;
          const short4v vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(kv + kv_off(n_lo, unit) + sub));
          const short4v vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(kv + kv_off(n_hi, unit) + sub));
          const half4 hlo = __builtin_bit_cast(half4, vlo);
          const half4 hhi = __builtin_bit_cast(half4, vhi);
          const half8 vf = half8{hlo[0], hlo[1], hlo[2], hlo[3], hhi[0], hhi[1], hhi[2], hhi[3]};
          acc_o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[kb], acc_o[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // kv and sbuf are overwritten by the next chunk
  }

  // Finish: total softmax sum of head c16 (same value in its 4 lanes).
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = l_tot + __shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  float* orow = a.out + ((int64_t)r * kHeads + c16) * kDv + 128 * wave + 4 * g;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    *reinterpret_cast<float4v*>(orow + 16 * nt) = acc_o[nt] * inv;
  }
  if (a.lse && wave == 0 && g == 0) {
    a.lse[(int64_t)r * kHeads + c16] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.n_q <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_kernel, dim3(a.n_q), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spmla
