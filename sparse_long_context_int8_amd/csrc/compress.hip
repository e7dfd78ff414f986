// Ratio-4 compression of raw latent rows on the GPU.
//
// Page "perf(ds4): extend sparse prefill scheduling to 10K", Summary: the
// indexer and attention read ratio-4 compressed rows kept in F16, and state
// is committed in chronological order. Compressed row j is the mean of raw
// rows 4j .. 4j+3, rounded once to fp16 (nearest, ties to even); only
// complete groups are built, so the newest n_raw mod 4 raw rows wait for
// their group to complete.
//
// Exactness: a finite fp16 value is an integer multiple of 2^-24 below 2^16,
// so four of them sum exactly in fp64 (and in a 64-bit integer counting
// units of 2^-24), and the mean is exact in fp64. The one rounding to fp16
// must come from that exact value: rounding it to float32 first can land on
// an fp16 tie and then round the wrong way. So the mean goes through float32
// only when float32 holds it exactly (the common case: nearby exponents);
// otherwise it is rounded from the integer sum. Zero results are -0 only
// when all four inputs are -0, and infinities / NaN follow IEEE addition.
//
// One thread per 8 dims of one compressed row: four 16-byte loads, one
// 16-byte store; HBM-bound (5 x 1,152 B per compressed row).
#include "spmla_internal.h"

namespace spmla {
namespace {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// Exact path: integer sum and round-to-nearest-even from its bits.
__device__ __noinline__ unsigned short mean4_fp16_exact(unsigned short h0, unsigned short h1, unsigned short h2,
                                                        unsigned short h3) {
  const unsigned short h[4] = {h0, h1, h2, h3};
  bool any_nan = false, pos_inf = false, neg_inf = false, all_neg_zero = true;
  long long sum = 0;  // units of 2^-24
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (h[i] >> 10) & 31;
    const int m = h[i] & 1023;
    const bool neg = h[i] >> 15;
    all_neg_zero &= h[i] == 0x8000;
    if (e == 31) {
      any_nan |= m != 0;
      pos_inf |= m == 0 && !neg;
      neg_inf |= m == 0 && neg;
      continue;
    }
    const long long mag = e == 0 ? (long long)m : (long long)(1024 + m) << (e - 1);
    sum += neg ? -mag : mag;
  }
  if (any_nan || (pos_inf && neg_inf)) return 0x7E00;
  if (pos_inf) return 0x7C00;
  if (neg_inf) return 0xFC00;
  if (sum == 0) return all_neg_zero ? 0x8000 : 0x0000;
  const unsigned short sign = sum < 0 ? 0x8000 : 0;
  const unsigned long long a = sum < 0 ? (unsigned long long)(-sum) : (unsigned long long)sum;
  // value = a * 2^-26. With p = bit length of a: normal numbers have p >= 13
  // (value >= 2^-14), exponent p - 27 and 11 significant bits a >> (p - 11);
  // subnormals are multiples of 2^-24, i.e. a >> 2.
  const int p = 64 - __clzll(a);
  const int shift = p <= 12 ? 2 : p - 11;
  unsigned long long q = a >> shift;
  const unsigned long long rem = a & ((1ull << shift) - 1);
  const unsigned long long half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (p <= 12) return sign | (unsigned short)q;  // q == 1024 encodes 2^-14
  int e = p - 12;                                 // biased exponent
  if (q == 2048) {
    q = 1024;
    ++e;
  }
  return sign | (unsigned short)(e << 10) | (unsigned short)(q - 1024);
}

__device__ __forceinline__ double h2d(unsigned short h) { return (double)(float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ unsigned short mean4_fp16(unsigned short h0, unsigned short h1, unsigned short h2,
                                                     unsigned short h3) {
  const double mean = (((h2d(h0) + h2d(h1)) + h2d(h2)) + h2d(h3)) * 0.25;  // exact
  const float f = (float)mean;
  if ((double)f == mean) return __builtin_bit_cast(unsigned short, (_Float16)f);  // the one rounding
  return mean4_fp16_exact(h0, h1, h2, h3);                                      // NaN, or not exact in f32
}

constexpr int kUnitsPerRow = kDqk / 8;  // 72 groups of 8 dims

__global__ __launch_bounds__(256) void compress_kernel(const unsigned short* __restrict__ raw,
                                                       unsigned short* __restrict__ comp, int comp_begin,
                                                       int n_new) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)n_new * kUnitsPerRow) return;
  const int64_t j = comp_begin + g / kUnitsPerRow;
  const int u = (int)(g % kUnitsPerRow);
  const u16x8* src = reinterpret_cast<const u16x8*>(raw + 4 * j * kDqk) + u;
  const u16x8 r0 = __builtin_nontemporal_load(src);
  const u16x8 r1 = __builtin_nontemporal_load(src + kUnitsPerRow);
  const u16x8 r2 = __builtin_nontemporal_load(src + 2 * kUnitsPerRow);
  const u16x8 r3 = __builtin_nontemporal_load(src + 3 * kUnitsPerRow);
  u16x8 o;
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = mean4_fp16(r0[d], r1[d], r2[d], r3[d]);
  reinterpret_cast<u16x8*>(comp + j * kDqk)[u] = o;
}

}  // namespace

hipError_t launch_compress(const uint16_t* kv_raw, uint16_t* kv_comp, int comp_begin, int n_comp,
                           hipStream_t stream) {
  const int n_new = n_comp - comp_begin;
  if (n_new <= 0) return hipSuccess;
  const int64_t items = (int64_t)n_new * kUnitsPerRow;
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const unsigned short*>(kv_raw), reinterpret_cast<unsigned short*>(kv_comp),
                     comp_begin, n_new);
  return hipGetLastError();
}

}  // namespace spmla
