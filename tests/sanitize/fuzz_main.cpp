// Seeded descriptor fuzz of the library's host code, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against host stubs of the
// HIP runtime and the kernel launchers (hip_stubs.cpp).
//
// Each case draws a descriptor (mostly consistent, with edge values: zero
// and one query, band edges, the largest top-k and compressed-row counts,
// positions near the int32 limit, and broken fields), registers exactly the
// regions the C ABI documents for it at fake device addresses, and calls
// every entry point. Return codes must be documented ones; on success every
// launch the call makes must stay inside the registered regions (checked by
// the stubs), and spmla_prefill must reject a workspace one byte short.
//
// usage: fuzz <cases> <seed>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "spmla.h"
#include "stub_regions.h"

namespace {

unsigned long long g_state;
unsigned long long next_u64() {  // splitmix64
  unsigned long long z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int pick(const int* v, int n) { return v[next_u64() % (unsigned long long)n]; }
int uniform(int lo, int hi) { return lo + (int)(next_u64() % (unsigned long long)(hi - lo + 1)); }

void fail(const char* what, const spmla_desc& d, int rc) {
  std::fprintf(stderr,
               "FAIL %s rc=%d: n_q=%d q_pos0=%d n_raw=%d n_comp=%d ratio=%d window=%d top_k=%d band=%d (%s)\n",
               what, rc, d.n_q, d.q_pos0, d.n_raw, d.n_comp, d.ratio, d.window, d.top_k, d.band,
               spmla_last_error());
  std::abort();
}

bool documented(int rc) {
  return rc == SPMLA_OK || rc == SPMLA_EINVAL || rc == SPMLA_EUNSUPPORTED || rc == SPMLA_EWORKSPACE;
}

// Fake device arrays, 1 TiB apart (never dereferenced).
uintptr_t fake(int slot) { return (uintptr_t)(slot + 1) << 40; }

spmla_desc draw() {
  static const int nqs[] = {0, 1, 2, 5, 63, 255, 256, 257, 300, 511, 512, 513, 941, 2047, 2048, 2049, 8192, 9133,
                            10240, 20000};
  static const int pos[] = {0, 1, 3, 4, 6000, 14336, 114687, 122874, 130000, 131000};
  static const int ks[] = {1, 2, 7, 32, 100, 271, 512, 2048, 4095, 4096};
  static const int wins[] = {1, 2, 64, 128, 200, 100000};
  static const int bands[] = {1, 2, 37, 256, 300, 1000, 2048, 4096, 1 << 30};
  spmla_desc d;
  d.n_q = next_u64() % 4 ? pick(nqs, 20) : uniform(0, 12000);
  d.q_pos0 = next_u64() % 4 ? pick(pos, 10) : uniform(0, 131000);
  d.ratio = next_u64() % 8 ? 4 : uniform(1, 5);
  d.window = pick(wins, 6);
  d.top_k = next_u64() % 4 ? pick(ks, 10) : uniform(1, 4096);
  d.band = next_u64() % 4 ? pick(bands, 9) : uniform(1, 5000);
  d.n_raw = d.q_pos0 + d.n_q + (next_u64() % 8 == 0 ? uniform(0, 9) : 0);
  d.n_comp = d.n_raw / d.ratio;
  d.n_heads = 16;
  d.d_qk = 576;
  d.d_v = 512;
  d.idx_heads = 4;
  d.idx_dim = 64;
  d.scale = 1.0f / 24.0f;
  // Broken or extreme fields, one at a time.
  switch (next_u64() % 24) {
    case 0: d.n_q = -1 - uniform(0, 5); break;
    case 1: d.q_pos0 = INT_MAX - uniform(0, 3); break;
    case 2: d.n_comp += 1; break;
    case 3: d.n_raw = d.q_pos0 + d.n_q - 1; break;
    case 4: d.ratio = uniform(-2, 0); break;
    case 5: d.window = uniform(-2, 0); break;
    case 6: d.top_k = next_u64() % 2 ? 0 : 4097; break;
    case 7: d.band = uniform(-3, 0); break;
    case 8: d.n_heads = 8; break;
    case 9: d.d_v = 600; break;
    case 10: d.scale = next_u64() % 2 ? NAN : -1.0f; break;
    case 11: d.idx_dim = 32; break;
    case 12:  // the most compressed rows the kernels cover, and one more
      d.q_pos0 = 4 * 32768 - d.n_q + (int)(next_u64() % 2) * 4;
      d.n_raw = d.q_pos0 + d.n_q;
      d.n_comp = d.n_raw / d.ratio;
      break;
    case 13: d.n_raw = INT_MAX; d.n_comp = d.n_raw / (d.ratio > 0 ? d.ratio : 1); break;
    default: break;
  }
  return d;
}

struct Arrays {
  const uint16_t *q, *kv_comp, *kv_raw;
  const int8_t *iq, *iw, *ik;
  int32_t *scores, *sel, *n_sel;
  float *out, *lse;
};

// Registers the documented extents of every argument of descriptor d.
Arrays register_arrays(const spmla_desc& d) {
  stub::clear();
  Arrays a;
  const size_t nq = d.n_q > 0 ? (size_t)d.n_q : 0, nc = d.n_comp > 0 ? (size_t)d.n_comp : 0;
  const size_t nr = d.n_raw > 0 ? (size_t)d.n_raw : 0, k = d.top_k > 0 ? (size_t)d.top_k : 0;
  a.q = (const uint16_t*)fake(0);
  stub::add("q", a.q, nq * 16 * 576 * 2);
  a.kv_comp = (const uint16_t*)fake(1);
  stub::add("kv_comp", a.kv_comp, nc * 576 * 2);
  a.kv_raw = (const uint16_t*)fake(2);
  stub::add("kv_raw", a.kv_raw, nr * 576 * 2);
  a.iq = (const int8_t*)fake(3);
  stub::add("iq", a.iq, nq * 4 * 64);
  a.iw = (const int8_t*)fake(4);
  stub::add("iw", a.iw, nq * 4);
  a.ik = (const int8_t*)fake(5);
  stub::add("ik", a.ik, nc * 64);
  a.scores = (int32_t*)fake(6);
  stub::add("scores", a.scores, nq * nc * 4);
  a.sel = (int32_t*)fake(7);
  stub::add("sel", a.sel, nq * k * 4);
  a.n_sel = (int32_t*)fake(8);
  stub::add("n_sel", a.n_sel, nq * 4);
  a.out = (float*)fake(9);
  stub::add("out", a.out, nq * 16 * 512 * 4);
  a.lse = (float*)fake(10);
  stub::add("lse", a.lse, nq * 16 * 4);
  return a;
}

void run_case(const spmla_desc& d) {
  const Arrays a = register_arrays(d);
  void* st = nullptr;
  int rc = spmla_check_desc(&d);
  if (!documented(rc)) fail("check_desc", d, rc);
  const int desc_rc = rc;
  rc = spmla_num_bands(&d);
  if (desc_rc == 0 && rc != (int)(((long long)d.n_q + d.band - 1) / d.band)) fail("num_bands", d, rc);
  if (desc_rc != 0 && rc != desc_rc) fail("num_bands code", d, rc);

  rc = spmla_indexer_scores(&d, a.iq, a.iw, a.ik, a.scores, st);
  if (rc != desc_rc) fail("indexer_scores", d, rc);
  rc = spmla_topk(&d, a.scores, a.sel, a.n_sel, st);
  if (rc != desc_rc) fail("topk", d, rc);
  rc = spmla_sparse_attn(&d, a.q, a.kv_comp, a.kv_raw, a.sel, a.out, a.lse, st);
  if (rc != desc_rc) fail("sparse_attn", d, rc);
  rc = spmla_sparse_attn_grouped(&d, a.q, a.kv_comp, a.kv_raw, a.sel, a.out, nullptr, st);
  if (rc != desc_rc) fail("sparse_attn_grouped", d, rc);
  if (desc_rc == 0 && d.n_comp > 0) {
    const int begin = uniform(0, d.n_comp);
    rc = spmla_compress(&d, a.kv_raw, (uint16_t*)a.kv_comp, begin, st);
    if (rc != (d.ratio == 4 ? 0 : SPMLA_EUNSUPPORTED)) fail("compress", d, rc);
  }

  size_t ws_bytes = 0;
  rc = spmla_prefill_workspace_bytes(&d, &ws_bytes);
  if (rc != desc_rc) fail("workspace_bytes", d, rc);
  if (desc_rc == 0) {
    void* ws = (void*)fake(11);
    stub::add("workspace", ws, ws_bytes);
    int32_t* sel_out = next_u64() % 2 ? a.sel : nullptr;
    float* lse = next_u64() % 2 ? a.lse : nullptr;
    rc = spmla_prefill(&d, a.q, a.kv_comp, a.kv_raw, a.iq, a.iw, a.ik, a.out, lse, sel_out, ws, ws_bytes, st);
    if (rc != 0) fail("prefill", d, rc);
    if (d.n_q > 0 && ws_bytes > 0) {
      rc = spmla_prefill(&d, a.q, a.kv_comp, a.kv_raw, a.iq, a.iw, a.ik, a.out, lse, sel_out, ws, ws_bytes - 1,
                         st);
      if (rc != SPMLA_EWORKSPACE) fail("prefill short workspace", d, rc);
    }
    stub::add("no-alloc scratch", (void*)stub::kScratchBase, (size_t)64 << 20);
    rc = spmla_prefill_noalloc(&d, a.q, a.kv_comp, a.kv_raw, a.iq, a.iw, a.ik, a.out, lse, sel_out, st);
    if (rc != 0) fail("prefill_noalloc", d, rc);
  } else {
    rc = spmla_prefill(&d, a.q, a.kv_comp, a.kv_raw, a.iq, a.iw, a.ik, a.out, a.lse, a.sel, (void*)fake(11),
                       (size_t)1 << 40, st);
    if (rc != desc_rc) fail("prefill (bad desc)", d, rc);
    rc = spmla_prefill_noalloc(&d, a.q, a.kv_comp, a.kv_raw, a.iq, a.iw, a.ik, a.out, a.lse, a.sel, st);
    if (rc != desc_rc) fail("prefill_noalloc (bad desc)", d, rc);
  }
  // A misaligned or missing pointer is refused before any launch.
  if (desc_rc == 0 && d.n_q > 0) {
    const long before = stub::g_launches;
    rc = spmla_sparse_attn(&d, (const uint16_t*)((uintptr_t)a.q + 2), a.kv_comp, a.kv_raw, a.sel, a.out, a.lse, st);
    if (rc != SPMLA_EINVAL) fail("misaligned q", d, rc);
    rc = spmla_prefill(&d, a.q, a.kv_comp, a.kv_raw, nullptr, a.iw, a.ik, a.out, a.lse, a.sel, (void*)fake(11),
                       (size_t)1 << 40, st);
    if (rc != SPMLA_EINVAL) fail("null iq", d, rc);
    if (stub::g_launches != before) fail("launch after a refused call", d, rc);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long cases = argc > 1 ? std::atol(argv[1]) : 2000;
  g_state = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1;
  long ok = 0;
  for (long i = 0; i < cases; ++i) {
    const spmla_desc d = draw();
    run_case(d);
    ok += spmla_check_desc(&d) == 0;
  }
  std::printf("fuzz: %ld cases, %ld valid descriptors, %ld stub launches checked\n", cases, ok, stub::g_launches);
  return 0;
}
