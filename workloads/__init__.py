"""Seeded synthetic inputs for one sparse-MLA prefill layer.

This module is shared by the CPU oracle and the HIP path's tests and benchmark.
It only draws random numbers and lays them out; it performs no step of the
attention method (no scoring, visibility, selection or softmax).

Layer shape (DeepSeek-style MLA as described on the pages "perf(ds4): extend
sparse prefill scheduling to 10K", Summary, and "perf(ds4): unify gfx1151
sparse-prefill stack", Validation completed): 16 query heads sharing one
576-wide latent per key row (512 value dims + 64 rope dims), ratio-4
compressed rows scored by a small int8 indexer, a sliding window of raw rows,
and independent 2,048-token query bands.

Value recipe (the pages print no tensors, so all values are synthetic):
  latents X and queries Q  ~ N(0, 1) drawn in float32, stored as float16
  indexer queries / keys   int8 uniform in [-8, 7]
  indexer weights          int8 uniform in [1, 4], one per (token, indexer head)
  compressed rows C        float16 mean of each group of 4 consecutive raw
                           latents (exact fp64 sum, x0.25, one round to fp16);
                           this is input construction, not a step of the path.
Draw order from numpy.random.default_rng(seed): X, Q, iq, ik, iw.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes of one sparse-MLA prefill call.

    Queries are the absolute positions q_pos0 .. q_pos0 + n_q - 1; the raw
    latent history holds every row up to the last query (n_raw rows).
    """

    name: str
    n_q: int
    q_pos0: int
    window: int
    top_k: int
    ratio: int = 4
    band: int = 2048
    n_heads: int = 16
    d_qk: int = 576
    d_v: int = 512
    idx_heads: int = 4
    idx_dim: int = 64

    @property
    def n_raw(self) -> int:
        return self.q_pos0 + self.n_q

    @property
    def n_comp(self) -> int:
        # Every complete group of `ratio` raw rows has one compressed row; a
        # trailing partial group (n_raw mod ratio rows) is not yet compressed.
        return self.n_raw // self.ratio

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# The five workloads used for parity and timing.
TINY_256 = LayerShape("tiny-256", n_q=256, q_pos0=0, window=64, top_k=32)
BAND_2048 = LayerShape("band-2048", n_q=2048, q_pos0=0, window=128, top_k=512)
PREFILL_8192 = LayerShape("prefill-8192", n_q=8192, q_pos0=0, window=128, top_k=512)
PREFILL_9133 = LayerShape("prefill-9133", n_q=9133, q_pos0=0, window=128, top_k=512)
CHUNK_8192_AT_114687 = LayerShape(
    "chunk-8192-after-114687", n_q=8192, q_pos0=114687, window=128, top_k=2048
)

# Decode and speculative verification at the end of the same long history:
# 1 or 5 new query tokens (lanes) whose last position is 122,878, so the
# history is 122,879 raw rows and 30,719 compressed rows as above.
DECODE_1 = LayerShape("decode-1-at-122878", n_q=1, q_pos0=122878, window=128, top_k=2048)
VERIFY_5 = LayerShape("verify-5-at-122874", n_q=5, q_pos0=122874, window=128, top_k=2048)

# The five-band frontier: five full 2,048-token bands, 10,240 tokens.
PREFILL_10240 = LayerShape("prefill-10240", n_q=10240, q_pos0=0, window=128, top_k=512)

WORKLOADS = [TINY_256, BAND_2048, PREFILL_8192, PREFILL_9133, CHUNK_8192_AT_114687, DECODE_1, VERIFY_5,
             PREFILL_10240]
BY_NAME = {w.name: w for w in WORKLOADS}
# Seed of each named workload: its position in WORKLOADS.
SEEDS = {w.name: i for i, w in enumerate(WORKLOADS)}


def compress_mean_fp16(x: np.ndarray, ratio: int) -> np.ndarray:
    """Input construction: fp16 mean of each complete group of `ratio` rows."""
    n_comp = x.shape[0] // ratio
    groups = x[: n_comp * ratio].astype(np.float64).reshape(n_comp, ratio, x.shape[1])
    return (groups.sum(axis=1) * (1.0 / ratio)).astype(np.float16)


def generate(shape: LayerShape, seed: int | None = None) -> dict:
    """Draw every input of one prefill call (host numpy arrays, C-contiguous).

    Returns a dict with
      q       float16 [n_q, n_heads, d_qk]
      kv_raw  float16 [n_raw, d_qk]
      kv_comp float16 [n_comp, d_qk]
      iq      int8    [n_q, idx_heads, idx_dim]
      ik      int8    [n_comp, idx_dim]
      iw      int8    [n_q, idx_heads]
    """
    if seed is None:
        seed = SEEDS.get(shape.name, 0)
    rng = np.random.default_rng(seed)
    s = shape
    kv_raw = rng.standard_normal((s.n_raw, s.d_qk), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((s.n_q, s.n_heads, s.d_qk), dtype=np.float32).astype(np.float16)
    iq = rng.integers(-8, 8, (s.n_q, s.idx_heads, s.idx_dim)).astype(np.int8)
    ik = rng.integers(-8, 8, (s.n_comp, s.idx_dim)).astype(np.int8)
    iw = rng.integers(1, 5, (s.n_q, s.idx_heads)).astype(np.int8)
    kv_comp = compress_mean_fp16(kv_raw, s.ratio)
    return {
        "q": np.ascontiguousarray(q),
        "kv_raw": np.ascontiguousarray(kv_raw),
        "kv_comp": np.ascontiguousarray(kv_comp),
        "iq": np.ascontiguousarray(iq),
        "ik": np.ascontiguousarray(ik),
        "iw": np.ascontiguousarray(iw),
    }
