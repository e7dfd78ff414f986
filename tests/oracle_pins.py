"""Checks that tie the CPU oracle to facts outside itself.

Each pin takes the oracle module as its argument so that the same checks can
be run against copies of the oracle with a planted mistake (see
test_oracle_mutants.py): every plausible slip must fail at least one pin.

Pins come from: values the pages print (tests/golden/*.json), brute force
written from the definitions with plain Python loops, closed forms, library
routines (torch's scaled_dot_product_attention, numpy integer matmul) for
special cases, and invariants of a top-k.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_inputs(rng, *, n_q, q_pos0, ratio, H, D, Hi, Di, value_range=8):
    n_raw = q_pos0 + n_q
    n_comp = n_raw // ratio
    kv_raw = rng.standard_normal((n_raw, D)).astype(np.float16)
    groups = kv_raw[: n_comp * ratio].astype(np.float64).reshape(n_comp, ratio, D)
    kv_comp = (groups.mean(axis=1)).astype(np.float16)
    return {
        "q": rng.standard_normal((n_q, H, D)).astype(np.float16),
        "kv_raw": kv_raw,
        "kv_comp": kv_comp,
        "iq": rng.integers(-value_range, value_range, (n_q, Hi, Di)).astype(np.int8),
        "ik": rng.integers(-value_range, value_range, (n_comp, Di)).astype(np.int8),
        "iw": rng.integers(1, 5, (n_q, Hi)).astype(np.int8),
    }


# ------------------------------------------------------------ visibility pins
def pin_visibility_brute_force(orc):
    """Explicit mask from the definition of a compressed row == analytic form.

    A compressed row j stands for raw rows ratio*j .. ratio*j+ratio-1; it
    exists once all of them exist and is visible to query t once all of them
    are at or before t (the explicit-mask versus analytic-mask check named on
    "perf(ds4): extend sparse prefill scheduling to 10K", Qualification).
    """
    for ratio in (1, 2, 3, 4, 5):
        for n_raw in range(0, 41):
            groups = []
            j = 0
            while True:
                members = [ratio * j + m for m in range(ratio)]
                if not all(x < n_raw for x in members):
                    break
                groups.append(members)
                j += 1
            assert orc.n_compressed(n_raw, ratio) == len(groups), (ratio, n_raw)
            for t in range(n_raw):
                explicit = [all(x <= t for x in g) for g in groups]
                nv = orc.n_visible(t, len(groups), ratio)
                assert explicit == [True] * nv + [False] * (len(groups) - nv), (ratio, n_raw, t)


def pin_window_brute_force(orc):
    """Window = the W most recent raw rows up to and including t."""
    for W in (1, 2, 3, 7, 64):
        for t in range(0, 80):
            rows = [s for s in range(t + 1) if t - s < W]
            lo, hi = orc.window_range(t, W)
            assert list(range(lo, hi)) == rows, (W, t)


def pin_mask_memory(orc):
    """The printed GiB of removed fp32 masks match T x (T + floor(T/4)) keys."""
    g = _golden("mask_memory.json")
    for case in g["cases"]:
        T = case["tokens"]
        keys = T + orc.n_compressed(T, g["ratio"])
        gib = g["layers"] * T * keys * 4 / 2**30
        assert abs(gib - case["gib_printed"]) <= 0.0005 + 1e-12, (T, gib)


# --------------------------------------------------------------- indexer pins
def _indexer_brute(iq, iw, ik, q_pos0, ratio):
    T, Hi, Di = iq.shape
    Nc = ik.shape[0]
    out = [[None] * Nc for _ in range(T)]
    for r in range(T):
        t = q_pos0 + r
        for j in range(Nc):
            if not all(ratio * j + m <= t for m in range(ratio)):
                out[r][j] = -(2**31)
                continue
            total = 0
            for h in range(Hi):
                dot = 0
                for d in range(Di):
                    dot += int(iq[r, h, d]) * int(ik[j, d])
                total += int(iw[r, h]) * (dot if dot > 0 else 0)
            out[r][j] = total
    return np.array(out, dtype=np.int64)


def pin_indexer_brute_force(orc):
    rng = np.random.default_rng(11)
    for (n_q, q_pos0, Hi, Di, ratio) in ((9, 0, 4, 64, 4), (7, 13, 3, 8, 4), (6, 5, 2, 5, 2)):
        inp = _tiny_inputs(rng, n_q=n_q, q_pos0=q_pos0, ratio=ratio, H=1, D=4, Hi=Hi, Di=Di)
        got = orc.indexer_scores(inp["iq"], inp["iw"], inp["ik"], q_pos0, ratio)
        want = _indexer_brute(inp["iq"], inp["iw"], inp["ik"], q_pos0, ratio)
        assert got.dtype == np.int32
        np.testing.assert_array_equal(got.astype(np.int64), want)
    # the whole int8 range, negative weights and the extreme dot products
    # (+-64*128*128 = +-2^20 per head, weighted sums up to 2^29) stay exact
    inp = _tiny_inputs(rng, n_q=8, q_pos0=40, ratio=4, H=1, D=4, Hi=4, Di=64, value_range=128)
    inp["iw"] = rng.integers(-128, 128, inp["iw"].shape).astype(np.int8)
    inp["iq"][0] = -128
    inp["ik"][0] = -128
    inp["iw"][0] = -128
    inp["iw"][1] = 127
    inp["iq"][1] = 127
    inp["ik"][1] = -128
    got = orc.indexer_scores(inp["iq"], inp["iw"], inp["ik"], 40, 4)
    want = _indexer_brute(inp["iq"], inp["iw"], inp["ik"], 40, 4)
    assert want[0, 0] == -128 * 4 * 64 * 128 * 128
    np.testing.assert_array_equal(got.astype(np.int64), want)


def pin_indexer_closed_forms(orc):
    """Special cases with a known answer.

    * all inputs >= 0: the ReLU never clips, so S = (sum_h w_h q_h) . k, an
      integer matmul;
    * q >= 0, k <= 0: every head dot is <= 0, so every visible score is 0;
    * weights that select one head: S = ReLU(q_h . k) for that head;
    * the extreme q = k = -8, w = 4 over 4 x 64 gives 4*4*64*64 = 65536.
    """
    rng = np.random.default_rng(12)
    T, Hi, Di, Nc, ratio, p0 = 12, 4, 64, 20, 4, 70
    iq = rng.integers(0, 8, (T, Hi, Di)).astype(np.int8)
    ik = rng.integers(0, 8, (Nc, Di)).astype(np.int8)
    iw = rng.integers(1, 5, (T, Hi)).astype(np.int8)
    got = orc.indexer_scores(iq, iw, ik, p0, ratio).astype(np.int64)
    comb = np.einsum("th,thd->td", iw.astype(np.int64), iq.astype(np.int64))
    want = comb @ ik.astype(np.int64).T
    for r in range(T):
        nv = min(Nc, (p0 + r + 1) // ratio)
        np.testing.assert_array_equal(got[r, :nv], want[r, :nv])
        assert (got[r, nv:] == -(2**31)).all()

    neg_k = (-ik).astype(np.int8)
    got0 = orc.indexer_scores(iq, iw, neg_k, p0, ratio)
    for r in range(T):
        nv = min(Nc, (p0 + r + 1) // ratio)
        assert (got0[r, :nv] == 0).all()

    iq2 = rng.integers(-8, 8, (T, Hi, Di)).astype(np.int8)
    ik2 = rng.integers(-8, 8, (Nc, Di)).astype(np.int8)
    for h0 in range(Hi):
        w = np.zeros((T, Hi), np.int8)
        w[:, h0] = 1
        got1 = orc.indexer_scores(iq2, w, ik2, p0, ratio).astype(np.int64)
        dots = iq2[:, h0, :].astype(np.int64) @ ik2.astype(np.int64).T
        for r in range(T):
            nv = min(Nc, (p0 + r + 1) // ratio)
            np.testing.assert_array_equal(got1[r, :nv], np.maximum(dots[r, :nv], 0))

    iq3 = np.full((1, 4, 64), -8, np.int8)
    ik3 = np.full((1, 64), -8, np.int8)
    iw3 = np.full((1, 4), 4, np.int8)
    assert int(orc.indexer_scores(iq3, iw3, ik3, 3, 4)[0, 0]) == 65536


# ----------------------------------------------------------------- top-k pins
def pin_topk_brute_force(orc):
    rng = np.random.default_rng(13)
    for trial in range(40):
        Nc = int(rng.integers(0, 40))
        T = 6
        p0 = int(rng.integers(0, 4 * Nc + 8))
        k = int(rng.integers(1, 12))
        hi = int(rng.integers(1, 6))  # few distinct values: many ties
        sc = rng.integers(0, hi, (T, Nc)).astype(np.int32)
        sel, n_sel = orc.topk_select(sc, p0, 4, k, Nc)
        for r in range(T):
            nv = min(Nc, (p0 + r + 1) // 4)
            want = sorted(range(nv), key=lambda j: (-int(sc[r, j]), j))[:k]
            assert n_sel[r] == len(want)
            assert list(sel[r, : len(want)]) == want, (trial, r)
            assert (sel[r, len(want):] == -1).all()


def pin_topk_closed_forms(orc):
    Nc, k = 50, 16
    t_last = 4 * Nc - 1  # every row visible
    flat = np.full((1, Nc), 7, np.int32)
    sel, n = orc.topk_select(flat, t_last, 4, k, Nc)
    assert list(sel[0]) == list(range(k))  # all tied: lowest indices, ascending
    inc = np.arange(Nc, dtype=np.int32)[None]
    sel, n = orc.topk_select(inc, t_last, 4, k, Nc)
    assert list(sel[0]) == list(range(Nc - 1, Nc - 1 - k, -1))
    dec = (1000 - np.arange(Nc, dtype=np.int32))[None]
    sel, n = orc.topk_select(dec, t_last, 4, k, Nc)
    assert list(sel[0]) == list(range(k))
    # fewer visible rows than k: all of them, padded with -1
    sel, n = orc.topk_select(inc, 4 * 5 - 1, 4, k, Nc)
    assert n[0] == 5 and list(sel[0, :5]) == [4, 3, 2, 1, 0] and (sel[0, 5:] == -1).all()
    # query 0..2 sees no compressed row at all
    sel, n = orc.topk_select(inc, 2, 4, k, Nc)
    assert n[0] == 0 and (sel[0] == -1).all()


def pin_topk_invariants(orc):
    """On a tiny-256-like workload: size, order, boundary and tie rules."""
    rng = np.random.default_rng(14)
    inp = _tiny_inputs(rng, n_q=256, q_pos0=0, ratio=4, H=1, D=4, Hi=4, Di=64)
    sc = orc.indexer_scores(inp["iq"], inp["iw"], inp["ik"], 0, 4)
    k = 32
    sel, n_sel = orc.topk_select(sc, 0, 4, k, 64)
    for r in range(256):
        nv = min(64, (r + 1) // 4)
        n = int(n_sel[r])
        assert n == min(k, nv)
        chosen = [int(x) for x in sel[r, :n]]
        assert len(set(chosen)) == n and all(0 <= j < nv for j in chosen)
        s = [int(sc[r, j]) for j in chosen]
        for a in range(n - 1):
            assert s[a] > s[a + 1] or (s[a] == s[a + 1] and chosen[a] < chosen[a + 1])
        rest = [j for j in range(nv) if j not in set(chosen)]
        if rest and chosen:
            assert max(int(sc[r, j]) for j in rest) <= s[-1]
            ties_out = [j for j in rest if int(sc[r, j]) == s[-1]]
            ties_in = [j for j in chosen if int(sc[r, j]) == s[-1]]
            assert not ties_out or min(ties_out) > max(ties_in)


# ------------------------------------------------------------- attention pins
def _attn_brute(q, kv_comp, kv_raw, sel, n_sel, q_pos0, W, scale, d_v):
    T, H, D = q.shape
    out = np.zeros((T, H, d_v))
    lse = np.zeros((T, H))
    for r in range(T):
        t = q_pos0 + r
        keys = [kv_comp[int(sel[r, i])] for i in range(int(n_sel[r]))]
        keys += [kv_raw[s] for s in range(t + 1) if t - s < W]
        for h in range(H):
            z = []
            for key in keys:
                z.append(scale * sum(float(q[r, h, d]) * float(key[d]) for d in range(D)))
            m = max(z)
            e = [math.exp(v - m) for v in z]
            den = sum(e)
            for c in range(d_v):
                out[r, h, c] = sum(e[i] * float(keys[i][c]) for i in range(len(keys))) / den
            lse[r, h] = m + math.log(den)
    return out, lse


def pin_attention_brute_force(orc):
    rng = np.random.default_rng(15)
    for (n_q, q_pos0, ratio, W, k, H, D, d_v) in ((10, 0, 2, 3, 2, 2, 6, 4), (6, 9, 4, 4, 3, 3, 5, 3)):
        inp = _tiny_inputs(rng, n_q=n_q, q_pos0=q_pos0, ratio=ratio, H=H, D=D, Hi=2, Di=4)
        nc = inp["kv_comp"].shape[0]
        sc = orc.indexer_scores(inp["iq"], inp["iw"], inp["ik"], q_pos0, ratio)
        sel, n_sel = orc.topk_select(sc, q_pos0, ratio, k, nc)
        scale = 1.0 / math.sqrt(D)
        got_o, got_l = orc.sparse_attention(inp["q"], inp["kv_comp"], inp["kv_raw"], sel, n_sel,
                                            q_pos0, W, scale, d_v)
        want_o, want_l = _attn_brute(inp["q"], inp["kv_comp"], inp["kv_raw"], sel, n_sel,
                                     q_pos0, W, scale, d_v)
        np.testing.assert_allclose(got_o, want_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(got_l, want_l, rtol=0, atol=1e-12)


def pin_attention_closed_forms(orc):
    """Closed forms of softmax attention.

    * query 0 sees exactly one key (its own raw row): out = that row's value
      dims and lse = scale * q.key;
    * q = 0: every logit is 0, out = mean of the key set's values, lse = log n;
    * all rows identical: out = that row's values;
    * a value column fixed to 1 returns 1 (the weights sum to one);
    * two keys (e, 0) against q = a*e: weight of the first is a logistic.
    """
    rng = np.random.default_rng(16)
    D, d_v, H, W, k, ratio = 8, 6, 3, 4, 3, 2
    inp = _tiny_inputs(rng, n_q=12, q_pos0=0, ratio=ratio, H=H, D=D, Hi=2, Di=4)
    nc = inp["kv_comp"].shape[0]
    sc = orc.indexer_scores(inp["iq"], inp["iw"], inp["ik"], 0, ratio)
    sel, n_sel = orc.topk_select(sc, 0, ratio, k, nc)
    scale = 0.37
    out, lse = orc.sparse_attention(inp["q"], inp["kv_comp"], inp["kv_raw"], sel, n_sel, 0, W,
                                    scale, d_v)
    x0 = inp["kv_raw"][0].astype(np.float64)
    np.testing.assert_array_equal(out[0], np.broadcast_to(x0[:d_v], (H, d_v)))
    np.testing.assert_allclose(lse[0], scale * (inp["q"][0].astype(np.float64) @ x0), atol=1e-12)

    qz = np.zeros_like(inp["q"])
    out, lse = orc.sparse_attention(qz, inp["kv_comp"], inp["kv_raw"], sel, n_sel, 0, W, scale, d_v)
    for r in range(12):
        keys = [inp["kv_comp"][int(sel[r, i])] for i in range(int(n_sel[r]))]
        keys += [inp["kv_raw"][s] for s in range(max(0, r - W + 1), r + 1)]
        mean = np.mean(np.array(keys, dtype=np.float64)[:, :d_v], axis=0)
        np.testing.assert_allclose(out[r], np.broadcast_to(mean, (H, d_v)), atol=1e-12)
        np.testing.assert_allclose(lse[r], math.log(len(keys)), atol=1e-12)

    v = rng.standard_normal(D).astype(np.float16)
    same_raw = np.broadcast_to(v, inp["kv_raw"].shape).copy()
    same_comp = np.broadcast_to(v, inp["kv_comp"].shape).copy()
    out, _ = orc.sparse_attention(inp["q"], same_comp, same_raw, sel, n_sel, 0, W, scale, d_v)
    np.testing.assert_allclose(out, np.broadcast_to(v[:d_v].astype(np.float64), out.shape),
                               atol=1e-12)

    ones_raw = inp["kv_raw"].copy()
    ones_comp = inp["kv_comp"].copy()
    ones_raw[:, 2] = 1.0
    ones_comp[:, 2] = 1.0
    out, _ = orc.sparse_attention(inp["q"], ones_comp, ones_raw, sel, n_sel, 0, W, scale, d_v)
    np.testing.assert_allclose(out[:, :, 2], 1.0, atol=1e-12)

    a = 1.75  # exact in fp16
    q2 = np.zeros((2, 1, D), np.float16)
    q2[1, 0, 0] = a
    raw2 = np.zeros((2, D), np.float16)
    raw2[0, 0] = 1.0  # key 0 = e0, key 1 = 0; both in query 1's window
    comp2 = np.zeros((0, D), np.float16)
    sel2 = np.full((2, 1), -1, np.int32)
    out, lse = orc.sparse_attention(q2, comp2, raw2, sel2, np.zeros(2, np.int32), 0, 2, scale, D)
    w0 = 1.0 / (1.0 + math.exp(-scale * a))
    np.testing.assert_allclose(out[1, 0, 0], w0, atol=1e-12)
    np.testing.assert_allclose(lse[1, 0], math.log(math.exp(scale * a) + 1.0), atol=1e-12)


def pin_sparse_equals_dense_sdpa(orc):
    """When k covers every visible compressed row, the sparse layer equals
    dense causal attention over [compressed ; raw] keys with an explicit
    boolean mask, computed by torch's scaled_dot_product_attention in fp64."""
    import torch

    rng = np.random.default_rng(17)
    n_q, q_pos0, ratio, W, H, D, d_v = 24, 9, 4, 5, 4, 16, 12
    inp = _tiny_inputs(rng, n_q=n_q, q_pos0=q_pos0, ratio=ratio, H=H, D=D, Hi=4, Di=8)
    nc = inp["kv_comp"].shape[0]
    k = nc  # covers every visible row
    sc = orc.indexer_scores(inp["iq"], inp["iw"], inp["ik"], q_pos0, ratio)
    sel, n_sel = orc.topk_select(sc, q_pos0, ratio, k, nc)
    scale = 1.0 / math.sqrt(D)
    got, _ = orc.sparse_attention(inp["q"], inp["kv_comp"], inp["kv_raw"], sel, n_sel, q_pos0, W,
                                  scale, d_v)
    n_raw = inp["kv_raw"].shape[0]
    keys = np.concatenate([inp["kv_comp"], inp["kv_raw"]]).astype(np.float64)
    mask = np.zeros((n_q, nc + n_raw), dtype=bool)
    for r in range(n_q):
        t = q_pos0 + r
        for j in range(nc):
            mask[r, j] = all(ratio * j + m <= t for m in range(ratio))
        for s in range(n_raw):
            mask[r, nc + s] = s <= t and t - s < W
    qt = torch.from_numpy(inp["q"].astype(np.float64)).permute(1, 0, 2).contiguous()  # [H, T, D]
    kt = torch.from_numpy(keys)[None].expand(H, -1, -1).contiguous()
    vt = torch.from_numpy(keys[:, :d_v].copy())[None].expand(H, -1, -1).contiguous()
    mt = torch.from_numpy(mask)[None].expand(H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    ref = ref.permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_band_independence(orc):
    """Each band run as its own call (its own q_pos0, history cut at the band's
    last query) gives the same result as one call over all queries: bands
    only schedule work ("perf(ds4): extend sparse prefill scheduling to 10K",
    Summary: independent 2K attention bands), and rows after the last query
    cannot matter (causality)."""
    rng = np.random.default_rng(18)
    n_q, q_pos0, ratio, band = 40, 6, 4, 16
    inp = _tiny_inputs(rng, n_q=n_q, q_pos0=q_pos0, ratio=ratio, H=2, D=8, Hi=4, Di=16)
    kw = dict(ratio=ratio, window=5, top_k=3, scale=0.3, d_v=6)
    full = orc.prefill(inp, q_pos0=q_pos0, **kw)
    parts = []
    for a in range(0, n_q, band):
        b = min(n_q, a + band)
        n_raw_b = q_pos0 + b
        nc_b = n_raw_b // ratio
        sub = {
            "q": inp["q"][a:b], "iq": inp["iq"][a:b], "iw": inp["iw"][a:b],
            "kv_raw": inp["kv_raw"][:n_raw_b], "kv_comp": inp["kv_comp"][:nc_b],
            "ik": inp["ik"][:nc_b],
        }
        parts.append(orc.prefill(sub, q_pos0=q_pos0 + a, chunk=5, **kw))
    for key in ("sel", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(full[key], np.concatenate([p[key] for p in parts]))


def _prefill_brute(inp, q_pos0, ratio, window, top_k, scale, d_v):
    """One whole layer from the definitions, in plain Python loops: visible
    compressed rows from their raw members, integer indexer scores, a
    sorted() top-k, and a math.exp softmax over the selected compressed rows
    followed by the window's raw rows. Returns (sel, out, lse) lists."""
    q, kv_comp, kv_raw = inp["q"], inp["kv_comp"], inp["kv_raw"]
    iq, iw, ik = inp["iq"], inp["iw"], inp["ik"]
    T, H, D = q.shape
    Hi, Di = iq.shape[1], iq.shape[2]
    sels, outs, lses = [], [], []
    for r in range(T):
        t = q_pos0 + r
        vis = [j for j in range(kv_comp.shape[0]) if all(ratio * j + m <= t for m in range(ratio))]
        score = {}
        for j in vis:
            total = 0
            for h in range(Hi):
                dot = sum(int(iq[r, h, d]) * int(ik[j, d]) for d in range(Di))
                total += int(iw[r, h]) * max(dot, 0)
            score[j] = total
        chosen = sorted(vis, key=lambda j: (-score[j], j))[:top_k]
        sels.append(chosen + [-1] * (top_k - len(chosen)))
        keys = [kv_comp[j] for j in chosen] + [kv_raw[s] for s in range(t + 1) if t - s < window]
        o_t, l_t = [], []
        for h in range(H):
            z = [scale * sum(float(q[r, h, d]) * float(key[d]) for d in range(D)) for key in keys]
            m = max(z)
            e = [math.exp(v - m) for v in z]
            den = sum(e)
            o_t.append([sum(e[i] * float(keys[i][c]) for i in range(len(keys))) / den for c in range(d_v)])
            l_t.append(m + math.log(den))
        outs.append(o_t)
        lses.append(l_t)
    return sels, outs, lses


def pin_prefill_end_to_end(orc):
    """The oracle's whole-layer entry point (the one the GPU path is compared
    with) against the plain-Python layer above: indexer, top-k and attention
    composed with the right arguments and query offsets, over several
    chunks of a call that starts mid-sequence, and over a sub-range of its
    queries. Window and top-k differ, so passing one for the other fails."""
    rng = np.random.default_rng(19)
    n_q, q_pos0, ratio = 13, 7, 4
    inp = _tiny_inputs(rng, n_q=n_q, q_pos0=q_pos0, ratio=ratio, H=2, D=6, Hi=3, Di=5)
    kw = dict(ratio=ratio, window=3, top_k=2, scale=0.41, d_v=4)
    sels, outs, lses = _prefill_brute(inp, q_pos0, **kw)
    full = orc.prefill(inp, q_pos0=q_pos0, chunk=5, **kw)
    np.testing.assert_array_equal(full["sel"], np.array(sels, dtype=np.int64))
    np.testing.assert_array_equal(full["n_sel"], [sum(1 for j in s if j >= 0) for s in sels])
    np.testing.assert_allclose(full["out"], np.array(outs), rtol=0, atol=1e-12)
    np.testing.assert_allclose(full["lse"], np.array(lses), rtol=0, atol=1e-12)
    part = orc.prefill(inp, q_pos0=q_pos0, q_begin=4, q_end=11, chunk=3, **kw)
    np.testing.assert_array_equal(part["sel"], np.array(sels[4:11], dtype=np.int64))
    np.testing.assert_allclose(part["out"], np.array(outs[4:11]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(part["lse"], np.array(lses[4:11]), rtol=0, atol=1e-12)


# ------------------------------------------------------ compression pins
def _fp16_bits_exact(v):
    """IEEE binary16 bits of the exact rational v rounded to nearest, ties
    to even (from the format's definition; v is finite and |v| <= 65504)."""
    from fractions import Fraction

    def rne(x):
        fl = x.numerator // x.denominator
        d = x - fl
        if d > Fraction(1, 2):
            return fl + 1
        if d < Fraction(1, 2):
            return fl
        return fl + (fl & 1)

    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = 0
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    if e < -14:  # subnormal: multiples of 2^-24
        m = rne(a * 2 ** 24)
        return sign | m  # m == 1024 is the smallest normal's encoding
    m = rne(a * Fraction(2) ** (10 - e))
    if m == 2048:
        m, e = 1024, e + 1
    return sign | ((e + 15) << 10) | (m - 1024)


def _fp16_value(bits):
    from fractions import Fraction

    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 31
    m = bits & 1023
    if e == 0:
        return s * Fraction(m, 2 ** 24)
    return s * Fraction(1024 + m, 2 ** 10) * Fraction(2) ** (e - 15)


def pin_compress_exact_rounding(orc):
    """Brute force: exact rational mean of each group, rounded by the format's
    definition, on values that hit subnormals, ties and wide exponent spans."""
    rng = np.random.default_rng(21)
    n_raw, D = 4 * 9 + 3, 24  # 9 complete groups and a 3-row tail
    bits = rng.integers(0, 0x7C00, (n_raw, D)).astype(np.uint16)  # finite
    bits[rng.random((n_raw, D)) < 0.5] |= 0x8000
    bits[:4, :4] = [[0x3C00, 0x1000, 0x0001, 0x0000]] * 4  # spans 2^0 .. 2^-24
    bits[4:8, 0] = [0x0001, 0x0001, 0x0000, 0x0000]  # 2^-25: tie at zero -> +0
    bits[4:8, 1] = [0x0001, 0x0001, 0x0001, 0x0000]  # 3 * 2^-26 -> 2^-24
    bits[4:8, 2] = [0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF]  # largest finite
    bits[4:8, 3] = [0x8000, 0x8000, 0x8000, 0x8000]  # all -0 -> -0
    bits[4:8, 4] = [0x3C00, 0xBC00, 0x8000, 0x8000]  # exact cancellation -> +0
    x = bits.view(np.float16)
    got = orc.compress_rows(x, 4).view(np.uint16)
    assert got.shape == (9, D)
    for j in range(9):
        for d in range(D):
            mean = sum(_fp16_value(int(bits[4 * j + i, d])) for i in range(4)) / 4
            want = _fp16_bits_exact(mean)
            if mean == 0:  # IEEE sum: -0 only when every term is -0
                want = 0x8000 if all(int(bits[4 * j + i, d]) == 0x8000 for i in range(4)) else 0
            assert int(got[j, d]) == want, (j, d, hex(int(got[j, d])), hex(want))


def pin_compress_closed_forms(orc):
    """Constant groups keep their value; a mean that lies just above a tie
    rounds up (one rounding, no stop at float32); the tail is not compressed;
    `begin` skips rows already committed."""
    x = np.zeros((4 * 3 + 2, 8), np.float16)
    x[0:4] = np.float16(1.5)
    x[4:8] = np.float16(-3.0e-5)
    # 1 + 2^-11 + 2^-24 over 4 = 0.25 + 2^-13 + 2^-26: just above the tie
    # between 0.25 and 0.25 + 2^-12; float32 would round it onto the tie first.
    x[8, 0], x[9, 0], x[10, 0] = np.float16(1.0), np.float16(2.0 ** -11), np.float16(2.0 ** -24)
    x[12:14] = np.float16(7.0)  # tail rows (ignored)
    c = orc.compress_rows(x, 4)
    assert c.shape == (3, 8)
    assert (c[0] == np.float16(1.5)).all()
    assert (c[1] == np.float16(-3.0e-5)).all()
    assert c[2, 0] == np.float16(0.25 + 2.0 ** -12)
    assert (c[2, 1:] == 0).all()
    assert (orc.compress_rows(x, 4, begin=2) == c[2:]).all()
    assert orc.compress_rows(x[:3], 4).shape == (0, 8)


PINS = [
    pin_visibility_brute_force,
    pin_window_brute_force,
    pin_mask_memory,
    pin_indexer_brute_force,
    pin_indexer_closed_forms,
    pin_topk_brute_force,
    pin_topk_closed_forms,
    pin_topk_invariants,
    pin_attention_brute_force,
    pin_attention_closed_forms,
    pin_sparse_equals_dense_sdpa,
    pin_band_independence,
    pin_prefill_end_to_end,
    pin_compress_exact_rounding,
    pin_compress_closed_forms,
]
