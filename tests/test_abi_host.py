"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function include/spmla.h declares, and its
argument checks reject bad calls before anything reaches the HIP runtime.
"""
import ctypes
import json
import os
import re
import subprocess

import pytest

import sparse_long_context_int8_amd as sp
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spmla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spmla_[a-z_]+)\s*\(", text)))


def desc_of(w, **kw):
    d = sp.make_desc(w.n_q, w.q_pos0, w.window, w.top_k, ratio=w.ratio, band=w.band)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_library_exports_every_declared_symbol():
    lib = sp.load_library()
    decl = declared_functions()
    assert decl == sorted(sp.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", sp.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (spmla_\w+)", out.stdout))
    for name in decl:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_abi_version():
    assert sp.spmla_abi_version() == 1


def test_struct_layout_matches_header():
    # 13 int32 fields then one float, no padding.
    assert ctypes.sizeof(sp.spmla_desc) == 14 * 4
    assert sp.spmla_desc.scale.offset == 13 * 4


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=[w.name for w in workloads.WORKLOADS])
def test_workload_descriptors_are_valid(w):
    assert sp.spmla_check_desc(desc_of(w)) == 0


BAD = [
    (dict(n_q=-1), sp.SPMLA_EINVAL, "n_q"),
    (dict(q_pos0=-5), sp.SPMLA_EINVAL, "q_pos0"),
    (dict(ratio=0), sp.SPMLA_EINVAL, "ratio"),
    (dict(window=0), sp.SPMLA_EINVAL, "window"),
    (dict(top_k=0), sp.SPMLA_EINVAL, "top_k"),
    (dict(band=0), sp.SPMLA_EINVAL, "band"),
    (dict(n_raw=100), sp.SPMLA_EINVAL, "n_raw"),
    (dict(n_comp=63), sp.SPMLA_EINVAL, "n_comp"),
    (dict(d_v=600), sp.SPMLA_EINVAL, "d_v"),
    (dict(scale=float("nan")), sp.SPMLA_EINVAL, "scale"),
    (dict(scale=0.0), sp.SPMLA_EINVAL, "scale"),
    (dict(scale=-0.5), sp.SPMLA_EINVAL, "scale"),
    (dict(n_heads=8), sp.SPMLA_EUNSUPPORTED, "n_heads"),
    (dict(d_qk=512, d_v=512), sp.SPMLA_EUNSUPPORTED, "d_qk"),
    (dict(idx_dim=32), sp.SPMLA_EUNSUPPORTED, "idx_dim"),
    (dict(top_k=4097), sp.SPMLA_EUNSUPPORTED, "top_k"),
]


@pytest.mark.parametrize("kw,code,word", BAD, ids=[b[2] for b in BAD])
def test_bad_descriptor_rejected(kw, code, word):
    d = desc_of(workloads.TINY_256, **kw)
    with pytest.raises(sp.SpmlaError) as e:
        sp.spmla_check_desc(d)
    assert e.value.code == code
    assert word in str(e.value)


def test_too_many_compressed_rows_unsupported():
    d = sp.make_desc(8, 131072, 128, 512)  # n_comp = 32770
    with pytest.raises(sp.SpmlaError) as e:
        sp.spmla_check_desc(d)
    assert e.value.code == sp.SPMLA_EUNSUPPORTED


def test_band_schedule_matches_pages():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "band_schedule.json")))
    for case in g["cases"]:
        T = case["tokens"]
        d = sp.make_desc(T, 0, 128, 512, band=g["band"])
        nb = sp.spmla_num_bands(d)
        assert nb == case["bands"]
        assert T - (nb - 1) * g["band"] == case["last_band"]
    assert g["max_bands"] * g["band"] == g["frontier_printed"]


def _up(x, a=256):
    return -(-x // a) * a


def test_workspace_bytes():
    """Scores of one selection group (consecutive bands whose score matrix
    fits 128 MiB) + that group's selections in two orders."""
    w = workloads.PREFILL_8192  # 16 MiB of scores per band: all four bands in one group
    nb = sp.spmla_prefill_workspace_bytes(desc_of(w))
    assert nb == 8192 * 2048 * 4 + 2 * 8192 * 512 * 4
    w = workloads.PREFILL_9133  # row stride 2,284; 18.7 MB per band: all five bands fit
    nb = sp.spmla_prefill_workspace_bytes(desc_of(w))
    assert nb == _up(9133 * 2284 * 4) + 2 * _up(9133 * 512 * 4)
    d = sp.make_desc(20480, 0, 128, 512)  # 5,120 rows: 40 MiB per band, 3 bands per group
    nb = sp.spmla_prefill_workspace_bytes(d)
    assert nb == 6144 * 5120 * 4 + 2 * 6144 * 512 * 4
    # long history: every band takes the fused handoff, whose thresholds, slot
    # counts and 60 spans x 128 candidate slots per query (126 MB per band)
    # fit 512 MiB four bands at a time; that exceeds one band of scores
    w4 = workloads.CHUNK_8192_AT_114687
    nb4 = sp.spmla_prefill_workspace_bytes(desc_of(w4))
    n, spans = 8192, 60
    fused = _up(n * 4) + _up(4) + _up(n * 4) + _up(n * spans * 4) + _up(n * spans * 128 * 8)
    assert fused > 2048 * 30720 * 4
    assert nb4 == fused + 2 * n * 2048 * 4


def test_workspace_covers_split_partials_and_fused_candidates():
    """Small calls need room for the attention's key-split partials (up to
    32 splits x [16][512] + (m, l) per query); long-history bands need the
    fused selection's slots; both fit the scratch the call reports."""
    per_split = (16 * 512 + 16 * 2) * 4
    for w in (workloads.DECODE_1, workloads.VERIFY_5):
        nb = sp.spmla_prefill_workspace_bytes(desc_of(w))
        splits = min(32, -(-1024 // w.n_q))
        assert nb >= w.n_q * splits * per_split
    d = sp.make_desc(300, 6000, 128, 512)  # 300 queries: 4 splits each
    assert sp.spmla_prefill_workspace_bytes(d) >= 300 * 4 * per_split
    w = workloads.CHUNK_8192_AT_114687
    nb = sp.spmla_prefill_workspace_bytes(desc_of(w))
    n_spans = -(-w.n_comp // 512)
    assert nb >= 2048 * n_spans * 128 * 8 + 2048 * n_spans * 4  # candidate slots + counts
    # a call too large for splits needs no partials: the group's scores dominate
    assert sp.spmla_prefill_workspace_bytes(desc_of(workloads.PREFILL_8192)) == 8192 * 2048 * 4 + 2 * 8192 * 512 * 4


def test_empty_call():
    """No queries: the workspace is empty and spmla_prefill returns at once,
    before any pointer is looked at."""
    lib = sp.load_library()
    d = sp.make_desc(0, 100, 128, 512)
    assert sp.spmla_check_desc(d) == 0
    assert sp.spmla_prefill_workspace_bytes(d) == 0
    assert sp.spmla_num_bands(d) == 0
    ptrs = [0] * 10
    assert lib.spmla_prefill(ctypes.byref(d), *[ctypes.c_void_p(p) for p in ptrs], ctypes.c_size_t(0), None) == sp.SPMLA_OK


A = 1 << 20  # an aligned fake address; never dereferenced by these calls


def _call_prefill(lib, d, ptrs, ws_bytes):
    return lib.spmla_prefill(ctypes.byref(d), *[ctypes.c_void_p(p) for p in ptrs],
                             ctypes.c_size_t(ws_bytes), None)


def test_null_and_misaligned_pointers_rejected_before_launch():
    lib = sp.load_library()
    d = desc_of(workloads.TINY_256)
    good = [A] * 10  # q kv_comp kv_raw iq iw ik out lse sel ws
    for i, name in enumerate(["q", "kv_comp", "kv_raw", "iq", "iw", "ik", "out"]):
        ptrs = list(good)
        ptrs[i] = 0
        assert _call_prefill(lib, d, ptrs, 1 << 30) == sp.SPMLA_EINVAL
        assert name in lib.spmla_last_error().decode()
        ptrs[i] = A + 4
        assert _call_prefill(lib, d, ptrs, 1 << 30) == sp.SPMLA_EINVAL
        assert "aligned" in lib.spmla_last_error().decode()
    assert _call_prefill(lib, d, good, 0) == sp.SPMLA_EWORKSPACE
    assert lib.spmla_sparse_attn(ctypes.byref(d), None, None, None, None, None, None, None) == sp.SPMLA_EINVAL
    assert lib.spmla_sparse_attn_grouped(ctypes.byref(d), None, None, None, None, None, None, None) == sp.SPMLA_EINVAL
    assert lib.spmla_topk(ctypes.byref(d), None, None, None, None) == sp.SPMLA_EINVAL
    assert lib.spmla_indexer_scores(ctypes.byref(d), None, None, None, None, None) == sp.SPMLA_EINVAL
    assert lib.spmla_check_desc(None) == sp.SPMLA_EINVAL


def test_compress_arguments_checked_before_launch():
    lib = sp.load_library()
    d = sp.make_desc(8, 100, 16, 4)  # n_raw 108 -> n_comp 27
    raw, comp = ctypes.c_void_p(A), ctypes.c_void_p(A)
    assert lib.spmla_compress(ctypes.byref(d), raw, comp, -1, None) == sp.SPMLA_EINVAL
    assert lib.spmla_compress(ctypes.byref(d), raw, comp, 28, None) == sp.SPMLA_EINVAL
    assert "comp_begin" in lib.spmla_last_error().decode()
    assert lib.spmla_compress(ctypes.byref(d), None, comp, 0, None) == sp.SPMLA_EINVAL
    assert lib.spmla_compress(ctypes.byref(d), raw, ctypes.c_void_p(A + 2), 0, None) == sp.SPMLA_EINVAL
    assert lib.spmla_compress(ctypes.byref(d), raw, comp, 27, None) == 0  # nothing new: no launch
    d8 = sp.make_desc(8, 100, 16, 4, ratio=8)
    assert lib.spmla_compress(ctypes.byref(d8), raw, comp, 0, None) == sp.SPMLA_EUNSUPPORTED


def test_empty_call_is_a_noop():
    lib = sp.load_library()
    d = sp.make_desc(0, 10, 64, 32)
    assert _call_prefill(lib, d, [0] * 10, 0) == 0
    assert lib.spmla_sparse_attn(ctypes.byref(d), None, None, None, None, None, None, None) == 0
    assert lib.spmla_last_error().decode() == ""


def test_generator_shapes_and_ranges():
    w = workloads.TINY_256
    x = workloads.generate(w)
    assert x["q"].shape == (256, 16, 576) and x["q"].dtype.name == "float16"
    assert x["kv_raw"].shape == (256, 576)
    assert x["kv_comp"].shape == (64, 576)
    assert x["iq"].shape == (256, 4, 64) and x["iq"].min() >= -8 and x["iq"].max() <= 7
    assert x["ik"].shape == (64, 64)
    assert x["iw"].shape == (256, 4) and x["iw"].min() >= 1 and x["iw"].max() <= 4
    y = workloads.generate(w)
    for k in x:
        assert (x[k] == y[k]).all()  # seeded


def _host_args(w):
    import torch

    d = desc_of(w)
    x = workloads.generate(w)
    t = {k: torch.from_numpy(v) for k, v in x.items()}
    t["out"] = torch.empty((w.n_q, 16, 512), dtype=torch.float32)
    t["lse"] = torch.empty((w.n_q, 16), dtype=torch.float32)
    t["sel"] = torch.empty((w.n_q, w.top_k), dtype=torch.int32)
    return d, t


def test_binding_checks_tensor_sizes_against_the_descriptor():
    """The library sees only pointers; the binding refuses a tensor shorter
    than the descriptor implies (and a wrong dtype) before any call, and
    only then asks for device memory."""
    import torch

    d, t = _host_args(workloads.TINY_256)
    args = [t["q"], t["kv_comp"], t["kv_raw"], t["sel"], t["out"], t["lse"]]
    with pytest.raises(ValueError, match="device tensor"):
        sp.spmla_sparse_attn(d, *args)
    for i, name in enumerate(["q", "kv_comp", "kv_raw", "sel", "out", "lse"]):
        short = list(args)
        short[i] = args[i].reshape(-1)[:-1]
        with pytest.raises(ValueError, match=f"{name} holds .* needs {args[i].numel()}"):
            sp.spmla_sparse_attn(d, *short)
        with pytest.raises(ValueError, match=f"{name} holds"):
            sp.spmla_sparse_attn_grouped(d, *short)
    with pytest.raises(ValueError, match="dtype"):
        sp.spmla_sparse_attn(d, t["q"].float(), *args[1:])
    with pytest.raises(ValueError, match="iq holds"):
        sp.spmla_indexer_scores(d, t["iq"][:-1], t["iw"], t["ik"], None)
    scores = torch.empty((d.n_q, d.n_comp - 1), dtype=torch.int32)
    with pytest.raises(ValueError, match="scores holds"):
        sp.spmla_indexer_scores(d, t["iq"], t["iw"], t["ik"], scores)
    with pytest.raises(ValueError, match="scores holds"):
        sp.spmla_topk(d, scores, t["sel"])
    with pytest.raises(ValueError, match="n_sel holds"):
        sp.spmla_topk(d, torch.empty((d.n_q, d.n_comp), dtype=torch.int32), t["sel"],
                      torch.empty((d.n_q - 1,), dtype=torch.int32))
    with pytest.raises(ValueError, match="kv_comp holds"):
        sp.spmla_compress(d, t["kv_raw"], t["kv_comp"][:-1])
    ws = torch.empty((64,), dtype=torch.uint8)
    pre = [t["q"], t["kv_comp"], t["kv_raw"], t["iq"], t["iw"], t["ik"], t["out"], t["lse"], t["sel"]]
    with pytest.raises(ValueError, match="exceeds the workspace"):
        sp.spmla_prefill(d, *pre, ws, 65)
    with pytest.raises(ValueError, match="ik holds"):
        sp.spmla_prefill(d, *pre[:5], t["ik"][:-1], *pre[6:], ws)
    with pytest.raises(ValueError, match="device tensor"):
        sp.spmla_prefill(d, *pre, ws)
