"""spmla_prefill_noalloc (device-resident scratch, no workspace argument)
against spmla_prefill, through the C ABI (needs a GPU).

Two calls in a row on the same device-resident scratch, the second with a
smaller input, then a call whose scratch only fits once its bands are
halved: selections, outputs and lse must be bit-identical to spmla_prefill
with a caller workspace (the same kernels run; only the grouping of queries
into launches differs, and results do not depend on it).
"""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sp():
    import torch

    import sparse_long_context_int8_amd as sp

    assert torch.cuda.is_available()
    sp.load_library()
    return sp


def _run_both(sp, w, seed):
    import torch

    x = workloads.generate(w, seed=seed)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    d = sp.make_desc(w.n_q, w.q_pos0, w.window, w.top_k, ratio=w.ratio, band=w.band)
    o_ref, l_ref, s_ref = sp.prefill(d, dev)
    out = torch.full((w.n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.n_q, 16), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((w.n_q, w.top_k), -7, dtype=torch.int32, device="cuda")
    sp.spmla_prefill_noalloc(d, dev["q"], dev["kv_comp"], dev["kv_raw"], dev["iq"], dev["iw"], dev["ik"],
                             out, lse, sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, s_ref), f"{w.name}: sel differs"
    assert torch.equal(out, o_ref), f"{w.name}: out differs"
    assert torch.equal(lse, l_ref), f"{w.name}: lse differs"


def test_noalloc_matches_prefill_two_calls(sp):
    """The benchmarked 8,192-query prefill (96 MiB of workspace by default,
    here selection groups of two bands), then 300 queries after 122,000
    tokens (fused selection, key-split attention) on the same scratch."""
    first = workloads.PREFILL_8192
    second = workloads.LayerShape("noalloc-small", n_q=300, q_pos0=122000, window=128, top_k=2048)
    assert second.n_q < first.n_q
    say(f"[noalloc] call 1: {first.name}")
    _run_both(sp, first, seed=None)
    say(f"[noalloc] call 2: {second.name}")
    _run_both(sp, second, seed=21)


def test_noalloc_halves_bands_to_fit(sp):
    """The long-context chunk needs 158 MB of scratch per 2,048-query band;
    the no-alloc call runs it in bands of 512 within 64 MiB."""
    w = workloads.CHUNK_8192_AT_114687
    say(f"[noalloc] {w.name}")
    _run_both(sp, w, seed=None)
