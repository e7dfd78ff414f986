"""On-device ratio-4 compression against the oracle (needs a GPU).

Bar: bit-exact fp16 for finite results, NaN where the oracle gives NaN.
"""
import sys

import numpy as np
import pytest

import oracle
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


def gpu_compress(sp, x, begin=0, comp_init=None):
    import torch

    n_raw = x.shape[0]
    d = sp.make_desc(1, n_raw - 1, 16, 1)  # only n_raw, n_comp, ratio, d_qk matter
    raw = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    comp = (torch.from_numpy(comp_init.copy()).cuda() if comp_init is not None
            else torch.full((d.n_comp, x.shape[1]), float("nan"), dtype=torch.float16, device="cuda"))
    sp.spmla_compress(d, raw, comp, begin)
    torch.cuda.synchronize()
    return comp.cpu().numpy()


def assert_same_fp16(got, want, what):
    gb, wb = got.view(np.uint16), want.view(np.uint16)
    nan_w = np.isnan(want)
    assert (np.isnan(got) == nan_w).all(), what
    mism = (gb != wb) & ~nan_w
    assert not mism.any(), (what, int(mism.sum()), np.argwhere(mism)[:5])


def test_random_rows_with_tail(sp):
    say("[compress] normal rows, 4003 raw rows")
    x = np.random.default_rng(3).standard_normal((4003, 576), dtype=np.float32).astype(np.float16)
    got = gpu_compress(sp, x)
    assert got.shape == (1000, 576)
    assert_same_fp16(got, oracle.compress_rows(x, 4), "normal rows")


def test_every_bit_pattern_class(sp):
    """Uniform random bit patterns (all exponents, subnormals, both signs),
    then hand-made groups: ties, wide spans, the largest value, signed
    zeros, infinities and NaN."""
    say("[compress] random bit patterns and special values")
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 0x10000, (4 * 512, 576), dtype=np.uint32).astype(np.uint16)
    bits[(bits & 0x7C00) == 0x7C00] &= 0xBFFF  # finite, except the special groups below
    special = [
        [0x3C00, 0x1000, 0x0001, 0x0000],  # 1 + 2^-11 + 2^-24: just above a tie
        [0x0001, 0x0001, 0x0000, 0x0000],  # 2^-25: ties to +0
        [0x0001, 0x0001, 0x0001, 0x0000],  # 3 * 2^-26 -> 2^-24
        [0x7BFF, 0x7BFF, 0x7BFF, 0x7BFF],  # largest finite
        [0xFBFF, 0x7BFF, 0x0000, 0x8000],  # exact cancellation -> +0
        [0x8000, 0x8000, 0x8000, 0x8000],  # all -0 -> -0
        [0x7C00, 0x3C00, 0x0000, 0x0000],  # +inf
        [0xFC00, 0x3C00, 0x0000, 0x0000],  # -inf
        [0x7C00, 0xFC00, 0x0000, 0x0000],  # +inf + -inf -> NaN
        [0x7E00, 0x3C00, 0x0000, 0x0000],  # NaN
        [0x03FF, 0x03FF, 0x03FF, 0x0001],  # subnormals carrying into 2^-14
    ]
    for c, grp in enumerate(special):
        bits[0:4, c] = grp
    x = bits.view(np.float16)
    with np.errstate(invalid="ignore", over="ignore"):
        want = oracle.compress_rows(x, 4)
    assert_same_fp16(gpu_compress(sp, x), want, "bit patterns")


def test_begin_leaves_committed_rows(sp):
    say("[compress] comp_begin keeps earlier rows")
    x = np.random.default_rng(5).standard_normal((4 * 300 + 1, 576), dtype=np.float32).astype(np.float16)
    init = np.full((300, 576), np.float16(7.0))
    got = gpu_compress(sp, x, begin=123, comp_init=init)
    assert (got[:123] == np.float16(7.0)).all()
    assert_same_fp16(got[123:], oracle.compress_rows(x, 4, begin=123), "begin 123")


def test_chronological_commit_equals_one_pass(sp):
    """Raw rows arrive in chunks of uneven length; each call compresses only
    the groups the chunk completed. The result equals one pass over all."""
    import torch

    say("[compress] chunked commit")
    x = np.random.default_rng(6).standard_normal((5003, 576), dtype=np.float32).astype(np.float16)
    raw = torch.from_numpy(x).cuda()
    comp = torch.full((5003 // 4, 576), float("nan"), dtype=torch.float16, device="cuda")
    done = 0
    for n_raw in (1, 2, 9, 10, 2047, 2048, 3001, 4096, 5003):
        d = sp.make_desc(1, n_raw - 1, 16, 1)
        sp.spmla_compress(d, raw[:n_raw], comp[: d.n_comp], done)
        done = d.n_comp
    torch.cuda.synchronize()
    assert_same_fp16(comp.cpu().numpy(), oracle.compress_rows(x, 4), "chunked")


@pytest.mark.parametrize("name", ["prefill-9133", "chunk-8192-after-114687"])
def test_full_size_matches_inputs(sp, name):
    """The workloads' compressed rows, rebuilt on the device (9,133 raw rows
    leave a 1-row tail; 122,879 leave 3)."""
    w = workloads.BY_NAME[name]
    say(f"[compress] {name}")
    x = workloads.generate(w)
    got = gpu_compress(sp, x["kv_raw"])
    assert got.shape == x["kv_comp"].shape
    assert_same_fp16(got, oracle.compress_rows(x["kv_raw"], 4), name)
