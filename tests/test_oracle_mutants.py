"""Plant plausible mistakes in copies of the oracle; each must fail a pin.

This shows the pins constrain every step of the oracle: a dropped term, a
wrong sign or index, an off-by-one boundary or a swapped operand in any step
is caught by at least one check that does not come from the oracle itself.
Mutants are made from the oracle's source text on the CPU; the real oracle
module is never modified.
"""
import os
import types

import pytest

import oracle.spmla_oracle as real
from tests.oracle_pins import PINS

SRC_PATH = real.__file__

# (name, original snippet, planted mistake)
MUTANTS = [
    ("ceil-compressed-count", "return n_raw // ratio", "return -(-n_raw // ratio)"),
    ("visibility-off-by-one", "(t + 1) // ratio)", "t // ratio)"),
    ("visibility-one-early", "(t + 1) // ratio)", "(t + 2) // ratio)"),
    ("window-too-long", "max(0, t - window + 1)", "max(0, t - window)"),
    ("window-excludes-self", "return max(0, t - window + 1), t + 1", "return max(0, t - window), t"),
    ("indexer-no-relu", "relu = np.maximum(dots, 0)", "relu = dots"),
    ("indexer-abs-not-relu", "relu = np.maximum(dots, 0)", "relu = np.abs(dots)"),
    ("indexer-no-weights", 'np.einsum("th,thj->tj", iw.astype(np.int64), relu)',
     'np.einsum("thj->tj", relu)'),
    ("indexer-weights-transposed", 'np.einsum("th,thj->tj", iw.astype(np.int64), relu)',
     'np.einsum("th,thj->tj", iw.astype(np.int64)[:, ::-1], relu)'),
    ("indexer-invisible-zero", "out[r, n_visible(q_pos0 + r, Nc, ratio):] = INVISIBLE",
     "out[r, n_visible(q_pos0 + r, Nc, ratio):] = 0"),
    ("topk-ascending", "np.lexsort((j, -s))", "np.lexsort((j, s))"),
    ("topk-tie-high-index", "np.lexsort((j, -s))", "np.lexsort((-j, -s))"),
    ("topk-index-order", "np.lexsort((j, -s))", "np.lexsort((-s, j))"),
    ("topk-drops-last", "order[: min(k, n_vis)]", "order[: min(k, n_vis) - 1]"),
    ("attn-no-scale", "z = scale * (q64 @ k64.T)", "z = (q64 @ k64.T)"),
    ("attn-keys-only-value-dims", "z = scale * (q64 @ k64.T)",
     "z = scale * (q64[:, :d_v] @ k64[:, :d_v].T)"),
    ("attn-unnormalised", "out = p @ k64[:, :d_v]", "out = e @ k64[:, :d_v]"),
    ("attn-values-from-tail", "out = p @ k64[:, :d_v]", "out = p @ k64[:, -d_v:]"),
    ("attn-lse-drops-max", "lse = m[:, 0] + np.log(denom[:, 0])", "lse = np.log(denom[:, 0])"),
    ("attn-compressed-from-raw", "keys = np.concatenate([kv_comp[comp_ids], kv_raw[raw_ids]], axis=0)",
     "keys = np.concatenate([kv_raw[comp_ids], kv_raw[raw_ids]], axis=0)"),
    ("attn-no-window", "keys = np.concatenate([kv_comp[comp_ids], kv_raw[raw_ids]], axis=0)",
     "keys = np.concatenate([kv_comp[comp_ids], kv_raw[raw_ids][-1:]], axis=0)"),
    ("attn-drops-a-selected-row", "sel_row[:n_sel]", "sel_row[:max(0, n_sel - 1)]"),
    ("attn-head-swap", "out[i], lse[i] = attend_one(q[r], keys, scale, d_v)",
     "out[i], lse[i] = attend_one(q[r][::-1], keys, scale, d_v)"),
    ("compress-via-float32", "return (total * (1.0 / ratio)).astype(np.float16)",
     "return (total * (1.0 / ratio)).astype(np.float32).astype(np.float16)"),
    ("compress-sum-not-mean", "return (total * (1.0 / ratio)).astype(np.float16)",
     "return total.astype(np.float16)"),
    ("compress-groups-shifted", "groups = kv_raw[ratio * begin: ratio * n_comp]",
     "groups = kv_raw[ratio * begin + 1: ratio * n_comp + 1]"),
    ("compress-drops-a-member", "for i in range(1, ratio):", "for i in range(2, ratio):"),
    ("compress-sum-reduction-sign", "    total = groups[:, 0]\n    for i in range(1, ratio):\n        total = total + groups[:, i]",
     "    total = groups.sum(axis=1)"),
    ("prefill-query-offset", "indexer_scores(iq[a:b], iw[a:b], ik, q_pos0 + a, ratio)",
     "indexer_scores(iq[a:b], iw[a:b], ik, q_pos0, ratio)"),
    ("prefill-topk-offset", "topk_select(sc, q_pos0 + a, ratio, top_k, n_comp)",
     "topk_select(sc, q_pos0, ratio, top_k, n_comp)"),
    ("prefill-topk-gets-window", "topk_select(sc, q_pos0 + a, ratio, top_k, n_comp)",
     "topk_select(sc, q_pos0 + a, ratio, window, n_comp)"),
    ("prefill-attn-offset", "sel, n_sel, q_pos0 + a,\n", "sel, n_sel, q_pos0,\n"),
    ("prefill-attn-gets-top-k", "                                    window, scale, d_v)",
     "                                    top_k, scale, d_v)"),
    ("prefill-ignores-q-begin", "for a in range(q_begin, q_end, chunk):", "for a in range(0, q_end - q_begin, chunk):"),
    ("prefill-chunk-overlap", "b = min(q_end, a + chunk)", "b = min(q_end, a + chunk + 1)"),
]


def _load_mutant(orig, mutated):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(orig) >= 1, f"snippet not found: {orig!r}"
    src = src.replace(orig, mutated)
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(src, SRC_PATH + "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,mutated", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, mutated):
    mod = _load_mutant(orig, mutated)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:  # any failure of the pin counts as a catch
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"


def test_unmutated_copy_passes():
    mod = _load_mutant("INVISIBLE = ", "INVISIBLE = ")
    for pin in PINS:
        pin(mod)
