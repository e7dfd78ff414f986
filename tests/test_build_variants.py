"""The attention kernel's template also instantiates configurations the
library does not ship (16-key chunks with a deeper ring, 8-wave workgroups
with three buffers). They were measured and rejected, but must keep
compiling: this builds them on the host (no GPU) and checks that each
kernel's host launch stub is defined, not just referenced."""
import os
import shutil
import subprocess

import pytest

import sparse_long_context_int8_amd.build as b

VARIANTS = [
    {"SPMLA_ATTN_WAVES": 4, "SPMLA_ATTN_CHUNK": 16, "SPMLA_ATTN_NBUF": 4, "SPMLA_ATTN_WPE": 2},
    {"SPMLA_ATTN_WAVES": 8, "SPMLA_ATTN_CHUNK": 32, "SPMLA_ATTN_NBUF": 3, "SPMLA_ATTN_WPE": 2},
]


def _hipcc():
    try:
        return b.hipcc()
    except RuntimeError:
        return None


@pytest.mark.skipif(_hipcc() is None or shutil.which("nm") is None, reason="needs hipcc and nm")
@pytest.mark.parametrize("cfg", VARIANTS, ids=lambda c: "w{SPMLA_ATTN_WAVES}c{SPMLA_ATTN_CHUNK}b{SPMLA_ATTN_NBUF}".format(**c))
def test_attention_variant_compiles(cfg, tmp_path):
    obj = tmp_path / "attn.o"
    defs = [f"-D{k}={v}" for k, v in cfg.items()]
    cmd = [_hipcc(), *b.common_flags(), *defs, "-x", "hip", "-c", os.path.join(b.CSRC, "attn.hip"), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    syms = subprocess.run(["nm", str(obj)], capture_output=True, text=True).stdout.splitlines()
    stubs = [ln for ln in syms if "__device_stub__attn_kernel" in ln]
    assert stubs, "no attention kernel stubs"
    undefined = [ln for ln in stubs if ln.split()[0] == "U"]
    assert not undefined, f"kernel stub referenced but not defined: {undefined}"
