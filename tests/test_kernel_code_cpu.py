"""CPU checks of the generated gfx950 code of the bf16 forward kernel (one
instance per copy placement, compiled to assembly here):

* M0 is written only by the LDS-DMA helpers, each write followed by its
  `buffer_load ... lds`, and read by nothing else.  The helpers declare M0
  clobbered, which clang does not honour for its own uses of the register;
  this pins that the compiler makes none.
* No scalar-cache stores or atomics, and no packed-FP32 arithmetic (the
  build disables it).
"""

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from block_sparse_flash_amd import build as B  # noqa: E402

INSTANCES = [
    # (DQK, DV, BN, NW, CAP, SPLIT, PACK): copies in the matrix phase (128-wide
    # heads) and in the softmax phase (192-wide heads, with a cap and segments)
    (128, 128, 64, 8, "false", "false", "false"),
    (192, 128, 64, 8, "true", "false", "false"),
]


def _asm(tmp_path, inst):
    src = tmp_path / "one.hip"
    src.write_text('#include "splash_fwd_bf16_kernel.h"\n'
                   "namespace splash {\n"
                   "void* one_instance() { return reinterpret_cast<void*>(&splash_fwd_bf16_kernel<"
                   + ", ".join(str(x) for x in inst) + ">); }\n}\n")
    out = tmp_path / "one.s"
    cmd = [B.hipcc(), *B.common_flags(), *B.EXTRA_FLAGS["splash_fwd_bf16.hip"],
           "--cuda-device-only", "-S", str(src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "clobber list contains reserved registers" not in r.stderr
    lines = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    return [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
@pytest.mark.parametrize("inst", INSTANCES, ids=lambda i: "x".join(map(str, i[:2])) + ("-cap" if i[4] == "true" else ""))
def test_m0_scalar_stores_and_packed_fp32(tmp_path, inst):
    code = _asm(tmp_path, inst)
    n_copies = 0
    for i, line in enumerate(code):
        op = line.split()[0]
        if re.search(r"\bm0\b", line):
            if op == "s_mov_b32" and re.match(r"s_mov_b32 m0, s\d+$", line):
                nxt = code[i + 1]
                assert nxt.startswith("buffer_load_dword") and nxt.endswith(" lds"), (line, nxt)
                n_copies += 1
            else:
                raise AssertionError(f"M0 used outside the copy helpers: {line}")
        assert not op.startswith(("s_store", "s_atomic", "s_buffer_store", "s_scratch_store",
                                  "s_dcache_wb", "s_dcache_discard")), line
        assert not re.match(r"v_pk_(fma|mul|add|mov)_f32", op), line
    assert n_copies > 0
