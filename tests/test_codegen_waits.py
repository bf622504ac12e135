"""The attention kernels' loads stay in flight together (gfx950 assembly, no GPU).

A load under a per-lane condition makes the compiler wait for every memory
operation in flight at the next use (`s_waitcnt vmcnt(0)`). In the gather
kernel that serialised its list, K and V loads; in the shared-key kernel it
made each tile wait for the next tile's just-issued prefetch before its first
MFMA. Both kernels are compiled here to gfx950 assembly with the library's own
flags and checked for those two patterns.
"""
import os
import re
import shutil
import subprocess

import pytest

from head_wise_dynamic_amd import _build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def _assembly(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    flags = [f for f in _build.FLAGS if f != "-fPIC"]
    cmd = ["hipcc"] + flags + ["--cuda-device-only", "-S", os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text().split("\n")


def _functions(lines):
    """(mangled name, list of instruction lines) per kernel."""
    fns, name = {}, None
    for line in lines:
        m = re.match(r"^(_Z[^:\s]+):", line)
        if m:
            name = m.group(1)
            fns[name] = []
        elif name is not None:
            t = line.strip()
            if t and not t.startswith(";") and not t.startswith("."):
                fns[name].append(t)
    return fns


def test_gather_kernel_loads_not_waited_one_by_one(tmp_path):
    fns = _functions(_assembly("attn_valu.hip", tmp_path))
    body = [v for k, v in fns.items() if "valu_attn_kernel" in k and "ItE" in k]  # the bf16 instantiation
    assert len(body) == 1
    ins = body[0]
    loads = [i for i, t in enumerate(ins) if t.startswith("global_load")]
    assert len(loads) >= 24  # 8 list reads, 8 K rows, 8 V rows per chunk
    serial = [i for i in loads if i + 1 < len(ins) and ins[i + 1].startswith("s_waitcnt") and "vmcnt(0)" in ins[i + 1]]
    assert not serial, [ins[i] for i in serial]


def test_shared_key_kernel_mfma_never_waits_for_all_loads(tmp_path):
    fns = _functions(_assembly("attn_mfma.hip", tmp_path))
    body = [v for k, v in fns.items() if "mfma_attn_kernel" in k]
    assert len(body) == 1
    ins = body[0]
    mfma = [i for i, t in enumerate(ins) if t.startswith("v_mfma")]
    assert len(mfma) >= 32
    waited = [i for i in mfma if ins[i - 1].startswith("s_waitcnt") and "vmcnt(0)" in ins[i - 1]]
    assert not waited, [ins[i - 1] for i in waited]
