"""The attention kernels' loads stay in flight together (gfx950 assembly, no GPU).

A load under a per-lane condition makes the compiler wait for every memory
operation in flight at the next use (`s_waitcnt vmcnt(0)`). In the gather
kernel that serialised its list, K and V loads; in the shared-key kernel it
made each tile wait for the next tile's just-issued prefetch before its first
MFMA. Both kernels are compiled here to gfx950 assembly with the library's own
flags and checked for those patterns.
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
    """The bf16 gather kernel requests the K and V rows of a chunk for every
    head of a group together: 3 heads x 4 rows x (K, V) = 24 loads in one run
    with no wait between them, and no key-row load waited for on its own."""
    fns = _functions(_assembly("attn_valu.hip", tmp_path))
    body = [v for k, v in fns.items() if "gather_attn_kernel" in k]
    assert len(body) == 1
    ins = body[0]
    run, best = 0, 0
    for t in ins:
        if t.startswith("global_load_dwordx4"):
            run += 1
            best = max(best, run)
        elif t.startswith("s_waitcnt") and "vmcnt" in t:
            run = 0
    assert best >= 24, best
    rows = [i for i, t in enumerate(ins) if t.startswith("global_load_dwordx4")]
    serial = [i for i in rows if i + 1 < len(ins) and ins[i + 1].startswith("s_waitcnt") and "vmcnt(0)" in ins[i + 1]
              and not (i > 0 and ins[i - 1].startswith("global_load_dwordx4"))]
    # a lone 16-byte load followed by a full wait may only be a head's query row
    assert len(serial) <= 6, [ins[i] for i in serial]


def test_shared_key_kernel_mfma_never_waits_for_all_loads(tmp_path):
    fns = _functions(_assembly("attn_mfma.hip", tmp_path))
    body = [v for k, v in fns.items() if "mfma_attn_kernel" in k]
    assert len(body) == 2  # the key-set kernel and its dense (contiguous keys) instantiation
    for ins in body:
        mfma = [i for i, t in enumerate(ins) if t.startswith("v_mfma")]
        assert len(mfma) >= 32
        waited = [i for i in mfma if ins[i - 1].startswith("s_waitcnt") and "vmcnt(0)" in ins[i - 1]]
        assert not waited, [ins[i - 1] for i in waited]


def test_bf16_dot2_reads_every_word_of_a_pack(tmp_path):
    """Each v_dot2 of a packed 8-channel product reads its own 32-bit word.
    When the four words of a 128-bit vector were bit-cast element by element,
    this compiler emitted all four dot2 on the first word (wrong sums with no
    error); the kernels extract the words first.  The gather kernel's q . k
    takes four dot2 per key row, dot2s that read the same registers as the
    one before would be that defect."""
    fns = _functions(_assembly("attn_valu.hip", tmp_path))
    ins = [v for k, v in fns.items() if "gather_attn_kernel" in k][0]
    dots = [re.split(r"[\s,]+", t)[1:4] for t in ins if t.startswith("v_dot2")]
    assert len(dots) >= 48, len(dots)
    repeats = [(a, b) for a, b in zip(dots, dots[1:]) if a[0] == b[0] and a[1:] == b[1:]]
    assert not repeats, repeats[:4]
