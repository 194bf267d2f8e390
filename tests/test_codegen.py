"""Code-generation checks on the gfx950 assembly of the batched MFMA kernels.

The batched GEMMs stream operands into an LDS ring with asynchronous
global->LDS copies and wait for them with explicit, counted `s_waitcnt vmcnt`
instructions.  The compiler cannot see those copies.  If any ordinary global
load is still pending where the stage loop reads the ring (for example one left
outstanding across a lane-divergent branch), the compiler guards the read with
its own `s_waitcnt vmcnt(...)`, and that wait also drains every copy in flight:
results stay correct, only the pipelining is lost.  This test compiles the
source to assembly (no GPU needed) and requires that no compiler-inserted
vmcnt wait sits directly in front of an LDS operand read in those kernels'
stage loops (the code up to the last MFMA; the epilogue after it runs once
the ring is drained and waits for its own loads once per row block).
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from activation_sparse_predictor_amd import build as B


def _assembly(tmp_path, src):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in B.CFLAGS if f != "-fPIC"]
    cmd = [B.HIPCC, *flags, "-S", "--cuda-device-only", src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().split("\n")


def _functions(lines):
    """(name, body lines) of every kernel in the assembly listing."""
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\w+):", lines[i])
        if not m:
            i += 1
            continue
        j = i + 1
        while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
            j += 1
        yield m.group(1), lines[i + 1:j]
        i = j


def _compiler_waits_before_lds_reads(body, window=4):
    """Compiler-inserted vmcnt waits within `window` lines before a ds_read
    that comes before the last MFMA of the kernel."""
    last_mfma = max((k for k, l in enumerate(body) if "v_mfma" in l), default=-1)
    in_asm = False
    asm_line = set()
    for k, line in enumerate(body):
        s = line.strip()
        if s == ";;#ASMSTART":
            in_asm = True
        elif s == ";;#ASMEND":
            in_asm = False
        elif in_asm:
            asm_line.add(k)
    hits = []
    for k, line in enumerate(body):
        if k > last_mfma or not line.strip().startswith("ds_read"):
            continue
        for q in range(max(0, k - window), k):
            if "s_waitcnt" in body[q] and "vmcnt" in body[q] and q not in asm_line:
                hits.append((q, body[q].strip(), line.strip()))
    return hits


def test_batched_mfma_loops_have_no_implicit_dma_drain(tmp_path):
    lines = _assembly(tmp_path, os.path.join(B.CSRC, "batch.hip"))
    checked = 0
    bad = {}
    for name, body in _functions(lines):
        if not any("v_mfma" in l for l in body):
            continue
        checked += 1
        hits = _compiler_waits_before_lds_reads(body)
        if hits:
            bad[name] = hits[:3]
    # up (relu, reglu), down, predictor hidden and logits kernels, 5 tile widths each
    assert checked >= 25, checked
    assert not bad, bad
