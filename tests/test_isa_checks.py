"""Static checks on the gfx950 assembly of every kernel (no GPU needed).

Each HIP source is compiled to device assembly with the library's own flags,
then two code-generation traps are looked for:

* flat loads: a read of LDS through a pointer the compiler cannot trace back
  to shared memory becomes a flat load, which also counts against vmcnt, so
  every wait for it would wait for the direct-to-LDS loads in flight too;
* an MFMA result read by the first instructions of a branch target that the
  MFMA branches to almost at once, with no s_nop in between: the compiler has
  been seen to omit the wait states a matrix-core result needs on such a path
  (the values read were then timing dependent).
"""
import os
import re
import shutil
import subprocess

import pytest

from trainable_block_sparse_mean_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
SOURCES = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not found")


def device_asm(src: str, tmp_path) -> list:
    out = tmp_path / (src + ".s")
    flags = [f for f in B.COMPILE_FLAGS if f != "-fPIC"]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def instructions(lines):
    """(labels -> index, [(kernel, instruction text)])"""
    labels, insts, kernel = {}, [], "?"
    for line in lines:
        t = line.strip()
        if not t or t.startswith(";"):
            continue
        m = re.match(r"^(\.LBB\w+):", t)
        if m:
            labels[m.group(1)] = len(insts)
            continue
        if t.startswith("."):
            continue
        if t.endswith(":"):
            kernel = t[:-1]
            continue
        insts.append((kernel, t.split(";")[0].strip()))
    return labels, insts


def mfma_reads_at_branch_target(labels, insts):
    hits = []
    for i, (kernel, t) in enumerate(insts):
        m = re.match(r"v_mfma\S* v\[(\d+):(\d+)\]", t)
        if not m:
            continue
        dst = {f"v{r}" for r in range(int(m.group(1)), int(m.group(2)) + 1)}
        for k in range(i + 1, min(i + 4, len(insts))):
            u = insts[k][1]
            if u.startswith("v_mfma") or u.startswith("s_nop"):
                break
            b = re.match(r"s_c?branch\w* (\.LBB\w+)", u)
            if not b or b.group(1) not in labels:
                continue
            tgt = labels[b.group(1)]
            for _, w in insts[tgt:tgt + 3]:
                if w.startswith("s_nop") or " " not in w:
                    break
                ops = w.split(" ", 1)[1]
                srcs = set(re.findall(r"v\d+", ops)[1:]) if w.startswith("v_") else set(re.findall(r"v\d+", ops))
                for a, c in re.findall(r"v\[(\d+):(\d+)\]", ops)[1 if w.startswith("v_") else 0:]:
                    srcs |= {f"v{r}" for r in range(int(a), int(c) + 1)}
                if dst & srcs:
                    hits.append(f"{kernel}: {t} -> {u} -> {w}")
                    break
    return hits


@pytest.mark.parametrize("src", SOURCES)
def test_kernels_have_no_flat_loads_and_no_unpadded_mfma_reads(src, tmp_path):
    labels, insts = instructions(device_asm(src, tmp_path))
    assert insts, "no instructions parsed"
    flat = [f"{k}: {t}" for k, t in insts if t.startswith("flat_load") or t.startswith("flat_store")]
    assert not flat, "flat memory instructions:\n" + "\n".join(flat[:10])
    hits = mfma_reads_at_branch_target(labels, insts)
    assert not hits, "MFMA results read at a branch target without wait states:\n" + "\n".join(hits[:10])
