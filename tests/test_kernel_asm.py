"""The gfx950 assembly that the kernel sources compile to (built here, no GPU
needed), checked for three properties the kernels rely on:

* M0 is written only by the DMA staging's own inline assembly, each write
  directly followed by the copy that reads it.  The compiler reserves M0
  and does not preserve it around that assembly, so a value of its own
  kept in M0 would be overwritten; it must keep none.
* No kernel writes through the scalar data cache (scalar stores, scalar
  atomics, write-back or discard of that cache): all stores are vector
  stores.
* The performance kernels (bf16 attention at head_dim 128, the gather, RoPE
  and the dense mask) spill no registers to scratch.

This file names scalar-cache write instructions only to check their absence;
no GPU run loads it.
"""

import os
import re
import subprocess

import pytest

from prefix_shared_tree_packed_amd import build as b

KERNEL_SOURCES = [s for s in b.HIP_SOURCES if s.startswith("kernels/")]
NO_SPILL = {"kernels/attn_fwd_bf16.hip", "kernels/attn_bwd_bf16.hip", "kernels/gather.hip",
            "kernels/rope.hip", "kernels/mask.hip"}
SCALAR_WRITE = re.compile(r"^s_(store|atomic|buffer_store|buffer_atomic|scratch_store|dcache_wb|dcache_discard)")


def _instructions(text):
    """Instruction lines of an assembly listing, comments and directives dropped."""
    out = []
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        out.append(s)
    return out


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("asm")
    hipcc = b._hipcc()
    res = {}
    for src in KERNEL_SOURCES:
        out = tmp / (os.path.basename(src) + ".s")
        cmd = [hipcc, *b.HIP_FLAGS, *b.FILE_FLAGS.get(src, []), "--cuda-device-only", "-S",
               os.path.join(b.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, f"{src}: {r.stdout[-2000:]}"
        res[src] = out.read_text()
    return res


def test_m0_written_only_by_dma_staging(listings):
    n_dma = 0
    for src, text in listings.items():
        ins = _instructions(text)
        for i, s in enumerate(ins):
            if not re.search(r"\bm0\b", s):
                continue
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", s), f"{src}: compiler use of m0: {s!r}"
            assert ins[i + 1] == "s_nop 0", f"{src}: {ins[i:i + 3]}"
            assert re.match(r"global_load_lds_dword(x4)? ", ins[i + 2]), f"{src}: {ins[i:i + 3]}"
            n_dma += 1
    assert n_dma > 0  # the attention kernels do stage through LDS DMA


def test_no_scalar_cache_writes(listings):
    for src, text in listings.items():
        bad = [s for s in _instructions(text) if SCALAR_WRITE.match(s)]
        assert not bad, f"{src}: {bad[:5]}"


def test_performance_kernels_do_not_spill(listings):
    for src in NO_SPILL:
        text = listings[src]
        names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
        spills = re.findall(r"^\s+\.(?:v|s)gpr_spill_count:\s+(\d+)", text, re.M)
        assert spills, src
        assert all(int(x) == 0 for x in spills), (src, list(zip(names, spills)))
