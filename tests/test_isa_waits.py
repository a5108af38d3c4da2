"""The tile kernel's hand-placed memory-counter waits hold only if the
compiler emits the instructions they count.  This compiles bi_gemm.hip for
gfx950 to assembly (this repository's own source, with the library's flags)
and checks, for the K-slice instantiation, that:

- every block of partial-sum stores is sixteen buffer stores in straight
  line (no branch can skip one, so the vmcnt(22) after a segment boundary
  counts exactly six loads, six loads and sixteen stores);
- the only vector-memory waits are the hand-placed ones.

CPU only: needs hipcc, not a GPU."""
import os
import re
import shutil
import subprocess

import pytest

from invariant_bi_gemm_02_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_bi_gemm_02_amd", "csrc")


@pytest.fixture(scope="module")
def slice_asm(tmp_path_factory):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "bi_gemm.s")
    flags = [f for f in lib_build.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = ["hipcc", *flags, "-S", "--cuda-device-only", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "bi_gemm.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = open(out).read()
    m = re.search(r"^(_ZN2bi16gemm_tile_kernelILb0ELb1E\w*):[^\n]*\n(.*?)s_endpgm", text, re.S | re.M)
    assert m, "K-slice tile kernel not found in the assembly"
    return m.group(2)


def test_partial_sum_stores_are_straight_line_blocks_of_sixteen(slice_asm):
    lines = [l.strip() for l in slice_asm.splitlines()]
    idx = [i for i, l in enumerate(lines) if l.startswith("buffer_store_dwordx4")]
    assert idx and len(idx) % 16 == 0, f"{len(idx)} partial-sum stores"
    for b in range(0, len(idx), 16):
        block = lines[idx[b]:idx[b + 15] + 1]
        assert not any(l.startswith(("s_cbranch", "s_branch")) or l.endswith(":")
                       for l in block), "a branch or label inside a store block"


def test_only_hand_placed_vector_memory_waits(slice_asm):
    waits = set(re.findall(r"s_waitcnt[^\n]*?vmcnt\((\d+)\)", slice_asm))
    assert "22" in waits and "6" in waits
    assert waits <= {"0", "6", "12", "22"}, waits
