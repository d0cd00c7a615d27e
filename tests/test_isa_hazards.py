"""Checks on the gfx950 assembly of the kernel sources, compiled with the library's own flags
(host-only: hipcc cross-compiles; about a minute).

The HBM-to-LDS loads are inline assembly, so the compiler's hazard checks do not see them.
A `buffer_load ... lds` takes its LDS address from M0, and the compiler writes M0 with a
scalar instruction just before each one; on gfx950 an LDS DMA must not read M0 in the
cycle after that write (the compiler pads its own LDS DMA with an `s_nop 0` there).  Every
LDS DMA must have at least one instruction after the last write of M0 before it.

No kernel may spill to scratch memory, except the block-mask head_dim-64 forward, whose
three-workgroups-per-CU register budget leaves three values (16 bytes) on the stack."""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "scaled_dot_product_05_amd"))
import build as B  # noqa: E402

pytestmark = pytest.mark.slow

DMA_SOURCES = ["fwd.hip", "bwd.hip", "bwd_dq128.hip"]


def _assembly(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    flags = [f for f in B.COMMON if f not in ("-fPIC",)]
    cmd = [B.HIPCC, *flags, *B.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out


def _m0_gaps(path):
    """For every LDS DMA: instructions between it and the last scalar write of M0."""
    ins = []
    for line in open(path):
        t = line.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            ins.append(t)
    gaps = []
    for i, t in enumerate(ins):
        if t.startswith("buffer_load") and t.endswith(" lds"):
            for j in range(i - 1, -1, -1):
                if re.match(r"^s_\w+\s+m0\b", ins[j]):
                    gaps.append(i - j - 1)
                    break
    return gaps


def _scratch(path):
    """{kernel symbol: private segment bytes} of every kernel in the assembly."""
    txt = open(path).read()
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", txt, re.S):
        out[m.group(1)] = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2)).group(1))
    return out


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("isa"))
    with ThreadPoolExecutor(max_workers=len(DMA_SOURCES)) as ex:
        return dict(zip(DMA_SOURCES, ex.map(lambda s: _assembly(s, d), DMA_SOURCES)))


def test_lds_dma_waits_one_state_after_m0(assembly):
    for src, path in assembly.items():
        gaps = _m0_gaps(path)
        assert gaps, f"{src}: no LDS DMA found"
        assert min(gaps) >= 1, f"{src}: {gaps.count(0)} LDS DMAs read M0 right after its write"


def test_no_kernel_spills(assembly):
    # the block-mask D64 forward: fwd16p_kernel<BF, 64, ..., BSM = true>
    allowed = re.compile(r"fwd16p_kernelILb[01]ELi64E.*ELb1EEEv")
    for src, path in assembly.items():
        sizes = _scratch(path)
        assert sizes, f"{src}: no kernels found"
        for name, n in sizes.items():
            limit = 16 if allowed.search(name) else 0
            assert n <= limit, f"{src}: {name} uses {n} bytes of scratch"
