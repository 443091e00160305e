"""Checks on the generated gfx950 code of the HIP kernels (no GPU needed:
hipcc cross-compiles to assembly here).

* The attention kernel's tile loads go straight to LDS through buffer
  descriptors with a range check: each is a `buffer_load_dwordx4 ... offen
  lds` whose whole offset is in the VGPR operand (SGPR offset 0, no immediate),
  the part the hardware range-checks, so an offset past a descriptor's size
  reads zeros instead of faulting. No unchecked pointer form
  (`global_load_lds_*`) is left in any kernel.
* M0 holds the LDS address of the direct-to-LDS tile loads, which are issued
  from inline assembly. The compiler does not treat M0 as clobbered by inline
  assembly, so the kernels are correct only while no compiler-generated
  instruction uses M0. Checked for every kernel source.
* No kernel spills to scratch memory (a spill in the attention loop would add
  HBM traffic per tile).
* Every kernel's LDS fits one compute unit (160 KiB).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_decode_attention_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def _flags():
    from quantized_decode_attention_03_amd import build as B
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    return flags + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("isa")
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        path = os.path.join(d, src + ".s")
        subprocess.run([HIPCC] + _flags() + ["-o", path, os.path.join(CSRC, src)], check=True,
                       stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        with open(path) as f:
            out[src] = f.read()
    return out


def test_m0_only_inside_inline_asm(asm):
    for src, text in asm.items():
        inside = False
        for line in text.split("\n"):
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                inside = True
            elif t.startswith(";;#ASMEND"):
                inside = False
            elif not inside and not t.startswith(";") and re.search(r"\bm0\b", t):
                pytest.fail(f"{src}: compiler-generated use of m0: {t}")


def test_dma_loads_only_in_inline_asm(asm):
    # the loads whose LDS address comes from M0 are exactly the inline-asm ones
    text = asm["kvq_attention.hip"]
    assert len(re.findall(r"buffer_load_dwordx4 .*\blds\b", text)) > 0
    inside = False
    for line in text.split("\n"):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
        elif t.startswith(";;#ASMEND"):
            inside = False
        elif re.search(r"_load_.*\blds\b", t) and not t.startswith(";"):
            assert inside, t


def test_dma_loads_are_range_checked(asm):
    # every LDS load is a raw buffer load with the whole offset in the VGPR
    # (SGPR offset 0, no immediate offset); no unchecked pointer form remains
    for src, text in asm.items():
        assert "global_load_lds" not in text, f"{src}: unchecked pointer DMA"
        for line in text.split("\n"):
            t = line.strip()
            if t.startswith(";") or not re.search(r"_load_.*\blds\b", t):
                continue
            assert re.fullmatch(r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], 0 offen lds", t), (src, t)


def _kernel_meta(text):
    """(name, private_segment_fixed_size, group_segment_fixed_size) per kernel."""
    names = re.findall(r"^\s*\.name:\s+(\S+)", text, re.M)
    priv = [int(x) for x in re.findall(r"^\s*\.private_segment_fixed_size:\s+(\d+)", text, re.M)]
    grp = [int(x) for x in re.findall(r"^\s*\.group_segment_fixed_size:\s+(\d+)", text, re.M)]
    return list(zip(names, priv, grp))


def test_no_scratch_and_lds_fits(asm):
    n = 0
    for src, text in asm.items():
        for name, priv, grp in _kernel_meta(text):
            n += 1
            assert priv == 0, f"{src}: {name} uses {priv} B of scratch"
            assert grp <= 160 * 1024, f"{src}: {name} needs {grp} B of LDS"
    assert n >= 108  # every attention variant plus the other kernels
