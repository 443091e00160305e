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
* The buffer descriptors of those loads take the base address's high half
  zero-extended: descriptor word 1 (address bits 32..47, stride 0) is the
  high half masked with 0xffff, never a sign fill of the low half (a
  sign-extended 32-bit value there would point the load far outside the
  cache). Traced through the register moves back to the definition, for every
  load of every kernel variant.
* Inline assembly holds only the tile loads, the M0 set-up and the waits
  (scalar instructions and buffer loads with an address operand): no vector
  ALU instruction. The compiler inserts the wait states a vector read of a
  matrix-core result needs only for instructions it emits itself, so an
  inline-asm ALU operation on a score fresh from an MFMA would read stale
  registers.
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


def test_inline_asm_has_no_vector_alu(asm):
    allowed = re.compile(r"(s_mov_b32 m0, s\d+|s_nop \d+|s_waitcnt (vmcnt|lgkmcnt)\(\d+\)|"
                         r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], 0 offen lds)")
    seen = 0
    for src, text in asm.items():
        inside = False
        for line in text.split("\n"):
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                inside = True
            elif t.startswith(";;#ASMEND"):
                inside = False
            elif inside and t and not t.startswith(";"):
                seen += 1
                assert allowed.fullmatch(t), f"{src}: inline assembly outside the allowed forms: {t}"
    assert seen > 0


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


# instructions whose first operand is a source, not a written SGPR
_NO_SDST = re.compile(r"s_(cmp|bitcmp|cbranch|branch|waitcnt|barrier|nop|endpgm|setprio|sleep|store|"
                      r"buffer_store|dcache|setreg|sendmsg|wait|trap|icache)")


def _sgprs(op):
    """SGPR numbers named by an operand (s5 or s[4:7]), else []."""
    m = re.fullmatch(r"s(\d+)", op)
    if m:
        return [int(m.group(1))]
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", op)
    return list(range(int(m.group(1)), int(m.group(2)) + 1)) if m else []


def _parse(lines):
    """(mnemonic, operands) per instruction line, None for other lines."""
    out = []
    for line in lines:
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            out.append(None)
            continue
        parts = t.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        out.append((parts[0], ops))
    return out


def _written(ins):
    """SGPRs an instruction writes (its first operand), else []."""
    if ins is None:
        return []
    mn, ops = ins
    if not ops or not (mn.startswith("s_") or mn.startswith("v_readfirstlane") or mn.startswith("v_readlane")):
        return []
    if _NO_SDST.match(mn):
        return []
    return _sgprs(ops[0])


def _def_chain(parsed, writes, lo, i, reg, depth=12):
    """Definitions reaching SGPR reg at line i (text order, not before line
    lo, the kernel's first line), following register moves: a list of
    (mnemonic, operands) from the nearest one outwards."""
    import bisect
    chain = []
    while depth > 0:
        depth -= 1
        w = writes.get(reg, [])
        k = bisect.bisect_left(w, i) - 1
        if k < 0 or w[k] < lo:
            chain.append(("<entry>", [f"s{reg}"]))
            return chain
        j = w[k]
        mn, ops = parsed[j]
        chain.append((mn, ops))
        src = _sgprs(ops[1]) if len(ops) > 1 else []
        if mn == "s_mov_b32" and len(src) == 1:
            i, reg = j, src[0]
        elif mn == "s_mov_b64" and len(src) == 2:
            i, reg = j, src[reg - _sgprs(ops[0])[0]]
        elif mn == "s_and_b32" and len(src) == 1:
            i, reg = j, src[0]
        else:
            return chain
    return chain


def _vgprs(op):
    m = re.fullmatch(r"v(\d+)", op)
    if m:
        return [int(m.group(1))]
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    return list(range(int(m.group(1)), int(m.group(2)) + 1)) if m else []


def _vwritten(ins):
    """VGPRs a vector ALU or load instruction writes (its first operand)."""
    if ins is None:
        return []
    mn, ops = ins
    if not ops or mn.startswith(("v_cmp", "v_readfirstlane", "v_readlane", "s_", "ds_write", "global_store",
                                 "buffer_store", "scratch_store")):
        return []
    return _vgprs(ops[0])


def _rsrc_word1_chains(text):
    """Per kernel, the distinct definition chains of descriptor word 1 of its
    direct-to-LDS loads; a chain that ends in a read of a VGPR also names
    that VGPR's definition."""
    import bisect
    lines = text.split("\n")
    parsed = _parse(lines)
    writes, vwrites = {}, {}
    for j, ins in enumerate(parsed):
        for r in _written(ins):
            writes.setdefault(r, []).append(j)
        for r in _vwritten(ins):
            vwrites.setdefault(r, []).append(j)

    def vdef(i, reg, lo):
        w = vwrites.get(reg, [])
        k = bisect.bisect_left(w, i) - 1
        return parsed[w[k]] if k >= 0 and w[k] >= lo else ("<entry>", [f"v{reg}"])
    kernels = {}
    name, lo = None, 0
    for i, ins in enumerate(parsed):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m:
            name, lo = m.group(1), i
        if ins and ins[0] == "buffer_load_dwordx4" and ins[1] and ins[1][-1].endswith("lds"):
            word1 = _sgprs(ins[1][1])[1]
            chain = _def_chain(parsed, writes, lo, i, word1)
            if chain[-1][0] == "v_readfirstlane_b32":
                # the line of that read: the last one writing its SGPR before i
                sreg = _sgprs(chain[-1][1][0])[0]
                w = writes[sreg]
                j = w[bisect.bisect_left(w, i) - 1]
                while parsed[j] != chain[-1]:
                    j = w[w.index(j) - 1]
                chain = chain + [vdef(j, _vgprs(chain[-1][1][1])[0], lo)]
            lst = kernels.setdefault(name, [])
            if chain not in lst:
                lst.append(chain)
    return kernels


def test_dma_descriptor_base_is_zero_extended(asm):
    kernels = _rsrc_word1_chains(asm["kvq_attention.hip"])
    assert len(kernels) >= 100
    for name, chains in kernels.items():
        for chain in chains:
            mns = [mn for mn, _ in chain]
            assert "s_and_b32" in mns, (name, chain)           # stride bits cleared
            k = mns.index("s_and_b32")
            assert chain[k][1][2] in ("0xffff", "0xFFFF", "65535"), (name, chain)
            for mn, ops in chain[k + 1:]:
                assert not (mn in ("s_ashr_i32", "v_ashrrev_i32") and "31" in ops), (name, chain)
                assert not mn.startswith(("s_bfe_i", "s_sext", "v_bfe_i32")), (name, chain)
            # the masked value comes from a zero-extended source: the high
            # half of a 64-bit address (read out of a VGPR that 64-bit address
            # arithmetic or a move wrote, loaded, or carried by 64-bit pointer
            # arithmetic)
            end = chain[-2][0] if chain[-1][0].startswith("v_") or chain[-1][0] == "<entry>" else chain[-1][0]
            assert end in ("v_readfirstlane_b32", "s_addc_u32", "s_load_dwordx2", "s_load_dwordx4",
                           "s_load_dword", "<entry>"), (name, chain)
