"""Code-generation invariants of the bf16 main kernel, checked on its gfx950 assembly (CPU).

The kernel keeps the O accumulator in AGPRs a0..a255 that only its inline asm
touches.  That is safe only if the compiler itself never allocates an AGPR and
never spills; the asm also relies on the wait states written into it.  These
checks rebuild the kernel's assembly with the library's flags and verify that.
"""

import os
import re
import subprocess

import pytest

from mla_decode_attention_flashmla_amd import build as Bd


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "main.s"
    src = os.path.join(Bd.CSRC, "mla_main_bf16.hip")
    cmd = [Bd.hipcc(), *Bd.compile_flags(), *Bd.EXTRA.get("mla_main_bf16.hip", []),
           "--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    return out.read_text()


# instantiations: <gathered pages, fp8 pages>; the paged one is the hot path
KINDS = {"paged": "ILb0ELb0E", "gathered": "ILb1ELb0E", "fp8": "ILb0ELb1E"}


def _kernel_bodies(asm):
    """The code of each instantiation of the kernel (paged, gathered and fp8 pages), in
    the order paged, gathered, fp8."""
    names = re.findall(r"^(_Z\w*mla_main_bf16_kernel\w*):", asm, re.M)
    assert len(names) == 3, names
    names = [next(n for n in names if tag in n) for tag in KINDS.values()]
    bodies = []
    for n in names:
        start = re.search(r"^" + re.escape(n) + r":", asm, re.M).start()
        bodies.append(asm[start:asm.index("s_endpgm", start)])
    return bodies


def test_no_spills_and_full_agpr_file(asm):
    assert len(re.findall(r"NumAgprs: 256\b", asm)) == 3
    assert len(re.findall(r"Occupancy: 1\b", asm)) == 3
    paged, gathered, fp8 = _kernel_bodies(asm)
    # the paged and gathered kernels never spill; the fp8 one spills a few values, read
    # back at most once per page
    assert "scratch_" not in paged and "scratch_" not in gathered
    lines = fp8.splitlines()
    mfma = [k for k, ln in enumerate(lines) if "v_mfma" in ln]
    in_loop = [k for k, ln in enumerate(lines) if "scratch_" in ln and mfma[0] < k < mfma[-1]]
    assert len(in_loop) <= 2, in_loop


@pytest.mark.parametrize("which", [0, 1, 2])
def test_compiler_code_never_touches_agprs(asm, which):
    inside, bad = False, []
    for ln in _kernel_bodies(asm)[which].splitlines():
        if ";;#ASMSTART" in ln:
            inside = True
            continue
        if ";;#ASMEND" in ln:
            inside = False
            continue
        code = ln.split(";")[0]
        if not inside and re.search(r"\ba\d+\b|\ba\[\d", code):
            bad.append(ln.strip())
    assert not bad, bad[:5]


@pytest.mark.parametrize("which", [0, 1, 2])
def test_mfma_count_and_no_packed_fp32(asm, which):
    body = _kernel_bodies(asm)[which]
    # 72 score + 64 PV MFMAs per page, emitted once
    assert len(re.findall(r"v_mfma_f32_32x32x16_bf16", body)) == 136
    assert not re.search(r"v_pk_(add|mul|fma)_f32", body)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_valu_writes_are_fenced_before_pv_mfmas(asm, which):
    """Between the scheduling fence before the first PV MFMA and that MFMA, only the
    wait-state nop and LDS/SALU work may appear (no VALU writes of P)."""
    body = _kernel_bodies(asm)[which]
    first_pv = body.index("v_mfma_f32_32x32x16_bf16 a[0:15]")
    fence = body.rindex("sched_barrier", 0, first_pv)
    seg = body[fence:first_pv]
    assert "s_nop 7" in seg
    for ln in seg.splitlines():
        code = ln.split(";")[0].strip()
        assert not code.startswith("v_cvt") and not code.startswith("v_mul"), ln


@pytest.mark.parametrize("which", [0, 1, 2])
def test_dma_base_address_is_not_sign_extended(asm, which):
    """The 64-bit page base handed to global_load_lds is rebuilt from two readfirstlane
    halves; the low half must be zero-extended (a sign extension turned addresses with
    bit 31 set into 0xffffffff........)."""
    body = _kernel_bodies(asm)[which]
    assert "global_load_lds_dwordx4" in body
    assert "s_bfe_i64" not in body
