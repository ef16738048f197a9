"""Code-generation invariants of the bf16 main kernel, checked on its gfx950 assembly (CPU).

The kernel keeps the O accumulator in AGPRs a0..a255 that only its inline asm
touches.  That is safe only if the compiler itself never allocates an AGPR and
never spills; the asm also relies on the wait states written into it.  These
checks rebuild the kernel's assembly with the library's flags and verify that.
"""

import os
import re
import subprocess
import sys

import pytest

from mla_decode_attention_flashmla_amd import build as Bd


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    # the compiler is started as a child process: never from a process that has already
    # initialised a GPU (a GPU test earlier in the same session)
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        pytest.skip("the assembly is rebuilt only in processes that have not used the GPU")
    out = tmp_path_factory.mktemp("isa") / "main.s"
    src = os.path.join(Bd.CSRC, "mla_main_bf16.hip")
    cmd = [Bd.hipcc(), *Bd.compile_flags(), *Bd.EXTRA.get("mla_main_bf16.hip", []),
           "--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    return out.read_text()


# instantiations: <gathered pages, fp8 pages, strided q / out rows>; the paged one is the
# hot path
KINDS = {"paged": "ILb0ELb0ELb0E", "gathered": "ILb1ELb0ELb0E", "fp8": "ILb0ELb1ELb0E",
         "strided": "ILb0ELb0ELb1E"}
WHICH = list(range(len(KINDS)))


def _kernel_bodies(asm):
    """The code of each instantiation of the kernel (paged, gathered and fp8 pages, paged
    with strided rows), in the order of KINDS."""
    names = re.findall(r"^(_Z\w*mla_main_bf16_kernel\w*):", asm, re.M)
    assert len(names) == len(KINDS), names
    names = [next(n for n in names if tag in n) for tag in KINDS.values()]
    bodies = []
    for n in names:
        start = re.search(r"^" + re.escape(n) + r":", asm, re.M).start()
        bodies.append(asm[start:asm.index("s_endpgm", start)])
    return bodies


def test_no_spills_and_full_agpr_file(asm):
    assert len(re.findall(r"NumAgprs: 256\b", asm)) == len(KINDS)
    assert len(re.findall(r"Occupancy: 1\b", asm)) == len(KINDS)
    paged, gathered, fp8, strided = _kernel_bodies(asm)
    # the paged, gathered and strided kernels never spill; the fp8 one spills a few
    # values, read back at most once per page
    assert "scratch_" not in paged and "scratch_" not in gathered
    assert "scratch_" not in strided
    lines = fp8.splitlines()
    mfma = [k for k, ln in enumerate(lines) if "v_mfma" in ln]
    in_loop = [k for k, ln in enumerate(lines) if "scratch_" in ln and mfma[0] < k < mfma[-1]]
    assert len(in_loop) <= 2, in_loop


@pytest.mark.parametrize("which", WHICH)
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


@pytest.mark.parametrize("which", WHICH)
def test_mfma_count_and_no_packed_fp32(asm, which):
    body = _kernel_bodies(asm)[which]
    # 72 score + 64 PV MFMAs per page, emitted once
    assert len(re.findall(r"v_mfma_f32_32x32x16_bf16", body)) == 136
    assert not re.search(r"v_pk_(add|mul|fma)_f32", body)


@pytest.mark.parametrize("which", WHICH)
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


@pytest.mark.parametrize("which", WHICH)
def test_dma_base_address_is_not_sign_extended(asm, which):
    """The 64-bit page base handed to global_load_lds is rebuilt from two readfirstlane
    halves; the low half must be zero-extended (a sign extension turned addresses with
    bit 31 set into 0xffffffff........)."""
    body = _kernel_bodies(asm)[which]
    assert "global_load_lds_dwordx4" in body
    assert "s_bfe_i64" not in body


def _regs(spec):
    """VGPR numbers named by an operand such as v7 or v[12:15]."""
    m = re.fullmatch(r"v(\d+)", spec) or re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def _valu_writes_too_close_to_mfma(lines):
    """(MFMA, VALU) pairs where a VALU instruction writes a VGPR that a later PV MFMA
    (accumulator in AGPRs) reads as its A or B operand with fewer than 2 wait states
    between them (an s_nop N counts N + 1, any other instruction 1)."""
    lines = [ln.split(";")[0].strip() for ln in lines]
    lines = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
    bad = []
    for k, ln in enumerate(lines):
        m = re.match(r"v_mfma_f32_32x32x16_bf16 a\[\d+:\d+\], (v\[\d+:\d+\]), (v\[\d+:\d+\])", ln)
        if not m:
            continue
        srcs = _regs(m.group(1)) | _regs(m.group(2))
        waits = 0
        for prev in reversed(lines[:k]):
            if waits >= 2:
                break
            op = prev.split()[0]
            if op == "s_nop":
                waits += int(prev.split()[1]) + 1
                continue
            if op.startswith("v_") and not op.startswith("v_mfma") and len(prev.split()) > 1:
                if _regs(prev.split()[1].rstrip(",")) & srcs:
                    bad.append((ln, prev))
                    break
            waits += 1
    return bad


def test_wait_state_check_sees_a_short_distance():
    close = ["v_cvt_pk_bf16_f32 v21, v3, v4", "v_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[18:21], a[0:15]"]
    assert _valu_writes_too_close_to_mfma(close)
    spaced = [close[0], "s_nop 1", close[1]]
    assert not _valu_writes_too_close_to_mfma(spaced)
    other = ["v_add_f32_e32 v30, v3, v4", close[1]]
    assert not _valu_writes_too_close_to_mfma(other)


@pytest.mark.parametrize("which", WHICH)
def test_pv_operands_written_by_valu_have_wait_states(asm, which):
    """Inside the PV loop the next chunk's P^T is computed by VALU between the MFMAs that
    read the current one.  An MFMA that reads a VGPR that a VALU instruction wrote needs
    2 wait states after that write; the MFMAs are inline asm, so the compiler does not
    insert them: check the distance in the emitted code."""
    bad = _valu_writes_too_close_to_mfma(_kernel_bodies(asm)[which].splitlines())
    assert not bad, bad[:3]


@pytest.mark.parametrize("which", WHICH)
def test_m0_is_set_only_by_the_copy_asm(asm, which):
    """The page copies set M0 (the LDS destination of direct-to-LDS loads) once per window
    of copies in inline asm and rely on it until the window's last copy: code the
    compiler emits must neither read nor write M0."""
    inside, bad = False, []
    for ln in _kernel_bodies(asm)[which].splitlines():
        if ";;#ASMSTART" in ln:
            inside = True
            continue
        if ";;#ASMEND" in ln:
            inside = False
            continue
        code = ln.split(";")[0]
        if not inside and re.search(r"\bm0\b", code):
            bad.append(ln.strip())
    assert not bad, bad[:5]
