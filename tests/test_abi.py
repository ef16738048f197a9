"""The C-ABI library loads, exports what include/mla_decode.h declares, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from mla_decode_attention_flashmla_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "mla_decode.h")


# These tests hand made-up device addresses to the compute entry points: a clean error
# code proves validation ran before any HIP call.  Where a GPU is visible, a validation
# regression would launch kernels on those addresses, so they run only without one.
GPU_VISIBLE = os.path.exists("/dev/kfd")
fake_pointers = pytest.mark.skipif(GPU_VISIBLE, reason="passes fake device pointers; "
                                   "runs only where no GPU is visible")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmla_decode.so not built (run __graft_entry__.build())")
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(B.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert B.status_string(B.MLA_OK) == "ok"
    for c in (B.MLA_ERR_INVALID_ARG, B.MLA_ERR_UNSUPPORTED, B.MLA_ERR_PLAN, B.MLA_ERR_HIP):
        assert B.status_string(c) not in ("ok", "unknown status code")
    assert B.status_string(12345) == "unknown status code"


def test_plan_size(lib):
    meta, ws = B.plan_size(64, 1, 128, 256)
    assert meta == (32 + 8 * 256 + 8 * 64) * 4
    assert ws == (256 + 64) * 128 * 513 * 4
    meta2, ws2 = B.plan_size(128, 2, 128, 256)   # two 128-row groups per sequence
    assert meta2 == (32 + 8 * 256 + 8 * 256) * 4
    with pytest.raises(B.MlaError) as e:
        B.plan_size(1, 2, 8193, 256)              # 16386 rows > MLA_MAX_ROWS
    assert e.value.code == B.MLA_ERR_UNSUPPORTED
    with pytest.raises(B.MlaError) as e:
        B.plan_size(1, 0, 16, 256)
    assert e.value.code == B.MLA_ERR_INVALID_ARG


def _fwd(lib, **kw):
    a = dict(dtype=B.MLA_DTYPE_BF16, q=4096, kv=8192, nblk=4, table=12288, maxb=4, lens=16384,
             batch=1, s_q=1, heads=16, causal=0, scale=0.1, out=20480, lse=24576, meta=28672,
             meta_bytes=1 << 20, nwg=8, ws=32768, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.mla_decode_fwd(a["dtype"], a["q"], a["kv"], a["nblk"], a["table"], a["maxb"],
                              a["lens"], a["batch"], a["s_q"], a["heads"], a["causal"],
                              a["scale"], a["out"], a["lse"], a["meta"], a["meta_bytes"], a["nwg"],
                              a["ws"], a["ws_bytes"], a["stream"])


@fake_pointers
def test_decode_rejects_bad_arguments_without_touching_hip(lib):
    # the pointers are fake: any call that got past validation would fail or fault,
    # so a clean error code proves validation ran first
    assert _fwd(lib, dtype=7) == B.MLA_ERR_UNSUPPORTED
    assert _fwd(lib, q=None) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, q=4100) == B.MLA_ERR_INVALID_ARG            # not 16-byte aligned
    assert _fwd(lib, out=None) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, scale=float("nan")) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, scale=float("inf")) == B.MLA_ERR_INVALID_ARG
    # the softmax scale is positive: the kernels take the row max on unscaled scores
    assert _fwd(lib, scale=0.0) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, scale=-0.1) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, causal=2) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, heads=0) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, s_q=2, heads=10000) == B.MLA_ERR_UNSUPPORTED
    assert _fwd(lib, nwg=0) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, nwg=70000) == B.MLA_ERR_UNSUPPORTED
    assert _fwd(lib, meta_bytes=16) == B.MLA_ERR_PLAN
    assert _fwd(lib, ws_bytes=1024) == B.MLA_ERR_PLAN
    assert _fwd(lib, ws=None) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, meta=None) == B.MLA_ERR_INVALID_ARG
    assert _fwd(lib, nblk=-1) == B.MLA_ERR_INVALID_ARG
    # an empty batch is a no-op: OK without any launch
    assert _fwd(lib, batch=0, q=None, out=None) == B.MLA_OK


@fake_pointers
def test_metadata_rejects_bad_arguments(lib):
    f = lib.mla_get_split_metadata
    assert f(None, 2, 1, 16, 0, 4, 8, 0, 4096, 1 << 20, None) == B.MLA_ERR_INVALID_ARG
    assert f(4096, 2, 1, 16, 0, 4, 8, 0, None, 1 << 20, None) == B.MLA_ERR_INVALID_ARG
    assert f(4096, 2, 1, 16, 0, 4, 8, 0, 8192, 8, None) == B.MLA_ERR_PLAN
    assert f(4096, 2, 1, 16, 3, 4, 8, 0, 8192, 1 << 20, None) == B.MLA_ERR_INVALID_ARG
    assert f(4096, 2, 1, 16, 0, -1, 8, 0, 8192, 1 << 20, None) == B.MLA_ERR_INVALID_ARG
    assert f(4096, 2, 1, 16, 0, 4, 8, -3, 8192, 1 << 20, None) == B.MLA_ERR_INVALID_ARG


@fake_pointers
def test_status_read_rejects_null(lib):
    v = ctypes.c_int32(0)
    assert lib.mla_read_status(None, None, ctypes.byref(v)) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_read_status(4096, None, None) == B.MLA_ERR_INVALID_ARG


def test_sparse_plan_size(lib):
    meta, ws = B.sparse_plan_size(64, 128, 2048, 256)
    assert meta == (32 + 8 * 256 + 8 * 64) * 4
    dense = (256 + 64) * 128 * 513 * 4
    rows = 64 * 2048
    a256 = lambda x: (x + 255) // 256 * 256
    assert ws == a256(dense) + a256(rows * 1152) + a256(rows * 4) + a256(rows // 64 * 4) + a256(64 * 4)
    for topk, code in ((0, B.MLA_ERR_INVALID_ARG), (100, B.MLA_ERR_INVALID_ARG),
                       (131072, B.MLA_ERR_UNSUPPORTED)):
        with pytest.raises(B.MlaError) as e:
            B.sparse_plan_size(2, 128, topk, 256)
        assert e.value.code == code


def _sparse(lib, **kw):
    a = dict(q=4096, kv=8192, nblk=4, table=12288, maxb=4, lens=16384, idx=20480, topk=128,
             batch=1, heads=16, scale=0.1, out=24576, lse=28672, meta=32768, meta_bytes=1 << 20,
             nwg=8, ws=36864, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.mla_decode_sparse_fwd(a["q"], a["kv"], a["nblk"], a["table"], a["maxb"], a["lens"],
                                     a["idx"], a["topk"], a["batch"], a["heads"], a["scale"],
                                     a["out"], a["lse"], a["meta"], a["meta_bytes"], a["nwg"],
                                     a["ws"], a["ws_bytes"], a["stream"])


@fake_pointers
def test_sparse_decode_rejects_bad_arguments_without_touching_hip(lib):
    assert _sparse(lib, topk=100) == B.MLA_ERR_INVALID_ARG       # not a multiple of 64
    assert _sparse(lib, topk=0) == B.MLA_ERR_INVALID_ARG
    assert _sparse(lib, topk=1 << 17) == B.MLA_ERR_UNSUPPORTED
    assert _sparse(lib, idx=None) == B.MLA_ERR_INVALID_ARG
    assert _sparse(lib, q=4100) == B.MLA_ERR_INVALID_ARG
    assert _sparse(lib, scale=0.0) == B.MLA_ERR_INVALID_ARG
    assert _sparse(lib, nblk=(1 << 25) + 1) == B.MLA_ERR_INVALID_ARG
    assert _sparse(lib, meta_bytes=16) == B.MLA_ERR_PLAN
    assert _sparse(lib, ws_bytes=1024) == B.MLA_ERR_PLAN
    assert _sparse(lib, heads=16385) == B.MLA_ERR_UNSUPPORTED
    assert _sparse(lib, batch=0, q=None, out=None) == B.MLA_OK


def _fp8(lib, **kw):
    a = dict(q=4096, kv=8192, nblk=4, table=12288, maxb=4, lens=16384, batch=1, s_q=1,
             heads=16, causal=0, scale=0.1, out=24576, lse=28672, meta=32768,
             meta_bytes=1 << 20, nwg=8, ws=36864, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.mla_decode_fp8_fwd(a["q"], a["kv"], a["nblk"], a["table"], a["maxb"], a["lens"],
                                  a["batch"], a["s_q"], a["heads"], a["causal"], a["scale"],
                                  a["out"], a["lse"], a["meta"], a["meta_bytes"], a["nwg"],
                                  a["ws"], a["ws_bytes"], a["stream"])


@fake_pointers
def test_fp8_decode_rejects_bad_arguments_without_touching_hip(lib):
    # the fp8 rows are widened inside the main kernel: the same plan as bf16 decode
    assert B.fp8_plan_size(2, 1, 128, 10, 256) == B.plan_size(2, 1, 128, 256)
    assert _fp8(lib, scale=0.0) == B.MLA_ERR_INVALID_ARG
    assert _fp8(lib, causal=3) == B.MLA_ERR_INVALID_ARG
    assert _fp8(lib, q=4100) == B.MLA_ERR_INVALID_ARG
    assert _fp8(lib, kv=8200) == B.MLA_ERR_INVALID_ARG         # rows need 16-byte alignment
    assert _fp8(lib, maxb=-1) == B.MLA_ERR_INVALID_ARG
    assert _fp8(lib, heads=16385) == B.MLA_ERR_UNSUPPORTED
    assert _fp8(lib, meta_bytes=16) == B.MLA_ERR_PLAN
    assert _fp8(lib, ws_bytes=1024) == B.MLA_ERR_PLAN
    assert _fp8(lib, batch=0, q=None, out=None) == B.MLA_OK


def _fwd_strided(lib, q_rs, o_rs, dtype=B.MLA_DTYPE_BF16):
    return lib.mla_decode_fwd_strided(dtype, 4096, q_rs, 8192, 4, 12288, 4, 16384, 1, 1, 16, 0,
                                      0.1, 20480, o_rs, 24576, 28672, 1 << 20, 8, 32768, 1 << 30,
                                      None)


@fake_pointers
def test_strided_decode_rejects_bad_strides_without_touching_hip(lib):
    # rows of q and out must be dense, 16-byte aligned, and not overlap
    assert _fwd_strided(lib, 575, 512) == B.MLA_ERR_INVALID_ARG
    assert _fwd_strided(lib, 580, 512) == B.MLA_ERR_INVALID_ARG      # bf16: multiple of 8
    assert _fwd_strided(lib, 576, 511) == B.MLA_ERR_INVALID_ARG
    assert _fwd_strided(lib, 576, 514) == B.MLA_ERR_INVALID_ARG      # multiple of 4
    assert _fwd_strided(lib, 576, 1 << 41) == B.MLA_ERR_INVALID_ARG
    assert _fwd_strided(lib, 578, 512, B.MLA_DTYPE_F32) == B.MLA_ERR_INVALID_ARG   # f32: of 4

    # valid strides pass on to the same validation as mla_decode_fwd (here a plan buffer
    # too small, so still no HIP call)
    def small_plan(dtype, q_rs, o_rs):
        return lib.mla_decode_fwd_strided(dtype, 4096, q_rs, 8192, 4, 12288, 4, 16384, 1, 1, 16,
                                          0, 0.1, 20480, o_rs, 24576, 28672, 16, 8, 32768,
                                          1 << 30, None)
    assert small_plan(B.MLA_DTYPE_BF16, 640, 520) == B.MLA_ERR_PLAN
    assert small_plan(B.MLA_DTYPE_F32, 580, 512) == B.MLA_ERR_PLAN


def test_row_strides_of_views():
    """The binding derives a row stride from a view whose rows are dense and evenly
    spaced, and refuses any other layout."""
    import torch

    assert B._row_stride(torch.zeros((2, 3, 4, 576))[..., :576], "q") == 576
    assert B._row_stride(torch.zeros((2, 3, 4, 640))[..., :576], "q") == 640
    assert B._row_stride(torch.zeros((2, 1, 1, 700))[..., 64:640], "q") == 700
    with pytest.raises(ValueError, match="evenly spaced"):
        B._row_stride(torch.zeros((2, 3, 5, 576))[:, :, :4], "q")    # gap after each token
    with pytest.raises(ValueError, match="contiguous"):
        B._row_stride(torch.zeros((2, 3, 512, 4)).transpose(2, 3), "out")


def test_strided_tensors_are_rejected_on_the_host():
    """The dense entry points take dense row-major buffers only (plain pointers, no
    strides): the binding refuses a strided view, e.g. q sliced out of a wider projection
    output or a transposed out, before any library call; such a q or out goes through
    decode_fwd_strided, anything else must be copied first."""
    import torch

    qw = torch.zeros((2, 1, 16, 640), dtype=torch.bfloat16)
    q = qw[..., :576]                                     # rows 640 elements apart
    kv = torch.zeros((4, 64, 576), dtype=torch.bfloat16)
    table = torch.zeros((2, 2), dtype=torch.int32)
    lens = torch.zeros(2, dtype=torch.int32)
    out = torch.zeros((2, 1, 16, 512))
    lse = torch.zeros((2, 1, 16))
    plan = B.Plan(torch.zeros(16, dtype=torch.int32), torch.zeros(16, dtype=torch.uint8),
                  2, 1, 16, 0, 2, 8)
    assert not q.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        B.decode_fwd(q, kv, table, lens, 0.1, out, lse, plan)
    out_t = torch.zeros((2, 1, 512, 16)).transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        B.decode_fwd(q.contiguous(), kv, table, lens, 0.1, out_t, lse, plan)
    with pytest.raises(ValueError, match="contiguous"):
        B.decode_fp8_fwd(q, torch.zeros((4, 64, 656), dtype=torch.uint8), table, lens, 0.1,
                         out, lse, plan)


def test_operand_types_and_devices_are_checked_on_the_host():
    """The C ABI sees plain pointers: the binding checks what they cannot carry (float32
    out and lse, int32 tables and lengths of the right count, GPU memory) before any
    library call, so a float16 out or an int64 length array never reaches a kernel."""
    import torch

    q = torch.zeros((2, 1, 16, 576), dtype=torch.bfloat16)
    kv = torch.zeros((4, 64, 576), dtype=torch.bfloat16)
    table = torch.zeros((2, 2), dtype=torch.int32)
    lens = torch.zeros(2, dtype=torch.int32)
    out = torch.zeros((2, 1, 16, 512))
    lse = torch.zeros((2, 1, 16))
    plan = B.Plan(torch.zeros(16, dtype=torch.int32), torch.zeros(16, dtype=torch.uint8),
                  2, 1, 16, 0, 2, 8)
    bad = [("out", dict(out=out.half()), "out must be float32"),
           ("lse", dict(lse=lse.double()), "lse must be float32"),
           ("lens int64", dict(lens=lens.long()), "seqlens must be int32"),
           ("lens count", dict(lens=torch.zeros(3, dtype=torch.int32)), "seqlens must be int32"),
           ("table int64", dict(table=table.long()), "block_table must be int32"),
           ("host memory", {}, "memory of the GPU")]
    for fn in (B.decode_fwd, B.decode_fwd_strided, B.decode_main):
        for what, repl, msg in bad:
            a = dict(q=q, kv=kv, table=table, lens=lens, out=out, lse=lse)
            a.update(repl)
            with pytest.raises(ValueError, match=msg):
                fn(a["q"], a["kv"], a["table"], a["lens"], 0.1, a["out"], a["lse"], plan)
    with pytest.raises(ValueError, match="seqlens"):
        B.get_split_metadata(lens.long(), plan)
    with pytest.raises(ValueError, match="seqlens"):
        B.get_split_metadata(lens, plan)          # host memory
    with pytest.raises(ValueError, match="memory of the GPU"):
        B.decode_fp8_fwd(q, torch.zeros((4, 64, 656), dtype=torch.uint8), table, lens, 0.1,
                         out, lse, plan)
    with pytest.raises(ValueError, match="indices must be int32"):
        B.decode_sparse_fwd(q, kv, table, lens, torch.zeros((2, 64), dtype=torch.int64), 0.1,
                            out, lse, plan)
    with pytest.raises(ValueError, match="memory of the GPU"):
        B.kv_append(torch.zeros((2, 1, 576), dtype=torch.bfloat16), kv, table, lens)


@fake_pointers
def test_c_caller_compiles_links_and_gets_the_documented_codes(tmp_path):
    """A C99 program (tests/abi_from_c.c) built against include/mla_decode.h and linked to
    the library: the header is C, every declared entry point links, and host-side checks
    return the documented codes without any GPU call."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(B.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I",
                    os.path.join(root, "include"), os.path.join(root, "tests", "abi_from_c.c"),
                    "-o", exe, "-L", lib_dir, "-lmla_decode", "-lm",
                    "-Wl,-rpath," + lib_dir, "-Wl,-rpath-link,/opt/rocm/lib"],
                   check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
