"""Thin ctypes binding over libmla_decode.so (same names as the C ABI).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  PyTorch supplies device memory (``tensor.data_ptr()``) and the current
stream; nothing here computes attention.  If the library is missing, every call
raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_PLAN = -3
MLA_ERR_HIP = -4
MLA_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 80 << 20
MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1
MLA_STATUS_BAD_SEQLEN = 1
MLA_STATUS_BAD_BLOCK = 2
MLA_STATUS_PLAN_MISMATCH = 4
MLA_STATUS_BAD_SCALE = 8
PAGE = 64
D_QK = 576
D_V = 512

EXPORTS = ("mla_device_workgroups", "mla_plan_size", "mla_get_split_metadata",
           "mla_decode_fwd", "mla_decode_main", "mla_decode_combine", "mla_sparse_plan_size",
           "mla_decode_sparse_fwd", "mla_fp8_plan_size", "mla_decode_fp8_fwd", "mla_kv_append",
           "mla_read_status", "mla_status_string", "mla_decode_fwd_noalloc",
           "mla_decode_fwd_strided")

_lib: Optional[ctypes.CDLL] = None


class MlaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libmla_decode.so from the package directory (built by build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m mla_decode_attention_flashmla_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_i64, c_sz, c_p, c_f = (ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_float)
    lib.mla_device_workgroups.argtypes = [c_int, ctypes.POINTER(c_int)]
    lib.mla_plan_size.argtypes = [c_int, c_int, c_int, c_int, ctypes.POINTER(c_sz),
                                  ctypes.POINTER(c_sz)]
    lib.mla_get_split_metadata.argtypes = [c_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                           c_p, c_sz, c_p]
    fwd_args = [c_int, c_p, c_p, c_i64, c_p, c_int, c_p, c_int, c_int, c_int, c_int, c_f, c_p,
                c_p, c_p, c_sz, c_int, c_p, c_sz, c_p]
    for fn in ("mla_decode_fwd", "mla_decode_main", "mla_decode_combine"):
        getattr(lib, fn).argtypes = fwd_args
    lib.mla_sparse_plan_size.argtypes = [c_int, c_int, c_int, c_int, ctypes.POINTER(c_sz),
                                         ctypes.POINTER(c_sz)]
    lib.mla_decode_sparse_fwd.argtypes = [c_p, c_p, c_i64, c_p, c_int, c_p, c_p, c_int, c_int,
                                          c_int, c_f, c_p, c_p, c_p, c_sz, c_int, c_p, c_sz, c_p]
    lib.mla_fp8_plan_size.argtypes = [c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(c_sz),
                                      ctypes.POINTER(c_sz)]
    lib.mla_decode_fp8_fwd.argtypes = [c_p, c_p, c_i64, c_p, c_int, c_p, c_int, c_int, c_int,
                                       c_int, c_f, c_p, c_p, c_p, c_sz, c_int, c_p, c_sz, c_p]
    lib.mla_kv_append.argtypes = [c_int, c_p, c_p, c_i64, c_p, c_int, c_p, c_int, c_int, c_p,
                                  c_p]
    lib.mla_decode_fwd_noalloc.argtypes = [c_int, c_p, c_p, c_i64, c_p, c_int, c_p, c_int,
                                           c_int, c_int, c_int, c_f, c_p, c_p, c_int, c_p]
    lib.mla_decode_fwd_strided.argtypes = [c_int, c_p, c_i64, c_p, c_i64, c_p, c_int, c_p, c_int,
                                           c_int, c_int, c_int, c_f, c_p, c_i64, c_p, c_p, c_sz,
                                           c_int, c_p, c_sz, c_p]
    lib.mla_read_status.argtypes = [c_p, c_p, ctypes.POINTER(ctypes.c_int32)]
    lib.mla_status_string.argtypes = [c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    for fn in EXPORTS:
        if fn != "mla_status_string":
            getattr(lib, fn).restype = c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().mla_status_string(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != MLA_OK:
        raise MlaError(fn, code)


def device_workgroups(device: int = 0) -> int:
    n = ctypes.c_int(0)
    _check("mla_device_workgroups", load().mla_device_workgroups(device, ctypes.byref(n)))
    return n.value


def plan_size(batch: int, s_q: int, heads: int, num_workgroups: int) -> tuple[int, int]:
    m, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_plan_size", load().mla_plan_size(batch, s_q, heads, num_workgroups,
                                                 ctypes.byref(m), ctypes.byref(w)))
    return m.value, w.value


def _stream(stream) -> Optional[int]:
    """The HIP stream handle: the given torch stream's, else the current device's current
    stream (torch's raw query: the Stream object costs ~3 us of host time per call)."""
    import torch
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Plan:
    """Device buffers of one split plan: metadata (int32) and partial workspace (bytes)."""
    meta: "object"
    workspace: "object"
    batch: int
    s_q: int
    heads: int
    causal: int
    max_blocks: int
    num_workgroups: int


def alloc_plan(batch: int, s_q: int, heads: int, causal: bool, max_blocks: int,
               num_workgroups: Optional[int] = None, device=None) -> Plan:
    """Allocate (with torch) the metadata and workspace buffers a plan needs."""
    import torch
    device = device or torch.device("cuda", torch.cuda.current_device())
    if num_workgroups is None:
        num_workgroups = device_workgroups(device.index or 0)
    mb, wb = plan_size(batch, s_q, heads, num_workgroups)
    meta = torch.empty(mb // 4, dtype=torch.int32, device=device)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=device)
    return Plan(meta, ws, batch, s_q, heads, int(bool(causal)), max_blocks, num_workgroups)


def get_split_metadata(seqlens, plan: Plan, min_split_blocks: int = 0, stream=None) -> None:
    """mla_get_split_metadata: fill plan.meta from seqlens (int32 device tensor)."""
    if (tuple(seqlens.shape) != (plan.batch,) or seqlens.dtype != torch_int32()
            or not seqlens.is_contiguous() or seqlens.get_device() < 0
            or seqlens.get_device() != plan.meta.get_device()):
        raise ValueError("seqlens must be a contiguous int32 [B] tensor on the plan's GPU")
    import torch
    if seqlens.get_device() != torch.cuda.current_device():
        raise ValueError("seqlens and the plan must be on the current device")
    _check("mla_get_split_metadata", load().mla_get_split_metadata(
        seqlens.data_ptr(), plan.batch, plan.s_q, plan.heads, plan.causal, plan.max_blocks,
        plan.num_workgroups, min_split_blocks, plan.meta.data_ptr(),
        plan.meta.numel() * 4, _stream(stream)))


def torch_int32():
    import torch
    return torch.int32


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MLA_DTYPE_F32
    raise MlaError("dtype", MLA_ERR_UNSUPPORTED)


def _check_operands(B: int, block_table, seqlens, floats=(), others=(), plan=None) -> None:
    """What the C ABI cannot see in plain pointers: element types, the lengths of the
    per-sequence arrays, and that every buffer is GPU memory of one device."""
    import torch
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if tuple(seqlens.shape) != (B,) or seqlens.dtype != torch.int32:
        raise ValueError("seqlens must be int32 [B]")
    for name, t in floats:
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    ts = [("block_table", block_table), ("seqlens", seqlens), *floats, *others]
    if plan is not None:
        ts += [("plan.meta", plan.meta), ("plan.workspace", plan.workspace)]
    dev = block_table.get_device()   # -1 for host memory
    for name, t in ts:
        if dev < 0 or t.get_device() != dev:
            raise ValueError(f"{name} must be in the memory of the GPU that holds block_table")
    # the library launches on the current device, with these pointers
    if dev != torch.cuda.current_device():
        raise ValueError(f"the tensors are on cuda:{dev} but cuda:{torch.cuda.current_device()} "
                         "is current; call under torch.cuda.device(...)")


def _decode(fn: str, q, kv_cache, block_table, seqlens, scale: float, out, lse, plan: Plan,
            stream=None) -> None:
    lib = load()
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seqlens", seqlens), ("out", out), ("lse", lse)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, s_q, H, D = q.shape
    if (D != D_QK or kv_cache.shape[1:] != (PAGE, D_QK) or block_table.shape[0] != B
            or tuple(out.shape) != (B, s_q, H, D_V) or tuple(lse.shape) != (B, s_q, H)
            or kv_cache.dtype != q.dtype):
        raise ValueError("shape/dtype mismatch with q [B,s_q,H,576], kv [n,64,576]")
    _check_operands(B, block_table, seqlens, (("out", out), ("lse", lse)),
                    (("q", q), ("kv_cache", kv_cache)), plan)
    _check(fn, getattr(lib, fn)(
        _dtype_code(q), q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
        block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(), B, s_q, H,
        plan.causal, float(scale), out.data_ptr(), lse.data_ptr(), plan.meta.data_ptr(),
        plan.meta.numel() * 4, plan.num_workgroups, plan.workspace.data_ptr(),
        plan.workspace.numel(), _stream(stream)))


def decode_fwd(q, kv_cache, block_table, seqlens, scale, out, lse, plan, stream=None):
    """mla_decode_fwd: main kernel + LSE combine into out [B,s_q,H,512] and lse [B,s_q,H]."""
    _decode("mla_decode_fwd", q, kv_cache, block_table, seqlens, scale, out, lse, plan, stream)


def _row_stride(t, name: str) -> int:
    """Elements between consecutive (b, t, h) rows of a [B, s_q, H, D] tensor whose rows
    are each dense and evenly spaced (e.g. a slice [..., :D] of a wider buffer)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    B, s_q, H, D = t.shape
    rs = t.stride(2) if H > 1 else (t.stride(1) if s_q > 1 else (t.stride(0) if B > 1 else D))
    for d, expect in ((2, rs), (1, H * rs), (0, s_q * H * rs)):
        if t.shape[d] > 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: rows must be evenly spaced (strides {t.stride()})")
    return rs


def decode_fwd_strided(q, kv_cache, block_table, seqlens, scale, out, lse, plan,
                       stream=None) -> None:
    """mla_decode_fwd_strided: as decode_fwd, with q and out allowed to be row-strided
    views (each 576- or 512-value row dense, rows evenly spaced, e.g. q = proj[..., :576]
    of a wider projection output); kv_cache, the tables and lse dense."""
    lib = load()
    for name, t in (("kv_cache", kv_cache), ("block_table", block_table),
                    ("seqlens", seqlens), ("lse", lse)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    q_rs, o_rs = _row_stride(q, "q"), _row_stride(out, "out")
    B, s_q, H, D = q.shape
    if (D != D_QK or kv_cache.shape[1:] != (PAGE, D_QK) or block_table.shape[0] != B
            or tuple(out.shape) != (B, s_q, H, D_V) or tuple(lse.shape) != (B, s_q, H)
            or kv_cache.dtype != q.dtype):
        raise ValueError("shape/dtype mismatch with q [B,s_q,H,576], kv [n,64,576]")
    _check_operands(B, block_table, seqlens, (("out", out), ("lse", lse)),
                    (("q", q), ("kv_cache", kv_cache)), plan)
    _check("mla_decode_fwd_strided", lib.mla_decode_fwd_strided(
        _dtype_code(q), q.data_ptr(), q_rs, kv_cache.data_ptr(), kv_cache.shape[0],
        block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(), B, s_q, H,
        plan.causal, float(scale), out.data_ptr(), o_rs, lse.data_ptr(), plan.meta.data_ptr(),
        plan.meta.numel() * 4, plan.num_workgroups, plan.workspace.data_ptr(),
        plan.workspace.numel(), _stream(stream)))


def decode_main(q, kv_cache, block_table, seqlens, scale, out, lse, plan, stream=None):
    _decode("mla_decode_main", q, kv_cache, block_table, seqlens, scale, out, lse, plan, stream)


def decode_combine(q, kv_cache, block_table, seqlens, scale, out, lse, plan, stream=None):
    _decode("mla_decode_combine", q, kv_cache, block_table, seqlens, scale, out, lse, plan,
            stream)


def decode_fwd_noalloc(q, kv_cache, block_table, seqlens, scale, out, lse, causal=False,
                       num_workgroups: Optional[int] = None, stream=None) -> None:
    """mla_decode_fwd_noalloc: plan, main kernel and combine in one call, with the plan and
    partial results in the library's static scratch (no device allocation, no plan
    buffers)."""
    lib = load()
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seqlens", seqlens), ("out", out), ("lse", lse)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, s_q, H, D = q.shape
    if (D != D_QK or kv_cache.shape[1:] != (PAGE, D_QK) or block_table.shape[0] != B
            or tuple(out.shape) != (B, s_q, H, D_V) or tuple(lse.shape) != (B, s_q, H)
            or kv_cache.dtype != q.dtype):
        raise ValueError("shape/dtype mismatch with q [B,s_q,H,576], kv [n,64,576]")
    _check_operands(B, block_table, seqlens, (("out", out), ("lse", lse)),
                    (("q", q), ("kv_cache", kv_cache)))
    if num_workgroups is None:
        num_workgroups = device_workgroups(q.device.index or 0)
    _check("mla_decode_fwd_noalloc", lib.mla_decode_fwd_noalloc(
        _dtype_code(q), q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
        block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(), B, s_q, H,
        int(bool(causal)), float(scale), out.data_ptr(), lse.data_ptr(), num_workgroups,
        _stream(stream)))


def sparse_plan_size(batch: int, heads: int, topk: int, num_workgroups: int) -> tuple[int, int]:
    m, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_sparse_plan_size", load().mla_sparse_plan_size(
        batch, heads, topk, num_workgroups, ctypes.byref(m), ctypes.byref(w)))
    return m.value, w.value


def alloc_sparse_plan(batch: int, heads: int, topk: int, num_workgroups: Optional[int] = None,
                      device=None) -> Plan:
    """Allocate (with torch) the metadata and workspace buffers of sparse decode."""
    import torch
    device = device or torch.device("cuda", torch.cuda.current_device())
    if num_workgroups is None:
        num_workgroups = device_workgroups(device.index or 0)
    mb, wb = sparse_plan_size(batch, heads, topk, num_workgroups)
    meta = torch.empty(mb // 4, dtype=torch.int32, device=device)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=device)
    return Plan(meta, ws, batch, 1, heads, 0, topk // PAGE, num_workgroups)


def decode_sparse_fwd(q, kv_cache, block_table, seqlens, indices, scale, out, lse, plan: Plan,
                      stream=None) -> None:
    """mla_decode_sparse_fwd: packing of the selected rows, scheduler, main kernel and
    combine into out [B,1,H,512] and lse [B,1,H]."""
    lib = load()
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seqlens", seqlens), ("indices", indices), ("out", out), ("lse", lse)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, s_q, H, D = q.shape
    topk = indices.shape[1]
    if (D != D_QK or s_q != 1 or kv_cache.shape[1:] != (PAGE, D_QK) or block_table.shape[0] != B
            or indices.shape[0] != B or tuple(out.shape) != (B, 1, H, D_V)
            or tuple(lse.shape) != (B, 1, H) or kv_cache.dtype != q.dtype
            or _dtype_code(q) != MLA_DTYPE_BF16):
        raise ValueError("shape/dtype mismatch with bf16 q [B,1,H,576], kv [n,64,576], "
                         "indices [B,topk]")
    if indices.dim() != 2 or indices.dtype != torch_int32():
        raise ValueError("indices must be int32 [B, topk]")
    _check_operands(B, block_table, seqlens, (("out", out), ("lse", lse)),
                    (("q", q), ("kv_cache", kv_cache), ("indices", indices)), plan)
    _check("mla_decode_sparse_fwd", lib.mla_decode_sparse_fwd(
        q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(),
        block_table.shape[1], seqlens.data_ptr(), indices.data_ptr(), topk, B, H, float(scale),
        out.data_ptr(), lse.data_ptr(), plan.meta.data_ptr(), plan.meta.numel() * 4,
        plan.num_workgroups, plan.workspace.data_ptr(), plan.workspace.numel(), _stream(stream)))


def fp8_plan_size(batch: int, s_q: int, heads: int, max_blocks: int,
                  num_workgroups: int) -> tuple[int, int]:
    m, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mla_fp8_plan_size", load().mla_fp8_plan_size(
        batch, s_q, heads, max_blocks, num_workgroups, ctypes.byref(m), ctypes.byref(w)))
    return m.value, w.value


def alloc_fp8_plan(batch: int, s_q: int, heads: int, causal: bool, max_blocks: int,
                   num_workgroups: Optional[int] = None, device=None) -> Plan:
    """Allocate (with torch) the metadata and workspace of decode over an fp8 cache."""
    import torch
    device = device or torch.device("cuda", torch.cuda.current_device())
    if num_workgroups is None:
        num_workgroups = device_workgroups(device.index or 0)
    mb, wb = fp8_plan_size(batch, s_q, heads, max_blocks, num_workgroups)
    meta = torch.empty(mb // 4, dtype=torch.int32, device=device)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=device)
    return Plan(meta, ws, batch, s_q, heads, int(causal), max_blocks, num_workgroups)


def decode_fp8_fwd(q, kv_fp8, block_table, seqlens, scale, out, lse, plan: Plan,
                   stream=None) -> None:
    """mla_decode_fp8_fwd: q bf16 [B,s_q,H,576], kv_fp8 uint8 [n,64,656] (fp8 latent codes,
    bf16 rope, fp32 row scale) -> out [B,s_q,H,512], lse [B,s_q,H]."""
    lib = load()
    for name, t in (("q", q), ("kv_fp8", kv_fp8), ("block_table", block_table),
                    ("seqlens", seqlens), ("out", out), ("lse", lse)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, s_q, H, D = q.shape
    if (D != D_QK or tuple(kv_fp8.shape[1:]) != (PAGE, 656) or kv_fp8.element_size() != 1
            or block_table.shape[0] != B or tuple(out.shape) != (B, s_q, H, D_V)
            or tuple(lse.shape) != (B, s_q, H) or _dtype_code(q) != MLA_DTYPE_BF16):
        raise ValueError("shape/dtype mismatch with bf16 q [B,s_q,H,576], kv_fp8 [n,64,656]")
    _check_operands(B, block_table, seqlens, (("out", out), ("lse", lse)),
                    (("q", q), ("kv_fp8", kv_fp8)), plan)
    _check("mla_decode_fp8_fwd", lib.mla_decode_fp8_fwd(
        q.data_ptr(), kv_fp8.data_ptr(), kv_fp8.shape[0], block_table.data_ptr(),
        block_table.shape[1], seqlens.data_ptr(), B, s_q, H, plan.causal, float(scale),
        out.data_ptr(), lse.data_ptr(), plan.meta.data_ptr(), plan.meta.numel() * 4,
        plan.num_workgroups, plan.workspace.data_ptr(), plan.workspace.numel(),
        _stream(stream)))


def kv_append(new_kv, kv_cache, block_table, seqlens, status=None, stream=None) -> None:
    """mla_kv_append: writes new_kv [B, s_new, 576] into the pages of kv_cache [n, 64, 576]
    at positions seqlens[b] - s_new + t (seqlens count the new tokens).  status: an
    optional device int32 tensor of one element that collects MLA_STATUS_* bits."""
    lib = load()
    for name, t in (("new_kv", new_kv), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seqlens", seqlens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, s_new, D = new_kv.shape
    if (D != D_QK or kv_cache.shape[1:] != (PAGE, D_QK) or block_table.shape[0] != B
            or seqlens.shape[0] != B or kv_cache.dtype != new_kv.dtype):
        raise ValueError("shape/dtype mismatch with new_kv [B,s_new,576], kv [n,64,576]")
    if status is not None and (status.dtype != torch_int32() or status.numel() < 1):
        raise ValueError("status must be an int32 tensor of at least one element")
    _check_operands(B, block_table, seqlens, (),
                    (("new_kv", new_kv), ("kv_cache", kv_cache))
                    + ((("status", status),) if status is not None else ()))
    _check("mla_kv_append", lib.mla_kv_append(
        _dtype_code(new_kv), new_kv.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
        block_table.data_ptr(), block_table.shape[1], seqlens.data_ptr(), B, s_new,
        status.data_ptr() if status is not None else None, _stream(stream)))


def read_status(plan: Plan, stream=None) -> int:
    v = ctypes.c_int32(0)
    _check("mla_read_status", load().mla_read_status(plan.meta.data_ptr(), _stream(stream),
                                                     ctypes.byref(v)))
    return v.value


def mla_decode(q, kv_cache, block_table, seqlens, scale, causal=False, plan=None,
               min_split_blocks: int = 0, num_workgroups: Optional[int] = None):
    """Convenience: plan + forward.  Returns (out, lse) float32 tensors."""
    import torch
    B, s_q, H, _ = q.shape
    if plan is None:
        plan = alloc_plan(B, s_q, H, causal, block_table.shape[1], num_workgroups, q.device)
        get_split_metadata(seqlens, plan, min_split_blocks)
    out = torch.empty((B, s_q, H, D_V), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q.device)
    decode_fwd(q, kv_cache, block_table, seqlens, scale, out, lse, plan)
    return out, lse
