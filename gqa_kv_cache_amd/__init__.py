"""Python binding of libgqa_decode (GQA decode over a KV cache on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgqa_decode.so``.  torch supplies device memory and the
current stream.  The names mirror the C ABI in ``include/gqa_decode.h``
and ``include/gqa_append.h``:

    gqa_decode_make_plan(params)              -> dict
    gqa_decode_workspace_size(params)         -> int
    gqa_decode_run(params, q, k_cache, ...)   -> None (writes o, lse)
    gqa_decode_run_noalloc(params, q, ...)    -> None (no workspace; library scratch)
    gqa_resolve_rows(params, ..., rows_out)   -> None
    gqa_kv_append_workspace_size(aparams)     -> int
    gqa_kv_append(aparams, k_new, v_new, ...) -> None (writes the cache rows)
    gqa_status_string(code), gqa_abi_version()

plus ``make_params(...)`` / ``make_append_params(...)`` and a convenience
``decode(...)`` that allocates the outputs and workspace with torch.  There is no fallback: if the library
is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa_decode.so")

LAYOUT_CONTIGUOUS, LAYOUT_RAGGED, LAYOUT_PAGED = 0, 1, 2
KV_BF16, KV_FP8_E4M3FN, KV_INT8 = 0, 1, 2
GATE_NONE, GATE_ELEMENTWISE, GATE_HEADWISE = 0, 1, 2
LAYOUTS = {"contiguous": LAYOUT_CONTIGUOUS, "ragged": LAYOUT_RAGGED, "paged": LAYOUT_PAGED}
KV_DTYPES = {"bf16": KV_BF16, "fp8_e4m3fn": KV_FP8_E4M3FN, "int8": KV_INT8}
GATE_MODES = {"none": GATE_NONE, "elementwise": GATE_ELEMENTWISE, "headwise": GATE_HEADWISE}
MATH = {"auto": 0, "mfma": 1, "valu": 2}
SCALE_POLICIES = {"given": 0, "first_block": 1}

STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED", 3: "GQA_ERR_ALIGNMENT",
          4: "GQA_ERR_WORKSPACE", 5: "GQA_ERR_HIP"}


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("max_seqlen_kv", ctypes.c_int32),
        ("seq_capacity", ctypes.c_int32), ("kv_rows", ctypes.c_int64), ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("topk", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("kv_chunk", ctypes.c_int32), ("num_cus", ctypes.c_int32),
        ("math", ctypes.c_int32), ("partial_event_begin", ctypes.c_void_p),
        ("partial_event_end", ctypes.c_void_p),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("row_blocks", ctypes.c_int32), ("kv_chunk", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("partial_workgroups", ctypes.c_int64),
        ("combine", ctypes.c_int32), ("math", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
    ]


class AppendParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("s_new", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("layout", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("scale_policy", ctypes.c_int32), ("seq_capacity", ctypes.c_int32), ("kv_rows", ctypes.c_int64),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 4),
    ]


_lib_handle = None


def load_library(path: Optional[str] = None):
    """Load libgqa_decode.so (once).  Raises if it is missing."""
    global _lib_handle
    if _lib_handle is not None and path is None:
        return _lib_handle
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libgqa_decode.so not found at {p}; build it with "
                           "`python -m gqa_kv_cache_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(Params)
    vp = ctypes.c_void_p
    lib.gqa_decode_make_plan.argtypes = [P, ctypes.POINTER(Plan)]
    lib.gqa_decode_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.gqa_decode_run.argtypes = [P] + [vp] * 13 + [ctypes.c_size_t, vp]
    lib.gqa_decode_run_noalloc.argtypes = [P] + [vp] * 12 + [vp]
    lib.gqa_resolve_rows.argtypes = [P, vp, vp, vp, vp, vp, vp]
    A = ctypes.POINTER(AppendParams)
    lib.gqa_kv_append_workspace_size.argtypes = [A, ctypes.POINTER(ctypes.c_size_t)]
    lib.gqa_kv_append.argtypes = [A] + [vp] * 10 + [ctypes.c_size_t, vp]
    for f in ("gqa_decode_make_plan", "gqa_decode_workspace_size", "gqa_decode_run", "gqa_decode_run_noalloc",
              "gqa_resolve_rows",
              "gqa_kv_append_workspace_size", "gqa_kv_append"):
        getattr(lib, f).restype = ctypes.c_int
    lib.gqa_status_string.argtypes = [ctypes.c_int]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_last_error.argtypes = []
    lib.gqa_last_error.restype = ctypes.c_char_p
    lib.gqa_abi_version.argtypes = []
    lib.gqa_abi_version.restype = ctypes.c_int
    if path is None:
        _lib_handle = lib
    return lib


def _check(lib, st: int):
    if st != 0:
        raise GqaError(st, lib.gqa_last_error().decode())


def gqa_abi_version() -> int:
    return load_library().gqa_abi_version()


def gqa_status_string(code: int) -> str:
    return load_library().gqa_status_string(code).decode()


def make_params(*, batch: int, s_q: int, h_q: int, h_kv: int, head_dim: int,
                layout="contiguous", kv_dtype="bf16", causal: bool = False,
                max_seqlen_kv: int, seq_capacity: int = 0, kv_rows: int,
                page_size: int = 16, max_pages_per_seq: int = 0, topk: int = 0,
                gate_mode="none", softmax_scale: Optional[float] = None,
                kv_chunk: int = 0, num_cus: int = 0, math="auto") -> Params:
    p = Params()
    p.batch, p.s_q, p.h_q, p.h_kv, p.head_dim = batch, s_q, h_q, h_kv, head_dim
    p.layout = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    p.kv_dtype = KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    p.causal = int(bool(causal))
    p.max_seqlen_kv = max_seqlen_kv
    p.seq_capacity = seq_capacity
    p.kv_rows = kv_rows
    p.page_size = page_size
    p.max_pages_per_seq = max_pages_per_seq
    p.topk = topk
    p.gate_mode = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    p.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    p.kv_chunk = kv_chunk
    p.num_cus = num_cus
    p.math = MATH[math] if isinstance(math, str) else int(math)
    return p


def gqa_decode_make_plan(params: Params) -> dict:
    lib = load_library()
    plan = Plan()
    _check(lib, lib.gqa_decode_make_plan(ctypes.byref(params), ctypes.byref(plan)))
    return {f: getattr(plan, f) for f, _ in Plan._fields_ if not f.startswith("reserved")}


def gqa_decode_workspace_size(params: Params) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib, lib.gqa_decode_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return int(n.value)


# Element types each tensor argument may have.  Raw bit containers are
# accepted for stored bf16 values (int16 / uint16 views of the bits) and for
# one-byte codes (uint8 / int8 bytes); index arrays, scales and LSE must be
# exactly the type the kernels read.
_DTYPES = None


def _dtypes(kind: str):
    global _DTYPES
    if _DTYPES is None:
        import torch
        bits16 = tuple(t for t in (torch.bfloat16, torch.int16, getattr(torch, "uint16", None)) if t is not None)
        fp8 = getattr(torch, "float8_e4m3fn", None)
        _DTYPES = {
            "bf16": (torch.bfloat16,),
            "bf16_bits": bits16,
            "fp8_codes": tuple(t for t in (torch.uint8, torch.int8, fp8) if t is not None),
            "int8_codes": (torch.int8, torch.uint8),
            "int32": (torch.int32,),
            "int64": (torch.int64,),
            "float32": (torch.float32,),
        }
    return _DTYPES[kind]


def _cache_kind(kv_dtype: int) -> str:
    return {KV_BF16: "bf16_bits", KV_FP8_E4M3FN: "fp8_codes", KV_INT8: "int8_codes"}.get(kv_dtype, "bf16_bits")


class _Checked:
    """Checks what the C ABI cannot see in a plain pointer: each tensor's
    element type, that it is contiguous, its size, and that every tensor
    sits on one CUDA device.  An int is taken as a raw device pointer and
    passed on unchecked.  Failures raise GqaError(GQA_ERR_INVALID_ARG)
    before anything reaches the library."""

    def __init__(self):
        self.devices = {}

    def ptr(self, x, name: str, kind: Optional[str] = None, *, exact: Optional[int] = None,
            at_least: Optional[int] = None, min_bytes: Optional[int] = None):
        if x is None or isinstance(x, int):
            return x
        if not hasattr(x, "data_ptr") or not hasattr(x, "is_contiguous"):
            raise GqaError(1, f"{name}: expected a torch tensor or an int device pointer, not {type(x).__name__}")
        if kind is not None and x.dtype not in _dtypes(kind):
            raise GqaError(1, f"{name}: dtype {x.dtype} is not one of {[str(t) for t in _dtypes(kind)]}")
        if not x.is_contiguous():
            raise GqaError(1, f"{name}: tensor is not contiguous")
        if exact is not None and x.numel() != exact:
            raise GqaError(1, f"{name}: {x.numel()} elements, expected {exact}")
        if at_least is not None and x.numel() < at_least:
            raise GqaError(1, f"{name}: {x.numel()} elements, at least {at_least} needed")
        if min_bytes is not None and x.numel() * x.element_size() < min_bytes:
            raise GqaError(1, f"{name}: {x.numel() * x.element_size()} bytes, at least {min_bytes} needed")
        self.devices[name] = x.get_device() if x.is_cuda else x.device
        return x.data_ptr()

    def same_cuda_device(self):
        devs = set(self.devices.values())
        for name, d in self.devices.items():
            if not isinstance(d, int):
                raise GqaError(1, f"{name}: tensor is on {d}, not on a CUDA device")
        if len(devs) > 1:
            raise GqaError(1, f"tensors are on different devices: {sorted(f'cuda:{d}' for d in devs)}")


def _nbytes(x) -> int:
    return x.numel() * x.element_size()


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gqa_decode_run(params: Params, q, k_cache, v_cache, seqlens=None, cu_seqlens=None,
                   block_table=None, topk_idx=None, k_scale=None, v_scale=None, gate=None,
                   o=None, lse=None, workspace=None, workspace_bytes: Optional[int] = None,
                   stream=None) -> None:
    """Enqueue one decode call.  Tensors are passed by device pointer; the
    caller keeps them alive until the stream has run the call.  Tensor
    arguments are checked first (element type, contiguity, size, one CUDA
    device); an int is a raw device pointer, passed on as it is.
    workspace_bytes defaults to the workspace tensor's own size; an int
    workspace pointer needs it given."""
    args = _decode_args(params, q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx, k_scale, v_scale,
                        gate, o, lse, workspace)
    if workspace_bytes is None:
        if isinstance(workspace, int):
            raise GqaError(1, "an int workspace pointer needs workspace_bytes")
        workspace_bytes = 0 if workspace is None else _nbytes(workspace)
    lib = load_library()
    st = lib.gqa_decode_run(ctypes.byref(params), *args, ctypes.c_size_t(workspace_bytes), _stream_handle(stream))
    _check(lib, st)


class DecodeCall:
    """One decode call's arguments, checked once (as gqa_decode_run checks
    them) and kept as device pointers, for callers that repeat the same call
    on the same buffers, such as a serving loop: run() only enqueues it.
    The object holds references to the tensors it was given, so they stay
    allocated while it lives; their contents may change between runs."""

    def __init__(self, params: Params, q, k_cache, v_cache, seqlens=None, cu_seqlens=None, block_table=None,
                 topk_idx=None, k_scale=None, v_scale=None, gate=None, o=None, lse=None, workspace=None,
                 workspace_bytes: Optional[int] = None):
        self.params = params
        self._keep = (q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx, k_scale, v_scale, gate, o,
                      lse, workspace)
        self._args = _decode_args(params, q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx,
                                  k_scale, v_scale, gate, o, lse, workspace)
        if workspace_bytes is None:
            if isinstance(workspace, int):
                raise GqaError(1, "an int workspace pointer needs workspace_bytes")
            workspace_bytes = 0 if workspace is None else _nbytes(workspace)
        self._ws = ctypes.c_size_t(workspace_bytes)
        self._pp = ctypes.byref(params)
        self._lib = load_library()

    def run(self, stream=None) -> None:
        _check(self._lib, self._lib.gqa_decode_run(self._pp, *self._args, self._ws, _stream_handle(stream)))


def _decode_args(p, q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx, k_scale, v_scale, gate, o, lse,
                 workspace=False):
    """Device pointers of a decode call's tensors, after the checks."""
    B, Sq, Hq, Hkv, d = p.batch, p.s_q, p.h_q, p.h_kv, p.head_dim
    esz = 2 if p.kv_dtype == KV_BF16 else 1
    c = _Checked()
    args = [
        c.ptr(q, "q", "bf16", exact=B * Sq * Hq * d),
        c.ptr(k_cache, "k_cache", _cache_kind(p.kv_dtype), min_bytes=p.kv_rows * Hkv * d * esz),
        c.ptr(v_cache, "v_cache", _cache_kind(p.kv_dtype), min_bytes=p.kv_rows * Hkv * d * esz),
        c.ptr(seqlens, "seqlens", "int32", at_least=B),
        c.ptr(cu_seqlens, "cu_seqlens", "int32", at_least=B + 1),
        c.ptr(block_table, "block_table", "int32", at_least=B * p.max_pages_per_seq),
        c.ptr(topk_idx, "topk_idx", "int32", at_least=B * p.topk),
        c.ptr(k_scale, "k_scale", "float32", at_least=B * Hkv),
        c.ptr(v_scale, "v_scale", "float32", at_least=B * Hkv),
        c.ptr(gate, "gate", "bf16", exact=B * Sq * Hq * (1 if p.gate_mode == GATE_HEADWISE else d)),
        c.ptr(o, "o", "bf16", exact=B * Sq * Hq * d),
        c.ptr(lse, "lse", "float32", exact=B * Hq * Sq),
    ]
    if workspace is not False:
        args.append(c.ptr(workspace, "workspace"))
    c.same_cuda_device()
    return args


NOALLOC_SCRATCH_BYTES = 32 << 20   # GQA_NOALLOC_SCRATCH_BYTES


def gqa_decode_run_noalloc(params: Params, q, k_cache, v_cache, seqlens=None, cu_seqlens=None,
                           block_table=None, topk_idx=None, k_scale=None, v_scale=None, gate=None,
                           o=None, lse=None, stream=None) -> None:
    """gqa_decode_run without a workspace: the split partials go to the
    library's per-device scratch array (at most NOALLOC_SCRATCH_BYTES; a
    larger plan raises GQA_ERR_WORKSPACE).  Calls that overlap on one
    device share that array and must be ordered by the caller."""
    args = _decode_args(params, q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx, k_scale, v_scale,
                        gate, o, lse)
    lib = load_library()
    st = lib.gqa_decode_run_noalloc(ctypes.byref(params), *args, _stream_handle(stream))
    _check(lib, st)


def gqa_resolve_rows(params: Params, seqlens=None, cu_seqlens=None, block_table=None,
                     topk_idx=None, rows_out=None, stream=None) -> None:
    p = params
    B = p.batch
    c = _Checked()
    args = [
        c.ptr(seqlens, "seqlens", "int32", at_least=B),
        c.ptr(cu_seqlens, "cu_seqlens", "int32", at_least=B + 1),
        c.ptr(block_table, "block_table", "int32", at_least=B * p.max_pages_per_seq),
        c.ptr(topk_idx, "topk_idx", "int32", at_least=B * p.topk),
        c.ptr(rows_out, "rows_out", "int64", exact=B * p.s_q * (p.topk if p.topk > 0 else p.max_seqlen_kv)),
    ]
    c.same_cuda_device()
    lib = load_library()
    st = lib.gqa_resolve_rows(ctypes.byref(params), *args, _stream_handle(stream))
    _check(lib, st)


def make_append_params(*, batch: int, s_new: int, h_kv: int, head_dim: int, layout="paged",
                       kv_dtype="fp8_e4m3fn", scale_policy="given", seq_capacity: int = 0,
                       kv_rows: int, page_size: int = 16, max_pages_per_seq: int = 0) -> AppendParams:
    p = AppendParams()
    p.batch, p.s_new, p.h_kv, p.head_dim = batch, s_new, h_kv, head_dim
    p.layout = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    p.kv_dtype = KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    p.scale_policy = SCALE_POLICIES[scale_policy] if isinstance(scale_policy, str) else int(scale_policy)
    p.seq_capacity = seq_capacity
    p.kv_rows = kv_rows
    p.page_size = page_size
    p.max_pages_per_seq = max_pages_per_seq
    return p


def gqa_kv_append_workspace_size(params: AppendParams) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib, lib.gqa_kv_append_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return int(n.value)


def gqa_kv_append(params: AppendParams, k_new, v_new, seqlens, seqlens_out=None, block_table=None,
                  k_cache=None, v_cache=None, k_scale=None, v_scale=None, workspace=None,
                  workspace_bytes: Optional[int] = None, stream=None) -> None:
    """Enqueue one append: the new rows go after each request's length.
    Tensor arguments are checked as in gqa_decode_run."""
    args = _append_args(params, k_new, v_new, seqlens, seqlens_out, block_table, k_cache, v_cache, k_scale, v_scale,
                        workspace)
    if workspace_bytes is None:
        if isinstance(workspace, int):
            raise GqaError(1, "an int workspace pointer needs workspace_bytes")
        workspace_bytes = 0 if workspace is None else _nbytes(workspace)
    lib = load_library()
    st = lib.gqa_kv_append(ctypes.byref(params), *args, ctypes.c_size_t(workspace_bytes), _stream_handle(stream))
    _check(lib, st)


def _append_args(params, k_new, v_new, seqlens, seqlens_out, block_table, k_cache, v_cache, k_scale, v_scale,
                 workspace):
    """Device pointers of an append call's tensors, after the checks."""
    p = params
    B, S, Hkv, d = p.batch, p.s_new, p.h_kv, p.head_dim
    esz = 2 if p.kv_dtype == KV_BF16 else 1
    c = _Checked()
    args = [
        c.ptr(k_new, "k_new", "bf16_bits", exact=B * S * Hkv * d),
        c.ptr(v_new, "v_new", "bf16_bits", exact=B * S * Hkv * d),
        c.ptr(seqlens, "seqlens", "int32", at_least=B),
        c.ptr(seqlens_out, "seqlens_out", "int32", at_least=B),
        c.ptr(block_table, "block_table", "int32", at_least=B * p.max_pages_per_seq),
        c.ptr(k_cache, "k_cache", _cache_kind(p.kv_dtype), min_bytes=p.kv_rows * Hkv * d * esz),
        c.ptr(v_cache, "v_cache", _cache_kind(p.kv_dtype), min_bytes=p.kv_rows * Hkv * d * esz),
        c.ptr(k_scale, "k_scale", "float32", at_least=B * Hkv),
        c.ptr(v_scale, "v_scale", "float32", at_least=B * Hkv),
        c.ptr(workspace, "workspace"),
    ]
    c.same_cuda_device()
    return args


class AppendCall:
    """One append call's arguments, checked once and kept as device
    pointers (see DecodeCall); run() only enqueues it."""

    def __init__(self, params: AppendParams, k_new, v_new, seqlens, seqlens_out=None, block_table=None, k_cache=None,
                 v_cache=None, k_scale=None, v_scale=None, workspace=None, workspace_bytes: Optional[int] = None):
        self.params = params
        self._keep = (k_new, v_new, seqlens, seqlens_out, block_table, k_cache, v_cache, k_scale, v_scale, workspace)
        self._args = _append_args(params, k_new, v_new, seqlens, seqlens_out, block_table, k_cache, v_cache, k_scale,
                                  v_scale, workspace)
        if workspace_bytes is None:
            if isinstance(workspace, int):
                raise GqaError(1, "an int workspace pointer needs workspace_bytes")
            workspace_bytes = 0 if workspace is None else _nbytes(workspace)
        self._ws = ctypes.c_size_t(workspace_bytes)
        self._pp = ctypes.byref(params)
        self._lib = load_library()

    def run(self, stream=None) -> None:
        _check(self._lib, self._lib.gqa_kv_append(self._pp, *self._args, self._ws, _stream_handle(stream)))


def decode(q, k_cache, v_cache, *, h_kv: Optional[int] = None, seqlens=None, cu_seqlens=None,
           block_table=None, topk_idx=None, k_scale=None, v_scale=None, gate=None,
           gate_mode: Optional[str] = None, causal: bool = False,
           softmax_scale: Optional[float] = None, max_seqlen_kv: Optional[int] = None,
           layout: Optional[str] = None, kv_chunk: int = 0, out=None, lse=None, workspace=None,
           stream=None, kv_dtype: Optional[str] = None):
    """Allocate O / LSE / workspace with torch and run one decode call.

    q: bf16 [B, S_q, H_q, d].  k_cache / v_cache: bf16, float8_e4m3fn or
    int8 tensors (or uint8 bytes, read as FP8 codes unless kv_dtype says
    "int8"), as [B, S_cap, H_kv, d] (contiguous),
    [N, H_kv, d] (ragged, with cu_seqlens) or [pages, P, H_kv, d] (paged,
    with block_table).  Returns (O bf16 [B, S_q, H_q, d], LSE fp32
    [B, H_q, S_q]).  ``max_seqlen_kv`` is required for the ragged layout;
    otherwise it defaults to the cache capacity (no device sync)."""
    import torch

    B, Sq, Hq, d = q.shape
    if layout is None:
        layout = "paged" if block_table is not None else ("ragged" if cu_seqlens is not None else "contiguous")
    if h_kv is None:
        h_kv = k_cache.shape[-2]
    if kv_dtype is None:
        if k_cache.dtype == torch.int8:
            kv_dtype = "int8"
        elif k_cache.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
            kv_dtype = "fp8_e4m3fn"
        else:
            kv_dtype = "bf16"
    if layout == "contiguous":
        cap = k_cache.shape[1]
        kv_rows = k_cache.shape[0] * cap
        mx = cap if max_seqlen_kv is None else max_seqlen_kv
        page, mpp = 16, 0
    elif layout == "ragged":
        if max_seqlen_kv is None:
            raise ValueError("ragged layout needs max_seqlen_kv")
        cap, kv_rows, mx, page, mpp = 0, k_cache.shape[0], max_seqlen_kv, 16, 0
    else:
        page = k_cache.shape[1]
        mpp = block_table.shape[1]
        cap, kv_rows = 0, k_cache.shape[0] * page
        mx = mpp * page if max_seqlen_kv is None else max_seqlen_kv
    if gate_mode is None:
        gate_mode = "none" if gate is None else ("headwise" if gate.dim() == 3 else "elementwise")
    params = make_params(batch=B, s_q=Sq, h_q=Hq, h_kv=h_kv, head_dim=d, layout=layout,
                         kv_dtype=kv_dtype, causal=causal, max_seqlen_kv=mx,
                         seq_capacity=cap, kv_rows=max(kv_rows, 1), page_size=page,
                         max_pages_per_seq=mpp,
                         topk=0 if topk_idx is None else topk_idx.shape[1], gate_mode=gate_mode,
                         softmax_scale=softmax_scale, kv_chunk=kv_chunk)
    dev = q.device
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    ws = gqa_decode_workspace_size(params)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    # the workspace's own size: the library rejects one that is too small
    gqa_decode_run(params, q, k_cache, v_cache, seqlens, cu_seqlens, block_table, topk_idx, k_scale,
                   v_scale, gate, out, lse, workspace, None if workspace is not None else 0, stream)
    return out, lse
