"""ctypes binding of libfp8q.so (the C ABI declared in include/fp8q.h).

Argument marshalling only: tensors are checked (dtype, device, contiguity, shape) and
their device pointers handed to the library together with the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no fallback path:
a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

FP8Q_OK = 0
FP8Q_CALIB_STAGE, FP8Q_CALIB_DECLINE, FP8Q_CALIB_FREEZE, FP8Q_CALIB_FROZEN = 0, 1, 2, 3

# Every symbol include/fp8q.h declares.
EXPORTS = (
    "fp8q_strerror", "fp8q_version", "fp8q_time_next_launch", "fp8q_reference_empty",
    "fp8q_reference_stream", "fp8q_reference_lds_stream", "fp8_group_quant", "fp8_block_quant", "fp8_e4m3_encode",
    "w8a8_block_gemm", "w8a8_block_gemm_workspace_size", "w8a8_block_gemm_ws",
    "w8a8_block_gemm_noalloc",
    "w8a8_block_gemm_prefill", "w8a8_block_gemm_grouped",
    "fp8_quant_w8a8_gemm_grouped", "w8a16_block_gemv", "w8a16_block_gemv_grouped",
    "fp8_kv_write", "fp8_kv_write_amax", "fp8_kv_read", "fp8_kv_amax",
    "fp8q_kv_calib_create", "fp8q_kv_calib_create_with_ops", "fp8q_kv_calib_observe",
    "fp8q_kv_calib_decide", "fp8q_kv_calib_scales", "fp8q_kv_calib_state",
    "fp8q_kv_calib_destroy",
)


class Fp8qError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


class KvTarget(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p), ("block_size", ctypes.c_int32),
        ("key_stride", ctypes.c_int32), ("value_stride", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("cache_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
    ]


class GemmProj(ctypes.Structure):
    _fields_ = [("w_q", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("n", ctypes.c_int32), ("ldc", ctypes.c_int32)]


class KvCalibInfo(ctypes.Structure):
    _fields_ = [
        ("window_tokens", ctypes.c_int32), ("requested_tokens", ctypes.c_int32),
        ("frozen", ctypes.c_int32), ("staged_batches", ctypes.c_int32),
        ("tokens_seen", ctypes.c_int64), ("staged_tokens", ctypes.c_int64),
        ("unstaged_tokens", ctypes.c_int64), ("replayed_tokens", ctypes.c_int64),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("k_amax", ctypes.c_float), ("v_amax", ctypes.c_float),
        ("headroom", ctypes.c_float), ("provisional_scale", ctypes.c_float),
    ]


_P, _I32, _I64, _U64, _F32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                              ctypes.c_float)


class KvCalibOps(ctypes.Structure):
    """fp8q_kv_calib_ops: the calibrator's device work as callbacks (see include/fp8q.h)."""
    DEVICE = ctypes.CFUNCTYPE(ctypes.c_int, _P, ctypes.POINTER(_I32))
    ALLOC = ctypes.CFUNCTYPE(ctypes.c_int, _P, _U64, ctypes.POINTER(_P), _P)
    RELEASE = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _P, _I32)
    ZERO = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _U64, _P)
    AMAX_ROWS = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P)
    COPY2D = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _P, _I64, _I64, _I64, _P)
    READ = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _P, _U64, _P)
    REPLAY = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _P, _P, _P, _I32, _I32,
                              ctypes.POINTER(KvTarget), _F32, _F32, _P)
    STAGE = ctypes.CFUNCTYPE(ctypes.c_int, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P,
                             _P, _P)
    _fields_ = [("ctx", _P), ("device", DEVICE), ("alloc", ALLOC), ("release", RELEASE),
                ("zero", ZERO), ("amax_rows", AMAX_ROWS), ("copy2d", COPY2D), ("read", READ),
                ("replay", REPLAY), ("stage", STAGE)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libfp8q.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "fp8q_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "fp8q_version": (ctypes.c_int, []),
        "fp8q_time_next_launch": (ctypes.c_int, [P, P]),
        "fp8q_reference_empty": (ctypes.c_int, [P]),
        "fp8q_reference_stream": (ctypes.c_int, [P, P, I64, P]),
        "fp8q_reference_lds_stream": (ctypes.c_int, [P, I64, I64, P]),
        "fp8_group_quant": (ctypes.c_int, [P, P, P, I64, I32, P]),
        "fp8_block_quant": (ctypes.c_int, [P, P, P, I32, I32, P]),
        "fp8_e4m3_encode": (ctypes.c_int, [P, P, I64, P]),
        "w8a8_block_gemm": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P]),
        "w8a8_block_gemm_workspace_size": (ctypes.c_int, [I32, I32, I32,
                                                          ctypes.POINTER(ctypes.c_uint64)]),
        "w8a8_block_gemm_ws": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P,
                                              ctypes.c_uint64, P]),
        "w8a8_block_gemm_noalloc": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P]),
        "w8a8_block_gemm_grouped": (ctypes.c_int, [P, P, ctypes.POINTER(GemmProj), I32, I32,
                                                   I32, P]),
        "fp8_quant_w8a8_gemm_grouped": (ctypes.c_int, [P, P, P, ctypes.POINTER(GemmProj), I32,
                                                       I32, I32, P]),
        "w8a8_block_gemm_prefill": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, P]),
        "w8a16_block_gemv": (ctypes.c_int, [P, P, P, P, I32, I32, I32, I32, P]),
        "w8a16_block_gemv_grouped": (ctypes.c_int, [P, ctypes.POINTER(GemmProj), I32, I32, I32,
                                                    P]),
        "fp8_kv_write": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, I64, F32, F32,
                                        I32, I32, I64, P]),
        "fp8_kv_write_amax": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, I32, I64, F32, F32,
                                             I32, I32, I64, P, P]),
        "fp8_kv_read": (ctypes.c_int, [P, P, P, I32, I32, I32, I32, I64, F32, F32, P, P,
                                       I32, I32, I64, P]),
        "fp8_kv_amax": (ctypes.c_int, [P, P, I64, P, P]),
        "fp8q_kv_calib_create": (ctypes.c_int, [I32, F32, F32, ctypes.POINTER(P)]),
        "fp8q_kv_calib_create_with_ops": (ctypes.c_int, [I32, F32, F32,
                                                         ctypes.POINTER(KvCalibOps),
                                                         ctypes.POINTER(P)]),
        "fp8q_kv_calib_observe": (ctypes.c_int, [P, P, P, I32, I32, I32,
                                                 ctypes.POINTER(KvTarget), P]),
        "fp8q_kv_calib_decide": (ctypes.c_int, [P, I32, I32]),
        "fp8q_kv_calib_scales": (ctypes.c_int, [P, ctypes.POINTER(F32), ctypes.POINTER(F32)]),
        "fp8q_kv_calib_state": (ctypes.c_int, [P, ctypes.POINTER(KvCalibInfo)]),
        "fp8q_kv_calib_destroy": (None, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().fp8q_strerror(status).decode()


def check(fn: str, status: int) -> None:
    if status != FP8Q_OK:
        raise Fp8qError(fn, status, strerror(status))


def current_stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, contiguous: bool = True) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live in GPU memory (got {t.device})")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn)


# ------------------------------------------------------------------------- entry points


def fp8_group_quant(x: torch.Tensor, q: torch.Tensor | None = None,
                    scales: torch.Tensor | None = None, stream: int | None = None):
    """bf16 [m, k] -> (E4M3 codes uint8 [m, k], fp32 scales [m, k/128])."""
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    if q is None:
        q = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, max(k // 128, 1)), dtype=torch.float32, device=x.device)
    if tuple(q.shape) != (m, k) or scales.numel() < m * (k // 128):
        raise ValueError("output shapes do not match x")
    st = load().fp8_group_quant(_dev(x, "x", _BF16), _dev(q, "q", _U8),
                                _dev(scales, "scales", torch.float32), m, k,
                                current_stream(x.device) if stream is None else stream)
    check("fp8_group_quant", st)
    return q, scales


def fp8_block_quant(w: torch.Tensor, wq: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, stream: int | None = None):
    """bf16 [n, k] -> (E4M3 codes [n, k], fp32 block scales [ceil(n/128), ceil(k/128)])."""
    n, k = w.shape
    if wq is None:
        wq = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if ws is None:
        ws = torch.empty(((n + 127) // 128, (k + 127) // 128), dtype=torch.float32,
                         device=w.device)
    if tuple(wq.shape) != (n, k) or ws.numel() < ((n + 127) // 128) * ((k + 127) // 128):
        raise ValueError("output shapes do not match w")
    st = load().fp8_block_quant(_dev(w, "w", _BF16), _dev(wq, "wq", _U8),
                                _dev(ws, "ws", torch.float32), n, k,
                                current_stream(w.device) if stream is None else stream)
    check("fp8_block_quant", st)
    return wq, ws


def fp8_e4m3_encode(x: torch.Tensor, q: torch.Tensor | None = None,
                    stream: int | None = None) -> torch.Tensor:
    """fp32 [...] -> E4M3 codes (saturating round-to-nearest-even, no scale)."""
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if q.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    st = load().fp8_e4m3_encode(_dev(x, "x", torch.float32), _dev(q, "q", _U8), x.numel(),
                                current_stream(x.device) if stream is None else stream)
    check("fp8_e4m3_encode", st)
    return q


def _w8a8(fn, a_q, a_scale, w_q, w_scale, out, ldc, stream):
    m, k = a_q.shape
    n = w_q.shape[0]
    if w_q.shape[1] != k:
        raise ValueError("a_q and w_q disagree on k")
    if a_scale.numel() != m * (k // 128) or w_scale.numel() != (n // 128) * (k // 128):
        raise ValueError("scale grids do not match the operand shapes")
    if out is None:
        ldc = n if ldc is None else ldc
        out = torch.empty((m, ldc), dtype=torch.bfloat16, device=a_q.device)
    else:
        ldc = out.shape[-1] if ldc is None else ldc
        if out.numel() < (m - 1) * ldc + n:
            raise ValueError("out is smaller than (m - 1) * ldc + n elements")
    st = getattr(load(), fn)(_dev(a_q, "a_q", _U8), _dev(a_scale, "a_scale", torch.float32),
                             _dev(w_q, "w_q", _U8), _dev(w_scale, "w_scale", torch.float32),
                             _dev(out, "out", _BF16), m, n, k, ldc,
                             current_stream(a_q.device) if stream is None else stream)
    check(fn, st)
    return out


def w8a8_block_gemm(a_q: torch.Tensor, a_scale: torch.Tensor, w_q: torch.Tensor,
                    w_scale: torch.Tensor, out: torch.Tensor | None = None,
                    ldc: int | None = None, stream: int | None = None) -> torch.Tensor:
    """E4M3 a_q [m <= 16, k] x E4M3 w_q [n, k]^T with block scales -> bf16 out [m, ldc]."""
    return _w8a8("w8a8_block_gemm", a_q, a_scale, w_q, w_scale, out, ldc, stream)


def w8a8_block_gemm_workspace_size(m: int, n: int, k: int) -> int:
    """Bytes of workspace w8a8_block_gemm_ws needs for this shape on the current device (0:
    the shape runs unsplit)."""
    b = ctypes.c_uint64()
    check("w8a8_block_gemm_workspace_size",
          load().w8a8_block_gemm_workspace_size(m, n, k, ctypes.byref(b)))
    return b.value


_WORKSPACES = {}  # (device index, stream) -> uint8 tensor whose counts are zero between calls


def gemm_workspace(nbytes: int, device=None, stream: int | None = None) -> torch.Tensor:
    """A zero-filled workspace of at least nbytes for calls on `stream`, kept and reused: a
    call leaves its counts at zero, so the buffer needs no clearing between calls on one
    stream (calls on other streams get their own)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    key = (dev.index, current_stream(dev) if stream is None else stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def w8a8_block_gemm_ws(a_q: torch.Tensor, a_scale: torch.Tensor, w_q: torch.Tensor,
                       w_scale: torch.Tensor, out: torch.Tensor | None = None,
                       ldc: int | None = None, workspace: torch.Tensor | None = None,
                       stream: int | None = None) -> torch.Tensor:
    """w8a8_block_gemm with K split across workgroups where the shape has too few 16-column
    strips to fill the CUs.  workspace: a uint8 tensor of at least
    w8a8_block_gemm_workspace_size(m, n, k) bytes whose counts are zero (torch.zeros); by
    default one kept per stream by this module."""
    m, k = a_q.shape
    n = w_q.shape[0]
    if w_q.shape[1] != k:
        raise ValueError("a_q and w_q disagree on k")
    if a_scale.numel() != m * (k // 128) or w_scale.numel() != (n // 128) * (k // 128):
        raise ValueError("scale grids do not match the operand shapes")
    if out is None:
        ldc = n if ldc is None else ldc
        out = torch.empty((m, ldc), dtype=torch.bfloat16, device=a_q.device)
    else:
        ldc = out.shape[-1] if ldc is None else ldc
        if out.numel() < (m - 1) * ldc + n:
            raise ValueError("out is smaller than (m - 1) * ldc + n elements")
    st_ = current_stream(a_q.device) if stream is None else stream
    need = w8a8_block_gemm_workspace_size(m, n, k)
    if workspace is None and need:
        workspace = gemm_workspace(need, a_q.device, st_)
    wp, wb = (0, 0) if workspace is None else (_dev(workspace, "workspace", torch.uint8),
                                               workspace.numel())
    st = load().w8a8_block_gemm_ws(_dev(a_q, "a_q", _U8), _dev(a_scale, "a_scale", torch.float32),
                                   _dev(w_q, "w_q", _U8), _dev(w_scale, "w_scale", torch.float32),
                                   _dev(out, "out", _BF16), m, n, k, ldc, wp or None, wb, st_)
    check("w8a8_block_gemm_ws", st)
    return out


def w8a8_block_gemm_noalloc(a_q: torch.Tensor, a_scale: torch.Tensor, w_q: torch.Tensor,
                            w_scale: torch.Tensor, out: torch.Tensor,
                            ldc: int | None = None, stream: int | None = None) -> torch.Tensor:
    """w8a8_block_gemm_ws with its split scratch in the library's static device array: the
    call allocates nothing (out must be given).  Calls overlapping on one GPU race."""
    if out is None:
        raise ValueError("w8a8_block_gemm_noalloc writes into a given out tensor")
    return _w8a8("w8a8_block_gemm_noalloc", a_q, a_scale, w_q, w_scale, out, ldc, stream)


def w8a8_block_gemm_prefill(a_q: torch.Tensor, a_scale: torch.Tensor, w_q: torch.Tensor,
                            w_scale: torch.Tensor, out: torch.Tensor | None = None,
                            ldc: int | None = None, stream: int | None = None) -> torch.Tensor:
    """The same block-scaled W8A8 GEMM for any row count (tiled for prefill widths)."""
    return _w8a8("w8a8_block_gemm_prefill", a_q, a_scale, w_q, w_scale, out, ldc, stream)


def _proj_array(m, k, projections, device):
    """projections: (w_q [n, k], w_scale, out) with out None, a contiguous [m, ldc] tensor,
    or a 2-D column view [m, n] of a wider row-major buffer (its row stride is the ldc)."""
    arr = (GemmProj * len(projections))()
    outs = []
    for i, (w_q, w_scale, out) in enumerate(projections):
        n = w_q.shape[0]
        if w_q.shape[1] != k or w_scale.numel() != (n // 128) * (k // 128):
            raise ValueError(f"projection {i} does not match the activation")
        if out is None:
            out = torch.empty((m, n), dtype=torch.bfloat16, device=device)
        if out.is_contiguous():
            ldc = out.shape[-1]
            room = out.numel()
        elif out.dim() == 2 and out.stride(1) == 1 and out.shape[1] >= n:
            ldc = out.stride(0)
            room = out.untyped_storage().nbytes() // out.element_size() - out.storage_offset()
        else:
            raise ValueError(f"projection {i}: out must be contiguous or a row-major column view")
        if ldc < n or room < (m - 1) * ldc + n:
            raise ValueError(f"projection {i}: out is smaller than (m - 1) * ldc + n")
        arr[i] = GemmProj(_dev(w_q, "w_q", _U8), _dev(w_scale, "w_scale", torch.float32),
                          _dev(out, "out", _BF16, False), n, ldc)
        outs.append(out)
    return arr, outs


def w8a8_block_gemm_grouped(a_q: torch.Tensor, a_scale: torch.Tensor, projections,
                            stream: int | None = None):
    """One launch over several projections of the same activation.  projections: list of
    (w_q [n, k], w_scale [n/128, k/128], out [m, ldc] or None); returns the outputs."""
    m, k = a_q.shape
    arr, outs = _proj_array(m, k, projections, a_q.device)
    if a_scale.numel() != m * (k // 128):
        raise ValueError("a_scale does not match a_q")
    st = load().w8a8_block_gemm_grouped(_dev(a_q, "a_q", _U8),
                                        _dev(a_scale, "a_scale", torch.float32), arr,
                                        len(projections), m, k,
                                        current_stream(a_q.device) if stream is None else stream)
    check("w8a8_block_gemm_grouped", st)
    return outs


def w8a16_block_gemv(a: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                     out: torch.Tensor | None = None, ldc: int | None = None,
                     stream: int | None = None) -> torch.Tensor:
    """bf16 a [m <= 4, k] x E4M3 w_q [n, k]^T with block scales -> bf16 out [m, ldc]."""
    m, k = a.shape
    n = w_q.shape[0]
    if w_q.shape[1] != k:
        raise ValueError("a and w_q disagree on k")
    if w_scale.numel() != (n // 128) * (k // 128):
        raise ValueError("w_scale does not match w_q")
    if out is None:
        ldc = n if ldc is None else ldc
        out = torch.empty((m, ldc), dtype=torch.bfloat16, device=a.device)
    else:
        ldc = out.shape[-1] if ldc is None else ldc
        if out.numel() < (m - 1) * ldc + n:
            raise ValueError("out is smaller than (m - 1) * ldc + n elements")
    st = load().w8a16_block_gemv(_dev(a, "a", _BF16), _dev(w_q, "w_q", _U8),
                                 _dev(w_scale, "w_scale", torch.float32), _dev(out, "out", _BF16),
                                 m, n, k, ldc, current_stream(a.device) if stream is None else stream)
    check("w8a16_block_gemv", st)
    return out


def w8a16_block_gemv_grouped(a: torch.Tensor, projections, stream: int | None = None):
    """One launch of the W8A16 tier over several projections of the same bf16 activation."""
    m, k = a.shape
    arr, outs = _proj_array(m, k, projections, a.device)
    st = load().w8a16_block_gemv_grouped(_dev(a, "a", _BF16), arr, len(projections), m, k,
                                         current_stream(a.device) if stream is None else stream)
    check("w8a16_block_gemv_grouped", st)
    return outs


def fp8_quant_w8a8_gemm_grouped(a: torch.Tensor, projections, q: torch.Tensor | None = None,
                                scales: torch.Tensor | None = None,
                                stream: int | None = None):
    """bf16 activation [m, k] -> group quant fused into the grouped GEMM (one launch).
    q / scales, if given, receive the codes and scales fp8_group_quant would produce."""
    m, k = a.shape
    arr, outs = _proj_array(m, k, projections, a.device)
    if (q is None) != (scales is None):
        raise ValueError("pass both q and scales, or neither")
    qp = _dev(q, "q", _U8) if q is not None else None
    sp = _dev(scales, "scales", torch.float32) if scales is not None else None
    if q is not None and (q.numel() < m * k or scales.numel() < m * (k // 128)):
        raise ValueError("q / scales too small")
    st = load().fp8_quant_w8a8_gemm_grouped(_dev(a, "a", _BF16), qp, sp, arr, len(projections),
                                            m, k,
                                            current_stream(a.device) if stream is None else stream)
    check("fp8_quant_w8a8_gemm_grouped", st)
    return outs


def _room(t: torch.Tensor) -> int:
    """Elements a kernel may address from t.data_ptr(): the tensor itself when contiguous,
    else the rest of its storage (row views of a wider buffer)."""
    if t.is_contiguous():
        return t.numel()
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _kv_num_blocks(k_cache, v_cache, cache_stride) -> int:
    if k_cache.numel() != v_cache.numel() or k_cache.numel() % cache_stride:
        raise ValueError("pools must be equal and a whole number of blocks")
    return k_cache.numel() // cache_stride


def _kv_tokens(slot_mapping, num_tokens) -> int:
    t = slot_mapping.numel() if num_tokens is None else num_tokens
    if t > slot_mapping.numel():
        raise ValueError(f"num_tokens ({t}) exceeds slot_mapping ({slot_mapping.numel()} slots)")
    return t


def _kv_rows_fit(pairs, t, e) -> None:
    for name, rows, stride in pairs:
        if t > 0 and _room(rows) < (t - 1) * stride + e:
            raise ValueError(f"{name} is smaller than its {t} rows")


def _kv_write(fn, k, v, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim, block_size,
              k_scale, v_scale, key_stride, value_stride, cache_stride, num_tokens, stream,
              amax2=None):
    e = num_kv_heads * head_dim
    t = _kv_tokens(slot_mapping, num_tokens)
    key_stride = e if key_stride is None else key_stride
    value_stride = e if value_stride is None else value_stride
    cache_stride = block_size * e if cache_stride is None else cache_stride
    num_blocks = _kv_num_blocks(k_cache, v_cache, cache_stride)
    _kv_rows_fit((("k", k, key_stride), ("v", v, value_stride)), t, e)
    st = getattr(load(), fn)(_dev(k, "k", _BF16, False), _dev(v, "v", _BF16, False),
                             _dev(k_cache, "k_cache", _U8), _dev(v_cache, "v_cache", _U8),
                             _dev(slot_mapping, "slot_mapping", torch.int64), t, num_kv_heads,
                             head_dim, block_size, num_blocks, k_scale, v_scale, key_stride,
                             value_stride, cache_stride,
                             *(() if amax2 is None else (_dev(amax2, "amax2", torch.float32),)),
                             current_stream(k.device) if stream is None else stream)
    check(fn, st)


def fp8_kv_write(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                 v_cache: torch.Tensor, slot_mapping: torch.Tensor, num_kv_heads: int,
                 head_dim: int, block_size: int, k_scale: float, v_scale: float,
                 key_stride: int | None = None, value_stride: int | None = None,
                 cache_stride: int | None = None, num_tokens: int | None = None,
                 stream: int | None = None) -> None:
    """Slot-mapped E4M3 scatter of bf16 K/V rows into paged pools [blocks, bs*H*D]."""
    _kv_write("fp8_kv_write", k, v, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
              block_size, k_scale, v_scale, key_stride, value_stride, cache_stride,
              num_tokens, stream)


def fp8_kv_write_amax(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor, num_kv_heads: int,
                      head_dim: int, block_size: int, k_scale: float, v_scale: float,
                      amax2: torch.Tensor, key_stride: int | None = None,
                      value_stride: int | None = None, cache_stride: int | None = None,
                      num_tokens: int | None = None, stream: int | None = None) -> torch.Tensor:
    """fp8_kv_write plus the batch's max|K|, max|V| folded into amax2, in one pass."""
    if amax2.numel() < 2:
        raise ValueError("amax2 holds two floats")
    _kv_write("fp8_kv_write_amax", k, v, k_cache, v_cache, slot_mapping, num_kv_heads,
              head_dim, block_size, k_scale, v_scale, key_stride, value_stride, cache_stride,
              num_tokens, stream, amax2=amax2)
    return amax2


def fp8_kv_read(k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                num_kv_heads: int, head_dim: int, block_size: int, k_scale: float,
                v_scale: float, k_out: torch.Tensor | None = None,
                v_out: torch.Tensor | None = None, out_key_stride: int | None = None,
                out_value_stride: int | None = None, cache_stride: int | None = None,
                num_tokens: int | None = None, stream: int | None = None):
    """Dequantizing gather of paged E4M3 K/V back to bf16 rows (k_out, v_out); rows of
    tokens whose slot is out of range are left as they were (zeros when allocated here)."""
    e = num_kv_heads * head_dim
    t = _kv_tokens(slot_mapping, num_tokens)
    out_key_stride = e if out_key_stride is None else out_key_stride
    out_value_stride = e if out_value_stride is None else out_value_stride
    cache_stride = block_size * e if cache_stride is None else cache_stride
    num_blocks = _kv_num_blocks(k_cache, v_cache, cache_stride)
    if k_out is None:
        k_out = torch.zeros((t, out_key_stride), dtype=torch.bfloat16, device=k_cache.device)
    if v_out is None:
        v_out = torch.zeros((t, out_value_stride), dtype=torch.bfloat16, device=k_cache.device)
    _kv_rows_fit((("k_out", k_out, out_key_stride), ("v_out", v_out, out_value_stride)), t, e)
    st = load().fp8_kv_read(_dev(k_cache, "k_cache", _U8), _dev(v_cache, "v_cache", _U8),
                            _dev(slot_mapping, "slot_mapping", torch.int64), t, num_kv_heads,
                            head_dim, block_size, num_blocks, k_scale, v_scale,
                            _dev(k_out, "k_out", _BF16, False), _dev(v_out, "v_out", _BF16, False),
                            out_key_stride, out_value_stride, cache_stride,
                            current_stream(k_cache.device) if stream is None else stream)
    check("fp8_kv_read", st)
    return k_out, v_out


def fp8_kv_amax(k: torch.Tensor, v: torch.Tensor, amax2: torch.Tensor,
                stream: int | None = None) -> torch.Tensor:
    """amax2[0] = max(amax2[0], max|k|), amax2[1] = max(amax2[1], max|v|) (packed k, v)."""
    if k.numel() != v.numel() or amax2.numel() < 2:
        raise ValueError("k and v must have equal sizes; amax2 holds two floats")
    st = load().fp8_kv_amax(_dev(k, "k", _BF16), _dev(v, "v", _BF16), k.numel(),
                            _dev(amax2, "amax2", torch.float32),
                            current_stream(k.device) if stream is None else stream)
    check("fp8_kv_amax", st)
    return amax2


class KvCalibrator:
    """One attention layer's online FP8 KV scale calibration (fp8q_kv_calib_*).  `ops`, if
    given, is a KvCalibOps table the library calls for the calibrator's device work (kept
    referenced here for the calibrator's lifetime); by default the library's HIP path."""

    def __init__(self, window_tokens: int, headroom: float = 1.0,
                 provisional_scale: float = 2.0, ops: KvCalibOps | None = None):
        lib = load()
        h = ctypes.c_void_p()
        if ops is None:
            st = lib.fp8q_kv_calib_create(window_tokens, headroom, provisional_scale,
                                          ctypes.byref(h))
        else:
            st = lib.fp8q_kv_calib_create_with_ops(window_tokens, headroom, provisional_scale,
                                                   ctypes.byref(ops), ctypes.byref(h))
        check("fp8q_kv_calib_create", st)
        self._h = h.value
        self._ops = ops

    def decide(self, num_tokens: int, elems_per_token: int) -> int:
        st = load().fp8q_kv_calib_decide(self._h, num_tokens, elems_per_token)
        if st < 0:
            check("fp8q_kv_calib_decide", st)
        return st

    def observe(self, k: torch.Tensor, v: torch.Tensor, num_kv_heads: int, head_dim: int,
                k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                block_size: int, key_stride: int | None = None,
                value_stride: int | None = None, cache_stride: int | None = None,
                stream: int | None = None) -> None:
        """Fold the batch of slot_mapping.numel() tokens in (k, v rows at their strides);
        the freeze replays into k_cache / v_cache."""
        e = num_kv_heads * head_dim
        cs = block_size * e if cache_stride is None else cache_stride
        ks = e if key_stride is None else key_stride
        vs = e if value_stride is None else value_stride
        t = slot_mapping.numel()
        num_blocks = _kv_num_blocks(k_cache, v_cache, cs)
        _kv_rows_fit((("k", k, ks), ("v", v, vs)), t, e)
        tgt = KvTarget(k_pool=_dev(k_cache, "k_cache", _U8),
                       v_pool=_dev(v_cache, "v_cache", _U8),
                       slot_mapping=_dev(slot_mapping, "slot_mapping", torch.int64),
                       block_size=block_size, key_stride=ks, value_stride=vs, reserved=0,
                       cache_stride=cs, num_blocks=num_blocks)
        st = load().fp8q_kv_calib_observe(
            self._h, _dev(k, "k", _BF16, False), _dev(v, "v", _BF16, False), t, num_kv_heads,
            head_dim, ctypes.byref(tgt), current_stream(k.device) if stream is None else stream)
        check("fp8q_kv_calib_observe", st)

    def scales(self):
        ks, vs = ctypes.c_float(), ctypes.c_float()
        check("fp8q_kv_calib_scales",
              load().fp8q_kv_calib_scales(self._h, ctypes.byref(ks), ctypes.byref(vs)))
        return ks.value, vs.value

    def info(self) -> dict:
        inf = KvCalibInfo()
        check("fp8q_kv_calib_state", load().fp8q_kv_calib_state(self._h, ctypes.byref(inf)))
        return {name: getattr(inf, name) for name, _ in KvCalibInfo._fields_}

    def close(self) -> None:
        if self._h:
            load().fp8q_kv_calib_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
