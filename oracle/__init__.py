"""CPU oracle for the FP8 (OCP E4M3) quantize-and-consume path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg
may import this package.  The product path (the HIP library and its Python binding) never
does, and the two share no code: this file wraps the plain C in ``fp8_oracle.c`` with
numpy arrays.  Every function states the passage of the pages it follows in the C source.

Functions (single-threaded, in the order the pages define them; the *_rows wrappers run the
same C routine on disjoint row ranges in parallel threads, so every element is computed by
exactly the arithmetic of the single-threaded call):
  e4m3_decode(codes)                 -> float64 values (NaN for S.1111.111)
  e4m3_encode(v), e4m3_encode_search(v) -> uint8 codes (two independent encoders)
  group_quant(x_bf16[m,k])           -> (q uint8[m,k], scales f32[m,k/128])
  block_quant(w_bf16[n,k])           -> (wq uint8[n,k], ws f32[ceil(n/128),ceil(k/128)])
  gemm(a_q, a_s, w_q, w_s)           -> float64[m,n] reference
  gemm_rows(a_q, a_s, w_q, w_s, threads) the same, rows split over host threads
  group_quant_rows(x_bf16, threads)  group_quant, rows split over host threads
  gemm_w8a16(a_bf16, w_q, w_s)       -> (float64[m,n] reference, float64[m,n] sum of |terms|)
  amax(x_bf16)                       -> float32
  kv_write(...)                      in-place on the uint8 pools
  kv_read(...)                       dequantizing gather of a paged history to bf16
  Calibrator                         one layer's online scale calibration model
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b

        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode_bits.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_bits.argtypes = [_f32]
    lib.oracle_e4m3_encode_search.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_search.argtypes = [_f32]
    lib.oracle_e4m3_encode_bits_n.argtypes = [_p, _p, _i64]
    lib.oracle_e4m3_encode_search_n.argtypes = [_p, _p, _i64]
    lib.oracle_e4m3_sweep_compare.restype = _i64
    lib.oracle_e4m3_sweep_compare.argtypes = [ctypes.c_uint32, ctypes.c_uint32,
                                              ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_group_quant.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_block_quant.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_gemm.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p]
    lib.oracle_gemm_w8a16.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
    lib.oracle_amax.argtypes = [_p, _i64, _p]
    lib.oracle_kv_write.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f32, _f32,
                                    _i64, _i64, _i64]
    lib.oracle_kv_read.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _f32, _f32, _p, _p,
                                   _i64, _i64, _i64]
    lib.oracle_calib_create.restype = _p
    lib.oracle_calib_create.argtypes = [_i64, _f32, _f32]
    lib.oracle_calib_destroy.argtypes = [_p]
    lib.oracle_calib_observe_and_write.restype = ctypes.c_int
    lib.oracle_calib_observe_and_write.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64,
                                                   _i64, _p, _p]
    lib.oracle_calib_info.argtypes = [_p, _p, _p]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle takes C-contiguous arrays"
    return a.ctypes.data


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 data is passed as its uint16 bit pattern"
    return a


# ------------------------------------------------------------------------------ E4M3


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    out = np.array([lib.oracle_e4m3_decode(int(b)) for b in range(256)], dtype=np.float64)
    return out[c].reshape(np.shape(codes))


def e4m3_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_e4m3_decode(b) for b in range(256)], dtype=np.float64)


def e4m3_encode(v) -> np.ndarray:
    """Encoder (i): binary32 bit surgery, round-to-nearest-even, saturating at 448."""
    lib = _load()
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_bits_n(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_encode_search(v) -> np.ndarray:
    """Encoder (ii): search of the sorted decode table with an explicit tie rule."""
    lib = _load()
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_search_n(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_sweep_compare(lo_bits: int, hi_bits: int):
    """Mismatch count of encoders (i) and (ii) over binary32 patterns [lo, hi], both signs."""
    lib = _load()
    first = ctypes.c_uint32(0)
    bad = lib.oracle_e4m3_sweep_compare(lo_bits, hi_bits, ctypes.byref(first))
    return int(bad), int(first.value)


# ----------------------------------------------------------------------- quantizers


def group_quant(x_bf16):
    lib = _load()
    x = _u16(x_bf16)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.uint8)
    s = np.empty((m, k // 128), dtype=np.float32)
    lib.oracle_group_quant(_ptr(x), m, k, _ptr(q), _ptr(s))
    return q, s


def block_quant(w_bf16):
    lib = _load()
    w = _u16(w_bf16)
    n, k = w.shape
    wq = np.empty((n, k), dtype=np.uint8)
    ws = np.empty(((n + 127) // 128, (k + 127) // 128), dtype=np.float32)
    lib.oracle_block_quant(_ptr(w), n, k, _ptr(wq), _ptr(ws))
    return wq, ws


# ----------------------------------------------------------------------------- GEMM


def gemm(a_q, a_s, w_q, w_s) -> np.ndarray:
    lib = _load()
    a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    m, k = a_q.shape
    n = w_q.shape[0]
    assert w_q.shape[1] == k and a_s.shape == (m, k // 128)
    assert w_s.shape == ((n + 127) // 128, k // 128)
    ref = np.empty((m, n), dtype=np.float64)
    lib.oracle_gemm(_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), m, n, k, _ptr(ref))
    return ref


MAX_THREADS = 16  # a single-GPU host's CPU share


def default_threads() -> int:
    """Host threads the *_rows wrappers use by default: the CPUs this process may run on,
    at most MAX_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _row_ranges(m, threads):
    threads = max(1, min(int(threads or default_threads()), m))
    step = -(-m // threads)
    return [(r, min(m, r + step)) for r in range(0, m, step)]


def gemm_rows(a_q, a_s, w_q, w_s, threads=None) -> np.ndarray:
    """gemm() with the rows of the result split over `threads` host threads (default:
    default_threads()); each range is one call of the same C routine, which keeps no shared
    state, so the result equals gemm()'s bit for bit."""
    from concurrent.futures import ThreadPoolExecutor

    lib = _load()
    a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    m, k = a_q.shape
    n = w_q.shape[0]
    assert w_q.shape[1] == k and a_s.shape == (m, k // 128)
    assert w_s.shape == ((n + 127) // 128, k // 128)
    ref = np.empty((m, n), dtype=np.float64)

    def run(rng):
        r0, r1 = rng
        lib.oracle_gemm(a_q[r0:].ctypes.data, a_s[r0:].ctypes.data, _ptr(w_q), _ptr(w_s),
                        r1 - r0, n, k, ref[r0:].ctypes.data)

    with ThreadPoolExecutor(len(_row_ranges(m, threads))) as ex:
        list(ex.map(run, _row_ranges(m, threads)))
    return ref


def group_quant_rows(x_bf16, threads=None):
    """group_quant() with the rows split over `threads` host threads (default:
    default_threads()); equal to group_quant() bit for bit."""
    from concurrent.futures import ThreadPoolExecutor

    lib = _load()
    x = _u16(x_bf16)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.uint8)
    s = np.empty((m, k // 128), dtype=np.float32)

    def run(rng):
        r0, r1 = rng
        lib.oracle_group_quant(x[r0:].ctypes.data, r1 - r0, k, q[r0:].ctypes.data,
                               s[r0:].ctypes.data)

    with ThreadPoolExecutor(len(_row_ranges(m, threads))) as ex:
        list(ex.map(run, _row_ranges(m, threads)))
    return q, s


def gemm_w8a16(a_bf16, w_q, w_s):
    """bf16 activation x block-scaled E4M3 weight, in double: (ref, sum of |terms|)."""
    lib = _load()
    a = _u16(a_bf16)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    m, k = a.shape
    n = w_q.shape[0]
    assert w_q.shape[1] == k and w_s.shape == ((n + 127) // 128, k // 128)
    ref = np.empty((m, n), dtype=np.float64)
    mag = np.empty((m, n), dtype=np.float64)
    lib.oracle_gemm_w8a16(_ptr(a), _ptr(w_q), _ptr(w_s), m, n, k, _ptr(ref), _ptr(mag))
    return ref, mag


# ------------------------------------------------------------------------------- KV


def amax(x_bf16, acc: float = 0.0) -> np.float32:
    lib = _load()
    x = _u16(x_bf16)
    out = np.array([acc], dtype=np.float32)
    lib.oracle_amax(_ptr(x), x.size, _ptr(out))
    return out[0]


def kv_write(k_bf16, v_bf16, k_cache, v_cache, slots, num_tokens, num_kv_heads, head_dim,
             block_size, k_scale, v_scale, key_stride, value_stride, cache_stride):
    """Sequential slot-mapped writer; k_bf16/v_bf16 are flat uint16 arrays read at the
    given element strides; the pools are uint8 arrays updated in place."""
    lib = _load()
    kx = _u16(k_bf16)
    vx = _u16(v_bf16)
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    assert k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]
    _check_slots(sl[:num_tokens], k_cache, v_cache, block_size, cache_stride)
    lib.oracle_kv_write(_ptr(kx), _ptr(vx), _ptr(k_cache), _ptr(v_cache), _ptr(sl),
                        num_tokens, num_kv_heads, head_dim, block_size, k_scale, v_scale,
                        key_stride, value_stride, cache_stride)


def _check_slots(sl, k_cache, v_cache, block_size, cache_stride):
    """The writer indexes the pools with every non-negative slot: refuse slots past the end
    (the C code has no pool size to check against)."""
    nslots = min(k_cache.size, v_cache.size) // cache_stride * block_size
    assert np.all(sl < nslots), "slot past the end of the pools"


def kv_read(k_cache, v_cache, slots, num_kv_heads, head_dim, block_size, num_blocks, k_scale,
            v_scale, k_out, v_out, key_stride, value_stride, cache_stride):
    """Dequantizing gather of a paged history; k_out / v_out (uint16 bf16 bits) updated in place."""
    lib = _load()
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    assert k_out.dtype == np.uint16 and v_out.dtype == np.uint16
    assert k_out.flags["C_CONTIGUOUS"] and v_out.flags["C_CONTIGUOUS"]
    lib.oracle_kv_read(_ptr(k_cache), _ptr(v_cache), _ptr(sl), sl.size, num_kv_heads, head_dim,
                       block_size, num_blocks, k_scale, v_scale, _ptr(k_out), _ptr(v_out),
                       key_stride, value_stride, cache_stride)


class Calibrator:
    """One attention layer's online FP8 KV scale calibration (oracle model)."""

    STAGED, DECLINED, FROZE, FROZEN = 0, 1, 2, 3

    def __init__(self, window_tokens: int, headroom: float = 1.0,
                 provisional: float = 2.0):
        self._lib = _load()
        self._c = self._lib.oracle_calib_create(window_tokens, headroom, provisional)

    def observe_and_write(self, k_bf16, v_bf16, slots, num_kv_heads, head_dim, block_size,
                          cache_stride, k_cache, v_cache) -> int:
        kx = _u16(k_bf16)
        vx = _u16(v_bf16)
        sl = np.ascontiguousarray(slots, dtype=np.int64)
        _check_slots(sl, k_cache, v_cache, block_size, cache_stride)
        return self._lib.oracle_calib_observe_and_write(
            self._c, _ptr(kx), _ptr(vx), _ptr(sl), sl.size, num_kv_heads, head_dim,
            block_size, cache_stride, _ptr(k_cache), _ptr(v_cache))

    def info(self) -> dict:
        cnt = np.zeros(7, dtype=np.int64)
        val = np.zeros(5, dtype=np.float32)
        self._lib.oracle_calib_info(self._c, _ptr(cnt), _ptr(val))
        keys = ["window", "tokens_seen", "staged_tokens", "staged_batches",
                "unstaged_tokens", "replayed_tokens", "frozen"]
        d = {k: int(v) for k, v in zip(keys, cnt)}
        d.update(k_scale=val[0], v_scale=val[1], k_max=val[2], v_max=val[3],
                 headroom=val[4])
        return d

    def close(self):
        if self._c:
            self._lib.oracle_calib_destroy(self._c)
            self._c = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
