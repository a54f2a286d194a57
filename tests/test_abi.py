"""CPU checks of the C-ABI boundary: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before anything is enqueued (these calls
never reach the GPU, so they run without one)."""
import ctypes
import os
import re

import pytest

import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

EINVAL, ENULL, EALIGN = -1, -2, -3
FAKE = 0x100000  # an aligned, never-dereferenced address: the checks return first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    text = re.sub(r"typedef struct \w+ \{.*?\} \w+;", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{()]*\)\s*;", text)))


def test_library_exports_every_declared_symbol():
    lib = fq.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    lib = fq.load()
    assert lib.fp8q_version() == 10200
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert fq.strerror(code) and fq.strerror(code) != "unknown status"
    assert fq.strerror(-99) == "unknown status"


def test_group_quant_argument_checks():
    lib = fq.load()
    assert lib.fp8_group_quant(FAKE, FAKE, FAKE, 4, 100, None) == EINVAL
    assert lib.fp8_group_quant(FAKE, FAKE, FAKE, 4, 0, None) == EINVAL
    assert lib.fp8_group_quant(FAKE, FAKE, FAKE, -1, 128, None) == EINVAL
    assert lib.fp8_group_quant(FAKE, FAKE, FAKE, 1 << 60, 1 << 20, None) == EINVAL
    assert lib.fp8_group_quant(None, FAKE, FAKE, 4, 128, None) == ENULL
    assert lib.fp8_group_quant(FAKE + 2, FAKE, FAKE, 4, 128, None) == EALIGN
    assert lib.fp8_group_quant(FAKE, FAKE + 8, FAKE, 4, 128, None) == EALIGN
    assert lib.fp8_group_quant(None, None, None, 0, 128, None) == 0  # m == 0: no-op


def test_gemm_argument_checks():
    lib = fq.load()
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE)
    for m, n, k, ldc in [(0, 128, 128, 128), (17, 128, 128, 128), (4, 192, 128, 192),
                         (4, 128, 192, 128), (4, 256, 128, 255), (4, 128, 131072 + 128, 128),
                         (4, -128, 128, 128)]:
        assert lib.w8a8_block_gemm(*ok, m, n, k, ldc, None) == EINVAL, (m, n, k, ldc)
    assert lib.w8a8_block_gemm(FAKE, FAKE, None, FAKE, FAKE, 4, 128, 128, 128, None) == ENULL
    assert lib.w8a8_block_gemm(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 4, 128, 128, 128, None) == EALIGN
    assert lib.w8a8_block_gemm(FAKE, FAKE, FAKE, FAKE, FAKE + 1, 4, 128, 128, 128, None) == EALIGN


def test_grouped_launches_take_one_to_eight_projections():
    """count outside [1, 8] is refused before anything is read or launched, by all three
    grouped entry points; a NULL projection table is ENULL."""
    lib = fq.load()
    projs = (_lib.GemmProj * 9)(*[_lib.GemmProj(FAKE, FAKE, FAKE, 128, 128) for _ in range(9)])
    for count in (0, 9, -1):
        assert lib.w8a8_block_gemm_grouped(FAKE, FAKE, projs, count, 4, 128, None) == EINVAL
        assert lib.fp8_quant_w8a8_gemm_grouped(FAKE, FAKE, FAKE, projs, count, 4, 128,
                                               None) == EINVAL
        assert lib.w8a16_block_gemv_grouped(FAKE, projs, count, 2, 128, None) == EINVAL
    assert lib.w8a8_block_gemm_grouped(FAKE, FAKE, None, 2, 4, 128, None) == ENULL
    assert lib.w8a16_block_gemv_grouped(FAKE, None, 2, 2, 128, None) == ENULL
    bad = (_lib.GemmProj * 2)(_lib.GemmProj(FAKE, FAKE, FAKE, 128, 128),
                              _lib.GemmProj(FAKE, FAKE, FAKE, 100, 128))
    assert lib.w8a8_block_gemm_grouped(FAKE, FAKE, bad, 2, 4, 128, None) == EINVAL


def test_workspace_gemm_and_reference_argument_checks():
    lib = fq.load()
    b = ctypes.c_uint64(7)
    assert lib.w8a8_block_gemm_workspace_size(16, 1024, 5120, None) == ENULL
    for m, n, k in [(0, 1024, 5120), (17, 1024, 5120), (16, 1000, 5120), (16, 1024, 5000),
                    (16, 1024, 131072 + 128)]:
        assert lib.w8a8_block_gemm_workspace_size(m, n, k, ctypes.byref(b)) == EINVAL
        assert b.value == 0
    assert lib.w8a8_block_gemm_workspace_size(16, 16384, 5120, ctypes.byref(b)) == 0
    assert b.value == 0  # enough strips: no split, no workspace
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.w8a8_block_gemm_ws(*ok, 17, 1024, 5120, 1024, FAKE, 1 << 30, None) == EINVAL
    assert lib.w8a8_block_gemm_ws(*ok, 16, 1024, 5120, 1000, FAKE, 1 << 30, None) == EINVAL
    assert lib.w8a8_block_gemm_ws(FAKE, None, FAKE, FAKE, FAKE, 16, 1024, 5120, 1024, FAKE,
                                  1 << 30, None) == ENULL
    assert lib.fp8q_reference_stream(FAKE, FAKE, 24, None) == EINVAL
    assert lib.fp8q_reference_stream(None, FAKE, 32, None) == ENULL
    assert lib.fp8q_reference_stream(FAKE + 8, FAKE, 32, None) == EALIGN
    assert lib.fp8q_reference_stream(None, None, 0, None) == 0
    assert lib.fp8q_reference_lds_stream(FAKE, 65536 + 16, 65536, None) == EINVAL
    assert lib.fp8q_reference_lds_stream(FAKE, 65536, 1000, None) == EINVAL
    assert lib.fp8q_reference_lds_stream(FAKE, 0x7FFF0000 + 65536, 65536, None) == EINVAL
    assert lib.fp8q_reference_lds_stream(None, 65536, 65536, None) == ENULL
    assert lib.fp8q_reference_lds_stream(FAKE + 8, 65536, 65536, None) == EALIGN
    assert lib.fp8q_reference_lds_stream(None, 65536, 0, None) == 0


def test_kv_write_argument_checks():
    lib = fq.load()
    p = (FAKE, FAKE, FAKE, FAKE, FAKE)
    good = dict(t=4, h=4, d=128, bs=16, nb=8, ks=2.0, vs=2.0, kst=512, vst=512, cs=8192)

    def call(ptrs=p, **over):
        a = dict(good, **over)
        return lib.fp8_kv_write(*ptrs, a["t"], a["h"], a["d"], a["bs"], a["nb"], a["ks"],
                                a["vs"], a["kst"], a["vst"], a["cs"], None)

    for over in [dict(t=-1), dict(h=0), dict(d=0), dict(bs=0), dict(nb=0), dict(kst=511),
                 dict(vst=100), dict(cs=8191), dict(ks=0.0), dict(vs=-1.0),
                 dict(ks=float("nan")), dict(vs=float("inf")), dict(ks=2.0 ** -65),
                 dict(vs=2.0 ** 65), dict(nb=1 << 62)]:
        assert call(**over) == EINVAL, over
    assert call(ptrs=(FAKE, None, FAKE, FAKE, FAKE)) == ENULL
    assert call(ptrs=(FAKE, FAKE, FAKE, FAKE, FAKE + 4)) == EALIGN
    assert call(ptrs=(None,) * 5, t=0) == 0  # zero tokens: no-op


def test_kv_amax_argument_checks():
    lib = fq.load()
    assert lib.fp8_kv_amax(FAKE, FAKE, -1, FAKE, None) == EINVAL
    assert lib.fp8_kv_amax(None, FAKE, 8, FAKE, None) == ENULL
    assert lib.fp8_kv_amax(FAKE, FAKE, 8, FAKE + 2, None) == EALIGN
    assert lib.fp8_kv_amax(None, None, 0, None, None) == 0


def test_encode_and_block_quant_argument_checks():
    lib = fq.load()
    assert lib.fp8_e4m3_encode(FAKE, FAKE, -1, None) == EINVAL
    assert lib.fp8_e4m3_encode(None, FAKE, 4, None) == ENULL
    assert lib.fp8_e4m3_encode(None, None, 0, None) == 0
    assert lib.fp8_block_quant(FAKE, FAKE, FAKE, 0, 128, None) == EINVAL
    assert lib.fp8_block_quant(FAKE, None, FAKE, 128, 128, None) == ENULL


def test_calibrator_host_logic_without_gpu():
    """create / decide / scales / info / destroy never touch the device."""
    lib = fq.load()
    h = ctypes.c_void_p()
    assert lib.fp8q_kv_calib_create(0, 1.0, 2.0, ctypes.byref(h)) == EINVAL  # window 0: none
    assert lib.fp8q_kv_calib_create(8, float("nan"), 2.0, ctypes.byref(h)) == EINVAL
    assert lib.fp8q_kv_calib_create(8, 1.0, 2.0, None) == ENULL
    cal = fq.KvCalibrator(10 ** 6, 0.25)
    info = cal.info()
    assert info["window_tokens"] == 4096 and info["requested_tokens"] == 10 ** 6
    assert info["headroom"] == 1.0 and info["frozen"] == 0
    assert cal.scales() == (2.0, 2.0) and info["provisional_scale"] == 2.0
    assert cal.decide(4095, 512) == fq.FP8Q_CALIB_STAGE
    assert cal.decide(4096, 512) == fq.FP8Q_CALIB_FREEZE
    with pytest.raises(fq.Fp8qError):
        cal.decide(-1, 512)
    cal.close()
    one = fq.KvCalibrator(1)
    assert one.decide(1, 512) == fq.FP8Q_CALIB_FREEZE
    one.close()
    w = fq.KvCalibrator(256)
    tgt = _lib.KvTarget(k_pool=FAKE, v_pool=FAKE, slot_mapping=FAKE, block_size=16,
                        key_stride=511, value_stride=512, reserved=0, cache_stride=8192,
                        num_blocks=8)
    assert lib.fp8q_kv_calib_observe(w._h, FAKE, FAKE, 4, 4, 128, ctypes.byref(tgt),
                                     None) == EINVAL
    assert lib.fp8q_kv_calib_observe(w._h, FAKE, FAKE, 4, 4, 128, None, None) == ENULL
    tgt.key_stride = 512
    assert lib.fp8q_kv_calib_observe(w._h, FAKE, FAKE, 0, 4, 128, ctypes.byref(tgt), None) == 0
    assert w.info()["tokens_seen"] == 0
    w.close()
    lib.fp8q_kv_calib_destroy(None)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libfp8q.so"))
    with pytest.raises(ImportError):
        _lib.load()
