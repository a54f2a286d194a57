"""CPU checks of the Python binding's extent checks: shapes that would let a kernel read or
write past a buffer are refused with ValueError before any pointer reaches the library (the
checks run before the tensors' device is even looked at, so CPU tensors exercise them)."""
import pytest
import torch

import fp8_e4m3_quantization_amd as fq

H, D, BS = 4, 128, 16
E = H * D
CS = BS * E


def _kv(t=8, blocks=4):
    k = torch.zeros((t, E), dtype=torch.bfloat16)
    v = torch.zeros((t, E), dtype=torch.bfloat16)
    kc = torch.zeros(blocks * CS, dtype=torch.uint8)
    vc = torch.zeros(blocks * CS, dtype=torch.uint8)
    slots = torch.arange(t, dtype=torch.int64)
    return k, v, kc, vc, slots


@pytest.mark.parametrize("fn", ["fp8_kv_write", "fp8_kv_write_amax"])
def test_write_refuses_more_tokens_than_slots(fn):
    k, v, kc, vc, slots = _kv()
    extra = (torch.zeros(2),) if fn == "fp8_kv_write_amax" else ()
    with pytest.raises(ValueError, match="num_tokens"):
        getattr(fq, fn)(k, v, kc, vc, slots[:4], H, D, BS, 1.0, 1.0, *extra, num_tokens=8)


def test_write_refuses_short_rows_and_unequal_pools():
    k, v, kc, vc, slots = _kv()
    with pytest.raises(ValueError, match="v is smaller"):
        fq.fp8_kv_write(k, v[:7], kc, vc, slots, H, D, BS, 1.0, 1.0)
    with pytest.raises(ValueError, match="k is smaller"):
        fq.fp8_kv_write(k, v, kc, vc, slots, H, D, BS, 1.0, 1.0, key_stride=E + 8)
    with pytest.raises(ValueError, match="pools"):
        fq.fp8_kv_write(k, v, kc, vc[:-CS], slots, H, D, BS, 1.0, 1.0)
    with pytest.raises(ValueError, match="pools"):
        fq.fp8_kv_write(k, v, kc[:-1], vc[:-1], slots, H, D, BS, 1.0, 1.0)


def test_read_refuses_more_tokens_than_slots_and_short_outputs():
    k, v, kc, vc, slots = _kv()
    with pytest.raises(ValueError, match="num_tokens"):
        fq.fp8_kv_read(kc, vc, slots[:2], H, D, BS, 1.0, 1.0, num_tokens=3)
    with pytest.raises(ValueError, match="v_out is smaller"):
        fq.fp8_kv_read(kc, vc, slots, H, D, BS, 1.0, 1.0, k_out=k, v_out=v[:5])
    with pytest.raises(ValueError, match="pools"):
        fq.fp8_kv_read(kc, vc[:CS], slots, H, D, BS, 1.0, 1.0, k_out=k, v_out=v)


def test_calibrator_observe_checks_pools_and_rows_before_the_library():
    """The freeze replays into the pools with num_blocks taken from k_cache: a smaller
    v_cache, a pool that is not whole blocks, or K/V with fewer rows than the batch's slots
    must be refused on the host."""
    cal = fq.KvCalibrator(256)
    k, v, kc, vc, slots = _kv()
    try:
        with pytest.raises(ValueError, match="pools"):
            cal.observe(k, v, H, D, kc, vc[:CS], slots, BS)
        with pytest.raises(ValueError, match="pools"):
            cal.observe(k, v, H, D, kc[:-8], vc[:-8], slots, BS)
        with pytest.raises(ValueError, match="k is smaller"):
            cal.observe(k[:7], v, H, D, kc, vc, slots, BS)
        with pytest.raises(ValueError, match="v is smaller"):
            cal.observe(k, v, H, D, kc, vc, slots, BS, value_stride=E + 64)
        assert cal.info()["tokens_seen"] == 0
    finally:
        cal.close()


def test_strided_row_views_are_measured_by_their_storage():
    """A column view of a wider buffer may address the rest of that buffer's storage."""
    wide = torch.zeros((8, 2 * E), dtype=torch.bfloat16)
    k = wide[:, :E]
    assert fq._lib._room(k) == 8 * 2 * E
    assert fq._lib._room(wide[2:, :E]) == 6 * 2 * E
