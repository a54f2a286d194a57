"""GPU parity of the persistent decode kernels' halved last round.  When the 16-column strips
leave a last round at most half full, its strips run as two 8-column items, each with an
8-row weight descriptor and only its own columns stored.

The shapes come from the device's CU count, so that the last round is a quarter full, half
full (both halved) and just over half full (not halved).  Each output is checked three ways:
  - against the FP64 oracle: W8A8 within 1e-2 |ref| + 1e-3 rms(ref); W8A16 within the
    bound derived in test_gpu_gemv;
  - bit for bit against a separate call on the last 512 columns' weights alone (32 strips,
    never halved): a column's arithmetic does not depend on the other columns;
  - for its extent, through a strided output whose padding must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import (DEV, bf16_dev, bf16_host_to_f64, f32_dev, gemm_tolerance_ok,
                            host, need_gpu, u8_dev)

pytestmark = pytest.mark.gpu
K = synth.DECODE_K
TAIL = 512  # columns recomputed alone


def setup_module(_):
    need_gpu()


def _n_for(last_round_strips):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rest = {"quarter": cus // 4, "half": cus // 2, "over_half": cus // 2 + 8}[last_round_strips]
    n = 16 * (2 * cus + rest)
    assert n % 128 == 0 and rest < cus
    return n


def _strided(n, m, fill):
    ldc = n + 40
    return torch.full((m * ldc,), fill, dtype=torch.bfloat16, device=DEV), ldc


def _rows(buf_bits, m, n, ldc):
    return np.stack([buf_bits[r * ldc:r * ldc + n] for r in range(m)])


def _padding_untouched(buf_bits, m, n, ldc, fill):
    mask = np.ones(buf_bits.size, dtype=bool)
    for r in range(m):
        mask[r * ldc:r * ldc + n] = False
    return bool(np.all(bf16_host_to_f64(buf_bits[mask]) == fill))


@pytest.mark.parametrize("last", ["quarter", "half", "over_half"])
@pytest.mark.parametrize("m", [16, 5])
def test_w8a8_halved_last_round(last, m):
    n = _n_for(last)
    a = synth.decode_activation(m, seed=6100 + m)
    wq, ws = oracle.block_quant(synth.decode_weight(n, K, seed=6200 + n))
    q, s = fq.fp8_group_quant(bf16_dev(a))
    buf, ldc = _strided(n, m, 3.0)
    fq.w8a8_block_gemm(q, s, u8_dev(wq), f32_dev(ws), out=buf, ldc=ldc)
    got_buf = host(buf)
    assert _padding_untouched(got_buf, m, n, ldc, 3.0)
    got = _rows(got_buf, m, n, ldc)
    q_ref, s_ref = oracle.group_quant(a)
    ok, worst = gemm_tolerance_ok(got, oracle.gemm(q_ref, s_ref, wq, ws))
    assert ok, f"worst error / bound = {worst:.3f}"
    alone = host(fq.w8a8_block_gemm(q, s, u8_dev(wq[n - TAIL:]),
                                    f32_dev(ws[(n - TAIL) // 128:])))
    assert np.array_equal(got[:, n - TAIL:], alone)


@pytest.mark.parametrize("last", ["quarter", "half", "over_half"])
def test_w8a8_fused_quant_halved_last_round(last):
    """The fused quantize + GEMM launch: codes and scales equal the quantizer's, outputs
    equal the unfused GEMM's bit for bit."""
    n, m = _n_for(last), 16
    a = synth.decode_activation(m, seed=6300)
    wq, ws = oracle.block_quant(synth.decode_weight(n, K, seed=6400 + n))
    wq_d, ws_d = u8_dev(wq), f32_dev(ws)
    q0, s0 = fq.fp8_group_quant(bf16_dev(a))
    plain = host(fq.w8a8_block_gemm(q0, s0, wq_d, ws_d))
    q = torch.empty((m, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((m, K // 128), dtype=torch.float32, device=DEV)
    (out,) = fq.fp8_quant_w8a8_gemm_grouped(bf16_dev(a), [(wq_d, ws_d, None)], q=q, scales=s)
    assert np.array_equal(host(q), host(q0)) and np.array_equal(host(s), host(s0))
    assert np.array_equal(host(out), plain)


def _within_w8a16(out_bits, ref, mag, k):
    got = bf16_host_to_f64(out_bits)
    bound = 2.0 ** -8 * np.abs(ref) + 2 * (k / 128 + 144) * 2.0 ** -24 * mag
    err = np.abs(got - ref)
    return bool(np.all(err <= bound)), float(np.max(err / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("last", ["quarter", "half", "over_half"])
@pytest.mark.parametrize("m", [1, 4])
def test_w8a16_halved_last_round(last, m):
    n = _n_for(last)
    a = synth.decode_activation(m, seed=6500 + m)
    wq, ws = oracle.block_quant(synth.decode_weight(n, K, seed=6600 + n))
    buf, ldc = _strided(n, m, -5.0)
    fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws), out=buf, ldc=ldc)
    got_buf = host(buf)
    assert _padding_untouched(got_buf, m, n, ldc, -5.0)
    got = _rows(got_buf, m, n, ldc)
    ref, mag = oracle.gemm_w8a16(a, wq, ws)
    ok, worst = _within_w8a16(got, ref, mag, K)
    assert ok, f"worst error / bound = {worst:.3f}"
    alone = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq[n - TAIL:]),
                                     f32_dev(ws[(n - TAIL) // 128:])))
    assert np.array_equal(got[:, n - TAIL:], alone)
