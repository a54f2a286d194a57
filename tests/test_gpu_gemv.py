"""GPU parity: the W8A16 decode tier (bf16 activation x block-scaled E4M3 weight, 1..4 rows)
against the FP64 oracle.

Bar, from the arithmetic: the products are exact in FP32 and every output is a sum of k of
them, accumulated in FP32 in at most k/128 + 144 rounded additions (a group's partial, its
scaling, the groups of a wave's K-slice, the 8 slices), then rounded once to bf16.  So
    |gpu - ref| <= 2^-8 |ref| + 2 (k/128 + 144) 2^-24 S,   S = sum_k |term|
(the first part covers the bf16 rounding, the second the FP32 accumulation with a factor 2
of margin).  Bit-exact where the sum is exact (small integers); a row's bits do not depend
on how many rows the call has."""
import numpy as np
import pytest

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import DEV, bf16_dev, bf16_host_to_f64, f32_dev, host, need_gpu, u8_dev

pytestmark = pytest.mark.gpu


def setup_module(_):
    need_gpu()


def _within(out_bits, ref, mag, k):
    got = bf16_host_to_f64(out_bits)
    bound = 2.0 ** -8 * np.abs(ref) + 2 * (k / 128 + 144) * 2.0 ** -24 * mag
    err = np.abs(got - ref)
    return bool(np.all(err <= bound)), float(np.max(err / np.maximum(bound, 1e-300)))


_W = {}


def _weights(n, k, seed):
    if (n, k, seed) not in _W:
        _W.clear()
        _W[(n, k, seed)] = oracle.block_quant(synth.decode_weight(n, k, seed=seed))
    return _W[(n, k, seed)]


@pytest.mark.parametrize("n", synth.DECODE_N)
@pytest.mark.parametrize("m", [1, 4])
def test_decode_projections_within_bound(n, m):
    k = synth.DECODE_K
    wq, ws = _weights(n, k, 2100 + n)
    a = synth.decode_activation(m, seed=2200 + m)
    out = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws)))
    ref, mag = oracle.gemm_w8a16(a, wq, ws)
    ok, worst = _within(out, ref, mag, k)
    assert ok, f"worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("m", [2, 3])
@pytest.mark.parametrize("k", [128, 384, 1152, 8192, 8320, 16384, 20608])
def test_row_counts_and_ragged_k(m, k):
    """k <= 8192 runs the persistent kernel, longer k the per-strip long-K kernel (20608 =
    161 groups: the 8 waves' slices and their last 4-group chunks are uneven)."""
    n = 384
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=k + m))
    a = synth.decode_activation(m, k=k, seed=k * 3 + m)
    out = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws)))
    ref, mag = oracle.gemm_w8a16(a, wq, ws)
    ok, worst = _within(out, ref, mag, k)
    assert ok, f"worst error / bound = {worst:.3f}"


def test_longest_k_within_bound():
    k, n, m = 131072, 128, 4
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=41))
    a = synth.decode_activation(m, k=k, seed=42)
    out = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws)))
    ref, mag = oracle.gemm_w8a16(a, wq, ws)
    ok, worst = _within(out, ref, mag, k)
    assert ok, f"worst error / bound = {worst:.3f}"


def test_small_integer_sums_are_exact():
    """Sums of small multiples of 1/4: every one the oracle finds bf16-representable must
    come back bit for bit (and nearly all are)."""
    rng = np.random.default_rng(31)
    m, n, k = 4, 512, 512
    a = synth.to_bf16_bits(rng.integers(-1, 2, size=(m, k)).astype(np.float64))
    code = np.array([0x00, 0x00, 0x00, 0x38, 0xB8, 0x40, 0xC0], dtype=np.uint8)  # 0,1,-1,2,-2
    wq = code[rng.integers(0, len(code), size=(n, k))]
    ws = (2.0 ** rng.integers(-2, 1, size=(n // 128, k // 128))).astype(np.float32)
    out = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws)))
    ref, _ = oracle.gemm_w8a16(a, wq, ws)
    rep = bf16_host_to_f64(synth.to_bf16_bits(ref)) == ref
    assert rep.mean() > 0.99
    assert np.array_equal(bf16_host_to_f64(out)[rep], ref[rep])


def test_identity_weight_returns_the_activation():
    rng = np.random.default_rng(6)
    k = 1024
    a = synth.to_bf16_bits(rng.normal(0, 7, size=(3, k)))
    wq = np.zeros((k, k), dtype=np.uint8)
    np.fill_diagonal(wq, 0x38)
    out = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(np.ones((8, 8), np.float32))))
    assert np.array_equal(out, a)


def test_a_row_does_not_depend_on_the_row_count():
    k, n = synth.DECODE_K, 1024
    wq, ws = _weights(n, k, 2100 + n)
    a = synth.decode_activation(4, seed=77)
    w, s = u8_dev(wq), f32_dev(ws)
    four = host(fq.w8a16_block_gemv(bf16_dev(a), w, s))
    for m in (1, 2, 3):
        part = host(fq.w8a16_block_gemv(bf16_dev(np.ascontiguousarray(a[:m])), w, s))
        assert np.array_equal(part, four[:m])
    for r in range(4):
        one = host(fq.w8a16_block_gemv(bf16_dev(np.ascontiguousarray(a[r:r + 1])), w, s))
        assert np.array_equal(one[0], four[r])


def test_grouped_and_strided_match_single_calls_bit_for_bit():
    import torch
    k, m = synth.DECODE_K, 3
    a = bf16_dev(synth.decode_activation(m, seed=91))
    projs, singles = [], []
    big = torch.full((m, 5120 + 1024 + 64), -7.0, dtype=torch.bfloat16, device=DEV)
    views = [big[:, :5120], big[:, 5120:5120 + 1024]]
    for i, n in enumerate((5120, 1024)):
        wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=300 + n))
        w, s = u8_dev(wq), f32_dev(ws)
        singles.append(host(fq.w8a16_block_gemv(a, w, s)))
        projs.append((w, s, views[i]))
    fq.w8a16_block_gemv_grouped(a, projs)
    got = host(big)
    assert np.array_equal(got[:, :5120], singles[0])
    assert np.array_equal(got[:, 5120:6144], singles[1])
    assert np.all(bf16_host_to_f64(got[:, 6144:]) == -7.0)  # columns past both outputs


@pytest.mark.parametrize("m", [1, 4])
def test_grouped_four_decode_projections_match_single_calls_and_oracle(m):
    """The four decode projections (2176 strips: the last round runs as 8-column halves on
    a 256-CU part) in one launch: every output equals its single call bit for bit and the
    oracle within the bound."""
    k = synth.DECODE_K
    a = synth.decode_activation(m, seed=2300 + m)
    ad = bf16_dev(a)
    projs, singles = [], []
    for n in synth.DECODE_N:
        wq, ws = _weights(n, k, 2100 + n)
        wq_d, ws_d = u8_dev(wq), f32_dev(ws)
        projs.append((wq_d, ws_d, None))
        singles.append((host(fq.w8a16_block_gemv(ad, wq_d, ws_d)), wq, ws))
    outs = fq.w8a16_block_gemv_grouped(ad, projs)
    for out, (single, wq, ws) in zip(outs, singles):
        got = host(out)
        assert np.array_equal(got, single)
        ref, mag = oracle.gemm_w8a16(a, wq, ws)
        ok, worst = _within(got, ref, mag, k)
        assert ok, f"worst error / bound = {worst:.3f}"


def test_strided_output_writes_exactly_its_extent():
    import torch
    k, n, m, ldc = 256, 256, 3, 300
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=5))
    a = synth.decode_activation(m, k=k, seed=6)
    buf = torch.full(((m + 1) * ldc,), 3.0, dtype=torch.bfloat16, device=DEV)
    fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws), out=buf, ldc=ldc)
    got = bf16_host_to_f64(host(buf))
    extent = (m - 1) * ldc + n
    written = np.zeros(buf.numel(), dtype=bool)
    for r in range(m):
        written[r * ldc:r * ldc + n] = True
    assert np.all(got[~written] == 3.0) and extent == written.nonzero()[0][-1] + 1
    ref, mag = oracle.gemm_w8a16(a, wq, ws)
    vals = np.stack([host(buf)[r * ldc:r * ldc + n] for r in range(m)])
    assert _within(vals, ref, mag, k)[0]


@pytest.mark.parametrize("m,n,k,ldc,code", [
    (0, 128, 128, 128, -1), (5, 128, 128, 128, -1), (1, 100, 128, 128, -1),
    (1, 128, 100, 128, -1), (1, 128, 131200, 128, -1), (1, 256, 128, 128, -1)])
def test_invalid_shapes_rejected_before_launch(m, n, k, ldc, code):
    import ctypes
    lib = fq.load()
    p = ctypes.c_void_p(16)
    assert lib.w8a16_block_gemv(p, p, p, p, m, n, k, ldc, None) == code
    assert lib.w8a16_block_gemv(None, p, p, p, 1, 128, 128, 128, None) == -2
