"""GPU parity over seeded pseudo-random shapes: sizes, ragged edges and tilings that the
hand-picked cases elsewhere do not name, for the group quantizer (bit-exact), the decode
GEMM, its grouped and fused forms and the prefill GEMM (tolerance, rows sampled for the
large ones).  The shapes come from a fixed seed, so every run checks the same set."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import bf16_dev, f32_dev, gemm_tolerance_ok, host, need_gpu, u8_dev

pytestmark = pytest.mark.gpu


def setup_module(_):
    need_gpu()


def _shapes(seed, count, m_range, n_groups, k_groups):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(*m_range)), 128 * int(rng.integers(*n_groups)),
             128 * int(rng.integers(*k_groups))) for _ in range(count)]


@pytest.mark.parametrize("m,_n,k", _shapes(9100, 8, (1, 3000), (1, 2), (1, 65)))
def test_group_quant_seeded_shapes(m, _n, k):
    x = synth.prefill_activation(k, m=m, seed=m + k)
    q, s = fq.fp8_group_quant(bf16_dev(x))
    q_ref, s_ref = oracle.group_quant(x)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("m,n,k", _shapes(9200, 8, (1, 17), (1, 97), (1, 49)))
def test_decode_gemm_seeded_shapes(m, n, k):
    a = synth.decode_activation(m, k=k, seed=m * 31 + k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=n + k))
    q, s = fq.fp8_group_quant(bf16_dev(a))
    out = host(fq.w8a8_block_gemm(q, s, u8_dev(wq), f32_dev(ws)))
    ok, worst = gemm_tolerance_ok(out, oracle.gemm(host(q), host(s), wq, ws))
    assert ok, f"worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("seed", [9300, 9301, 9302, 9303])
def test_fused_grouped_seeded_projection_sets(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 17))
    k = 128 * int(rng.integers(1, 65))
    ns = [128 * int(x) for x in rng.integers(1, 41, size=int(rng.integers(1, 6)))]
    a = synth.decode_activation(m, k=k, seed=seed)
    w = [oracle.block_quant(synth.decode_weight(n, k, seed=seed + n)) for n in ns]
    dev = [(u8_dev(wq), f32_dev(ws), None) for wq, ws in w]
    outs = fq.fp8_quant_w8a8_gemm_grouped(bf16_dev(a), dev)
    q_ref, s_ref = oracle.group_quant(a)
    for (wq, ws), out in zip(w, outs):
        ok, worst = gemm_tolerance_ok(host(out), oracle.gemm(q_ref, s_ref, wq, ws))
        assert ok, f"m={m} k={k} n={wq.shape[0]}: worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("m,n,k", _shapes(9400, 10, (17, 9000), (1, 65), (1, 17)))
def test_prefill_gemm_seeded_shapes_on_sampled_rows(m, n, k):
    a = synth.prefill_activation(k, m=m, seed=m + 3 * k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=n * 5 + k))
    q, s = fq.fp8_group_quant(bf16_dev(a))
    out = fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws))
    rng = np.random.default_rng(m)
    rows = np.unique(np.r_[0:3, m - 3:m, rng.integers(0, m, size=10)].clip(0, m - 1))
    idx = torch.from_numpy(rows).to(q.device)
    got = host(out.index_select(0, idx))
    ref = oracle.gemm(host(q.index_select(0, idx)), host(s.index_select(0, idx)), wq, ws)
    ok, worst = gemm_tolerance_ok(got, ref)
    assert ok, f"worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("seed", range(9500, 9512))
def test_kv_write_and_read_seeded_geometries(seed):
    # heads, head dims, block sizes, row and pool paddings and slot maps (with skipped
    # slots) drawn from the seed; every kernel form (wide, 8-element, element-wise) is hit
    rng = np.random.default_rng(seed)
    h = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([8, 16, 24, 40, 64, 80, 128, 256]))
    bs = int(rng.choice([1, 4, 16, 32]))
    nblk = int(rng.integers(4, 65))
    e = h * d
    t = int(rng.integers(1, min(nblk * bs, 300) + 1))
    ks, vs = e + int(rng.choice([0, 8, 64, 3])), e + int(rng.choice([0, 8, 5]))
    cs = bs * e + int(rng.choice([0, 128, 16]))
    k = synth.to_bf16_bits(rng.normal(0, 3, size=t * ks))
    v = synth.to_bf16_bits(rng.normal(0, 3, size=t * vs))
    slots = rng.permutation(nblk * bs)[:t].astype(np.int64)
    slots[rng.random(t) < 0.05] = -1
    k_scale, v_scale = float(2.0 ** rng.uniform(-4, 4)), float(2.0 ** rng.uniform(-4, 4))
    kc = np.full(nblk * cs, 0xA5, dtype=np.uint8)
    vc = np.full(nblk * cs, 0x5A, dtype=np.uint8)
    kcd, vcd = torch.from_numpy(kc.copy()).cuda(), torch.from_numpy(vc.copy()).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    fq.fp8_kv_write(bf16_dev(k), bf16_dev(v), kcd, vcd, dev(slots), h, d, bs, k_scale, v_scale,
                    key_stride=ks, value_stride=vs, cache_stride=cs, num_tokens=t)
    oracle.kv_write(k, v, kc, vc, slots, t, h, d, bs, k_scale, v_scale, ks, vs, cs)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)
    # read the pools back through the same slots into padded rows
    kos, vos = e + int(rng.choice([0, 8, 2])), e + int(rng.choice([0, 16]))
    ko = np.full(t * kos, 0x1234, dtype=np.uint16)
    vo = np.full(t * vos, 0x1234, dtype=np.uint16)
    kod, vod = bf16_dev(ko), bf16_dev(vo)
    fq.fp8_kv_read(kcd, vcd, dev(slots), h, d, bs, k_scale, v_scale, k_out=kod, v_out=vod,
                   out_key_stride=kos, out_value_stride=vos, cache_stride=cs, num_tokens=t)
    oracle.kv_read(kc, vc, slots, h, d, bs, nblk, k_scale, v_scale, ko, vo, kos, vos, cs)
    assert np.array_equal(host(kod), ko) and np.array_equal(host(vod), vo)


@pytest.mark.parametrize("m,n,k", _shapes(9600, 8, (1, 5), (1, 97), (1, 97)))
def test_w8a16_seeded_shapes(m, n, k):
    # the W8A16 tier's bound from its own arithmetic (tests/test_gpu_gemv.py): products exact
    # in FP32, at most k/128 + 144 rounded additions, one bf16 rounding
    a = synth.decode_activation(m, k=k, seed=m * 17 + k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=n + 3 * k))
    out = host(fq.w8a16_block_gemv(bf16_dev(a), u8_dev(wq), f32_dev(ws)))
    ref, mag = oracle.gemm_w8a16(a, wq, ws)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 2 * (k / 128 + 144) * 2.0 ** -24 * mag
    assert np.all(np.abs(got - ref) <= bound)
