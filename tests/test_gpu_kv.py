"""GPU parity: paged FP8 KV write, K/V absmax and the online scale calibrator against the
CPU oracle -- pool bytes, scales and counters bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import DEV, bf16_dev, host, i64_dev, need_gpu

pytestmark = pytest.mark.gpu

H, D, BS, NB = synth.KV_HEADS, synth.KV_HEAD_DIM, synth.KV_BLOCK_SIZE, synth.KV_NUM_BLOCKS
E = H * D
CS = BS * E


def setup_module(_):
    need_gpu()


def _pools(fill_k=0xAA, fill_v=0x55, nblk=NB, cs=CS):
    kc = np.full(nblk * cs, fill_k, dtype=np.uint8)
    vc = np.full(nblk * cs, fill_v, dtype=np.uint8)
    return kc, vc, torch.from_numpy(kc.copy()).to(DEV), torch.from_numpy(vc.copy()).to(DEV)


@pytest.mark.parametrize("pattern", ["permutation", "block_runs"])
def test_full_pool_write_matches_oracle(pattern):
    b = synth.kv_full_pool()
    slots = b.slots if pattern == "permutation" else synth.kv_block_runs()
    kc, vc, kcd, vcd = _pools()
    ks, vs = 3.0 * 17.0 / 448.0, 0.0625
    fq.fp8_kv_write(bf16_dev(b.k), bf16_dev(b.v), kcd, vcd, i64_dev(slots), H, D, BS, ks, vs)
    oracle.kv_write(b.k, b.v, kc, vc, slots, len(slots), H, D, BS, ks, vs, E, E, CS)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


def test_batches_provisional_scale_and_skips():
    batches, _ = synth.kv_batches(num_tokens_total=400, seed=5010)
    kc, vc, kcd, vcd = _pools()
    for i, b in enumerate(batches):
        slots = b.slots.copy()
        if i % 3 == 0:
            slots[0] = -1                   # padding token
        if i % 4 == 1:
            slots[-1] = NB * BS + 5         # outside the pool: skipped, never written
        fq.fp8_kv_write(bf16_dev(b.k), bf16_dev(b.v), kcd, vcd, i64_dev(slots), H, D, BS,
                        2.0, 2.0)
        valid = np.where((slots >= 0) & (slots < NB * BS), slots, -1)
        oracle.kv_write(b.k, b.v, kc, vc, valid, len(slots), H, D, BS, 2.0, 2.0, E, E, CS)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


def test_strided_sources_and_padded_pool_stride():
    rng = np.random.default_rng(3)
    t, ks, vs, cs = 50, E + 64, E + 8, CS + 128
    k = synth.to_bf16_bits(rng.normal(0, 3, size=t * ks))
    v = synth.to_bf16_bits(rng.normal(0, 3, size=t * vs))
    slots = rng.permutation(64 * BS)[:t].astype(np.int64)
    kc, vc, kcd, vcd = _pools(nblk=64, cs=cs)
    fq.fp8_kv_write(bf16_dev(k), bf16_dev(v), kcd, vcd, i64_dev(slots), H, D, BS, 0.3, 0.7,
                    key_stride=ks, value_stride=vs, cache_stride=cs, num_tokens=t)
    oracle.kv_write(k, v, kc, vc, slots, t, H, D, BS, 0.3, 0.7, ks, vs, cs)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


@pytest.mark.parametrize("h,d,offset", [(3, 5, 0), (2, 64, 1), (1, 8, 3)])
def test_elementwise_path_odd_geometry_and_alignment(h, d, offset):
    rng = np.random.default_rng(h * d + offset)
    e, t, bs, nblk = h * d, 37, 4, 16
    ks = e + 3
    kbuf = synth.to_bf16_bits(rng.normal(0, 3, size=t * ks + offset))
    vbuf = synth.to_bf16_bits(rng.normal(0, 3, size=t * ks + offset))
    slots = rng.permutation(nblk * bs)[:t].astype(np.int64)
    cs = bs * e
    kc, vc, kcd, vcd = _pools(nblk=nblk, cs=cs)
    kd, vd = bf16_dev(kbuf)[offset:], bf16_dev(vbuf)[offset:]
    fq.fp8_kv_write(kd, vd, kcd, vcd, i64_dev(slots), h, d, bs, 0.5, 3.0, key_stride=ks,
                    value_stride=ks, num_tokens=t)
    oracle.kv_write(kbuf[offset:].copy(), vbuf[offset:].copy(), kc, vc, slots, t, h, d, bs,
                    0.5, 3.0, ks, ks, cs)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


def test_scale_far_below_values_saturates_with_sign():
    rng = np.random.default_rng(9)
    k = synth.to_bf16_bits(rng.normal(0, 1e3, size=(8, E)))
    slots = np.arange(8, dtype=np.int64)
    kc, vc, kcd, vcd = _pools(nblk=1)
    fq.fp8_kv_write(bf16_dev(k), bf16_dev(k), kcd, vcd, i64_dev(slots), H, D, BS, 2.0 ** -60,
                    2.0 ** 60)
    oracle.kv_write(k, k, kc, vc, slots, 8, H, D, BS, 2.0 ** -60, 2.0 ** 60, E, E, CS)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


def test_amax_matches_oracle_and_accumulates():
    batches, _ = synth.kv_batches(num_tokens_total=300, seed=5020)
    amax2 = torch.zeros(2, dtype=torch.float32, device=DEV)
    km = vm = np.float32(0)
    for b in batches:
        fq.fp8_kv_amax(bf16_dev(b.k), bf16_dev(b.v), amax2)
        km = max(km, oracle.amax(b.k))
        vm = max(vm, oracle.amax(b.v))
        assert host(amax2).tolist() == [float(km), float(vm)]
    odd = synth.to_bf16_bits(np.random.default_rng(1).normal(0, 1e4, size=1001))
    fq.fp8_kv_amax(bf16_dev(odd), bf16_dev(odd), amax2)
    assert host(amax2)[0] == max(km, oracle.amax(odd))


def _calibrate_on_gpu(batches, window, headroom=1.0, decline_at=None):
    kc, vc, kcd, vcd = _pools()
    cal = fq.KvCalibrator(window, headroom)
    for i, b in enumerate(batches):
        if i == decline_at:
            k2, v2 = np.ascontiguousarray(b.k[:, :256]), np.ascontiguousarray(b.v[:, :256])
            kd, vd, h = bf16_dev(k2), bf16_dev(v2), 2
        else:
            kd, vd, h = bf16_dev(b.k), bf16_dev(b.v), H
        sd = i64_dev(b.slots)
        cal.observe(kd, vd, h, D, kcd, vcd, sd, BS, cache_stride=CS)
        ks, vs = cal.scales()
        fq.fp8_kv_write(kd, vd, kcd, vcd, sd, h, D, BS, ks, vs, cache_stride=CS)
    info = cal.info()
    cal.close()
    return host(kcd), host(vcd), info


def _calibrate_oracle(batches, window, headroom=1.0, decline_at=None):
    kc, vc, _, _ = _pools()
    cal = oracle.Calibrator(window, headroom)
    for i, b in enumerate(batches):
        if i == decline_at:
            k2, v2 = np.ascontiguousarray(b.k[:, :256]), np.ascontiguousarray(b.v[:, :256])
            cal._lib.oracle_calib_observe_and_write(
                cal._c, k2.ctypes.data, v2.ctypes.data, b.slots.ctypes.data, len(b.slots),
                2, D, BS, CS, kc.ctypes.data, vc.ctypes.data)
        else:
            cal.observe_and_write(b.k, b.v, b.slots, H, D, BS, CS, kc, vc)
    info = cal.info()
    cal.close()
    return kc, vc, info


@pytest.mark.parametrize("window,headroom,seed", [(256, 1.0, 5000), (256, 1.5, 5001),
                                                  (1, 1.0, 5002), (100, 0.5, 5003)])
def test_calibration_matches_oracle(window, headroom, seed):
    batches, reuse = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=seed)
    kc, vc, info = _calibrate_on_gpu(batches, window, headroom)
    kc_ref, vc_ref, ref = _calibrate_oracle(batches, window, headroom)
    assert info["frozen"] == 1 and ref["frozen"] == 1
    for key in ("k_scale", "v_scale", "k_amax", "v_amax"):
        ref_key = key.replace("amax", "max")
        assert np.float32(info[key]) == ref[ref_key], key
    assert info["tokens_seen"] == ref["tokens_seen"]
    assert info["replayed_tokens"] == ref["replayed_tokens"]
    assert info["staged_batches"] == ref["staged_batches"]
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)


@pytest.mark.parametrize("k_pad,v_pad", [(64, 8), (3, 1)])
def test_calibration_from_strided_rows_matches_oracle(k_pad, v_pad):
    """K / V rows inside wider buffers: strides that keep 16-byte rows take the one-kernel
    staging (absmax + packed copy + slots), odd strides the absmax pass and 2-D copies; both
    stage the same packed rows, so the pools and scales equal the oracle's on packed input."""
    batches, _ = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=5030 + k_pad)
    ks, vs = E + k_pad, E + v_pad
    _, _, kcd, vcd = _pools()
    cal = fq.KvCalibrator(synth.KV_WINDOW)
    for b in batches:
        n = len(b.slots)
        # padding of bf16 2^127: a read past a row would show in the maxima and the codes
        kw = torch.full((n, ks), 0x7F00, dtype=torch.int16, device=DEV)
        vw = torch.full((n, vs), 0x7F00, dtype=torch.int16, device=DEV)
        kw[:, :E] = torch.from_numpy(b.k.view(np.int16)).to(DEV)
        vw[:, :E] = torch.from_numpy(b.v.view(np.int16)).to(DEV)
        kd, vd = kw.view(torch.bfloat16)[:, :E], vw.view(torch.bfloat16)[:, :E]
        sd = i64_dev(b.slots)
        cal.observe(kd, vd, H, D, kcd, vcd, sd, BS, key_stride=ks, value_stride=vs,
                    cache_stride=CS)
        k_scale, v_scale = cal.scales()
        fq.fp8_kv_write(kd, vd, kcd, vcd, sd, H, D, BS, k_scale, v_scale, key_stride=ks,
                        value_stride=vs, cache_stride=CS)
    info = cal.info()
    cal.close()
    kc_ref, vc_ref, ref = _calibrate_oracle(batches, synth.KV_WINDOW)
    assert info["frozen"] == 1 and info["replayed_tokens"] == ref["replayed_tokens"] > 0
    for key in ("k_scale", "v_scale", "k_amax", "v_amax"):
        assert np.float32(info[key]) == ref[key.replace("amax", "max")], key
    assert np.array_equal(host(kcd), kc_ref) and np.array_equal(host(vcd), vc_ref)


def test_calibration_with_a_declined_batch_matches_oracle():
    batches, _ = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=5004)
    kc, vc, info = _calibrate_on_gpu(batches, synth.KV_WINDOW, decline_at=1)
    kc_ref, vc_ref, ref = _calibrate_oracle(batches, synth.KV_WINDOW, decline_at=1)
    assert info["unstaged_tokens"] == ref["unstaged_tokens"] == len(batches[1].slots)
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)


def test_calibration_reuse_inside_window_equals_single_pass():
    """A slot rewritten after free/re-allocation inside the window: the replayed pools
    equal one chronological pass over every batch at the frozen scales."""
    batches, reuse = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=5000)
    kc, vc, info = _calibrate_on_gpu(batches, synth.KV_WINDOW)
    cross = int(np.searchsorted(np.cumsum([len(b.slots) for b in batches]), synth.KV_WINDOW))
    assert any(bi <= cross for bi, _ in reuse)
    kc2, vc2, _, _ = _pools()
    for b in batches:
        oracle.kv_write(b.k, b.v, kc2, vc2, b.slots, len(b.slots), H, D, BS, info["k_scale"],
                        info["v_scale"], E, E, CS)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)


def test_calibration_replay_with_heavy_slot_reuse_matches_oracle():
    """Staged batches that keep rewriting a few dozen slots (plus padding slots), over several
    64-token tiles: the one-launch replay keeps each slot's last staged writer, exactly as
    the oracle's in-order replay."""
    rng = np.random.default_rng(5020)
    batches = []
    for i in range(40):
        n = int(rng.integers(1, 65))
        slots = rng.permutation(96)[:n].astype(np.int64) * 7 % (NB * BS)
        if i % 5 == 0:
            slots[0] = -1
        k = synth.to_bf16_bits(rng.normal(0, 3, size=(n, E)))
        v = synth.to_bf16_bits(rng.normal(0, 3, size=(n, E)))
        batches.append(synth.KvBatch(k=k, v=v, slots=slots))
    window = sum(len(b.slots) for b in batches[:-1]) + 1  # the last batch crosses
    kc, vc, info = _calibrate_on_gpu(batches, window)
    kc_ref, vc_ref, ref = _calibrate_oracle(batches, window)
    assert info["frozen"] == 1 and info["replayed_tokens"] == ref["replayed_tokens"] > 64
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)


def test_calibrator_destroyed_inside_the_window_releases_its_staging():
    """Staging allocated in stream order and never frozen: destroy waits for the device and
    releases it; a second calibrator on the same pools then runs to the oracle's result."""
    batches, _ = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=5030)
    kc, vc, kcd, vcd = _pools()
    first = fq.KvCalibrator(synth.KV_WINDOW)
    for b in batches[:3]:
        first.observe(bf16_dev(b.k), bf16_dev(b.v), H, D, kcd, vcd, i64_dev(b.slots), BS)
    assert first.info()["staged_tokens"] == sum(len(b.slots) for b in batches[:3])
    first.close()
    got_k, got_v, info = _calibrate_on_gpu(batches, synth.KV_WINDOW)
    kc_ref, vc_ref, ref = _calibrate_oracle(batches, synth.KV_WINDOW)
    assert info["replayed_tokens"] == ref["replayed_tokens"]
    assert np.array_equal(got_k, kc_ref) and np.array_equal(got_v, vc_ref)


def test_calibrator_frozen_scale_out_of_range_is_refused_on_the_gpu():
    """headroom 2^64 over |K| ~ 1e4 puts the frozen scale above 2^64: the freezing observe
    fails with EINVAL and nothing is replayed or frozen."""
    rng = np.random.default_rng(31)
    k = synth.to_bf16_bits(rng.normal(0, 1e4, size=(8, E)))
    v = synth.to_bf16_bits(rng.normal(0, 1, size=(8, E)))
    kc, vc, kcd, vcd = _pools()
    cal = fq.KvCalibrator(8, 2.0 ** 64)
    with pytest.raises(fq.Fp8qError) as err:
        cal.observe(bf16_dev(k), bf16_dev(v), H, D, kcd, vcd, i64_dev(np.arange(8)), BS)
    assert err.value.status == -1
    info = cal.info()
    assert info["frozen"] == 0 and info["tokens_seen"] == 0 and cal.scales() == (2.0, 2.0)
    cal.close()
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


def test_calibrators_freezing_concurrently_on_two_streams_match_the_oracle():
    """Two calibrators driven from two host threads, each on its own stream, over different
    batch sequences: their freezes share the process's page-locked read buffer and must each
    read their own running maximum (scales, counters and pools equal the oracle's)."""
    import threading

    seqs = [synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 64, seed=seed)[0]
            for seed in (5040, 5041)]
    results, errors = [None, None], []

    def drive(idx):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                _, _, kcd, vcd = _pools()
                cal = fq.KvCalibrator(synth.KV_WINDOW)
                for b in seqs[idx]:
                    kd, vd, sd = bf16_dev(b.k), bf16_dev(b.v), i64_dev(b.slots)
                    cal.observe(kd, vd, H, D, kcd, vcd, sd, BS, cache_stride=CS)
                    ks, vs = cal.scales()
                    fq.fp8_kv_write(kd, vd, kcd, vcd, sd, H, D, BS, ks, vs, cache_stride=CS)
                stream.synchronize()
                results[idx] = (host(kcd), host(vcd), cal.info())
                cal.close()
        except Exception as exc:  # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=drive, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for idx in range(2):
        kc, vc, info = results[idx]
        kc_ref, vc_ref, ref = _calibrate_oracle(seqs[idx], synth.KV_WINDOW)
        assert info["frozen"] == 1 and info["replayed_tokens"] == ref["replayed_tokens"]
        for key in ("k_scale", "v_scale", "k_amax", "v_amax"):
            assert np.float32(info[key]) == ref[key.replace("amax", "max")], (idx, key)
        assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)


# ------------------------------------------------------------------ dequantizing read


def _read_both(kc, vc, slots, h, d, bs, nblk, ks, vs, kos, vos, cs, t, fill=0x1234,
               offset=0):
    """GPU read (through the C ABI) and oracle read of the same pools; the output rows start
    as `fill` so rows of skipped tokens can be checked."""
    ko = np.full(t * kos, fill, dtype=np.uint16)
    vo = np.full(t * vos, fill, dtype=np.uint16)
    kod = bf16_dev(np.concatenate([np.zeros(offset, np.uint16), ko]))[offset:]
    vod = bf16_dev(np.concatenate([np.zeros(offset, np.uint16), vo]))[offset:]
    fq.fp8_kv_read(torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV), i64_dev(slots),
                   h, d, bs, ks, vs, k_out=kod, v_out=vod, out_key_stride=kos,
                   out_value_stride=vos, cache_stride=cs, num_tokens=t)
    oracle.kv_read(kc, vc, slots, h, d, bs, nblk, ks, vs, ko, vo, kos, vos, cs)
    return host(kod), host(vod), ko, vo


def test_read_full_pool_every_code_matches_oracle():
    """The whole 2048-block pool (every byte value, NaN codes included) read back through a
    permuted slot map with padding and out-of-range slots."""
    rng = np.random.default_rng(77)
    kc = rng.integers(0, 256, size=NB * CS, dtype=np.uint8)
    vc = rng.integers(0, 256, size=NB * CS, dtype=np.uint8)
    slots = rng.permutation(NB * BS).astype(np.int64)
    slots[5] = -1
    slots[-3] = NB * BS + 7
    t = len(slots)
    kg, vg, ko, vo = _read_both(kc, vc, slots, H, D, BS, NB, 0.0234375, 3.0e-3, E, E, CS, t)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo)
    assert np.all(kg[5 * E:6 * E] == 0x1234) and np.all(vg[(t - 3) * E:(t - 2) * E] == 0x1234)


def test_read_full_pool_block_runs_matches_oracle():
    """The pool read back through the slots of a paged prefill (blocks in random order, 16
    consecutive tokens each)."""
    rng = np.random.default_rng(78)
    kc = rng.integers(0, 256, size=NB * CS, dtype=np.uint8)
    vc = rng.integers(0, 256, size=NB * CS, dtype=np.uint8)
    slots = synth.kv_block_runs(NB, BS)
    t = len(slots)
    kg, vg, ko, vo = _read_both(kc, vc, slots, H, D, BS, NB, 0.0234375, 3.0e-3, E, E, CS, t)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo)


@pytest.mark.parametrize("t", [1, 2, 37, 129])
def test_read_ragged_token_counts(t):
    rng = np.random.default_rng(t)
    nblk = 16
    kc = rng.integers(0, 256, size=nblk * CS, dtype=np.uint8)
    vc = rng.integers(0, 256, size=nblk * CS, dtype=np.uint8)
    slots = rng.permutation(nblk * BS)[:t].astype(np.int64)
    kg, vg, ko, vo = _read_both(kc, vc, slots, H, D, BS, nblk, 1.7e9, 2.0 ** -64, E, E, CS, t)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo)


def test_read_strided_outputs_and_padded_pool_stride():
    rng = np.random.default_rng(4)
    t, kos, vos, cs, nblk = 50, E + 64, E + 8, CS + 128, 64
    kc = rng.integers(0, 256, size=nblk * cs, dtype=np.uint8)
    vc = rng.integers(0, 256, size=nblk * cs, dtype=np.uint8)
    slots = rng.permutation(nblk * BS)[:t].astype(np.int64)
    kg, vg, ko, vo = _read_both(kc, vc, slots, H, D, BS, nblk, 0.3, 0.7, kos, vos, cs, t)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo)


@pytest.mark.parametrize("h,d,offset", [(3, 5, 0), (2, 64, 1), (1, 8, 3), (8, 128, 0), (1, 8, 0),
                                          (3, 8, 0)])
def test_read_elementwise_and_wide_rows(h, d, offset):
    """Odd geometry and misaligned outputs take the element-wise path; 8 x 128 rows take the
    vector path with a token spanning several waves."""
    rng = np.random.default_rng(h * d + offset)
    e, t, bs, nblk = h * d, 37, 4, 16
    cs = bs * e
    kc = rng.integers(0, 256, size=nblk * cs, dtype=np.uint8)
    vc = rng.integers(0, 256, size=nblk * cs, dtype=np.uint8)
    slots = rng.permutation(nblk * bs)[:t].astype(np.int64)
    slots[0] = -1
    kg, vg, ko, vo = _read_both(kc, vc, slots, h, d, bs, nblk, 0.5, 3.0, e + 3 * (offset > 0),
                                e + 3 * (offset > 0), cs, t, offset=offset)
    assert np.array_equal(kg, ko) and np.array_equal(vg, vo)


def test_write_then_read_round_trip_on_device():
    """GPU write then GPU read at the same scales reproduces the oracle's write + read."""
    b = synth.kv_full_pool()
    t = len(b.slots)
    kc, vc, kcd, vcd = _pools()
    ks = float(np.float32(oracle.amax(b.k)) / np.float32(448))
    vs = float(np.float32(oracle.amax(b.v)) / np.float32(448))
    fq.fp8_kv_write(bf16_dev(b.k), bf16_dev(b.v), kcd, vcd, i64_dev(b.slots), H, D, BS, ks, vs)
    kod, vod = fq.fp8_kv_read(kcd, vcd, i64_dev(b.slots), H, D, BS, ks, vs)
    oracle.kv_write(b.k, b.v, kc, vc, b.slots, t, H, D, BS, ks, vs, E, E, CS)
    ko = np.zeros((t, E), dtype=np.uint16)
    vo = np.zeros((t, E), dtype=np.uint16)
    oracle.kv_read(kc, vc, b.slots, H, D, BS, NB, ks, vs, ko, vo, E, E, CS)
    assert np.array_equal(host(kod), ko) and np.array_equal(host(vod), vo)


def test_read_argument_errors():
    kcd = torch.zeros(NB * CS, dtype=torch.uint8, device=DEV)
    s = i64_dev(np.zeros(4, dtype=np.int64))
    with pytest.raises(fq.Fp8qError):
        fq.fp8_kv_read(kcd, kcd, s, H, D, BS, 0.0, 1.0)
    with pytest.raises(fq.Fp8qError):
        fq.fp8_kv_read(kcd, kcd, s, H, D, BS, 1.0, float("nan"))
    ko, vo = fq.fp8_kv_read(kcd, kcd, s, H, D, BS, 1.0, 1.0, num_tokens=0)
    assert ko.shape == (0, E)


# ------------------------------------------------------ write + absmax in one pass


@pytest.mark.parametrize("h,d", [(H, D), (2, 64), (3, 5)])
def test_write_amax_equals_write_then_amax(h, d):
    """Per batch: pools as fp8_kv_write leaves them, amax2 the running max over every row of
    the batch -- a padding token's data included (its slot is -1 and it is not written)."""
    batches, _ = synth.kv_batches(num_tokens_total=300, seed=5030)
    e = h * d
    nblk, bs = 64, BS
    cs = bs * e
    kc = np.full(nblk * cs, 0x11, dtype=np.uint8)
    vc = np.full(nblk * cs, 0x22, dtype=np.uint8)
    kcd, vcd = torch.from_numpy(kc.copy()).to(DEV), torch.from_numpy(vc.copy()).to(DEV)
    amax2 = torch.zeros(2, dtype=torch.float32, device=DEV)
    km = vm = np.float32(0.0)
    for i, b in enumerate(batches):
        kk = np.ascontiguousarray(b.k[:, :e])
        vv = np.ascontiguousarray(b.v[:, :e])
        slots = b.slots % (nblk * bs)
        if i == 2:
            slots = slots.copy()
            slots[0] = -1
            kk = kk.copy()
            kk[0, 0] = synth.to_bf16_bits(np.array([-5000.0]))[0]
        fq.fp8_kv_write_amax(bf16_dev(kk), bf16_dev(vv), kcd, vcd, i64_dev(slots), h, d, bs,
                             0.375, 0.5, amax2)
        oracle.kv_write(kk, vv, kc, vc, slots, len(slots), h, d, bs, 0.375, 0.5, e, e, cs)
        km = max(km, oracle.amax(kk))
        vm = max(vm, oracle.amax(vv))
        assert host(amax2).tolist() == [float(km), float(vm)]
    assert km == synth.bf16_bits_to_f32(synth.to_bf16_bits(np.array([5000.0])))[0]  # 4992
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)


def test_write_amax_full_pool():
    b = synth.kv_full_pool()
    kc, vc, kcd, vcd = _pools()
    amax2 = torch.zeros(2, dtype=torch.float32, device=DEV)
    fq.fp8_kv_write_amax(bf16_dev(b.k), bf16_dev(b.v), kcd, vcd, i64_dev(b.slots), H, D, BS,
                         0.1, 0.2, amax2)
    oracle.kv_write(b.k, b.v, kc, vc, b.slots, len(b.slots), H, D, BS, 0.1, 0.2, E, E, CS)
    assert np.array_equal(host(kcd), kc) and np.array_equal(host(vcd), vc)
    assert host(amax2).tolist() == [float(oracle.amax(b.k)), float(oracle.amax(b.v))]
