"""The calibrator's state machine on the CPU: libfp8q.so's own calibrator (window, stage,
decline, freeze formula and range check, replay order, counters) driven through a table of
callbacks backed by host memory, whose writes and absmax are the oracle's.  Its pools,
scales and counters must equal oracle.Calibrator's byte for byte (calib: observe, the freeze
formula, the window and headroom clamps; staging: stage, decline, replay in write order)."""
import ctypes

import numpy as np
import pytest

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import _lib, synth

H, D, BS, NB = synth.KV_HEADS, synth.KV_HEAD_DIM, synth.KV_BLOCK_SIZE, synth.KV_NUM_BLOCKS
E = H * D
CS = BS * E
EINVAL, ENULL, EHIP = -1, -2, -5


def _u16_at(addr, count):
    return np.ctypeslib.as_array((ctypes.c_uint16 * count).from_address(addr))


def _i64_at(addr, count):
    return np.ctypeslib.as_array((ctypes.c_int64 * count).from_address(addr))


def _rows(addr, rows, elems, stride):
    """Packed copy of `rows` bf16 rows of `elems` at `stride` elements, read from host memory."""
    if rows == 0:
        return np.zeros((0, elems), np.uint16)
    flat = _u16_at(addr, (rows - 1) * stride + elems)
    return np.stack([flat[r * stride:r * stride + elems] for r in range(rows)])


class HostOps:
    """fp8q_kv_calib_ops over host memory: allocations are numpy buffers (filled with 0xCD so
    a read of memory the calibrator never initialized shows), the absmax and the replay's
    write are the oracle's, the replay writes the staged tokens one after another."""

    def __init__(self, pools, with_stage=False):
        self.bufs = {}
        self.pools = pools  # address -> numpy pool the target points at
        self.reads = 0
        self.releases = []
        self.errors = []
        self.fail_alloc_over = None  # bytes: larger allocations fail (EHIP)
        ops = _lib.KvCalibOps
        self.table = ops(
            None, ops.DEVICE(self._guard(self.device)), ops.ALLOC(self._guard(self.alloc)),
            ops.RELEASE(self._guard(self.release)), ops.ZERO(self._guard(self.zero)),
            ops.AMAX_ROWS(self._guard(self.amax_rows)), ops.COPY2D(self._guard(self.copy2d)),
            ops.READ(self._guard(self.read)), ops.REPLAY(self._guard(self.replay)),
            ops.STAGE(self._guard(self.stage)) if with_stage else ops.STAGE())

    def _guard(self, fn):
        def call(*a):
            try:
                return fn(*a)
            except Exception as exc:  # surfaced by the test, never swallowed
                self.errors.append(exc)
                return EHIP
        return call

    def device(self, ctx, dev):
        dev[0] = 0
        return 0

    def alloc(self, ctx, nbytes, out, stream):
        if self.fail_alloc_over is not None and nbytes > self.fail_alloc_over:
            return EHIP
        buf = np.full(nbytes, 0xCD, dtype=np.uint8)
        self.bufs[buf.ctypes.data] = buf
        out[0] = buf.ctypes.data
        return 0

    def release(self, ctx, p, stream, at_destroy):
        if p:
            del self.bufs[p]
            self.releases.append(bool(at_destroy))
        return 0

    def zero(self, ctx, p, nbytes, stream):
        ctypes.memset(p, 0, nbytes)
        return 0

    def amax_rows(self, ctx, k, v, rows, elems, ks, vs, amax2, stream):
        acc = np.ctypeslib.as_array((ctypes.c_float * 2).from_address(amax2))
        acc[0] = oracle.amax(_rows(k, rows, elems, ks), acc=float(acc[0]))
        acc[1] = oracle.amax(_rows(v, rows, elems, vs), acc=float(acc[1]))
        return 0

    def copy2d(self, ctx, dst, src, src_pitch, row_bytes, rows, stream):
        for r in range(rows):
            ctypes.memmove(dst + r * row_bytes, src + r * src_pitch, row_bytes)
        return 0

    def stage(self, ctx, k, v, slots, rows, elems, ks, vs, dk, dv, dslots, amax2, stream):
        """The optional one-call staging: absmax, packed rows, slots."""
        self.amax_rows(ctx, k, v, rows, elems, ks, vs, amax2, stream)
        packed_k = np.ascontiguousarray(_rows(k, rows, elems, ks))  # held until copied
        packed_v = np.ascontiguousarray(_rows(v, rows, elems, vs))
        ctypes.memmove(dk, packed_k.ctypes.data, packed_k.nbytes)
        ctypes.memmove(dv, packed_v.ctypes.data, packed_v.nbytes)
        ctypes.memmove(dslots, slots, rows * 8)
        self.staged_calls = getattr(self, "staged_calls", 0) + 1
        return 0

    def read(self, ctx, host_dst, src, nbytes, stream):
        self.reads += 1
        ctypes.memmove(host_dst, src, nbytes)
        return 0

    def replay(self, ctx, k, v, slots, scratch, n, elems, target, k_scale, v_scale, stream):
        t = target.contents
        kk = _rows(k, n, elems, elems)
        vv = _rows(v, n, elems, elems)
        sl = _i64_at(slots, n).copy()
        oracle.kv_write(kk, vv, self.pools[t.k_pool], self.pools[t.v_pool], sl, n, 1, elems,
                        t.block_size, k_scale, v_scale, elems, elems, t.cache_stride)
        return 0


def _pools():
    return (np.full(NB * CS, 0xAA, dtype=np.uint8), np.full(NB * CS, 0x55, dtype=np.uint8))


def _batch_input(b, narrow):
    if narrow:  # a batch with half the heads: the staging declines it
        return np.ascontiguousarray(b.k[:, :E // 2]), np.ascontiguousarray(b.v[:, :E // 2]), H // 2
    return b.k, b.v, H


def _run_library(batches, window, headroom=1.0, provisional=2.0, decline_at=None,
                 with_stage=False):
    kc, vc = _pools()
    ops = HostOps({kc.ctypes.data: kc, vc.ctypes.data: vc}, with_stage)
    lib = fq.load()
    cal = fq.KvCalibrator(window, headroom, provisional, ops=ops.table)
    steps = []
    for i, b in enumerate(batches):
        k, v, h = _batch_input(b, i == decline_at)
        e = h * D
        steps.append(cal.decide(len(b.slots), e))
        tgt = _lib.KvTarget(k_pool=kc.ctypes.data, v_pool=vc.ctypes.data,
                            slot_mapping=b.slots.ctypes.data, block_size=BS, key_stride=e,
                            value_stride=e, reserved=0, cache_stride=CS, num_blocks=NB)
        st = lib.fp8q_kv_calib_observe(cal._h, k.ctypes.data, v.ctypes.data, len(b.slots), h,
                                       D, ctypes.byref(tgt), None)
        assert st == 0 and not ops.errors, (i, st, ops.errors)
        ks, vs = cal.scales()
        # the caller's own write of the batch at the scales now in force
        oracle.kv_write(k, v, kc, vc, b.slots, len(b.slots), h, D, BS, ks, vs, e, e, CS)
    info = cal.info()
    left = dict(ops.bufs)
    cal.close()
    return kc, vc, info, steps, ops, left


def _run_oracle(batches, window, headroom=1.0, provisional=2.0, decline_at=None):
    kc, vc = _pools()
    cal = oracle.Calibrator(window, headroom, provisional)
    steps = []
    for i, b in enumerate(batches):
        k, v, h = _batch_input(b, i == decline_at)
        steps.append(cal.observe_and_write(k, v, b.slots, h, D, BS, CS, kc, vc))
    info = cal.info()
    cal.close()
    return kc, vc, info, steps


def _same(lib_run, ora_run):
    kc, vc, info, steps, ops, left = lib_run
    kc_ref, vc_ref, ref, ref_steps = ora_run
    assert steps == ref_steps
    assert info["frozen"] == ref["frozen"] == 1
    for key, ref_key in (("k_scale", "k_scale"), ("v_scale", "v_scale"), ("k_amax", "k_max"),
                         ("v_amax", "v_max"), ("headroom", "headroom")):
        assert np.float32(info[key]) == ref[ref_key], key
    for key in ("tokens_seen", "replayed_tokens", "staged_batches", "unstaged_tokens"):
        assert info[key] == ref[key], key
    assert info["window_tokens"] == ref["window"]
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    # one host read (at the freeze); the staging was released in stream order there, and
    # only the 8-byte running maximum stayed until destroy
    assert ops.reads == 1
    assert len(left) == 1 and next(iter(left.values())).nbytes == 8
    assert not any(ops.releases[:-1]) and ops.releases[-1]
    assert not ops.bufs


@pytest.mark.parametrize("window,headroom,seed", [(256, 1.0, 5000), (256, 1.5, 5001),
                                                  (1, 1.0, 5002), (100, 0.5, 5003)])
@pytest.mark.parametrize("with_stage", [False, True])
def test_library_calibrator_equals_oracle(window, headroom, seed, with_stage):
    """With and without the optional one-call staging callback."""
    batches, reuse = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=seed)
    if window == 256 and seed == 5000:  # the 256-token window at seed 5000 rewrites a freed slot
        cross = int(np.searchsorted(np.cumsum([len(b.slots) for b in batches]), window))
        assert any(bi <= cross for bi, _ in reuse)
    run = _run_library(batches, window, headroom, with_stage=with_stage)
    _same(run, _run_oracle(batches, window, headroom))
    if with_stage and window > 1:
        assert run[4].staged_calls == run[2]["staged_batches"]


def test_window_one_freezes_on_the_first_observe_and_stages_nothing():
    batches, _ = synth.kv_batches(num_tokens_total=40, seed=5006)
    run = _run_library(batches, 1)
    assert run[3][0] == fq.FP8Q_CALIB_FREEZE and run[2]["replayed_tokens"] == 0
    assert run[2]["staged_batches"] == 0
    _same(run, _run_oracle(batches, 1))


def test_declined_batch_keeps_the_provisional_scale():
    batches, _ = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=5004)
    run = _run_library(batches, synth.KV_WINDOW, decline_at=1)
    assert run[3][1] == fq.FP8Q_CALIB_DECLINE
    assert run[2]["unstaged_tokens"] == len(batches[1].slots)
    _same(run, _run_oracle(batches, synth.KV_WINDOW, decline_at=1))


def test_window_clamped_to_4096_staged_tokens():
    batches, _ = synth.kv_batches(num_tokens_total=4096 + 96, seed=5007, num_blocks=NB)
    run = _run_library(batches, 10 ** 6)
    assert run[2]["window_tokens"] == 4096 and run[2]["requested_tokens"] == 10 ** 6
    assert run[2]["replayed_tokens"] > 4000
    _same(run, _run_oracle(batches, 10 ** 6))


def test_provisional_scale_is_an_argument():
    batches, _ = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 32, seed=5008)
    run = _run_library(batches, synth.KV_WINDOW, provisional=0.5)
    _same(run, _run_oracle(batches, synth.KV_WINDOW, provisional=0.5))


def test_frozen_scale_out_of_range_fails_and_leaves_the_calibrator_unchanged():
    """headroom 2^64 over |x| ~ 1e4: (amax * 2^64) / 448 exceeds the write's 2^64 range, so
    the freezing observe returns EINVAL and the calibrator stays unfrozen."""
    rng = np.random.default_rng(9)
    kc, vc = _pools()
    ops = HostOps({kc.ctypes.data: kc, vc.ctypes.data: vc})
    lib = fq.load()
    cal = fq.KvCalibrator(8, 2.0 ** 64, ops=ops.table)
    k = synth.to_bf16_bits(rng.normal(0, 1e4, size=(8, E)))
    v = synth.to_bf16_bits(rng.normal(0, 1, size=(8, E)))
    slots = np.arange(8, dtype=np.int64)
    tgt = _lib.KvTarget(k_pool=kc.ctypes.data, v_pool=vc.ctypes.data,
                        slot_mapping=slots.ctypes.data, block_size=BS, key_stride=E,
                        value_stride=E, reserved=0, cache_stride=CS, num_blocks=NB)
    before = cal.info()
    for _ in range(2):
        st = lib.fp8q_kv_calib_observe(cal._h, k.ctypes.data, v.ctypes.data, 8, H, D,
                                       ctypes.byref(tgt), None)
        assert st == EINVAL and not ops.errors
        assert cal.info() == before and cal.scales() == (2.0, 2.0)
    assert np.all(kc == 0xAA) and np.all(vc == 0x55)
    cal.close()
    assert not ops.bufs


def test_failed_staging_allocation_leaves_the_calibrator_unchanged():
    """The staging cannot be allocated: observe fails with the callback's status before any
    state changes, and every buffer allocated on the way is released."""
    batches, _ = synth.kv_batches(num_tokens_total=64, seed=5009)
    kc, vc = _pools()
    ops = HostOps({kc.ctypes.data: kc, vc.ctypes.data: vc})
    lib = fq.load()
    cal = fq.KvCalibrator(256, ops=ops.table)
    b = batches[0]
    tgt = _lib.KvTarget(k_pool=kc.ctypes.data, v_pool=vc.ctypes.data,
                        slot_mapping=b.slots.ctypes.data, block_size=BS, key_stride=E,
                        value_stride=E, reserved=0, cache_stride=CS, num_blocks=NB)
    ops.fail_alloc_over = 256 * 8  # the running maximum and the slot buffers fit, rows do not
    st = lib.fp8q_kv_calib_observe(cal._h, b.k.ctypes.data, b.v.ctypes.data, len(b.slots), H,
                                   D, ctypes.byref(tgt), None)
    assert st == EHIP and not ops.errors
    info = cal.info()
    assert info["tokens_seen"] == 0 and info["staged_batches"] == 0 and info["frozen"] == 0
    assert len(ops.bufs) == 1  # only the running maximum
    ops.fail_alloc_over = None
    st = lib.fp8q_kv_calib_observe(cal._h, b.k.ctypes.data, b.v.ctypes.data, len(b.slots), H,
                                   D, ctypes.byref(tgt), None)
    assert st == 0 and cal.info()["staged_tokens"] == len(b.slots)
    cal.close()
    assert not ops.bufs


def test_create_bounds():
    lib = fq.load()
    h = ctypes.c_void_p()
    assert lib.fp8q_kv_calib_create(8, 2.0 ** 65, 2.0, ctypes.byref(h)) == EINVAL
    assert lib.fp8q_kv_calib_create(8, float("inf"), 2.0, ctypes.byref(h)) == EINVAL
    assert lib.fp8q_kv_calib_create(8, 1.0, 0.0, ctypes.byref(h)) == EINVAL
    assert lib.fp8q_kv_calib_create(8, 1.0, 2.0 ** 65, ctypes.byref(h)) == EINVAL
    assert lib.fp8q_kv_calib_create(8, 1.0, float("nan"), ctypes.byref(h)) == EINVAL
    assert lib.fp8q_kv_calib_create_with_ops(8, 1.0, 2.0, None, ctypes.byref(h)) == ENULL
    partial = _lib.KvCalibOps()  # every callback NULL
    assert lib.fp8q_kv_calib_create_with_ops(8, 1.0, 2.0, ctypes.byref(partial),
                                             ctypes.byref(h)) == ENULL
    assert lib.fp8q_kv_calib_create(8, 2.0 ** 64, 2.0 ** -64, ctypes.byref(h)) == 0
    lib.fp8q_kv_calib_destroy(h.value)
