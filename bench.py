"""Benchmark of the FP8 (E4M3) quantize-and-consume path on one MI355X.

One step = one pass of the whole hot path over one decode batch:
  per-token 1x128 group quant of the activation [16 x 5120] (bf16 -> E4M3 + scales, a
  launch of its own), the four decode projections sharing it (W8A8 block-scaled GEMM,
  M=16, K=5120, N = 16384, 12288, 5120, 1024) in one grouped launch, the K/V absmax and the
  paged FP8 KV write of the batch's 16 new tokens (4 KV heads x 128 dims) at the calibrated
  scale in one launch.  The same step with the quantizer fused into the GEMM launch is
  reported beside it.
Steps are issued eagerly through the library's API (the same step replayed as one HIP
graph per buffer set is reported beside it); inputs rotate over >= 1 GB of buffer sets so
the 256 MB MALL cannot serve repeated reads.  value = algorithmic bytes per step /
measured step time (GB/s).

Also measured (same process, same rotation rule): each kernel on its own, timed with HIP
events around every launch while the stream is held busy so no host latency leaks into
an interval -- the group quantizer on the 4593-token prefill (K = 5120 and 16384), the
GEMM at each N, the quant+GEMM pair at M = 5, 8, 12, 16 (N = 16384; as two launches and as
one fused launch), the KV write, absmax and dequantizing read over a full 2048-block pool
(slots a random permutation of all 32768; the write and read again with the slots of a
paged prefill, blocks in random order and 16 consecutive tokens per block), and the
per-batch latency of the decode-time write (absmax fused in) for 1, 4, 16 and 64 tokens.
The K-split entry point is timed at each N beside the plain GEMM; the prefill GEMM's
operands rotate over >= 1 GB like every other leg.  Reference rows: an empty kernel and a
plain 2:1 read/write stream of the group quantizer's and the KV write's bytes, timed by the
same hook.  The calibration window (256 tokens of seeded paged batches) reports the latency
of an in-window observe and of the freezing observe.  The roofline object covers the step's
dominant kernel (the four-projection grouped GEMM); cpu_baseline times the CPU oracle
on full steps, single-threaded and with quant and GEMM split by rows over the host threads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, published
ROTATE_BYTES = 1 << 30     # >= 4x the 256 MB MALL
COPY_CALIB_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--iters", type=int, default=100, help="launches per kernel measurement")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="",
                   help="comma list of sections: step,gemm,grouped,sweep,gemv,prefill,quant,"
                        "kv,calib (default all)")
    return p.parse_args()


# ------------------------------------------------------------------ algorithmic bytes

M_DECODE, K_DECODE = 16, 5120
N_DECODE = (16384, 12288, 5120, 1024)
KV_H, KV_D, KV_BS, KV_NB = 4, 128, 16, 2048


def quant_bytes(m, k):
    return m * k * 2 + m * k + m * (k // 128) * 4


def gemm_bytes(m, n, k):
    g = k // 128
    return n * k + (n // 128) * g * 4 + m * k + m * g * 4 + m * n * 2


def gemv_bytes(m, n, k):
    """W8A16 tier: weight codes + block scales, bf16 activation, bf16 output."""
    return n * k + (n // 128) * (k // 128) * 4 + m * k * 2 + m * n * 2


def gemm_weight_bytes(n, k):
    return n * k + (n // 128) * (k // 128) * 4


def kv_write_bytes(t, e=KV_H * KV_D):
    return t * (2 * e * 2 + 2 * e + 8)


def kv_read_bytes(t, e=KV_H * KV_D):
    return t * (2 * e + 2 * e * 2 + 8)


def kv_amax_bytes(t, e=KV_H * KV_D):
    return 2 * t * e * 2


def prefill_copy_bytes(m, n, k, cus):
    """Bytes the prefill GEMM moves from global memory into LDS per launch: every output tile
    copies its activation and weight tile of each 128-wide group, plus 1 KB of scales when
    the scales go through LDS (the launch rule of w8a8_block_gemm_prefill: 256 x 256 tiles,
    the last round's tiles split into two 256 x 128 halves when it would leave half the CUs
    idle, the scales loaded into registers when the group count is a multiple of eight;
    else 128 x 128 tiles)."""
    g = k // 128
    big_m, big_n = -(-m // 256), -(-n // 256)
    big = big_m * big_n
    if 2 * big >= cus:
        tail = big % cus
        split = tail if (tail and 2 * tail <= cus) else 0
        whole = big - split
        scales = 0 if g % 8 == 0 else 1024
        return g * (whole * (2 * 256 * 128 + scales) + split * 2 * (256 * 128 + 128 * 128 + scales))
    tiles = -(-m // 128) * -(-n // 128)
    return g * tiles * (2 * 128 * 128 + 512)


def grouped_gemm_bytes(m, ns, k):
    """Several projections of one activation in one launch: the activation is read once."""
    return sum(gemm_bytes(m, n, k) for n in ns) - (len(ns) - 1) * (m * k + m * (k // 128) * 4)


def fused_step_gemm_bytes(m, ns, k):
    """Fused quant + grouped GEMM: bf16 activation read once, codes and scales written once,
    weights, weight scales and outputs as in the grouped GEMM."""
    return (m * k * 2 + m * k + m * (k // 128) * 4
            + sum(gemm_weight_bytes(n, k) + m * n * 2 for n in ns))


def step_bytes():
    """One decode step: the group quant launch (bf16 read, codes and scales written), the
    grouped GEMM reading those codes and scales once, then the KV batch's rows read once for
    both its absmax and its write (+ the 8-byte running max)."""
    return (quant_bytes(M_DECODE, K_DECODE) + grouped_gemm_bytes(M_DECODE, N_DECODE, K_DECODE)
            + kv_write_bytes(M_DECODE) + 8)


def fused_step_bytes():
    """The same step with the quantizer fused into the GEMM launch (codes and scales still
    written out, the activation read once as bf16)."""
    return fused_step_gemm_bytes(M_DECODE, N_DECODE, K_DECODE) + kv_write_bytes(M_DECODE) + 8


# ------------------------------------------------------------------------- timing


class Timer:
    """Kernel durations from HIP events recorded by the kernel dispatch itself: the library
    launches its next kernel with hipExtLaunchKernelGGL(start, stop) after
    fp8q_time_next_launch, so an event pair spans exactly one kernel's execution."""

    def __init__(self, torch, lib):
        import ctypes

        self.torch = torch
        self.lib = lib
        self.hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.ct = ctypes
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = [self._event() for _ in range(2 * 512)]

    def _event(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def kernel_us(self, launches, iters):
        """launches: callables each enqueueing one library kernel, cycled over; returns
        (mean_us, median_us) of the kernels' own durations."""
        assert iters <= len(self.pool) // 2
        # untimed warm-up: every buffer set at least once and ~20 launches in all, so that
        # first-touch effects and an idle GPU's clock ramp stay out of the timed launches
        for i in range(max(len(launches), 20)):
            launches[i % len(launches)]()
        self.torch.cuda.synchronize()
        for i in range(iters):
            a, b = self.pool[2 * i], self.pool[2 * i + 1]
            self.lib.fp8q_time_next_launch(a, b)
            launches[i % len(launches)]()
        self.torch.cuda.synchronize()
        us = []
        ms = self.ct.c_float()
        for i in range(iters):
            a, b = self.pool[2 * i], self.pool[2 * i + 1]
            self.hip.hipEventSynchronize(b)
            self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
            us.append(ms.value * 1e3)
        us.sort()
        return sum(us) / len(us), us[len(us) // 2]


def rotation_sets(bytes_per_set):
    return max(2, -(-ROTATE_BYTES // bytes_per_set))


# ---------------------------------------------------------------------- workloads


def bf16_dev(torch, bits):
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def build_decode(torch, fq, synth):
    """Rotation sets for the decode step: activation, quantized weights per N, outputs,
    KV batch, pools."""
    import numpy as np

    w_master = {}
    for n in N_DECODE:
        w = bf16_dev(torch, synth.decode_weight(n, K_DECODE, seed=2100 + n))
        w_master[n] = fq.fp8_block_quant(w)
        del w
    per_set = sum(gemm_bytes(M_DECODE, n, K_DECODE) for n in N_DECODE)
    nsets = rotation_sets(per_set)
    rng = np.random.default_rng(2900)
    sets = []
    e = KV_H * KV_D
    kc = torch.zeros(KV_NB * KV_BS * e, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    for i in range(nsets):
        s = {}
        s["a"] = bf16_dev(torch, synth.decode_activation(M_DECODE, seed=2000 + i))
        s["q"] = torch.empty((M_DECODE, K_DECODE), dtype=torch.uint8, device="cuda")
        s["s"] = torch.empty((M_DECODE, K_DECODE // 128), dtype=torch.float32, device="cuda")
        s["w"] = {n: (wq.clone(), ws.clone()) for n, (wq, ws) in w_master.items()}
        s["out"] = {n: torch.empty((M_DECODE, n), dtype=torch.bfloat16, device="cuda")
                    for n in N_DECODE}
        s["k"] = bf16_dev(torch, synth.to_bf16_bits(rng.normal(0, 3, size=(M_DECODE, e))))
        s["v"] = bf16_dev(torch, synth.to_bf16_bits(rng.normal(0, 3, size=(M_DECODE, e))))
        s["slots"] = torch.from_numpy(
            rng.permutation(KV_NB * KV_BS)[:M_DECODE].astype(np.int64)).cuda()
        s["amax"] = torch.zeros(2, dtype=torch.float32, device="cuda")
        sets.append(s)
    return sets, kc, vc, w_master


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU (got --gpus {args.gpus}): a sharded run executes "
              "these same kernels on each GPU's share of the shapes; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fp8_e4m3_quantization_amd as fq
    from fp8_e4m3_quantization_amd import synth

    torch.cuda.set_device(0)
    fq.load()
    timer = Timer(torch, fq.load())
    only = (set(args.only.split(",")) if args.only
            else {"step", "gemm", "grouped", "sweep", "gemv", "prefill", "quant", "kv", "calib"})
    kernels = {}

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # A plain device copy of known size: the reference that scales the rocprofv3 HBM
    # counters (FETCH_SIZE / WRITE_SIZE) to bytes.
    calib_src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    # ---------------------------------------------------------------- decode step
    log("building decode-step buffers")
    sets, kc, vc, w_master = build_decode(torch, fq, synth)
    cal = fq.KvCalibrator(1)  # frozen after its first observe (window of one token)
    e = KV_H * KV_D
    s0 = sets[0]
    cal.observe(s0["k"], s0["v"], KV_H, KV_D, kc, vc, s0["slots"], KV_BS)
    k_scale, v_scale = cal.scales()

    def run_step_fused(s):
        # group quant fused into the grouped GEMM: one launch quantizes the activation (codes
        # and scales also written out) and computes the four projections
        fq.fp8_quant_w8a8_gemm_grouped(s["a"], [(s["w"][n][0], s["w"][n][1], s["out"][n])
                                                for n in N_DECODE], q=s["q"], scales=s["s"])
        cal.observe(s["k"], s["v"], KV_H, KV_D, kc, vc, s["slots"], KV_BS)  # frozen: no-op
        # the batch's K/V absmax and its paged write, one pass over the rows
        fq.fp8_kv_write_amax(s["k"], s["v"], kc, vc, s["slots"], KV_H, KV_D, KV_BS, k_scale,
                             v_scale, s["amax"])

    def run_step(s):
        # the quantizer as a launch of its own (fp8_group_quant's codes and scales), then the
        # four projections in one grouped launch, then the KV absmax and write in one launch
        fq.fp8_group_quant(s["a"], s["q"], s["s"])
        fq.w8a8_block_gemm_grouped(s["q"], s["s"], [(s["w"][n][0], s["w"][n][1], s["out"][n])
                                                    for n in N_DECODE])
        cal.observe(s["k"], s["v"], KV_H, KV_D, kc, vc, s["slots"], KV_BS)  # frozen: no-op
        fq.fp8_kv_write_amax(s["k"], s["v"], kc, vc, s["slots"], KV_H, KV_D, KV_BS, k_scale,
                             v_scale, s["amax"])

    def time_steps(fn):
        for i in range(args.warmup):
            fn(sets[i % len(sets)])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(sets[i % len(sets)])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    result = {}
    if "step" in only:
        fms = time_steps(run_step_fused)
        result["step_fused"] = dict(ms=fms, gbs=fused_step_bytes() / (fms * 1e-3) / 1e9)
        log(f"step with the quantizer fused into the GEMM launch: {fms * 1e3:.2f} us")
        # Timed region: exactly K steps issued eagerly through the library's API (the host
        # issues a step's three launches well ahead of the GPU's ~38 us, so the stream never
        # runs dry), synchronized on both sides.
        for i in range(args.warmup):
            run_step(sets[i % len(sets)])
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(args.steps):
            run_step(sets[i % len(sets)])
        ev1.record()
        torch.cuda.synchronize()
        step_ms = ev0.elapsed_time(ev1) / args.steps
        sb = step_bytes()
        result["step"] = dict(ms=step_ms, bytes=sb, gbs=sb / (step_ms * 1e-3) / 1e9)
        log(f"step: {step_ms * 1e3:.2f} us, {result['step']['gbs']:.1f} GB/s")
        # Reported beside it: the same step captured in one HIP graph per buffer set and
        # replayed (each replay adds the graph launch's own gap on this stack).
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for s in sets:
                run_step(s)  # eager warm-up of every launch on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(s)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        ev1.record()
        torch.cuda.synchronize()
        result["step_graph"] = dict(ms=ev0.elapsed_time(ev1) / args.steps)
        log(f"step as one graph replay per step: {result['step_graph']['ms'] * 1e3:.2f} us")
        del graphs

    # ------------------------------------------------------------- GEMM per N
    if "gemm" in only:
        for n in N_DECODE:
            launches = [(lambda s=s, n=n: fq.w8a8_block_gemm(s["q"], s["s"], s["w"][n][0],
                                                             s["w"][n][1], s["out"][n]))
                        for s in sets]
            for s in sets:
                fq.fp8_group_quant(s["a"], s["q"], s["s"])
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            b = gemm_bytes(M_DECODE, n, K_DECODE)
            fl = 2.0 * M_DECODE * n * K_DECODE
            kernels[f"w8a8_gemm_m16_n{n}_k5120"] = dict(
                us=round(mean_us, 3), us_median=round(med_us, 3),
                gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
                frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                weight_gbs=round(gemm_weight_bytes(n, K_DECODE) / (mean_us * 1e-6) / 1e9, 1),
                tflops=round(fl / (mean_us * 1e-6) / 1e12, 2), bytes=b)
            log(f"gemm n={n}: {mean_us:.2f} us (median {med_us:.2f}) "
                f"{kernels[f'w8a8_gemm_m16_n{n}_k5120']['gbs']} GB/s")
            # the same projection through the K-split entry point (its own workspace per
            # stream; shapes with enough strips run the kernel above unchanged)
            ws_bytes = fq.w8a8_block_gemm_workspace_size(M_DECODE, n, K_DECODE)
            launches = [(lambda s=s, n=n: fq.w8a8_block_gemm_ws(s["q"], s["s"], s["w"][n][0],
                                                                s["w"][n][1], s["out"][n]))
                        for s in sets]
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            kernels[f"w8a8_gemm_ws_m16_n{n}_k5120"] = dict(
                us=round(mean_us, 3), us_median=round(med_us, 3),
                gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
                frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                tflops=round(fl / (mean_us * 1e-6) / 1e12, 2), bytes=b,
                workspace_bytes=ws_bytes, split=ws_bytes > 0)
            log(f"gemm (K-split entry) n={n}: {mean_us:.2f} us, workspace {ws_bytes} B, "
                f"{kernels[f'w8a8_gemm_ws_m16_n{n}_k5120']['gbs']} GB/s")

    if "grouped" in only:
        for s in sets:
            fq.fp8_group_quant(s["a"], s["q"], s["s"])
        launches = [(lambda s=s: fq.w8a8_block_gemm_grouped(
            s["q"], s["s"], [(s["w"][n][0], s["w"][n][1], s["out"][n]) for n in N_DECODE]))
            for s in sets]
        mean_us, med_us = timer.kernel_us(launches, args.iters)
        b = grouped_gemm_bytes(M_DECODE, N_DECODE, K_DECODE)
        kernels["w8a8_gemm_grouped_m16_k5120_4proj"] = dict(
            us=round(mean_us, 3), us_median=round(med_us, 3),
            gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
            frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), bytes=b,
            tflops=round(2.0 * M_DECODE * sum(N_DECODE) * K_DECODE / (mean_us * 1e-6) / 1e12, 2))
        log(f"grouped gemm (4 projections): {mean_us:.2f} us "
            f"{kernels['w8a8_gemm_grouped_m16_k5120_4proj']['gbs']} GB/s")
        launches = [(lambda s=s: fq.fp8_quant_w8a8_gemm_grouped(
            s["a"], [(s["w"][n][0], s["w"][n][1], s["out"][n]) for n in N_DECODE],
            q=s["q"], scales=s["s"])) for s in sets]
        mean_us, med_us = timer.kernel_us(launches, args.iters)
        b = fused_step_gemm_bytes(M_DECODE, N_DECODE, K_DECODE)
        kernels["quant_w8a8_gemm_fused_m16_k5120_4proj"] = dict(
            us=round(mean_us, 3), us_median=round(med_us, 3),
            gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
            frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), bytes=b)
        log(f"fused quant + grouped gemm: {mean_us:.2f} us "
            f"{kernels['quant_w8a8_gemm_fused_m16_k5120_4proj']['gbs']} GB/s")

    # ------------------------------------------------------ W8A16 tier (1..4 rows)
    if "gemv" in only:
        n = 16384
        for m in (1, 2, 4):
            acts = [bf16_dev(torch, synth.decode_activation(m, seed=4500 + m + 10 * i))
                    for i in range(len(sets))]
            outs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in sets]
            launches = [(lambda i=i: fq.w8a16_block_gemv(acts[i], sets[i]["w"][n][0],
                                                         sets[i]["w"][n][1], outs[i]))
                        for i in range(len(sets))]
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            b = gemv_bytes(m, n, K_DECODE)
            kernels[f"w8a16_gemv_m{m}_n{n}_k5120"] = dict(
                us=round(mean_us, 3), us_median=round(med_us, 3),
                gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
                frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), bytes=b)
            log(f"w8a16 gemv m={m} n={n}: {mean_us:.2f} us "
                f"{kernels[f'w8a16_gemv_m{m}_n{n}_k5120']['gbs']} GB/s")
            del acts, outs

    # --------------------------------------- W8A8 GEMM at the 4593-token prefill width
    if "prefill" in only:
        # operands and outputs rotate over >= 1 GB of sets (codes, scales, weights, output)
        # the 4593-token prefill at the four decode widths, and a short (256-token) prefill
        m_full = synth.PREFILL_TOKENS
        a = bf16_dev(torch, synth.prefill_activation(K_DECODE, seed=3100))
        q_full, s_full = fq.fp8_group_quant(a)
        del a
        for m, n in [(m_full, n) for n in N_DECODE] + [(256, 16384)]:
            q0, s0 = q_full[:m].contiguous(), s_full[:m].contiguous()
            wq0, ws0 = sets[0]["w"][n]
            per = m * K_DECODE + n * K_DECODE + m * n * 2
            nset = rotation_sets(per)
            ps = [(q0.clone(), s0.clone(), wq0.clone(), ws0.clone(),
                   torch.empty((m, n), dtype=torch.bfloat16, device="cuda")) for _ in range(nset)]
            launches = [(lambda p=p: fq.w8a8_block_gemm_prefill(*p[:4], p[4])) for p in ps]
            launches[0]()
            mean_us, med_us = timer.kernel_us(launches, min(args.iters, 50))
            fl = 2.0 * m * n * K_DECODE
            key = f"w8a8_gemm_prefill_m{m}_n{n}_k5120"
            kernels[key] = dict(us=round(mean_us, 3), us_median=round(med_us, 3),
                                tflops=round(fl / (mean_us * 1e-6) / 1e12, 1),
                                frac_mfma_fp8=round(fl / (mean_us * 1e-6) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4),
                                rotation_sets=nset)
            log(f"prefill gemm m={m} n={n}: {mean_us:.1f} us {kernels[key]['tflops']} TFLOP/s "
                f"({kernels[key]['frac_mfma_fp8']:.3f} of fp8 MFMA peak, {nset} operand sets)")
            kernels[key]["copy_bytes"] = prefill_copy_bytes(
                m, n, K_DECODE, torch.cuda.get_device_properties(0).multi_processor_count)
            del ps, launches, q0, s0
        del q_full, s_full
        m = m_full
        # The copy path alone (global -> LDS, the GEMM's own copy instructions and slices, no
        # MFMA) moving the N = 16384 launch's operand bytes, from an L2-resident span and from
        # HBM, beside the launch's MFMA time at the fp8 peak: the floors the GEMM is read
        # against (overlapped perfectly it takes the larger, serialized their sum).
        lib = fq.load()
        stream = torch.cuda.current_stream().cuda_stream
        key = f"w8a8_gemm_prefill_m{m}_n16384_k5120"
        total = kernels[key]["copy_bytes"] // 65536 * 65536
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        path = {}
        for name, span in (("l2_2MB", 2 << 20), ("hbm_1GB", 1 << 30)):
            mean_us, med_us = timer.kernel_us(
                [lambda sp=span: lib.fp8q_reference_lds_stream(src.data_ptr(), sp, total, stream)],
                10)
            path[name] = dict(us=round(mean_us, 2), us_median=round(med_us, 2),
                              gbs=round(total / (mean_us * 1e-6) / 1e9, 1))
            log(f"reference global->LDS copy of {total / 1e9:.2f} GB from {name}: {mean_us:.1f} us "
                f"({path[name]['gbs']:.0f} GB/s)")
        mfma_us = 2.0 * m * 16384 * K_DECODE / (FP8_MFMA_PEAK_TFLOPS * 1e12) * 1e6
        path["mfma_at_peak_us"] = round(mfma_us, 2)
        path["gemm_us"] = kernels[key]["us"]
        path["floor_overlapped_us"] = round(max(mfma_us, path["l2_2MB"]["us"]), 2)
        path["floor_serialized_us"] = round(mfma_us + path["l2_2MB"]["us"], 2)
        path["bytes"] = total
        kernels["prefill_copy_path_n16384"] = path
        del src

    # ----------------------------------------------------------- width sweep
    if "sweep" in only:
        n = 16384
        sweep = {}
        for m in synth.SWEEP_M:
            acts = [bf16_dev(torch, synth.decode_activation(m, seed=4000 + m + 10 * i))
                    for i in range(len(sets))]
            qs = [torch.empty((m, K_DECODE), dtype=torch.uint8, device="cuda") for _ in sets]
            ss = [torch.empty((m, K_DECODE // 128), dtype=torch.float32, device="cuda")
                  for _ in sets]
            outs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in sets]

            lq = [(lambda i=i: fq.fp8_group_quant(acts[i], qs[i], ss[i])) for i in range(len(sets))]
            lg = [(lambda i=i: fq.w8a8_block_gemm(qs[i], ss[i], sets[i]["w"][n][0],
                                                  sets[i]["w"][n][1], outs[i]))
                  for i in range(len(sets))]
            # the same pair as one launch: group quant fused into the GEMM
            lf = [(lambda i=i: fq.fp8_quant_w8a8_gemm_grouped(
                acts[i], [(sets[i]["w"][n][0], sets[i]["w"][n][1], outs[i])]))
                  for i in range(len(sets))]
            for f in lq:
                f()
            tq, _ = timer.kernel_us(lq, args.iters)
            tg, _ = timer.kernel_us(lg, args.iters)
            tf, _ = timer.kernel_us(lf, args.iters)
            wb = gemm_weight_bytes(n, K_DECODE)
            t = tq + tg
            sweep[str(m)] = dict(us_quant=round(tq, 3), us_gemm=round(tg, 3), us=round(t, 3),
                                 weight_gbs=round(wb / (t * 1e-6) / 1e9, 1),
                                 frac_hbm=round(wb / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 gemm_gbs=round(gemm_bytes(m, n, K_DECODE) / (tg * 1e-6) / 1e9, 1),
                                 us_fused=round(tf, 3),
                                 weight_gbs_fused=round(wb / (tf * 1e-6) / 1e9, 1),
                                 frac_hbm_fused=round(wb / (tf * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
            log(f"sweep m={m}: quant {tq:.2f} us + gemm {tg:.2f} us, "
                f"{sweep[str(m)]['weight_gbs']} GB/s of weights; fused in one launch "
                f"{tf:.2f} us, {sweep[str(m)]['weight_gbs_fused']} GB/s of weights")
        kernels["quant_gemm_pair_n16384_k5120"] = sweep

    # ------------------------------------------------------------- prefill quant
    if "quant" in only:
        for k in synth.PREFILL_K:
            m = synth.PREFILL_TOKENS
            x_master = bf16_dev(torch, synth.prefill_activation(k, seed=3000 + k))
            nset = rotation_sets(quant_bytes(m, k))
            xs = [x_master.clone() for _ in range(nset)]
            qs = [torch.empty((m, k), dtype=torch.uint8, device="cuda") for _ in range(nset)]
            ss = [torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
                  for _ in range(nset)]
            launches = [(lambda i=i: fq.fp8_group_quant(xs[i], qs[i], ss[i])) for i in range(nset)]
            for f in launches:
                f()
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            b = quant_bytes(m, k)
            kernels[f"group_quant_m{m}_k{k}"] = dict(
                us=round(mean_us, 3), us_median=round(med_us, 3),
                gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
                frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), bytes=b)
            log(f"group quant k={k}: {mean_us:.2f} us {kernels[f'group_quant_m{m}_k{k}']['gbs']} GB/s")
            del xs, qs, ss, x_master

    # ---------------------------------------------------------------- KV pool
    if "kv" in only:
        full = synth.kv_full_pool()
        t = len(full.slots)
        per = kv_write_bytes(t) + KV_NB * KV_BS * e * 2 + 2 * t * e * 2
        nset = rotation_sets(per)
        kd = bf16_dev(torch, full.k)
        vd = bf16_dev(torch, full.v)
        sd = torch.from_numpy(full.slots).cuda()
        bufs = [(kd.clone(), vd.clone(), sd.clone(), torch.zeros_like(kc), torch.zeros_like(vc),
                 torch.zeros(2, dtype=torch.float32, device="cuda"), torch.empty_like(kd),
                 torch.empty_like(vd)) for _ in range(nset)]
        ks_, vs_ = 3.0 * 20.0 / 448.0, 3.0 * 20.0 / 448.0
        wl = [(lambda b=b: fq.fp8_kv_write(b[0], b[1], b[3], b[4], b[2], KV_H, KV_D, KV_BS,
                                           ks_, vs_)) for b in bufs]
        al = [(lambda b=b: fq.fp8_kv_amax(b[0], b[1], b[5])) for b in bufs]
        rl = [(lambda b=b: fq.fp8_kv_read(b[3], b[4], b[2], KV_H, KV_D, KV_BS, ks_, vs_,
                                          k_out=b[6], v_out=b[7])) for b in bufs]
        for f in wl + al + rl:
            f()
        for name, launches, b in (("kv_write_full_pool", wl, kv_write_bytes(t)),
                                  ("kv_amax_full_pool", al, kv_amax_bytes(t)),
                                  ("kv_read_full_pool", rl, kv_read_bytes(t))):
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            kernels[f"{name}_t{t}"] = dict(
                us=round(mean_us, 3), us_median=round(med_us, 3),
                gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
                frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), bytes=b)
            log(f"{name}: {mean_us:.2f} us {kernels[f'{name}_t{t}']['gbs']} GB/s")
        # per-batch latency of a decode-time write (absmax fused in) for 1..64 tokens: the
        # first T rows of each buffer set onto their (distinct) slots
        lat = {}
        for tb in (1, 4, 16, 64):
            bl = [(lambda b=b, tb=tb: fq.fp8_kv_write_amax(
                b[0][:tb], b[1][:tb], b[3], b[4], b[2][:tb], KV_H, KV_D, KV_BS, ks_, vs_, b[5]))
                for b in bufs]
            mean_us, med_us = timer.kernel_us(bl, args.iters)
            lat[str(tb)] = dict(us=round(mean_us, 3), us_median=round(med_us, 3),
                                bytes=kv_write_bytes(tb))
        kernels["kv_write_amax_batch_latency"] = lat
        log("kv write+absmax batch latency: " + ", ".join(
            f"{tb} tok {v['us']:.2f} us" for tb, v in lat.items()))
        # the same write and read with the slots of a paged prefill: blocks in random order,
        # 16 consecutive tokens per block (8 KB contiguous per block and pool)
        runs = torch.from_numpy(synth.kv_block_runs()).cuda()
        run_slots = [runs.clone() for _ in bufs]
        wl = [(lambda b=b, r=r: fq.fp8_kv_write(b[0], b[1], b[3], b[4], r, KV_H, KV_D, KV_BS,
                                                ks_, vs_)) for b, r in zip(bufs, run_slots)]
        rl = [(lambda b=b, r=r: fq.fp8_kv_read(b[3], b[4], r, KV_H, KV_D, KV_BS, ks_, vs_,
                                               k_out=b[6], v_out=b[7]))
              for b, r in zip(bufs, run_slots)]
        for name, launches, b in (("kv_write_block_runs", wl, kv_write_bytes(t)),
                                  ("kv_read_block_runs", rl, kv_read_bytes(t))):
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            kernels[f"{name}_t{t}"] = dict(
                us=round(mean_us, 3), us_median=round(med_us, 3),
                gbs=round(b / (mean_us * 1e-6) / 1e9, 1),
                frac_hbm=round(b / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), bytes=b)
            log(f"{name}: {mean_us:.2f} us {kernels[f'{name}_t{t}']['gbs']} GB/s")
        del bufs, run_slots

    # ------------------------------------------------- measurement references
    # What a launch costs with no work, and a plain 2:1 read/write stream of the same bytes
    # as the group quantizer and the KV write (no arithmetic), timed by the same hook: the
    # ceiling the bandwidth kernels are read against.
    if "quant" in only or "kv" in only:
        lib = fq.load()
        stream = torch.cuda.current_stream().cuda_stream
        mean_us, med_us = timer.kernel_us([lambda: lib.fp8q_reference_empty(stream)], args.iters)
        refs = {"empty_kernel": dict(us=round(mean_us, 3), us_median=round(med_us, 3))}
        log(f"reference empty kernel: {mean_us:.2f} us (median {med_us:.2f})")
        shapes = {f"group_quant_m{synth.PREFILL_TOKENS}_k{k}": (quant_bytes(synth.PREFILL_TOKENS, k),
                                                               synth.PREFILL_TOKENS * k * 2)
                  for k in synth.PREFILL_K}
        shapes["kv_write_full_pool_t32768"] = (kv_write_bytes(KV_NB * KV_BS), 2 * KV_NB * KV_BS * e * 2)
        for name, (alg_bytes, read_bytes) in shapes.items():
            nset = rotation_sets(read_bytes * 3 // 2)
            bufs = [(torch.ones(read_bytes // 2, dtype=torch.int16, device="cuda"),
                     torch.empty(read_bytes // 2, dtype=torch.uint8, device="cuda"))
                    for _ in range(nset)]
            launches = [(lambda b=b, rb=read_bytes: lib.fp8q_reference_stream(
                b[0].data_ptr(), b[1].data_ptr(), rb, stream)) for b in bufs]
            mean_us, med_us = timer.kernel_us(launches, args.iters)
            moved = read_bytes * 3 // 2
            ent = dict(us=round(mean_us, 3), us_median=round(med_us, 3), bytes=moved,
                       gbs=round(moved / (mean_us * 1e-6) / 1e9, 1),
                       frac_hbm=round(moved / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
            refs[f"stream_2to1_as_{name}"] = ent
            if name in kernels:
                kernels[name]["frac_of_stream_reference"] = round(ent["us"] / kernels[name]["us"], 4)
            log(f"reference 2:1 stream for {name}: {mean_us:.2f} us, {ent['frac_hbm']:.3f} of HBM")
            del bufs, launches
        kernels["references"] = refs

    # ----------------------------------------- calibration window (one layer, 256 tokens)
    if "calib" in only:
        kernels["calibration_window"] = calib_window(torch, fq, synth, log)

    # ---------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline and "step" in only:
        cpu = cpu_baseline(synth, log)

    # --------------------------------------------------------------- report
    dom_name = "w8a8_gemm_grouped_m16_k5120_4proj"
    dom = kernels.get(dom_name)
    roof = None
    if dom:
        roof = dict(bound="hbm", achieved=dom["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(dom["gbs"] / HBM_PEAK_GBS, 4),
                    traffic=profiled_traffic(dom_name),
                    kernel="w8a8_staged_kernel<5, false, 3> (4 decode projections, one "
                           "launch)",
                    bytes_per_launch=dom["bytes"], us_per_launch=dom["us"])
    st = result.get("step")
    line = {
        "metric": "HBM GB/s (% of 8 TB/s) for W8A8 decode GEMM M=16 and group quant",
        "value": round(st["gbs"], 1) if st else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["ms"], 5) if st else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> f32 (quantizer f32)",
        "data": "synthetic (seeded; weights ~N(0,0.02) block-quantized on the GPU)",
        "config": {
            "workload": "decode step: group quant [16x5120] + W8A8 GEMM M=16 K=5120 "
                        "N=16384,12288,5120,1024 + KV amax/write 16 tokens (4x128, bs 16)",
            "M": M_DECODE, "K": K_DECODE, "N": list(N_DECODE), "kv_tokens": M_DECODE,
            "kv_heads": KV_H, "head_dim": KV_D, "block_size": KV_BS,
            "bytes_per_step": step_bytes(), "rotation_sets": len(sets),
            "parallelism": "single GPU",
        },
        "frac_hbm": round(st["gbs"] / HBM_PEAK_GBS, 4) if st else None,
        "step_launch": {"eager_us": round(st["ms"] * 1e3, 2) if st else None,
                        "graph_replay_us": round(result["step_graph"]["ms"] * 1e3, 2)
                        if "step_graph" in result else None,
                        "quantizer_fused_into_gemm_us": round(result["step_fused"]["ms"] * 1e3, 2)
                        if "step_fused" in result else None,
                        "quantizer_fused_into_gemm_gbs": round(result["step_fused"]["gbs"], 1)
                        if "step_fused" in result else None},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


def profiled_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic.txt: '<kernel key> <bytes per launch> <source files, comma-separated>
    <sha256 of their contents>'), if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    try:
        with open(path) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 4 and parts[0] == name:
                    if sources_sha(parts[2].split(",")) == parts[3]:
                        return int(parts[1])
                    return None
    except OSError:
        return None
    return None


def sources_sha(rels):
    h = hashlib.sha256()
    for rel in rels:
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    return h.hexdigest()


def calib_window(torch, fq, synth, log, repeats=5):
    """One layer's calibration over the 256-token window of the seeded paged batches (4 KV
    heads x 128, block 16, 2048 blocks), through the library's calibrator: per in-window
    observe (absmax folded on the device + staging copies, no host wait) and for the
    freezing observe (the one 8-byte read, the last-writer mask, the one-launch replay and
    the stream-ordered release), the host time of the call and the GPU time of the work it
    enqueued (events around the call on an otherwise idle stream).  Beside them, what the
    per-observe synchronization of a design that reads the absmax back every batch costs
    here: the same absmax kernel, then a blocking 8-byte read."""
    import numpy as np

    e = KV_H * KV_D
    batches, _ = synth.kv_batches(num_tokens_total=synth.KV_WINDOW + 96, seed=5000)
    dev = [(bf16_dev(torch, b.k), bf16_dev(torch, b.v), torch.from_numpy(b.slots).cuda())
           for b in batches]
    kc = torch.zeros(KV_NB * KV_BS * e, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stage_host, stage_gpu, freeze_host, freeze_gpu, sync_host = [], [], [], [], []
    for rep in range(repeats + 1):  # the first pass warms up allocations and code
        cal = fq.KvCalibrator(synth.KV_WINDOW)
        for (k, v, sl), b in zip(dev, batches):
            step = cal.decide(len(b.slots), e)
            if step == fq.FP8Q_CALIB_FROZEN:
                break
            torch.cuda.synchronize()
            ev0.record()
            t0 = time.perf_counter()
            cal.observe(k, v, KV_H, KV_D, kc, vc, sl, KV_BS)
            t1 = time.perf_counter()
            ev1.record()
            ks, vs = cal.scales()
            fq.fp8_kv_write(k, v, kc, vc, sl, KV_H, KV_D, KV_BS, ks, vs)
            torch.cuda.synchronize()
            if rep == 0:
                continue
            host_us, gpu_us = (t1 - t0) * 1e6, ev0.elapsed_time(ev1) * 1e3
            if step == fq.FP8Q_CALIB_STAGE:
                stage_host.append(host_us)
                stage_gpu.append(gpu_us)
            elif step == fq.FP8Q_CALIB_FREEZE:
                freeze_host.append(host_us)
                freeze_gpu.append(gpu_us)
        staged = cal.info()["replayed_tokens"]
        cal.close()
        if rep > 0:
            amax2 = torch.zeros(2, dtype=torch.float32, device="cuda")
            for k, v, sl in dev[:8]:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                fq.fp8_kv_amax(k, v, amax2)
                amax2.cpu()  # blocking 8-byte read
                sync_host.append((time.perf_counter() - t0) * 1e6)
    res = dict(window_tokens=synth.KV_WINDOW, batches_in_window=len(stage_host) // repeats,
               replayed_tokens=staged, repeats=repeats,
               observe_in_window=dict(host_us=round(float(np.mean(stage_host)), 2),
                                      gpu_us=round(float(np.mean(stage_gpu)), 2),
                                      host_waits=0),
               observe_freeze=dict(host_us=round(float(np.mean(freeze_host)), 2),
                                   gpu_us=round(float(np.mean(freeze_gpu)), 2), host_waits=1),
               per_observe_sync_removed=dict(host_us=round(float(np.mean(sync_host)), 2),
                                             what="absmax kernel + blocking 8-byte read"))
    log(f"calibration window: in-window observe host {res['observe_in_window']['host_us']} us, "
        f"gpu {res['observe_in_window']['gpu_us']} us; freeze host "
        f"{res['observe_freeze']['host_us']} us, gpu {res['observe_freeze']['gpu_us']} us; "
        f"a per-observe sync would cost {res['per_observe_sync_removed']['host_us']} us")
    return res


def cpu_baseline(synth, log):
    """The CPU oracle, as it stands, on full decode steps: single-threaded (about 10 s in
    all), and with the group quant and the GEMM split by rows over the host threads (the
    oracle's row-parallel wrappers; the KV write stays sequential, its order is part of its
    definition)."""
    import numpy as np

    import oracle

    log("cpu baseline: oracle on full decode steps")
    a = synth.decode_activation(M_DECODE, seed=2000)
    ws = {n: oracle.block_quant(synth.decode_weight(n, K_DECODE, seed=2100 + n))
          for n in N_DECODE}
    rng = np.random.default_rng(2900)
    e = KV_H * KV_D
    k = synth.to_bf16_bits(rng.normal(0, 3, size=(M_DECODE, e)))
    v = synth.to_bf16_bits(rng.normal(0, 3, size=(M_DECODE, e)))
    slots = rng.permutation(KV_NB * KV_BS)[:M_DECODE].astype(np.int64)
    kc = np.zeros(KV_NB * KV_BS * e, dtype=np.uint8)
    vc = np.zeros_like(kc)
    threads = oracle.default_threads()

    def step(parallel):
        if parallel:
            q, s = oracle.group_quant_rows(a, threads)
            for n in N_DECODE:
                oracle.gemm_rows(q, s, *ws[n], threads=threads)
        else:
            q, s = oracle.group_quant(a)
            for n in N_DECODE:
                oracle.gemm(q, s, *ws[n])
        oracle.amax(k)
        oracle.amax(v)
        oracle.kv_write(k, v, kc, vc, slots, M_DECODE, KV_H, KV_D, KV_BS, 0.1, 0.1, e, e,
                        KV_BS * e)

    def timed(parallel, budget, max_steps):
        steps, total = 0, 0.0
        while steps < 1 or (total < budget and steps < max_steps):
            t0 = time.perf_counter()
            step(parallel)
            total += time.perf_counter() - t0
            steps += 1
        return steps, total / steps

    n1, dt1 = timed(False, 10.0, 10)
    np_, dtp = timed(True, 5.0, 40)
    gbs1, gbsp = step_bytes() / dt1 / 1e9, step_bytes() / dtp / 1e9
    log(f"cpu baseline: 1 thread {n1} steps, {dt1:.2f} s per step, {gbs1:.4f} GB/s; "
        f"{threads} threads {np_} steps, {dtp:.3f} s per step, {gbsp:.4f} GB/s")
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    return dict(value=round(gbsp, 5), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{np_} full decode steps (same shapes as the GPU step), {dtp:.3f} s "
                       f"each, C oracle with group quant and FP64 GEMM split by rows over "
                       f"{threads} threads, KV write sequential",
                single_thread=dict(value=round(gbs1, 5), unit="GB/s", cores=1,
                                   sample=f"{n1} full decode steps, {dt1:.2f} s each"),
                cpu_model=model, host_cpus=os.cpu_count())


if __name__ == "__main__":
    main()
