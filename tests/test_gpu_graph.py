"""The decode step (fused and with the quantizer as its own launch) captured in a HIP graph:
every replay gives the eager bytes.

The step (fused group quant + four projections, then the KV batch's absmax and write) is
captured once; the graph is replayed several times with eager library calls and
synchronizations in between, and every replay's outputs must equal the eager run's
exactly (codes, scales, GEMM outputs, pools, running max)."""
import numpy as np
import pytest
import torch

import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import DEV, bf16_dev, host, i64_dev, need_gpu

pytestmark = pytest.mark.gpu

NS = (1024, 512, 256)
K = 1024
M = 16
H, D, BS, NB = 4, 128, 16, 64


def setup_module(_):
    need_gpu()


def _state():
    w = {n: fq.fp8_block_quant(bf16_dev(synth.decode_weight(n, K, seed=700 + n))) for n in NS}
    rng = np.random.default_rng(71)
    st = dict(
        a=bf16_dev(synth.decode_activation(M, k=K, seed=72)),
        q=torch.empty((M, K), dtype=torch.uint8, device=DEV),
        s=torch.empty((M, K // 128), dtype=torch.float32, device=DEV),
        out={n: torch.empty((M, n), dtype=torch.bfloat16, device=DEV) for n in NS},
        k=bf16_dev(synth.to_bf16_bits(rng.normal(0, 3, size=(M, H * D)))),
        v=bf16_dev(synth.to_bf16_bits(rng.normal(0, 3, size=(M, H * D)))),
        slots=i64_dev(rng.permutation(NB * BS)[:M].astype(np.int64)),
        kc=torch.zeros(NB * BS * H * D, dtype=torch.uint8, device=DEV),
        vc=torch.zeros(NB * BS * H * D, dtype=torch.uint8, device=DEV),
        amax=torch.zeros(2, dtype=torch.float32, device=DEV),
    )
    return w, st


def _step(w, st, fused=True):
    if fused:
        fq.fp8_quant_w8a8_gemm_grouped(st["a"], [(w[n][0], w[n][1], st["out"][n]) for n in NS],
                                       q=st["q"], scales=st["s"])
    else:  # the quantizer as a launch of its own, then the grouped GEMM on its codes
        fq.fp8_group_quant(st["a"], st["q"], st["s"])
        fq.w8a8_block_gemm_grouped(st["q"], st["s"], [(w[n][0], w[n][1], st["out"][n])
                                                      for n in NS])
    fq.fp8_kv_write_amax(st["k"], st["v"], st["kc"], st["vc"], st["slots"], H, D, BS, 0.05,
                         0.07, st["amax"])


def _snapshot(st):
    return [host(st["q"]), host(st["s"]), *[host(st["out"][n]) for n in NS], host(st["kc"]),
            host(st["vc"]), host(st["amax"])]


def _clear(st):
    for key in ("q", "s", "kc", "vc", "amax"):
        st[key].zero_()
    for n in NS:
        st["out"][n].zero_()


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_equal_eager(fused):
    w, st = _state()
    _step(w, st, fused)
    want = _snapshot(st)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(w, st, fused)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, st, fused)
    for rep in range(4):
        _clear(st)
        # eager library work between replays
        fq.fp8_group_quant(bf16_dev(synth.decode_activation(3, k=K, seed=rep)))
        torch.cuda.synchronize()
        g.replay()
        got = _snapshot(st)
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {rep} differs"
