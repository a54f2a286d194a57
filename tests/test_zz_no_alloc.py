"""GPU: the allocation-free K-split decode GEMM (w8a8_block_gemm_noalloc), called through the
C ABI, against the workspace entry point it mirrors (w8a8_block_gemm_ws: same split, same
bits) and against the oracle's tolerance, on two calls in a row (the second with a smaller
input), then again on the first shape (the static array's counts were left at zero)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import fp8_e4m3_quantization_amd as fq
from fp8_e4m3_quantization_amd import synth
from tests.gpu_util import DEV, f32_dev, gemm_tolerance_ok, host, need_gpu, u8_dev

pytestmark = pytest.mark.gpu


def setup_module(_):
    need_gpu()


def _operands(m, n, k, seed):
    a = synth.decode_activation(m, k=k, seed=seed)
    q, s = oracle.group_quant(a)
    wq, ws = oracle.block_quant(synth.decode_weight(n, k, seed=seed + 1))
    return q, s, wq, ws


def _noalloc(args, out, m, n, k):
    lib = fq.load()
    rc = lib.w8a8_block_gemm_noalloc(*(t.data_ptr() for t in args), out.data_ptr(), m, n, k, n,
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fq.strerror(rc)
    return host(out)


def test_noalloc_equals_the_workspace_entry_point_on_consecutive_calls():
    results = []
    for m, n, k, seed in [(16, 1024, 5248, 7100), (5, 128, 5248, 7200), (16, 1024, 5248, 7100)]:
        assert fq.w8a8_block_gemm_workspace_size(m, n, k) > 0, "shape takes the split path"
        q, s, wq, ws = _operands(m, n, k, seed)
        args = (u8_dev(q), f32_dev(s), u8_dev(wq), f32_dev(ws))
        out = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=DEV)
        got = _noalloc(args, out, m, n, k)
        want = host(fq.w8a8_block_gemm_ws(*args))
        assert np.array_equal(got, want)
        ok, worst = gemm_tolerance_ok(got, oracle.gemm(q, s, wq, ws))
        assert ok, worst
        results.append(got)
    assert np.array_equal(results[0], results[2])


def test_noalloc_unsplit_shape_is_w8a8_block_gemm():
    m, n, k = 16, 16384, 5120
    q, s, wq, ws = _operands(m, n, k, 7300)
    args = (u8_dev(q), f32_dev(s), u8_dev(wq), f32_dev(ws))
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    assert np.array_equal(_noalloc(args, out, m, n, k), host(fq.w8a8_block_gemm(*args)))


def test_noalloc_argument_errors_enqueue_nothing():
    lib = fq.load()
    p = ctypes.c_void_p(1 << 20)
    assert lib.w8a8_block_gemm_noalloc(p, p, p, p, p, 17, 1024, 5120, 1024, None) == -1
    assert lib.w8a8_block_gemm_noalloc(p, None, p, p, p, 16, 1024, 5120, 1024, None) == -2
    assert lib.w8a8_block_gemm_noalloc(p, p, p, p, p, 16, 1024, 5120, 1000, None) == -1
