"""FP8 (OCP E4M3) quantize-and-consume path for AMD MI355X (gfx950).

The compute lives in ``libfp8q.so`` (HIP kernels behind the C ABI in ``include/fp8q.h``);
this package is its thin Python binding (argument marshalling on torch tensors) plus the
seeded synthetic workload generators in ``synth``.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    FP8Q_CALIB_DECLINE,
    FP8Q_CALIB_FREEZE,
    FP8Q_CALIB_FROZEN,
    FP8Q_CALIB_STAGE,
    Fp8qError,
    KvCalibOps,
    KvCalibrator,
    KvTarget,
    fp8_block_quant,
    fp8_e4m3_encode,
    fp8_group_quant,
    fp8_kv_amax,
    fp8_kv_read,
    fp8_kv_write,
    fp8_kv_write_amax,
    fp8_quant_w8a8_gemm_grouped,
    load,
    strerror,
    gemm_workspace,
    w8a8_block_gemm,
    w8a8_block_gemm_noalloc,
    w8a8_block_gemm_workspace_size,
    w8a8_block_gemm_ws,
    w8a8_block_gemm_prefill,
    w8a8_block_gemm_grouped,
    w8a16_block_gemv,
    w8a16_block_gemv_grouped,
)
