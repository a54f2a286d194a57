"""CPU checks of bench.py's algorithmic byte counts (the numerators of every GB/s figure and
of the roofline's `achieved`) against the per-unit figures they are built from, and of its
single-GPU guard."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_group_quant_bytes_per_group():
    # one 1x128 group: 256 B of bf16 read, 128 codes and one fp32 scale written
    assert bench.quant_bytes(1, 128) == 256 + 128 + 4
    assert bench.quant_bytes(4593, 5120) == 4593 * 40 * 388


def test_kv_bytes_per_token():
    # 4 heads x 128: K and V rows of 512 bf16 read, 512 codes each written, one int64 slot
    assert bench.kv_write_bytes(1) == 2 * 512 * 2 + 2 * 512 + 8 == 3080
    assert bench.kv_read_bytes(1) == 3080
    assert bench.kv_amax_bytes(32768) == 2 * 32768 * 512 * 2


def test_gemm_bytes_decompose_into_strips_activation_and_output():
    m, n, k = 16, 16384, 5120
    strips = n // 16
    per_strip = 16 * k + (k // 128) * 4 / 8      # a 128-column scale row serves 8 strips
    weights = strips * per_strip
    assert bench.gemm_weight_bytes(n, k) == weights == n * k + (n // 128) * (k // 128) * 4
    assert bench.gemm_bytes(m, n, k) == weights + m * k + m * (k // 128) * 4 + m * n * 2
    assert bench.gemv_bytes(m, n, k) == weights + m * k * 2 + m * n * 2


def test_grouped_and_fused_read_the_activation_once():
    m, k, ns = 16, 5120, bench.N_DECODE
    act_q = m * k + m * (k // 128) * 4
    singles = sum(bench.gemm_bytes(m, n, k) for n in ns)
    assert bench.grouped_gemm_bytes(m, ns, k) == singles - (len(ns) - 1) * act_q
    # fused: bf16 read once, codes and scales written once, then weights and outputs
    fused = m * k * 2 + act_q + sum(bench.gemm_weight_bytes(n, k) + m * n * 2 for n in ns)
    assert bench.fused_step_gemm_bytes(m, ns, k) == fused
    assert bench.fused_step_bytes() == fused + bench.kv_write_bytes(16) + 8
    # the headline step: the quantizer's own launch, then the grouped GEMM reading its
    # codes and scales once
    grouped = bench.grouped_gemm_bytes(m, ns, k)
    assert bench.step_bytes() == (m * k * 2 + act_q) + grouped + bench.kv_write_bytes(16) + 8


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def test_prefill_copy_bytes_follow_the_launch_rule():
    # 4593 x 16384 on 256 CUs: 18 x 64 = 1152 tiles of 256 x 256, a last round of 128 tiles
    # (half the CUs) split into 256 x 128 halves; per 128-wide group a whole tile copies its
    # two 32 KB operand tiles, a half 32 KB + 16 KB (40 groups, a multiple of eight: the
    # scales go to registers, not LDS)
    g = 5120 // 128
    whole, split = 1152 - 128, 128
    assert bench.prefill_copy_bytes(4593, 16384, 5120, 256) == g * (
        whole * 2 * 32768 + split * 2 * (32768 + 16384))
    # with a group count that is not a multiple of eight 1 KB of scales per tile goes
    # through LDS too
    g = 5248 // 128
    assert bench.prefill_copy_bytes(4593, 16384, 5248, 256) == g * (
        whole * (2 * 32768 + 1024) + split * 2 * (32768 + 16384 + 1024))
    # a last round more than half full (712 = 2 x 256 + 200 tiles) is not split
    assert bench.prefill_copy_bytes(256 * 4, 256 * 178, 128, 256) == 712 * (2 * 32768 + 1024)
    g = 5120 // 128
    # fewer tiles than half the CUs: 128 x 128 tiles, 16 KB per operand + 512 B of scales
    assert bench.prefill_copy_bytes(4593, 1024, 5120, 256) == g * 36 * 8 * (2 * 16384 + 512)
