"""Helpers for the GPU parity tests: move the generators' numpy bit patterns to and from
the device as torch tensors (no arithmetic happens here)."""
import numpy as np
import pytest
import torch

DEV = torch.device("cuda:0")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i64_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_host_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_tolerance_ok(got_bits: np.ndarray, ref: np.ndarray):
    """|gpu - ref| <= 1e-2 |ref| + 1e-3 rms(ref), element-wise, rms over the call's output."""
    got = bf16_host_to_f64(got_bits)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref)
    bound = 1e-2 * np.abs(ref) + 1e-3 * rms
    ok = err <= bound
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    return bool(np.all(ok)), worst
