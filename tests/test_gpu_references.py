"""GPU checks of the measurement references the bench reads the path against: the 2:1
stream writes exactly the word its definition names for every 16 bytes read, the copy-path
stream and the empty kernel run to completion, and each refuses bad sizes before launching.
(They are references, not steps of the path, so their check is their own definition.)"""
import numpy as np
import pytest
import torch

import fp8_e4m3_quantization_amd as fq
from tests.gpu_util import DEV, host, need_gpu

pytestmark = pytest.mark.gpu
EINVAL = -1


def setup_module(_):
    need_gpu()


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("words", [1, 255, 4096 * 3 + 7, 1 << 20])
def test_stream_reference_writes_xor_of_word_pairs(words):
    lib = fq.load()
    rng = np.random.default_rng(words)
    src = rng.integers(0, 2 ** 32, size=words * 4, dtype=np.uint32)
    src_d = torch.from_numpy(src.view(np.int32)).to(DEV)
    dst_d = torch.full((words * 2,), -1, dtype=torch.int32, device=DEV)
    assert lib.fp8q_reference_stream(src_d.data_ptr(), dst_d.data_ptr(), words * 16, _stream()) == 0
    got = host(dst_d).view(np.uint32).reshape(words, 2)
    w = src.reshape(words, 4)
    assert np.array_equal(got[:, 0], w[:, 0] ^ w[:, 1])
    assert np.array_equal(got[:, 1], w[:, 2] ^ w[:, 3])


def test_lds_stream_and_empty_references_complete():
    lib = fq.load()
    span = 2 << 20
    src = torch.ones(span, dtype=torch.uint8, device=DEV)
    for total in (65536, 64 * 65536, 1024 * 65536 + 3 * 65536):
        assert lib.fp8q_reference_lds_stream(src.data_ptr(), span, total, _stream()) == 0
    assert lib.fp8q_reference_empty(_stream()) == 0
    torch.cuda.synchronize()
    assert lib.fp8q_reference_lds_stream(src.data_ptr(), span + 16, 65536, _stream()) == EINVAL
    assert lib.fp8q_reference_lds_stream(src.data_ptr(), span, 65536 + 1, _stream()) == EINVAL
    assert lib.fp8q_reference_stream(src.data_ptr(), src.data_ptr(), 24, _stream()) == EINVAL
