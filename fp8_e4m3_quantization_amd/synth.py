"""Seeded synthetic inputs shaped like the workloads the FP8 pages describe.

This module only draws random numbers and rounds them to bfloat16; it holds none of the
quantization arithmetic, so both the HIP path's tests/benchmark and the CPU oracle read the
same bf16 bits from here.

Recipe (all workloads):
  * numpy ``default_rng(seed)``; values drawn in float64, rounded to float32, then to
    bfloat16 with round-to-nearest-even (torch's CPU conversion);
  * an "outlier" is an independent Bernoulli(p) mask per entry that multiplies the entry
    by a factor, keeping its sign.
Workloads (sizes from the pages: 16-row decode projections at K=5120, a 4593-token
prefill, a 4-head x 128-dim FP8 KV cache paged in blocks of 16 tokens):
  tiny_e2e            A bf16 [16 x 512] ~N(0,1), 1% x20 outliers; W bf16 [1024 x 512] ~N(0,0.02)
  decode_projection   A bf16 [M x 5120] ~N(0,1), 0.5% x30 outliers; W bf16 [N x 5120] ~N(0,0.02)
  prefill_activation  bf16 [4593 x K], rows ~N(0,1) x exp(U(ln 0.01, ln 100)), 0.1% x50 outliers
  kv_batches          K/V bf16 [T, 4*128] ~N(0,1)*3, 0.2% x40 outliers, T ~ U{1..64},
                      int64 slots from a paged block allocator with free / re-allocation
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

DECODE_K = 5120
DECODE_N = (16384, 12288, 5120, 1024)
PREFILL_TOKENS = 4593
PREFILL_K = (5120, 16384)
SWEEP_M = (5, 8, 12, 16)
KV_HEADS = 4
KV_HEAD_DIM = 128
KV_BLOCK_SIZE = 16
KV_NUM_BLOCKS = 2048
KV_WINDOW = 256


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64/float32 array -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_with_outliers(rng: np.random.Generator, shape, std: float, p: float,
                         factor: float) -> np.ndarray:
    x = rng.normal(0.0, std, size=shape)
    mask = rng.random(size=shape) < p
    return np.where(mask, x * factor, x)


# ----------------------------------------------------------------------- activations


def tiny_e2e(seed: int = 0):
    """Tiny end-to-end case: returns (A bf16 bits [16,512], W bf16 bits [1024,512])."""
    rng = np.random.default_rng(seed)
    a = normal_with_outliers(rng, (16, 512), 1.0, 0.01, 20.0)
    w = rng.normal(0.0, 0.02, size=(1024, 512))
    return to_bf16_bits(a), to_bf16_bits(w)


def decode_activation(m: int, k: int = DECODE_K, seed: int = 2000) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bf16_bits(normal_with_outliers(rng, (m, k), 1.0, 0.005, 30.0))


def decode_weight(n: int, k: int = DECODE_K, seed: int = 2100) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.normal(0.0, 0.02, size=(n, k)))


def prefill_activation(k: int, m: int = PREFILL_TOKENS, seed: int = 3000) -> np.ndarray:
    rng = np.random.default_rng(seed)
    mag = np.exp(rng.uniform(np.log(0.01), np.log(100.0), size=(m, 1)))
    x = rng.normal(0.0, 1.0, size=(m, k)) * mag
    mask = rng.random(size=(m, k)) < 0.001
    return to_bf16_bits(np.where(mask, x * 50.0, x))


def random_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return to_bf16_bits(rng.normal(0.0, std, size=shape))


# ------------------------------------------------------------------------- KV cache


@dataclasses.dataclass
class KvBatch:
    k: np.ndarray      # bf16 bits [T, H*D]
    v: np.ndarray      # bf16 bits [T, H*D]
    slots: np.ndarray  # int64 [T]


class BlockAllocator:
    """Paged-cache block allocator: a free stack whose top few entries are picked at
    random, so freed blocks are re-allocated soon (as a serving allocator does)."""

    def __init__(self, rng: np.random.Generator, num_blocks: int, pick_window: int = 4):
        self.rng = rng
        self.free = list(rng.permutation(num_blocks)[::-1])
        self.pick_window = pick_window

    def alloc(self) -> int:
        if not self.free:
            raise RuntimeError("KV pool exhausted")
        w = min(self.pick_window, len(self.free))
        i = len(self.free) - 1 - int(self.rng.integers(0, w))
        return int(self.free.pop(i))

    def release(self, blocks):
        self.free.extend(blocks)


def kv_batches(num_tokens_total: int = KV_WINDOW + 64, seed: int = 5000,
               heads: int = KV_HEADS, head_dim: int = KV_HEAD_DIM,
               block_size: int = KV_BLOCK_SIZE, num_blocks: int = KV_NUM_BLOCKS,
               max_batch: int = 64, seq_len_range=(4, 48)):
    """Batches of U{1..max_batch} tokens until ``num_tokens_total`` tokens are produced.

    Tokens come from sequences of random length; each token appends to a live sequence
    (a new block is allocated at every block boundary); a sequence that reaches its length
    frees its blocks, which later batches re-allocate.  Slots within one batch are
    distinct.  Returns (batches, reuse) where ``reuse`` lists (batch, slot) pairs written
    again after their block was freed and re-allocated."""
    rng = np.random.default_rng(seed)
    alloc = BlockAllocator(rng, num_blocks)
    e = heads * head_dim
    live = []  # dicts: blocks, pos, length
    written = {}  # slot -> batch index of the latest write
    freed_blocks = set()
    reuse = []
    batches = []
    produced = 0
    bidx = 0
    while produced < num_tokens_total:
        t = int(rng.integers(1, max_batch + 1))
        t = min(t, num_tokens_total - produced)
        slots = []
        finished = []
        while len(slots) < t:
            if not live or rng.random() < 0.15:
                live.append(dict(blocks=[], pos=0,
                                 length=int(rng.integers(seq_len_range[0],
                                                         seq_len_range[1] + 1))))
            s = live[int(rng.integers(0, len(live)))]
            # one token per sequence per batch keeps slots distinct within the batch,
            # except a sequence may add a short run of consecutive tokens (a prefill chunk)
            run = int(rng.integers(1, 5))
            for _ in range(run):
                if len(slots) >= t or s["pos"] >= s["length"]:
                    break
                if s["pos"] % block_size == 0:
                    blk = alloc.alloc()
                    if blk in freed_blocks:
                        freed_blocks.discard(blk)
                    s["blocks"].append(blk)
                slot = s["blocks"][s["pos"] // block_size] * block_size + s["pos"] % block_size
                if slot in written:
                    reuse.append((bidx, slot))
                written[slot] = bidx
                slots.append(slot)
                s["pos"] += 1
            if s["pos"] >= s["length"]:
                live.remove(s)
                finished.append(s)
        # a finished sequence's blocks return to the pool after the batch that ended it
        for s in finished:
            alloc.release(s["blocks"])
            freed_blocks.update(s["blocks"])
        slots = np.asarray(slots, dtype=np.int64)
        assert len(set(slots.tolist())) == len(slots), "slots repeat within a batch"
        k = to_bf16_bits(normal_with_outliers(rng, (t, e), 3.0, 0.002, 40.0))
        v = to_bf16_bits(normal_with_outliers(rng, (t, e), 3.0, 0.002, 40.0))
        batches.append(KvBatch(k=k, v=v, slots=slots))
        produced += t
        bidx += 1
    return batches, reuse


def kv_full_pool(seed: int = 5100, heads: int = KV_HEADS, head_dim: int = KV_HEAD_DIM,
                 block_size: int = KV_BLOCK_SIZE, num_blocks: int = KV_NUM_BLOCKS):
    """One batch covering every slot of the pool once, in random order (bandwidth shape)."""
    rng = np.random.default_rng(seed)
    t = block_size * num_blocks
    e = heads * head_dim
    slots = rng.permutation(t).astype(np.int64)
    k = to_bf16_bits(normal_with_outliers(rng, (t, e), 3.0, 0.002, 40.0))
    v = to_bf16_bits(normal_with_outliers(rng, (t, e), 3.0, 0.002, 40.0))
    return KvBatch(k=k, v=v, slots=slots)


def kv_block_runs(num_blocks: int = KV_NUM_BLOCKS, block_size: int = KV_BLOCK_SIZE,
                  seed: int = 5101) -> np.ndarray:
    """Slots of a prefill that fills every block of the pool: blocks handed out in random
    order, each taking block_size consecutive tokens (offsets 0..block_size-1)."""
    rng = np.random.default_rng(seed)
    blocks = rng.permutation(num_blocks).astype(np.int64)
    return (blocks[:, None] * block_size + np.arange(block_size, dtype=np.int64)).ravel()


