"""Seeded synthetic inputs for sliding-window GQA attention.

This module only draws numbers and lays out shapes; it holds none of the
attention arithmetic.  Both the GPU tests/benchmark and the CPU oracle read
the same arrays produced here.

Element values are N(0, 1) drawn as float32 from numpy's PCG64 generator and,
for bf16 runs, rounded to bf16 with round-to-nearest-even (stored as uint16
bit patterns).

Named workloads (shapes follow the pages' own measurement shapes):
  decode_single_d256     one decode step, B=1, Hq=4, Hkv=2, D=256, W=1024,
                         1088-row ring, query at position 3000
  prefill_4x1024_mha_d128  4 packed documents of 1024 tokens, Hq=Hkv=32,
                         D=128, W=1024, causal
  decode_b64_d256        64 sequences, Hq=8, Hkv=4, D=256, W=1024, 1088-row
                         rings, positions ~U[1, 32768], left pad 0..63,
                         70 steps spanning one 64-token roll
  prefill_16k_gqa_d512   one 16384-token document, Hq=16, Hkv=8, D=512,
                         W=4096, causal
  prefill_vlm_4096_d256  4096 tokens with 8 image blocks of 256 at seeded
                         offsets, Hq=8, Hkv=4, D=256, W=1024, window AND
                         (causal OR same image block)
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

CAUSAL = 0
BLOCKWISE = 1


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = 0x7FFF + ((u >> 16) & 1)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws: float32 for dtype 'f32', bf16 bit patterns for 'bf16'."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- prefill
@dataclass
class PrefillCase:
    name: str
    cu_seqlens: np.ndarray  # int32 [ndocs + 1]
    hq: int
    hkv: int
    d: int
    window: int
    mode: int
    ids: Optional[np.ndarray] = None  # int32 [T], -1 = text
    seed: int = 0

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens))) if self.cu_seqlens.size > 1 else 0

    def tensors(self, dtype: str = "bf16", seed: Optional[int] = None):
        """q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D] drawn in that order."""
        rng = rng_for(self.seed if seed is None else seed)
        q = normal(rng, (self.T, self.hq, self.d), dtype)
        k = normal(rng, (self.T, self.hkv, self.d), dtype)
        v = normal(rng, (self.T, self.hkv, self.d), dtype)
        return q, k, v


def image_block_ids(T: int, n_blocks: int, block_len: int, seed: int) -> np.ndarray:
    """ids [T]: n_blocks non-overlapping runs of block_len tokens with ids
    0..n_blocks-1 in order, the rest -1.  Placement: sort n_blocks uniform
    draws u from {0..T - n_blocks*block_len}; block k starts at u_(k) + k*block_len."""
    free = T - n_blocks * block_len
    if free < 0:
        raise ValueError("blocks do not fit")
    rng = rng_for(seed)
    u = np.sort(rng.integers(0, free + 1, size=n_blocks))
    ids = np.full(T, -1, dtype=np.int32)
    for kk in range(n_blocks):
        s = int(u[kk]) + kk * block_len
        ids[s:s + block_len] = kk
    return ids


def prefill_4x1024_mha_d128() -> PrefillCase:
    return PrefillCase("prefill_4x1024_mha_d128",
                       np.array([0, 1024, 2048, 3072, 4096], dtype=np.int32),
                       hq=32, hkv=32, d=128, window=1024, mode=CAUSAL, seed=2)


def prefill_16k_gqa_d512() -> PrefillCase:
    return PrefillCase("prefill_16k_gqa_d512", np.array([0, 16384], dtype=np.int32),
                       hq=16, hkv=8, d=512, window=4096, mode=CAUSAL, seed=4)


def prefill_16k_mha_d128_w4k() -> PrefillCase:
    """One 16K-token document, 32 MHA heads of size 128, window 4K: the
    Llama-7B-shaped windowed row of the [SDPA] Benchmark table (timed there
    as forward + backward)."""
    return PrefillCase("prefill_16k_mha_d128_w4k", np.array([0, 16384], dtype=np.int32),
                       hq=32, hkv=32, d=128, window=4096, mode=CAUSAL, seed=7)


def prefill_vlm_4096_d256() -> PrefillCase:
    return PrefillCase("prefill_vlm_4096_d256", np.array([0, 4096], dtype=np.int32),
                       hq=8, hkv=4, d=256, window=1024, mode=BLOCKWISE,
                       ids=image_block_ids(4096, 8, 256, seed=5), seed=5)


def prefill_4x1024_gqa_d320() -> PrefillCase:
    """The packed 4 x 1024-token causal shape with the non-power-of-two head
    size 320 ([SDPA] Test plan) and GQA 16/8."""
    return PrefillCase("prefill_4x1024_gqa_d320",
                       np.array([0, 1024, 2048, 3072, 4096], dtype=np.int32),
                       hq=16, hkv=8, d=320, window=1024, mode=CAUSAL, seed=6)


def prefill_16k_gqa4_d128_w4k() -> PrefillCase:
    """The 16K window-4K D=128 shape with 8 kv heads shared by groups of 4
    query heads ([SDPA] Summary: grouped-query attention); with its group-of-2
    twin below it shows whether K/V bytes read from memory depend on the
    group size."""
    return PrefillCase("prefill_16k_gqa4_d128_w4k", np.array([0, 16384], dtype=np.int32),
                       hq=32, hkv=8, d=128, window=4096, mode=CAUSAL, seed=8)


def prefill_16k_gqa2_d128_w4k() -> PrefillCase:
    return PrefillCase("prefill_16k_gqa2_d128_w4k", np.array([0, 16384], dtype=np.int32),
                       hq=16, hkv=8, d=128, window=4096, mode=CAUSAL, seed=9)


PREFILL_WORKLOADS = {
    "prefill_4x1024_mha_d128": prefill_4x1024_mha_d128,
    "prefill_16k_gqa_d512": prefill_16k_gqa_d512,
    "prefill_vlm_4096_d256": prefill_vlm_4096_d256,
    "prefill_4x1024_gqa_d320": prefill_4x1024_gqa_d320,
    "prefill_16k_mha_d128_w4k": prefill_16k_mha_d128_w4k,
    "prefill_16k_gqa4_d128_w4k": prefill_16k_gqa4_d128_w4k,
    "prefill_16k_gqa2_d128_w4k": prefill_16k_gqa2_d128_w4k,
}


def ragged_cu_seqlens(rng: np.random.Generator, T: int, ndocs: int) -> np.ndarray:
    """ndocs documents of random (possibly tiny) lengths summing to T."""
    cuts = np.sort(rng.integers(0, T + 1, size=ndocs - 1))
    return np.concatenate([[0], cuts, [T]]).astype(np.int32)


# ---------------------------------------------------------------- decode
@dataclass
class DecodeCase:
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    window: int
    ring_rows: int
    prompt_lens: np.ndarray  # int32 [B]: prompt length L_b (positions 0..L_b-1)
    left_pad: np.ndarray  # int32 [B]
    tail_lens: np.ndarray  # int32 [B]: prompt rows handed to compaction (the last ones)
    steps: int
    seed: int
    pre_appends: int = 0  # decode-token appends before the measured steps

    @property
    def cu_tail(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.tail_lens)]).astype(np.int32)

    def prompt_tail(self, dtype: str = "bf16"):
        """Packed prompt-tail K and V [sum(tail_lens), Hkv, D]."""
        rng = rng_for(self.seed)
        n = int(self.tail_lens.sum())
        k = normal(rng, (n, self.hkv, self.d), dtype)
        v = normal(rng, (n, self.hkv, self.d), dtype)
        return k, v

    def step_inputs(self, step: int, dtype: str = "bf16"):
        """Query and new K/V rows of decode step `step` (seed 100*seed+step).
        Steps < 0 are the pre-appends."""
        rng = rng_for(100 * self.seed + step + 1000 if step < 0 else 100 * self.seed + step)
        q = normal(rng, (self.batch, self.hq, self.d), dtype)
        k = normal(rng, (self.batch, self.hkv, self.d), dtype)
        v = normal(rng, (self.batch, self.hkv, self.d), dtype)
        return q, k, v


def decode_single_d256() -> DecodeCase:
    """Query at position 3000: compaction of a 2944-token prompt then 56
    pre-appended tokens, so the measured step appends position 3000."""
    return DecodeCase("decode_single_d256", batch=1, hq=4, hkv=2, d=256, window=1024,
                      ring_rows=1088, prompt_lens=np.array([2944], np.int32),
                      left_pad=np.array([0], np.int32), tail_lens=np.array([1024], np.int32),
                      steps=1, seed=1, pre_appends=56)


def decode_b64_d256(steps: int = 70) -> DecodeCase:
    rng = rng_for(3)
    pos = rng.integers(1, 32768 + 1, size=64).astype(np.int32)
    lo = np.array([rng.integers(0, min(63, int(p) - 1) + 1) for p in pos], dtype=np.int32)
    tail = np.minimum(pos, 1024).astype(np.int32)
    return DecodeCase("decode_b64_d256", batch=64, hq=8, hkv=4, d=256, window=1024,
                      ring_rows=1088, prompt_lens=pos, left_pad=lo, tail_lens=tail,
                      steps=steps, seed=3)


DECODE_WORKLOADS = {
    "decode_single_d256": decode_single_d256,
    "decode_b64_d256": decode_b64_d256,
}
