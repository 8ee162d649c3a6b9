"""Seeded synthetic inputs for the attention backward, shared by the tests, the benchmark and the
CPU oracle's callers.

This module holds no arithmetic of the attention method: it draws random numbers, rounds them to
bfloat16 (round-to-nearest-even, from the definition of the format) or to IEEE binary16 (numpy's
own round-to-nearest-even conversion) and describes the workload shapes.  It imports nothing else from this package, so it can be used without the GPU library.
The forward outputs O and LSE that the backward consumes are not made here; the caller obtains
them from a forward pass of its choice.
"""
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One attention-backward problem: shapes, mask and mode."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    Dqk: int
    Dv: int
    causal: bool
    window_left: int = -1
    deterministic: bool = False
    padded: bool = False          # per-batch seq_q = seq_kv lengths drawn uniformly
    len_lo: int = 0               # inclusive lower bound of the drawn lengths
    input_scale: float = 1.0      # Q, K, V, dO ~ input_scale * N(0, 1)
    seed: int = 0
    scale: Optional[float] = None  # None: 1/sqrt(Dqk)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.Dqk)


# The five workloads of the attention-backward study, the NVFP4-QAT example shape and one GPU's
# share of the causal GQA workload, seeded by their index.
WORKLOADS = {
    "mha_s128_d64": Workload("mha_s128_d64", 1, 2, 2, 128, 128, 64, 64, causal=False, seed=1),
    "mha_causal_s2048_d128": Workload("mha_causal_s2048_d128", 2, 16, 16, 2048, 2048, 128, 128,
                                      causal=True, seed=2),
    "gqa_causal_s4096_d128": Workload("gqa_causal_s4096_d128", 1, 32, 8, 4096, 4096, 128, 128,
                                      causal=True, seed=3),
    "mha_det_s8192_d256": Workload("mha_det_s8192_d256", 1, 8, 8, 8192, 8192, 256, 256,
                                   causal=False, deterministic=True, input_scale=0.5, seed=4),
    "mla_window_padded_s4096": Workload("mla_window_padded_s4096", 4, 16, 16, 4096, 4096, 192, 128,
                                        causal=True, window_left=1024, padded=True, len_lo=1024,
                                        seed=5),
    # the NVFP4 attention-QAT example shape ("NVFP4 Attention QAT Backward", "High-level wrapper"):
    # non-causal MHA, head dim 128
    "qat_mha_s4096_d128": Workload("qat_mha_s4096_d128", 1, 16, 16, 4096, 4096, 128, 128,
                                   causal=False, seed=6),
    # one GPU's share of the causal GQA S=4096 workload split over 8 GPUs by KV-head group: one KV
    # head and its 4 query heads
    "gqa_causal_s4096_d128_1of8": Workload("gqa_causal_s4096_d128_1of8", 1, 4, 1, 4096, 4096, 128,
                                           128, causal=True, seed=7),
}


def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("bf16_bits expects finite values")
    u = f.view(np.uint32)
    # finite inputs stay below 2**32 after adding the rounding bias
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def fp16_bits(x) -> np.ndarray:
    """Round float32 values to IEEE binary16 (round to nearest, ties to even); uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("fp16_bits expects finite values")
    h = f.astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("fp16_bits: value outside the binary16 range")
    return h.view(np.uint16)


def fp16_to_f32(bits) -> np.ndarray:
    """Exact float32 value of binary16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bits_to_f32(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float32 value of 16-bit patterns of the given io type ("bf16" or "fp16")."""
    return fp16_to_f32(bits) if dtype == "fp16" else bf16_to_f32(bits)


def round_bf16(x) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


@dataclass
class Inputs:
    """Drawn inputs: bf16 bit patterns (uint16) plus optional per-batch lengths (int32)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    seq_q_lens: Optional[np.ndarray] = None
    seq_kv_lens: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


def draw_inputs(w: Workload, seed: Optional[int] = None, dtype: str = "bf16") -> Inputs:
    """Q, K, V, dO iid input_scale * N(0,1) in float32, rounded to bf16 (or to fp16 with
    dtype="fp16"); lengths drawn first.

    Lengths (padded workloads) are uniform integers in [len_lo, Sq], seq_q = seq_kv.  Rows past a
    batch entry's length are still filled with random values, so any leak through the padding
    mask shows up in the outputs.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    lens = None
    if w.padded:
        lens = rng.integers(w.len_lo, w.Sq + 1, size=w.B).astype(np.int32)

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.input_scale != 1.0:
            x *= np.float32(w.input_scale)
        return fp16_bits(x) if dtype == "fp16" else bf16_bits(x)

    q = draw((w.B, w.Hq, w.Sq, w.Dqk))
    k = draw((w.B, w.Hkv, w.Skv, w.Dqk))
    v = draw((w.B, w.Hkv, w.Skv, w.Dv))
    do = draw((w.B, w.Hq, w.Sq, w.Dv))
    return Inputs(q, k, v, do, lens, None if lens is None else lens.copy())


def small_variant(w: Workload, **overrides) -> Workload:
    """A copy of a workload with some fields replaced (used for reduced-size parity cases)."""
    d = dict(w.__dict__)
    d.update(overrides)
    return Workload(**d)
