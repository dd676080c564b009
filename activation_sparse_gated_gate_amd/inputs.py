"""Seeded synthetic inputs for the sparse gated-FFN forward.

This module is shared by the HIP path's tests/benchmark and by the CPU
oracle's tests. It holds no arithmetic of the method itself: it only draws
random numbers and stores them in the dtype the layer uses.

Recipe (one recipe for every workload):
  * every tensor draws from ``numpy.random.default_rng(SeedSequence([seed,
    tensor_id]))`` with ``standard_normal(shape, dtype=float32)``, is scaled in
    fp32 by its standard deviation, and is filled in storage order;
  * tensor ids: x = 0, W_gate = 1, W_up = 2, W_down = 3, LoPA A = 4,
    LoPA B = 5, the shared component of correlated prefill tokens = 6;
  * weight matrices are stored channel-major, ``[d_ff][d_model]`` (row i is
    channel i), for W_gate, W_up and W_down alike; LoPA's A is stored as its
    transpose ``[rank][d_model]`` and B as ``[d_ff][rank]``;
  * a weight with input dimension d_in has variance 1/d_in (d_model for the
    gate and up matrices, d_ff for the down matrix), so the gate
    pre-activation of a unit-variance token is N(0, 1) given the weights;
  * LoPA's A and B both have variance 1/sqrt(d_model * rank), which gives the
    low-rank gate pre-activation unit variance in expectation, so no
    data-dependent rescale is applied;
  * bf16 storage rounds the fp32 draw to nearest-even and keeps the 16-bit
    pattern (``uint16``); the activations x use the weights' dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

TENSOR_IDS = {"x": 0, "w_gate": 1, "w_up": 2, "w_down": 3, "lopa_a": 4, "lopa_b": 5, "shared": 6}

F32 = "f32"
BF16 = "bf16"


def draw_normal(seed: int, tensor_id: int, shape: Tuple[int, ...], std: float) -> np.ndarray:
    """fp32 N(0, std^2) draw for one tensor, in storage (row-major) order."""
    rng = np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id)]))
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32 (used by generator self-tests)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_x(seed: int, n: int, d: int, dtype: str, correlated: bool = False) -> np.ndarray:
    """Token activations ``[n][d]``.

    Independent tokens are N(0, 1) per coordinate. Correlated (prefill) tokens
    mix a shared N(0, 1) vector s with a per-token N(0, 1) vector e_t as
    (0.7 s + 0.3 e_t) / sqrt(0.7^2 + 0.3^2), which keeps unit variance per
    coordinate.
    """
    e = draw_normal(seed, TENSOR_IDS["x"], (n, d), 1.0)
    if correlated:
        s = draw_normal(seed, TENSOR_IDS["shared"], (1, d), 1.0)
        e = (np.float32(0.7) * s + np.float32(0.3) * e) / np.float32(math.sqrt(0.7 * 0.7 + 0.3 * 0.3))
        e = e.astype(np.float32)
    return store(e, dtype)


@dataclasses.dataclass
class Layer:
    d_model: int
    d_ff: int
    dtype: str
    rank: int
    w_gate: Optional[np.ndarray]
    w_up: np.ndarray
    w_down: np.ndarray
    lopa_a: Optional[np.ndarray] = None  # [rank][d_model]
    lopa_b: Optional[np.ndarray] = None  # [d_ff][rank]


def make_layer(seed: int, d: int, f: int, dtype: str, rank: int = 0, with_gate: bool = True) -> Layer:
    """One FFN layer's weights, channel-major, in the layer's storage dtype."""
    wg = store(draw_normal(seed, TENSOR_IDS["w_gate"], (f, d), 1.0 / math.sqrt(d)), dtype) if with_gate else None
    wu = store(draw_normal(seed, TENSOR_IDS["w_up"], (f, d), 1.0 / math.sqrt(d)), dtype)
    wd = store(draw_normal(seed, TENSOR_IDS["w_down"], (f, d), 1.0 / math.sqrt(f)), dtype)
    a = b = None
    if rank > 0:
        std = (1.0 / math.sqrt(d * rank)) ** 0.5
        a = store(draw_normal(seed, TENSOR_IDS["lopa_a"], (rank, d), std), dtype)
        b = store(draw_normal(seed, TENSOR_IDS["lopa_b"], (f, rank), std), dtype)
    return Layer(d, f, dtype, rank, wg, wu, wd, a, b)


# ---------------------------------------------------------------------------
# Workloads. Names say what each is, with its sizes.
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d_model: int
    d_ff: int
    dtype: str
    mode: str                 # "threshold" | "topk" | "lopa"
    tokens: Tuple[int, ...]
    taus: Tuple[float, ...] = ()
    ks: Tuple[int, ...] = ()
    ranks: Tuple[int, ...] = ()
    correlated: bool = False


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny_swiglu_fp32_d256_f1024", 256, 1024, F32, "threshold", (1, 8), taus=(1.2816,)),
        Workload("llama7b_ffn_bf16_d4096_f11008", 4096, 11008, BF16, "threshold", (1,),
                 taus=(0.0, 0.674, 1.2816, 1.645, 2.326)),
        Workload("lopa_gate_bf16_d4096_f11008", 4096, 11008, BF16, "lopa", (1, 4), taus=(1.2816,),
                 ranks=(256, 512, 1024)),
        Workload("moc_topk_bf16_d2048_f5632", 2048, 5632, BF16, "topk", (1, 16, 64), ks=(704, 1408)),
        Workload("prefill70b_ffn_bf16_d8192_f28672", 8192, 28672, BF16, "threshold", (256, 2048),
                 taus=(1.645,), correlated=True),
    )
}
