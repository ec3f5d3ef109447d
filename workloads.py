"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module draws random numbers and rounds them to the storage types the
library accepts.  It holds none of the method's arithmetic: no split, no
projection, no scales, no packing, no product.  Both sides of every parity
check receive the same arrays from here.

Shapes follow LLaMA-2 7B's linear layers (hidden 4096, MLP 11008, 32 layers),
which is the model the Fairy2i-W2 model card quantizes ("Model details":
base model LLaMA-2 7B).  Weights are N(0, 0.02^2) in fp32; activations are
N(0, 1), cast to bf16 with round-to-nearest-even.  Where a workload asks for
outliers, 1% of the weight entries (chosen by a second seed) are multiplied by
10 in fp32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

WEIGHT_STD = np.float32(0.02)


def weight(rows: int, cols: int, seed: int, outlier_seed: int | None = None) -> np.ndarray:
    """fp32 [rows][cols] ~ N(0, 0.02^2); optional 1% outliers x10 (second seed)."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((rows, cols), dtype=np.float32) * WEIGHT_STD
    if outlier_seed is not None:
        mask = np.random.default_rng(outlier_seed).random((rows, cols)) < 0.01
        R[mask] *= np.float32(10.0)
    return np.ascontiguousarray(R, dtype=np.float32)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the raw uint16 bits.

    Inputs are finite draws from a normal distribution, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Activations:
    """One activation batch: `values` is the exact fp32 value of every element
    (already rounded to bf16 when dtype == 'bf16'); `bf16_bits` holds the raw
    uint16 pattern for the GPU side when dtype == 'bf16'."""
    values: np.ndarray          # fp32 [B][2m]
    dtype: str                  # 'bf16' or 'f32'
    bf16_bits: np.ndarray | None = None


def activations(batch: int, two_m: int, seed: int, dtype: str = "bf16") -> Activations:
    """x [batch][2m] ~ N(0,1): fp32, or rounded to bf16 (RNE) when dtype == 'bf16'."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((batch, two_m), dtype=np.float32)
    if dtype == "f32":
        return Activations(values=np.ascontiguousarray(v), dtype="f32")
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = f32_to_bf16_bits(v)
    return Activations(values=bf16_bits_to_f32(bits), dtype="bf16", bf16_bits=bits)


def random_codes(T: int, n: int, m: int, seed: int) -> np.ndarray:
    """Uniform 2-bit codes uint8 [T][2][n][m] (inputs for pack/unpack and GEMM-only cases)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 4, size=(T, 2, n, m), dtype=np.uint8)


def random_scales(n: int, T: int, seed: int) -> np.ndarray:
    """Positive fp32 axis scales [n][T][2][2], magnitudes like a 0.02-std weight's residual."""
    rng = np.random.default_rng(seed)
    return (rng.random((n, T, 2, 2), dtype=np.float32) * np.float32(0.02) + np.float32(0.001)).astype(np.float32)


# ---------------------------------------------------------------------------
# The five workloads (shapes and seeds).  R is [2n][2m] like nn.Linear.weight [out][in].
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    rows: int          # 2n
    cols: int          # 2m
    seed: int
    outlier_seed: int | None = None

    @property
    def n(self) -> int:
        return self.rows // 2

    @property
    def m(self) -> int:
        return self.cols // 2

    def weight(self) -> np.ndarray:
        return weight(self.rows, self.cols, self.seed, self.outlier_seed)


TINY = Layer("tiny 256x256", 256, 256, seed=101)
TINY_X_SEED = 102

ATTN = Layer("attention projection 4096x4096", 4096, 4096, seed=201)
ATTN_X_SEEDS = {1: 202, 4: 203, 16: 204}

MLP_GATE_UP = Layer("mlp gate/up 11008x4096", 11008, 4096, seed=301, outlier_seed=311)
MLP_DOWN = Layer("mlp down 4096x11008", 4096, 11008, seed=302, outlier_seed=312)
MLP_X_SEEDS = {"gate_up": 321, "down": 322}

PREFILL_LAYERS = (Layer("prefill 4096x4096", 4096, 4096, seed=401),
                  Layer("prefill 11008x4096", 11008, 4096, seed=402))
PREFILL_X_SEED = 411
PREFILL_TOKENS = 2048

STACK_LAYERS = 32
STACK_SHAPES = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))


def stack_layer(layer: int, p: int) -> Layer:
    """Layer `layer` (0..31), projection p (0..6 in q,k,v,o,gate,up,down order)."""
    name, rows, cols = STACK_SHAPES[p]
    return Layer(f"L{layer}.{name}", rows, cols, seed=5000 + 7 * layer + p)


def stack_x_seed(layer: int, p: int) -> int:
    return 6000 + 7 * layer + p
