"""Seeded input generators for the sparse ternary BitLinear workloads.

Every generator draws from numpy's PCG64 (``numpy.random.default_rng``) and
returns host numpy arrays.  Activations that a workload defines as bfloat16 are
returned as float32 arrays whose values are exactly bfloat16-representable
(IEEE round-to-nearest-even onto the bfloat16 grid), together with the raw
bfloat16 bit patterns so a device buffer can be filled without another cast.

Workload shapes follow the layer shapes the pages train and serve: BitNet-2B
style FFN projections for decode, LLaMA-7B gate/up for prefill, Qwen2.5/3B-style
decoder projections for the training step (Sparse-BitNet page, results on the
Qwen-2.5 family; BitNet b1.58 page, LLaMA-alike stack).  The master weights
are fp32 N(0, 0.02^2).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

MASTER_SIGMA = 0.02


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def to_bf16(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns ``(values_as_float32, bits_as_uint16)``.  Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    bits = r.astype(np.uint16)
    vals = (r << 16).astype(np.uint32).view(np.float32)
    return vals.reshape(x.shape), bits.reshape(x.shape)


def master_weights(g: np.random.Generator, n: int, K: int, sigma: float = MASTER_SIGMA) -> np.ndarray:
    """fp32 master weights, n out-features x K in-features, N(0, sigma^2)."""
    return g.normal(0.0, sigma, size=(n, K)).astype(np.float32)


def act_normal(g: np.random.Generator, T: int, K: int) -> np.ndarray:
    """Activations ~ N(0, 1), float32 (caller may cast to bf16)."""
    return g.standard_normal(size=(T, K)).astype(np.float32)


def act_student_t(g: np.random.Generator, T: int, K: int, nu: float = 4.0, scale: float = 0.5) -> np.ndarray:
    """Heavy-tailed activations: scale * Student-t(nu), float32."""
    return (scale * g.standard_t(nu, size=(T, K))).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    n: int      # out features
    K: int      # in features
    N: int = 2  # kept per group
    M: int = 4  # group size


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    title: str
    layers: Tuple[Layer, ...]
    tokens: Tuple[int, ...]
    act: str          # "normal" | "student_t"
    act_dtype: str    # "fp32" | "bf16"


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "single BitLinear 16x256 -> 256, 2:4",
                     (Layer("w", 256, 256),), (16,), "normal", "fp32"),
    "decode": Workload("decode", "decode GEMV, FFN up 6912x2560 and down 2560x6912, 2:4",
                       (Layer("up", 6912, 2560), Layer("down", 2560, 6912)), (1, 4, 16), "normal", "bf16"),
    "prefill": Workload("prefill", "prefill GEMM 4096 tokens x 4096 -> 11008, 2:4",
                        (Layer("gate_up", 11008, 4096),), (4096,), "student_t", "bf16"),
    "six_eight": Workload("six_eight", "6:8 as 3 overlapping 2:4 windows, 2048 x 4096 -> 4096",
                          (Layer("w", 4096, 4096, 6, 8),), (2048,), "normal", "bf16"),
    "train_step": Workload("train_step", "3B-alike decoder layer set, hidden 3200, intermediate 8640, 8192 tokens",
                           (Layer("q", 3200, 3200), Layer("k", 3200, 3200), Layer("v", 3200, 3200),
                            Layer("o", 3200, 3200), Layer("gate", 8640, 3200), Layer("up", 8640, 3200),
                            Layer("down", 3200, 8640)), (8192,), "normal", "bf16"),
}


def workload_inputs(key: str, seed: int = 0, layers: List[str] | None = None,
                    tokens: int | None = None) -> Dict[str, np.ndarray]:
    """Draw a workload's tensors in a fixed order: masters in listed order, then activations.

    Returns a dict with ``W:<layer>`` (fp32 masters) and ``X:<K>`` activation
    matrices (one per distinct in-feature size, shared by the layers that read
    it), plus ``Xbits:<K>`` (uint16 bf16 bits) when the workload is bf16.
    ``tokens`` overrides the largest token count (activations are drawn at that
    count; smaller counts use leading rows).
    """
    wl = WORKLOADS[key]
    g = rng(seed)
    out: Dict[str, np.ndarray] = {}
    for L in wl.layers:
        W = master_weights(g, L.n, L.K)
        if layers is None or L.name in layers:
            out[f"W:{L.name}"] = W
    T = tokens if tokens is not None else max(wl.tokens)
    for K in sorted({L.K for L in wl.layers}, key=lambda k: [L.K for L in wl.layers].index(k)):
        x = act_student_t(g, T, K) if wl.act == "student_t" else act_normal(g, T, K)
        if wl.act_dtype == "bf16":
            x, bits = to_bf16(x)
            out[f"Xbits:{K}"] = bits
        out[f"X:{K}"] = x
    return out


GRAD_SIGMA = 2.0 ** -10


def grad_bf16(g: np.random.Generator, T: int, n: int, sigma: float = GRAD_SIGMA):
    """Output gradients dY ~ N(0, sigma^2) on the bfloat16 grid: (values as float32, uint16 bits)."""
    return to_bf16((g.standard_normal(size=(T, n)) * sigma).astype(np.float32))


def grad_int_bf16(g: np.random.Generator, T: int, n: int, lim: int = 8):
    """Integer output gradients in [-lim, lim] (exact in bfloat16): (float32 values, uint16 bits)."""
    return to_bf16(g.integers(-lim, lim + 1, size=(T, n)).astype(np.float32))


def workload_grads(key: str, seed: int = 0, tokens: int | None = None) -> Dict[str, np.ndarray]:
    """Output gradients of a workload's layers, ``dY:<layer>`` (values) and ``dYbits:<layer>``.

    Drawn from a stream of their own (seed sequence [seed, 1]) so the masters and activations of
    ``workload_inputs`` stay as they are.
    """
    wl = WORKLOADS[key]
    g = np.random.default_rng([seed, 1])
    T = tokens if tokens is not None else max(wl.tokens)
    out: Dict[str, np.ndarray] = {}
    for L in wl.layers:
        out[f"dY:{L.name}"], out[f"dYbits:{L.name}"] = grad_bf16(g, T, L.n)
    return out
