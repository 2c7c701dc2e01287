"""Seeded synthetic inputs for the projection -> residual-add -> RMSNorm workloads.

This module is shared by the tests, the benchmark and the oracle's callers.  It holds only
random draws and the rounding of those draws to their storage types (bf16 bit patterns,
fp32).  None of the method's arithmetic (projection, residual add, normalisation) lives here,
so neither the oracle nor the HIP path depends on the other through it.

Workload shapes follow the decoder-layer fusion sites of the vLLM "TPSP Design" page
(section 3, "Fusion regions": o_proj and down_proj, each followed by residual add and an
RMSNorm), at Llama-3-8B-like and Gemma-like sizes; the distributions are the plainest reading
of a randomly initialised layer (x ~ N(0,1), W ~ N(0, 1/K), residual ~ N(0,1)).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

NORM_STANDARD = 0
NORM_GEMMA = 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens (rows of x, residual, out)
    K: int                 # projection input size as laid out in memory (multiple of 64)
    H: int                 # hidden size (projection output size, normalised dim)
    K_real: int            # columns of K that carry data; [K_real, K) are zero in x and W
    x_dist: str            # "normal" or "silu_mul" (the SiluAndMul output feeding down_proj)
    eps: float
    norm_kind: int         # NORM_STANDARD (gain w) or NORM_GEMMA (gain 1 + w)
    microchunks: Tuple[int, ...]


SWEEP_T = (128, 512, 2048, 8192, 32768)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 64, 512, 512, 512, "normal", 1e-6, NORM_STANDARD, (16,)),
    "o_proj": Workload("o_proj", 2048, 4096, 4096, 4096, "normal", 1e-5, NORM_STANDARD,
                       (256, 512)),
    "down_proj": Workload("down_proj", 4096, 14336, 4096, 14336, "silu_mul", 1e-5,
                          NORM_STANDARD, (256, 512, 1024)),
    # Intermediate size 16360 zero-padded to 16384 (a multiple of 64); padding is inert.
    "gemma": Workload("gemma", 3000, 16384, 3072, 16360, "normal", 1e-6, NORM_GEMMA,
                      (256, 512, 1024)),
}
for _t in SWEEP_T:
    WORKLOADS[f"sweep_T{_t}"] = Workload(f"sweep_T{_t}", _t, 8192, 8192, 8192, "normal", 1e-5,
                                         NORM_STANDARD,
                                         tuple(m for m in (512, 1024, 2048) if m <= _t) or (_t,))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) and return the bit patterns.

    Used only to store drawn inputs in bf16.  NaN maps to a quiet NaN.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(wl: Workload, seed: int = 0, T: Optional[int] = None) -> dict:
    """Draw one workload's inputs.

    Draw order with numpy's PCG64 ``default_rng(seed)``: x (for silu_mul: a, then b), W,
    residual, norm weight.  Returns bf16 bit patterns for x [T,K] and the nn.Linear-layout
    weight W [H,K]; fp32 residual [T,H] and norm weight [H].
    """
    T = wl.T if T is None else T
    K, H, Kr = wl.K, wl.H, wl.K_real
    rng = np.random.default_rng(seed)
    if wl.x_dist == "normal":
        xr = rng.standard_normal((T, Kr), dtype=np.float32)
    elif wl.x_dist == "silu_mul":
        a = rng.standard_normal((T, Kr), dtype=np.float32)
        b = rng.standard_normal((T, Kr), dtype=np.float32)
        xr = (a / (np.float32(1.0) + np.exp(-a))) * b
        del a, b
    else:
        raise ValueError(wl.x_dist)
    x = np.zeros((T, K), dtype=np.uint16)
    x[:, :Kr] = f32_to_bf16_bits(xr)
    del xr
    wr = rng.standard_normal((H, Kr), dtype=np.float32) * np.float32(1.0 / np.sqrt(Kr))
    W = np.zeros((H, K), dtype=np.uint16)
    W[:, :Kr] = f32_to_bf16_bits(wr)
    del wr
    residual = rng.standard_normal((T, H), dtype=np.float32)
    nw = rng.standard_normal(H, dtype=np.float32) * np.float32(0.1)
    if wl.norm_kind == NORM_STANDARD:
        nw = nw + np.float32(1.0)
    return {"x": x, "W": W, "residual": residual, "norm_w": nw.astype(np.float32),
            "eps": float(np.float32(wl.eps)), "norm_kind": wl.norm_kind,
            "T": T, "K": K, "H": H, "K_real": Kr}


def make_custom(T: int, K: int, H: int, seed: int = 0, norm_kind: int = NORM_STANDARD,
                eps: float = 1e-5, x_dist: str = "normal", K_real: Optional[int] = None) -> dict:
    """Inputs for an arbitrary shape with the same recipe (used for small parity cases)."""
    wl = Workload("custom", T, K, H, K if K_real is None else K_real, x_dist, eps, norm_kind,
                  ())
    return make_inputs(wl, seed)


def gate_up_inputs(T: int, K: int, H: int, seed: int = 0, K_real: Optional[int] = None,
                   eps: float = 1e-5) -> dict:
    """Inputs of the down_proj block taken from the merged gate/up projection output:
    gate_up [T, 2K] bf16 (gate in columns [0, K), up in [K, 2K); gate, up ~ N(0,1)), the
    nn.Linear weight W [H, K] ~ N(0, 1/K_real), residual ~ N(0,1), norm weight 1 + N(0, 0.1).
    Columns [K_real, K) of gate, up and W are zero: the load-time padding of the intermediate
    size.  Drawn in that order with PCG64 ``default_rng(seed)``."""
    Kr = K if K_real is None else K_real
    rng = np.random.default_rng(seed)
    gu = np.zeros((T, 2 * K), dtype=np.uint16)
    gu[:, :Kr] = f32_to_bf16_bits(rng.standard_normal((T, Kr), dtype=np.float32))
    gu[:, K:K + Kr] = f32_to_bf16_bits(rng.standard_normal((T, Kr), dtype=np.float32))
    W = np.zeros((H, K), dtype=np.uint16)
    W[:, :Kr] = f32_to_bf16_bits(rng.standard_normal((H, Kr), dtype=np.float32) *
                                 np.float32(1.0 / np.sqrt(Kr)))
    residual = rng.standard_normal((T, H), dtype=np.float32)
    nw = rng.standard_normal(H, dtype=np.float32) * np.float32(0.1) + np.float32(1.0)
    return {"gate_up": gu, "W": W, "residual": residual, "norm_w": nw.astype(np.float32),
            "eps": float(np.float32(eps)), "norm_kind": NORM_STANDARD, "T": T, "K": K, "H": H,
            "K_real": Kr}


def tiled_inputs(T: int, K: int, H: int, period: int, seed: int = 0) -> dict:
    """Inputs for shapes whose x is too large to draw in full on the host: x is a block of
    `period` drawn rows (N(0,1), bf16), repeated down the T rows, so token t's row is block row
    t % period.  W ~ N(0, 1/K), the residual ~ N(0,1) and the norm weight 1 + N(0, 0.1) are
    drawn in full, in that order after the block, with PCG64 ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    xb = f32_to_bf16_bits(rng.standard_normal((period, K), dtype=np.float32))
    W = f32_to_bf16_bits(rng.standard_normal((H, K), dtype=np.float32) *
                         np.float32(1.0 / np.sqrt(K)))
    residual = rng.standard_normal((T, H), dtype=np.float32)
    nw = rng.standard_normal(H, dtype=np.float32) * np.float32(0.1) + np.float32(1.0)
    return {"x_block": xb, "x_period": period, "W": W, "residual": residual,
            "norm_w": nw.astype(np.float32), "eps": float(np.float32(1e-5)),
            "norm_kind": NORM_STANDARD, "T": T, "K": K, "H": H, "K_real": K}


def integer_inputs(T: int, K: int, H: int, seed: int = 0, lo: int = -4, hi: int = 4) -> dict:
    """Small-integer x and W (exact in bf16), integer residual, unit norm weight.

    With |sum| < 2**24 every partial sum of the projection is an integer exactly representable
    in fp32, so any summation order gives the same result.
    """
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=(T, K)).astype(np.float32)
    W = rng.integers(lo, hi + 1, size=(H, K)).astype(np.float32)
    residual = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    return {"x": f32_to_bf16_bits(x), "W": f32_to_bf16_bits(W), "residual": residual,
            "norm_w": np.ones(H, dtype=np.float32), "eps": float(np.float32(1e-5)),
            "norm_kind": NORM_STANDARD, "T": T, "K": K, "H": H, "K_real": K}
