"""CPU oracle for projection -> residual add -> RMSNorm, in float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module; the library never calls it, and it shares no code with the HIP
path.  It is the plain definition of what the path computes, written to be checked by eye:

* projection  y = x . W^T for an nn.Linear weight W [H,K]  (spyre-inference "Plugin
  Architecture" page, section "Transposed linear weights": F.linear computes x @ W^T; the
  weight may be stored transposed, which does not change the result);
* residual add  r' = r + y  (vLLM "TPSP Design" page, section 1 Motivation: the row-parallel
  projection is followed by a residual addition; section 3 "Fusion regions": the fused path
  updates the residual);
* RMSNorm  out = r' / sqrt(mean_h(r'^2) + eps) * g, with g = w (standard RMSNorm, no bias:
  "TPSP Design" section 4 Constraints) or g = 1 + w (the Gemma form, "Plugin Architecture"
  custom-op table, GemmaRMSNorm row), the weight multiply done in fp32 or wider;
* the microchunk partition ("TPSP Design" section 3 "Microchunk pipeline"): chunks of mc
  rows, the last padded, and only valid rows update residual and output;
* SiluAndMul, the step before down_proj ("Plugin Architecture" page, SiluAndMul row):
  x = silu(gate) * up from the merged gate/up projection output.

Two modes fix where the projection output may be rounded:
* ``fused``: the projection result enters the add unrounded;
* ``conventional``: the projection emits the model dtype (bf16, round to nearest even) first,
  as a stand-alone projection layer does before the residual add.

Everything is float64; inputs are the exact bf16 / fp32 values widened.  The pages print no
worked numeric example, so every function here is pinned by closed forms, invariants,
brute force and hand-worked cases in the tests.
"""
from __future__ import annotations

import math

import numpy as np

NORM_STANDARD = 0
NORM_GEMMA = 1


# --------------------------------------------------------------------------------------------
# storage types
# --------------------------------------------------------------------------------------------
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact): a bf16 value is the top 16 bits of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def widen_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even; returns float64.

    bf16 has an 8-bit exponent like fp32 and 8 significant bits.  For a normal value with
    binary exponent e (2^e <= |v| < 2^(e+1)) the spacing is 2^(e-7); below the smallest
    normal (2^-126) the spacing stays 2^-133.  np.rint rounds half to even.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    finite = np.isfinite(v) & (v != 0)
    a = np.abs(v[finite])
    _, e = np.frexp(a)              # a = m * 2^e, 0.5 <= m < 1  =>  binary exponent e-1
    e = np.maximum(e - 1, -126)
    q = np.ldexp(1.0, e - 7)        # spacing of bf16 values around a
    r = np.rint(a / q) * q
    r[r >= 2.0 ** 128 * (1 - 2.0 ** -9)] = np.inf  # overflow to infinity
    out[finite] = np.sign(v[finite]) * r
    out[~np.isfinite(v)] = v[~np.isfinite(v)]
    return out


def bf16_bits_of(v: np.ndarray) -> np.ndarray:
    """Bit patterns of float64 values that are already exact bf16 values."""
    f32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------------------------
# the three steps
# --------------------------------------------------------------------------------------------
def projection(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y[t,h] = sum_k x[t,k] * W[h,k], W in nn.Linear [out, in] layout, float64 matmul."""
    return x @ W.T


def residual_add(r: np.ndarray, y: np.ndarray) -> np.ndarray:
    """r'[t,h] = r[t,h] + y[t,h]."""
    return r + y


def norm_gain(w: np.ndarray, norm_kind: int) -> np.ndarray:
    """Per-column gain: w for standard RMSNorm, 1 + w for the Gemma form."""
    if norm_kind == NORM_STANDARD:
        return w
    if norm_kind == NORM_GEMMA:
        return 1.0 + w
    raise ValueError(f"unknown norm kind {norm_kind}")


def rms_norm(rp: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """out[t,h] = rp[t,h] / sqrt(mean_h rp[t,:]^2 + eps) * g[h]  (no mean subtraction, no bias)."""
    ms = np.mean(rp * rp, axis=-1, keepdims=True)
    return rp / np.sqrt(ms + eps) * g


def silu_mul(gate_up_bits: np.ndarray, K: int) -> np.ndarray:
    """SiluAndMul on the merged gate/up projection output ("Plugin Architecture" page, model
    table, SiluAndMul row, and section "Fused projections stay fused": the merged projection
    returns [..., 2d] and SiluAndMul slices gate and up out of it).  Each token's row holds gate
    in columns [0, K) and up in [K, 2K); x = silu(gate) * up with silu(g) = g / (1 + e^-g),
    evaluated in float64 and rounded once to bf16 (the model dtype), returned as bf16 bits
    [T, K].  Zero-padded columns (gate = up = 0) give x = 0, which is why the page's load-time
    padding of the intermediate size is inert."""
    gu = widen_bf16(gate_up_bits)
    g, u = gu[:, :K], gu[:, K:2 * K]
    with np.errstate(over="ignore"):
        x = g / (1.0 + np.exp(-g)) * u
    return bf16_bits_of(round_bf16(x))


# --------------------------------------------------------------------------------------------
# whole region
# --------------------------------------------------------------------------------------------
def proj_add_rmsnorm(x_bits, W_bits, residual, norm_w, eps, norm_kind=NORM_STANDARD,
                     mode="fused"):
    """Reference result of one call.

    x_bits [T,K] and W_bits [H,K] are bf16 bit patterns (W in nn.Linear layout), residual [T,H]
    and norm_w [H] fp32, eps the fp32 value the call receives.  Returns (r_new, out) in
    float64; ``out`` is unrounded (the device's bf16 output is compared against it).
    """
    x = widen_bf16(x_bits)
    W = widen_bf16(W_bits)
    r = widen_f32(residual)
    g = norm_gain(widen_f32(norm_w), norm_kind)
    e = float(np.float32(eps))
    y = projection(x, W)
    if mode == "conventional":
        y = round_bf16(y)
    elif mode != "fused":
        raise ValueError(mode)
    rp = residual_add(r, y)
    return rp, rms_norm(rp, g, e)


def proj_add_rmsnorm_chunked(x_bits, W_bits, residual, norm_w, eps, norm_kind, microchunk,
                             mode="fused", pad_value=np.nan):
    """The same call taken through the microchunk partition.

    Chunk c covers rows [c*mc, min(T, (c+1)*mc)); each chunk is processed as a full mc-row
    block whose rows past the end are padding (filled with ``pad_value``), and only the valid
    rows of the chunk are written back to the residual and the output.
    """
    x = widen_bf16(x_bits)
    W = widen_bf16(W_bits)
    r_new = widen_f32(residual).copy()
    g = norm_gain(widen_f32(norm_w), norm_kind)
    e = float(np.float32(eps))
    T, K = x.shape
    H = W.shape[0]
    mc = int(microchunk)
    out = np.full((T, H), np.nan)
    n_chunks = math.ceil(T / mc) if T > 0 else 0
    for c in range(n_chunks):
        lo = c * mc
        valid = min(mc, T - lo)
        xc = np.full((mc, K), pad_value)
        xc[:valid] = x[lo:lo + valid]
        rc = np.full((mc, H), pad_value)
        rc[:valid] = r_new[lo:lo + valid]
        yc = projection(xc, W)
        if mode == "conventional":
            yc = round_bf16(yc)
        rc = residual_add(rc, yc)
        oc = rms_norm(rc, g, e)
        r_new[lo:lo + valid] = rc[:valid]
        out[lo:lo + valid] = oc[:valid]
    return r_new, out


# --------------------------------------------------------------------------------------------
# comparison against a device result
# --------------------------------------------------------------------------------------------
OUT_MAX_ABS = 2e-2      # bf16 output: max |delta|
OUT_REL_L2 = 5e-3       # bf16 output: ||delta||_2 / ||ref||_2
RES_REL_L2 = 1e-3       # fp32 residual: ||delta||_2 / ||ref||_2


def compare(r_dev, out_dev_bits, r_ref, out_ref):
    """Error figures of a device result against the oracle (out_dev_bits are bf16 bits)."""
    out_dev = widen_bf16(out_dev_bits)
    r_dev = widen_f32(r_dev)
    d_out = out_dev - out_ref
    d_r = r_dev - r_ref
    nref_out = float(np.linalg.norm(out_ref)) or 1.0
    nref_r = float(np.linalg.norm(r_ref)) or 1.0
    return {
        "out_max_abs": float(np.max(np.abs(d_out))) if d_out.size else 0.0,
        "out_rel_l2": float(np.linalg.norm(d_out)) / nref_out,
        "res_rel_l2": float(np.linalg.norm(d_r)) / nref_r,
        "res_max_abs": float(np.max(np.abs(d_r))) if d_r.size else 0.0,
        "finite": bool(np.all(np.isfinite(out_dev)) and np.all(np.isfinite(r_dev))),
    }


def within_tolerance(err) -> bool:
    return (err["finite"] and err["out_max_abs"] <= OUT_MAX_ABS
            and err["out_rel_l2"] <= OUT_REL_L2 and err["res_rel_l2"] <= RES_REL_L2)
