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
  x = silu(gate) * up from the merged gate/up projection output;
* FP8 dense projections ("TPSP Design" page, section 5 To-do: quantized projections with
  their scales handled across microchunks).  The page names no format, so these functions
  take the plainest one the MI355X matrix cores run: OCP E4M3 (4 exponent bits, bias 7, 3
  mantissa bits, no infinities, S.1111.111 the only NaN, largest finite 448); the weight has one
  scale per tensor, the activations one per group of consecutive rows (a microchunk), each
  scale = the group's largest magnitude / 448 (1 for an all-zero group), and a code is the
  value divided by its scale in fp32, rounded to the nearest E4M3 value (ties to even) and
  clamped to +-448.  The quantised projection is y = s_x * s_w * sum_k dec(q_x) dec(q_w).

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
# FP8 (OCP E4M3) projection inputs
# --------------------------------------------------------------------------------------------
E4M3_MAX = 448.0


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64, exactly.  Bit 7 is the sign, bits 6..3 the biased
    exponent e (bias 7), bits 2..0 the mantissa m.  e = 0: subnormal m * 2^-9; e > 0:
    (8 + m) * 2^(e - 10), i.e. 1.m * 2^(e-7); e = 15 with m = 7 is NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
    out = sign * mag
    out[(e == 15) & (m == 7)] = np.nan
    return out


def _e4m3_grid():
    """All non-negative finite E4M3 values in code order (codes 0x00 .. 0x7E); the values
    increase with the code."""
    return decode_e4m3(np.arange(0x7F, dtype=np.uint8))


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """float values -> OCP E4M3 codes: the nearest representable magnitude, a tie going to
    the even code (the even mantissa), magnitudes above 448 clamped to 448; the sign bit is
    kept (-0 -> 0x80); NaN -> 0x7F."""
    v = np.asarray(v, dtype=np.float64)
    grid = _e4m3_grid()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(grid, a, side="left")         # first grid value >= a
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(grid[hi] == a, hi, pick)           # exact hits (also a == 0)
    code = pick.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    code[np.isnan(v)] = 0x7F
    return code


def quantize_fp8(src_bits: np.ndarray, group_rows: int):
    """Scaled E4M3 quantisation of a bf16 matrix [R, C] (bit patterns) by groups of
    `group_rows` consecutive rows (the last group may be shorter).  For group g: amax = the
    largest |value| in its rows; scale = amax / 448 computed in fp32 (1 when amax = 0); each
    code = encode_e4m3(value / scale), the quotient taken in fp32 (the precision the device
    takes this integer decision in).  Returns (codes uint8 [R, C], scales float32 [groups])."""
    x32 = widen_bf16(src_bits).astype(np.float32)     # bf16 values are exact in fp32
    R = x32.shape[0]
    G = int(group_rows)
    n_groups = -(-R // G) if R else 0
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.ones(n_groups, dtype=np.float32)
    for g in range(n_groups):
        rows = slice(g * G, min(R, (g + 1) * G))
        amax = np.float32(np.max(np.abs(x32[rows]))) if x32[rows].size else np.float32(0)
        scale = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
        scales[g] = scale
        codes[rows] = encode_e4m3((x32[rows] / scale).astype(np.float32))
    return codes, scales


def projection_fp8(xq: np.ndarray, x_scales: np.ndarray, group_rows: int, wq: np.ndarray,
                   w_scale: float) -> np.ndarray:
    """y[t,h] = s_x[t // group_rows] * s_w * sum_k dec(xq[t,k]) * dec(wq[h,k]) in float64
    (wq in nn.Linear [out, in] layout)."""
    x = decode_e4m3(xq)
    W = decode_e4m3(wq)
    sx = np.repeat(np.asarray(x_scales, np.float64), int(group_rows))[:x.shape[0]]
    return (x @ W.T) * sx[:, None] * float(np.float32(w_scale))


def proj_add_rmsnorm_fp8(xq, x_scales, group_rows, wq, w_scale, residual, norm_w, eps,
                         norm_kind=NORM_STANDARD):
    """The fused region with the FP8 projection: y enters the residual add unrounded, as
    in the bf16 fused mode; residual add and RMSNorm as there.  Returns (r_new, out) in
    float64, out unrounded."""
    r = widen_f32(residual)
    g = norm_gain(widen_f32(norm_w), norm_kind)
    e = float(np.float32(eps))
    y = projection_fp8(xq, x_scales, group_rows, wq, w_scale)
    rp = residual_add(r, y)
    return rp, rms_norm(rp, g, e)


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
# the conventional mode's rounding as a device takes it
# --------------------------------------------------------------------------------------------
FP32_UNIT_ROUNDOFF = 2.0 ** -24


def conventional_roundings(x_bits, W_bits):
    """The bf16 values a conventional projection may correctly emit for y = x . W^T.

    The projection layer rounds its own fp32 sum of the K products to bf16, not the exact y
    ("TPSP Design" section 1: the conventional region's projection emits the model dtype).
    The products of two bf16 values are exact in fp32, and an fp32 sum of K terms, in any
    order, differs from the exact sum by at most K * 2^-24 * sum_k |x_k w_k|.  So every bf16
    value that rounds (to nearest) some number within that distance of y is a correct
    result: the range [round(y - bound), round(y + bound)].  Returns (y, lo, hi), float64.
    """
    x = widen_bf16(x_bits)
    W = widen_bf16(W_bits)
    y = projection(x, W)
    bound = W.shape[1] * FP32_UNIT_ROUNDOFF * projection(np.abs(x), np.abs(W))
    return y, round_bf16(y - bound), round_bf16(y + bound)


def proj_add_rmsnorm_conventional_taken(x_bits, W_bits, residual, norm_w, eps, norm_kind,
                                        r_dev):
    """The conventional mode with each element's bf16 y taken as the device rounded it, where
    that rounding is a correct one (``conventional_roundings``).

    The device adds its bf16 y to the fp32 residual in fp32, so its residual is fl32(r + yhat).
    Its yhat is read back as the bf16 rounding of (r_dev - r) and kept where it lies in
    [lo, hi] and fl32(r + yhat) reproduces r_dev exactly; every other element keeps the
    round-to-nearest value of y, and the comparison then shows the device's error there.
    Returns (r_new, out) in float64, as ``proj_add_rmsnorm``.
    """
    y, lo, hi = conventional_roundings(x_bits, W_bits)
    r32 = np.asarray(residual, dtype=np.float32)
    r = r32.astype(np.float64)
    rd32 = np.asarray(r_dev, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        taken = round_bf16(rd32.astype(np.float64) - r)
        ok = ((taken >= lo) & (taken <= hi)
              & ((r32 + taken.astype(np.float32)) == rd32))
    yhat = np.where(ok, taken, round_bf16(y))
    rp = residual_add(r, yhat)
    g = norm_gain(widen_f32(norm_w), norm_kind)
    return rp, rms_norm(rp, g, float(np.float32(eps)))


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
