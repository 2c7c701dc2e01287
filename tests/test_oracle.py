"""Pins for the CPU oracle: each check fixes it against something other than itself.

Brute force on tiny shapes (pure Python, math.fsum), hand-worked values (tests/golden),
closed forms of RMSNorm, invariants named by the method (unit RMS, scale invariance, padded
rows untouched, chunked == unchunked) and a library routine (torch rms_norm in float64,
torch's bf16 cast).  Shapes are non-square so that a transposed operand or a mean over the
wrong axis fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _brute(x, W, r, w, eps, kind, conventional=False):
    """Pure-Python loops over the definition, with exactly rounded sums."""
    T, K = len(x), len(x[0])
    H = len(W)
    r_new = [[0.0] * H for _ in range(T)]
    out = [[0.0] * H for _ in range(T)]
    for t in range(T):
        for h in range(H):
            y = math.fsum(x[t][k] * W[h][k] for k in range(K))
            if conventional:
                y = float(torch.tensor(y, dtype=torch.float64).to(torch.float32)
                          .to(torch.bfloat16).to(torch.float64))
            r_new[t][h] = r[t][h] + y
        ms = math.fsum(v * v for v in r_new[t]) / H
        inv = 1.0 / math.sqrt(ms + eps)
        for h in range(H):
            g = w[h] if kind == 0 else 1.0 + w[h]
            out[t][h] = r_new[t][h] * inv * g
    return np.array(r_new), np.array(out)


# ----------------------------------------------------------------------------------- golden
def test_golden_exact_case():
    case = json.load(open(GOLDEN))["cases"][0]
    x, W = _bits(case["x"]), _bits(case["W"])
    r = np.array(case["residual"], dtype=np.float32)
    for kind, key in ((oracle.NORM_STANDARD, "norm_w_standard"),
                      (oracle.NORM_GEMMA, "norm_w_gemma")):
        w = np.array(case[key], dtype=np.float32)
        for mode in ("fused", "conventional"):
            r_new, out = oracle.proj_add_rmsnorm(x, W, r, w, case["eps"], kind, mode)
            np.testing.assert_array_equal(r_new, np.array(case["residual_out"]))
            np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-15)


def test_golden_conventional_rounding():
    case = json.load(open(GOLDEN))["cases"][1]
    x, W = _bits(case["x"]), _bits(case["W"])
    r = np.array(case["residual"], dtype=np.float32)
    w = np.ones(2, dtype=np.float32)
    rf, _ = oracle.proj_add_rmsnorm(x, W, r, w, 1e-5, 0, "fused")
    rc, _ = oracle.proj_add_rmsnorm(x, W, r, w, 1e-5, 0, "conventional")
    np.testing.assert_array_equal(rf, np.array(case["residual_out_fused"]))
    np.testing.assert_array_equal(rc, np.array(case["residual_out_conventional"]))


def test_golden_bf16_rne_table():
    table = json.load(open(GOLDEN))["bf16_rne"]["values"]
    vals = np.array([v for v, _ in table], dtype=np.float64)
    want = np.array([int(b, 16) for _, b in table], dtype=np.uint16)
    got = oracle.bf16_bits_of(oracle.round_bf16(vals))
    np.testing.assert_array_equal(got, want)
    # widening the expected patterns gives back exactly the rounded values
    np.testing.assert_array_equal(oracle.widen_bf16(want), oracle.round_bf16(vals))


def test_round_bf16_matches_torch_cast():
    """torch's fp32 -> bf16 cast is round-to-nearest-even; on fp32-exact inputs it must agree."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39,  # fp32 / bf16 subnormals
                        [0.0, -0.0, 1.0, 3.0, 1e38, -3.3e38]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_widen_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3EAB, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, 0.333984375, 3.140625]
    np.testing.assert_array_equal(oracle.widen_bf16(bits), want)


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("T,K,H,kind,mode", [
    (3, 5, 7, 0, "fused"), (4, 8, 3, 1, "fused"), (2, 6, 9, 0, "conventional"),
    (5, 3, 4, 1, "conventional"), (1, 16, 16, 0, "fused")])
def test_brute_force_tiny(T, K, H, kind, mode):
    rng = np.random.default_rng(T * 100 + K * 10 + H)
    x = _bits(rng.standard_normal((T, K)))
    W = _bits(rng.standard_normal((H, K)) / np.sqrt(K))
    r = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal(H) * 0.1 + (1.0 if kind == 0 else 0.0)).astype(np.float32)
    eps = float(np.float32(1e-5))
    r_ref, out_ref = oracle.proj_add_rmsnorm(x, W, r, w, eps, kind, mode)
    xf = oracle.widen_bf16(x).tolist()
    Wf = oracle.widen_bf16(W).tolist()
    r_b, out_b = _brute(xf, Wf, r.astype(np.float64).tolist(), w.astype(np.float64).tolist(),
                        eps, kind, conventional=(mode == "conventional"))
    np.testing.assert_allclose(r_ref, r_b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out_ref, out_b, rtol=1e-12, atol=1e-13)


def test_integer_projection_exact():
    d = synth.integer_inputs(7, 24, 11, seed=5)
    y = oracle.projection(oracle.widen_bf16(d["x"]), oracle.widen_bf16(d["W"]))
    xi = oracle.widen_bf16(d["x"]).astype(np.int64)
    Wi = oracle.widen_bf16(d["W"]).astype(np.int64)
    want = np.array([[sum(int(xi[t, k]) * int(Wi[h, k]) for k in range(24)) for h in range(11)]
                     for t in range(7)])
    np.testing.assert_array_equal(y, want)


def test_one_hot_row_selects_weight_column():
    K, H = 6, 5
    rng = np.random.default_rng(1)
    W = oracle.widen_bf16(_bits(rng.standard_normal((H, K))))
    for j in range(K):
        x = np.zeros((1, K))
        x[0, j] = 1.0
        np.testing.assert_array_equal(oracle.projection(x, W)[0], W[:, j])


# ---------------------------------------------------------------------------- RMSNorm forms
def test_zero_weight_leaves_residual_and_normalises_it():
    rng = np.random.default_rng(2)
    T, K, H = 4, 8, 12
    x = _bits(rng.standard_normal((T, K)))
    W = np.zeros((H, K), dtype=np.uint16)
    r = rng.standard_normal((T, H)).astype(np.float32)
    w = np.ones(H, dtype=np.float32)
    r_new, out = oracle.proj_add_rmsnorm(x, W, r, w, 0.0, 0)
    np.testing.assert_array_equal(r_new, r.astype(np.float64))
    rms = np.sqrt(np.mean(r.astype(np.float64) ** 2, axis=1, keepdims=True))
    np.testing.assert_allclose(out, r / rms, rtol=1e-14)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2, 3.0])
def test_unit_rms_closed_form(eps):
    rng = np.random.default_rng(4)
    rp = rng.standard_normal((6, 40)) * rng.uniform(0.1, 5, (6, 1))
    out = oracle.rms_norm(rp, np.ones(40), eps)
    ms = np.mean(rp ** 2, axis=1)
    got = np.sqrt(np.mean(out ** 2, axis=1))
    np.testing.assert_allclose(got, np.sqrt(ms / (ms + eps)), rtol=1e-14)


def test_scale_invariance_up_to_eps():
    rng = np.random.default_rng(5)
    rp = rng.standard_normal((5, 32))
    g = 1 + 0.1 * rng.standard_normal(32)
    for alpha in (0.5, 3.0, 1000.0):
        np.testing.assert_allclose(oracle.rms_norm(alpha * rp, g, 0.0), oracle.rms_norm(rp, g, 0.0),
                                   rtol=1e-13, atol=1e-15)
        eps = 1e-4
        diff = np.abs(oracle.rms_norm(alpha * rp, g, eps) - oracle.rms_norm(rp, g, eps))
        ms = np.mean(rp ** 2, axis=1, keepdims=True)
        bound = eps / (2 * ms) * abs(1 - 1 / alpha ** 2) * np.abs(oracle.rms_norm(rp, g, 0.0))
        assert np.all(diff <= 1.01 * bound + 1e-15)


def test_constant_and_one_hot_rows():
    H = 16
    g = np.linspace(0.5, 1.5, H)
    for c in (-3.0, 0.25, 7.0):
        out = oracle.rms_norm(np.full((1, H), c), g, 1e-3)
        np.testing.assert_allclose(out[0], c / math.sqrt(c * c + 1e-3) * g, rtol=1e-14)
    for j, v in ((0, 2.0), (7, -5.0), (15, 0.5)):
        rp = np.zeros((1, H))
        rp[0, j] = v
        out = oracle.rms_norm(rp, g, 1e-2)
        want = np.zeros(H)
        want[j] = v / math.sqrt(v * v / H + 1e-2) * g[j]
        np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=0)


def test_matches_torch_rms_norm_float64():
    rng = np.random.default_rng(6)
    rp = rng.standard_normal((9, 48)) * 3
    w = rng.standard_normal(48)
    for eps in (1e-6, 1e-2):
        want = torch.nn.functional.rms_norm(torch.from_numpy(rp), (48,), torch.from_numpy(w),
                                            eps=eps).numpy()
        np.testing.assert_allclose(oracle.rms_norm(rp, w, eps), want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("mode", ["fused", "conventional"])
def test_identity_weight_gives_rms_norm_of_x(kind, mode):
    """W = I (K = H) and r = 0: the projection returns x itself, exactly in both modes since x
    is bf16, so the updated residual is x and the output is RMSNorm(x) with gain w or 1 + w
    (torch rms_norm in float64 as the reference)."""
    rng = np.random.default_rng(9)
    T, H = 5, 24
    x = _bits(rng.standard_normal((T, H)) * 2)
    W = _bits(np.eye(H))
    r = np.zeros((T, H), dtype=np.float32)
    w = (0.1 * rng.standard_normal(H)).astype(np.float32)
    eps = float(np.float32(1e-5))
    r_new, out = oracle.proj_add_rmsnorm(x, W, r, w, eps, kind, mode)
    x64 = oracle.widen_bf16(x)
    np.testing.assert_array_equal(r_new, x64)
    g = w.astype(np.float64) + (1.0 if kind == 1 else 0.0)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x64), (H,), torch.from_numpy(g),
                                        eps=eps).numpy()
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)


def test_gemma_is_standard_with_one_plus_w():
    rng = np.random.default_rng(7)
    T, K, H = 3, 16, 10
    x = _bits(rng.standard_normal((T, K)))
    W = _bits(rng.standard_normal((H, K)))
    r = rng.standard_normal((T, H)).astype(np.float32)
    # offsets on a 2^-10 grid, so that 1 + w is exact in fp32 as well
    w = (np.round(0.1 * rng.standard_normal(H) * 1024) / 1024).astype(np.float32)
    _, out_g = oracle.proj_add_rmsnorm(x, W, r, w, 1e-6, oracle.NORM_GEMMA)
    _, out_s = oracle.proj_add_rmsnorm(x, W, r, (1.0 + w.astype(np.float64)), 1e-6,
                                       oracle.NORM_STANDARD)
    np.testing.assert_allclose(out_g, out_s, rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.norm_gain(w, 2)


# -------------------------------------------------------------------------- microchunking
@pytest.mark.parametrize("T,mc", [(10, 3), (10, 5), (10, 10), (10, 16), (1, 4), (17, 8)])
@pytest.mark.parametrize("mode", ["fused", "conventional"])
def test_chunked_equals_unchunked_and_padding_is_inert(T, mc, mode):
    rng = np.random.default_rng(T * 31 + mc)
    K, H = 12, 20
    x = _bits(rng.standard_normal((T, K)))
    W = _bits(rng.standard_normal((H, K)) / np.sqrt(K))
    r = rng.standard_normal((T, H)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    r_u, out_u = oracle.proj_add_rmsnorm(x, W, r, w, 1e-5, 0, mode)
    for pad in (np.nan, 1e30, 0.0):
        r_c, out_c = oracle.proj_add_rmsnorm_chunked(x, W, r, w, 1e-5, 0, mc, mode, pad_value=pad)
        np.testing.assert_array_equal(r_c, r_u)
        np.testing.assert_array_equal(out_c, out_u)


def test_chunked_empty():
    r_c, out_c = oracle.proj_add_rmsnorm_chunked(np.zeros((0, 8), np.uint16),
                                                 np.zeros((4, 8), np.uint16),
                                                 np.zeros((0, 4), np.float32),
                                                 np.ones(4, np.float32), 1e-5, 0, 4)
    assert r_c.shape == (0, 4) and out_c.shape == (0, 4)


def test_padded_k_columns_are_inert():
    """Zero columns appended to x and W (the 64-element padding of an intermediate size)."""
    rng = np.random.default_rng(8)
    T, Kr, K, H = 4, 10, 64, 6
    xr = rng.standard_normal((T, Kr))
    Wr = rng.standard_normal((H, Kr))
    x = np.zeros((T, K), np.uint16)
    W = np.zeros((H, K), np.uint16)
    x[:, :Kr] = _bits(xr)
    W[:, :Kr] = _bits(Wr)
    r = rng.standard_normal((T, H)).astype(np.float32)
    w = (0.1 * rng.standard_normal(H)).astype(np.float32)
    a = oracle.proj_add_rmsnorm(x, W, r, w, 1e-6, 1)
    b = oracle.proj_add_rmsnorm(x[:, :Kr], W[:, :Kr], r, w, 1e-6, 1)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ------------------------------------------------------------------------------ comparison
def test_compare_accepts_own_rounding_and_rejects_planted_errors():
    d = synth.make_custom(32, 64, 128, seed=9)
    r_ref, out_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"], d["eps"])
    out_bits = oracle.bf16_bits_of(oracle.round_bf16(out_ref))
    r32 = r_ref.astype(np.float32)
    assert oracle.within_tolerance(oracle.compare(r32, out_bits, r_ref, out_ref))
    bad = out_bits.copy()
    bad[3, 5] ^= 0x4000          # flip an exponent bit in one output element
    assert not oracle.within_tolerance(oracle.compare(r32, bad, r_ref, out_ref))
    r_bad = r32.copy()
    r_bad[:, 7] += 1.0           # one column's residual off by one
    assert not oracle.within_tolerance(oracle.compare(r_bad, out_bits, r_ref, out_ref))
    # a transposed / misread projection: residual without y added
    r_noy = d["residual"].astype(np.float32)
    assert not oracle.within_tolerance(oracle.compare(r_noy, out_bits, r_ref, out_ref))


# ------------------------------------------------- conventional rounding as the device takes it
def _fp32_sum(products, order):
    """The fp32 sum of exact products, added one at a time in the given order."""
    acc = np.float32(0.0)
    for i in order:
        acc = np.float32(acc + np.float32(products[i]))
    return float(acc)


def test_conventional_roundings_bound_holds_for_any_fp32_order():
    """Brute force: fp32 sums of the K exact bf16 products, in sequential, reversed, pairwise
    and random orders, always round (to bf16, nearest) into [lo, hi], and lie within the
    bound of the exact y.  Cancellation-heavy rows (x and -x halves) are included."""
    rng = np.random.default_rng(77)
    T, K, H = 6, 96, 5
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[3, K // 2:] = -x[3, :K // 2]          # a row that nearly cancels
    W = (rng.standard_normal((H, K)) / 8).astype(np.float32)
    xb, Wb = _bits(x), _bits(W)
    y, lo, hi = oracle.conventional_roundings(xb, Wb)
    xw, Ww = oracle.widen_bf16(xb), oracle.widen_bf16(Wb)
    bound = K * 2.0 ** -24 * (np.abs(xw) @ np.abs(Ww).T)
    for t in range(T):
        for h in range(H):
            p = xw[t] * Ww[h]
            assert math.fsum(p) == pytest.approx(y[t, h], abs=1e-12)
            orders = [range(K), range(K - 1, -1, -1)] + [rng.permutation(K) for _ in range(20)]
            sums = [_fp32_sum(p, o) for o in orders]
            # pairwise (tree) order
            level = [np.float32(v) for v in p]
            while len(level) > 1:
                level = [np.float32(level[i] + level[i + 1]) if i + 1 < len(level) else level[i]
                         for i in range(0, len(level), 2)]
            sums.append(float(level[0]))
            for v in sums:
                assert abs(v - y[t, h]) <= bound[t, h]
                rb = oracle.round_bf16(np.array([v]))[0]
                assert lo[t, h] <= rb <= hi[t, h]
            assert lo[t, h] <= oracle.round_bf16(y[t, h:h + 1])[0] <= hi[t, h]


def test_conventional_taken_equals_round_to_nearest_when_the_device_rounds_so():
    d = synth.make_custom(24, 128, 64, seed=21)
    r_ref, out_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"], d["eps"],
                                             0, "conventional")
    # the device's residual: fp32 add of the round-to-nearest bf16 y
    y = oracle.round_bf16(oracle.projection(oracle.widen_bf16(d["x"]), oracle.widen_bf16(d["W"])))
    r_dev = d["residual"].astype(np.float32) + y.astype(np.float32)
    r2, out2 = oracle.proj_add_rmsnorm_conventional_taken(d["x"], d["W"], d["residual"],
                                                          d["norm_w"], d["eps"], 0, r_dev)
    np.testing.assert_array_equal(r2, r_ref)
    np.testing.assert_array_equal(out2, out_ref)


def test_conventional_taken_accepts_the_other_neighbour_only_near_a_midpoint():
    """One element's y is placed a hair below the midpoint between two bf16 values: a device
    that rounded up (its fp32 sum landed past the midpoint) is accepted and its output is
    recomputed from its choice; a device two bf16 steps away is not, and the comparison then
    fails; an element far from any midpoint admits only the nearest value."""
    K = 4
    # y[0,0] = 1 + 2^-8 - 2^-25: the midpoint of 1 and 1 + 2^-7 minus less than the fp32
    # summation bound (4 * 2^-24 * (1 + 2^-8 + 2^-25), about 2^-22)
    x = np.array([[1.0, 2.0 ** -8, -(2.0 ** -25), 0.0], [0.75, 0.0, 0.0, 0.0]], np.float32)
    W = np.array([[1.0, 1.0, 1.0, 1.0], [1.0, 0.0, 0.0, 0.0]], np.float32)
    xb, Wb = _bits(x), _bits(W)
    y, lo, hi = oracle.conventional_roundings(xb, Wb)
    assert y[0, 0] == 1.0 + 2.0 ** -8 - 2.0 ** -25
    assert lo[0, 0] == 1.0 and hi[0, 0] == 1.0 + 2.0 ** -7     # both neighbours are correct
    assert lo[1, 0] == hi[1, 0] == 0.75                       # exact: only one
    r = np.array([[0.5, -0.25], [2.0, 1.0]], np.float32)
    w = np.array([1.0, 1.0], np.float32)
    eps = 1e-6
    up = np.array([[1.0 + 2.0 ** -7, y[0, 1]], [0.75, y[1, 1]]])
    r_dev = (r.astype(np.float64) + oracle.round_bf16(up)).astype(np.float32)
    rp, out = oracle.proj_add_rmsnorm_conventional_taken(xb, Wb, r, w, eps, 0, r_dev)
    assert rp[0, 0] == 0.5 + 1.0 + 2.0 ** -7
    expect = rp[0] / math.sqrt((rp[0, 0] ** 2 + rp[0, 1] ** 2) / 2 + float(np.float32(eps)))
    np.testing.assert_allclose(out[0], expect, rtol=1e-15)
    # two steps up: not a correct rounding, so the nearest value is kept and the residual
    # comparison shows the device's error
    far = r_dev.copy()
    far[0, 0] = np.float32(0.5 + 1.0 + 2 * 2.0 ** -7)
    rp2, out2 = oracle.proj_add_rmsnorm_conventional_taken(xb, Wb, r, w, eps, 0, far)
    assert rp2[0, 0] == 0.5 + 1.0
    out_bits = oracle.bf16_bits_of(oracle.round_bf16(out2))
    assert not oracle.within_tolerance(oracle.compare(far, out_bits, rp2, out2))


# -------------------------------------------------------------------------------- SiluAndMul
def test_silu_mul_hand_worked():
    """Hand-derived values.  silu(1) * 2 = 2 / (1 + e^-1) = 1.46211715...; bf16 spacing in [1, 2)
    is 2^-7, 1.46211715 / 2^-7 = 187.15 -> 187 -> 1 + 59/128 -> 0x3FBB.  silu(-1) * 1 =
    -1 / (1 + e) = -0.26894142...; spacing in [1/4, 1/2) is 2^-9, 0.26894142 / 2^-9 = 137.70
    -> 138 -> 2^-2 * (1 + 10/128) -> 0xBE8A.  silu(2) * 1 = 1.76159416 -> 225.48 -> 225 -> 0x3FE1.
    Gate comes first in the row: swapping the halves would give silu(2) * 1 in the first
    column instead."""
    gu = synth.f32_to_bf16_bits(np.array([[1.0, -1.0, 2.0, 2.0, 1.0, 1.0]], dtype=np.float32))
    assert oracle.silu_mul(gu, 3)[0].tolist() == [0x3FBB, 0xBE8A, 0x3FE1]


def test_silu_mul_matches_torch_silu_and_padding_is_inert():
    """torch's silu in float64 times up, rounded by round_bf16 (itself pinned against torch's
    cast); zero gate and up columns (the load-time padding) give exact zeros; large positive
    gates pass through (silu(g) = g to double precision), large negative ones vanish."""
    rng = np.random.default_rng(21)
    T, K, pad = 7, 40, 8
    g = rng.standard_normal((T, K)) * 3
    u = rng.standard_normal((T, K))
    g[:, K - pad:] = 0.0
    u[:, K - pad:] = 0.0
    g[0, 0], u[0, 0] = 80.0, 1.5
    g[0, 1], u[0, 1] = -80.0, 1.5
    gu = synth.f32_to_bf16_bits(np.concatenate([g, u], axis=1).astype(np.float32))
    got = oracle.silu_mul(gu, K)
    gw, uw = oracle.widen_bf16(gu[:, :K]), oracle.widen_bf16(gu[:, K:])
    want = torch.nn.functional.silu(torch.from_numpy(gw)).numpy() * uw
    np.testing.assert_array_equal(got, oracle.bf16_bits_of(oracle.round_bf16(want)))
    assert np.all(got[:, K - pad:] == 0)
    assert oracle.widen_bf16(got[0, 0]) == oracle.round_bf16(np.array(80.0 * 1.5))
    assert abs(oracle.widen_bf16(got[0, 1])) < 1e-30


def test_tiled_inputs_repeat_the_block():
    d = synth.tiled_inputs(10, 64, 128, period=3, seed=1)
    assert d["x_block"].shape == (3, 64) and d["x_block"].dtype == np.uint16
    assert d["W"].shape == (128, 64) and d["residual"].shape == (10, 128)
    x = oracle.widen_bf16(d["x_block"])
    assert abs(float(np.mean(x))) < 0.2 and 0.8 < float(np.std(x)) < 1.2
    again = synth.tiled_inputs(10, 64, 128, period=3, seed=1)
    np.testing.assert_array_equal(again["x_block"], d["x_block"])


def test_workload_inputs_statistics():
    """The recipes produce the stated distributions (W variance 1/K, silu*mul second moment)."""
    d = synth.make_inputs(synth.WORKLOADS["tiny"], seed=0)
    W = oracle.widen_bf16(d["W"])
    assert abs(W.var() * d["K"] - 1.0) < 0.02
    assert d["x"].shape == (64, 512) and d["residual"].dtype == np.float32
    g = synth.make_inputs(synth.WORKLOADS["gemma"], seed=0, T=8)
    assert np.all(g["x"][:, 16360:] == 0) and np.all(g["W"][:, 16360:] == 0)
    assert abs(float(np.mean(g["norm_w"]))) < 0.02     # Gemma offset weight centred on 0
    dp = synth.make_inputs(synth.WORKLOADS["down_proj"], seed=0, T=64)
    x = oracle.widen_bf16(dp["x"])
    assert 0.3 < float(np.mean(x * x)) < 0.42          # E[(silu(a) b)^2] ~ 0.356



# ------------------------------------------------------------------------------- FP8 (E4M3)
GOLDEN_E4M3 = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand.json")


def _golden_value(v):
    if v == "nan":
        return np.nan
    if v == "-0":
        return -0.0
    return float(v)


def test_e4m3_decode_hand_table():
    """Hand-derived bit-field values: subnormals, the smallest normal, ones, the largest finite,
    both NaN codes and the signed zero."""
    g = json.load(open(GOLDEN_E4M3))
    for e in g["decode"]:
        got = oracle.decode_e4m3(np.array([int(e["code"], 16)], np.uint8))[0]
        want = _golden_value(e["value"])
        if np.isnan(want):
            assert np.isnan(got), e
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (e, got)


def test_e4m3_decode_matches_torch_for_every_code():
    """All 256 codes against torch's float8_e4m3fn (a library routine of the same format)."""
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_e4m3_encode_hand_table():
    """Ties to the even mantissa (normal and subnormal), clamping above 448, the kept sign."""
    g = json.load(open(GOLDEN_E4M3))
    for e in g["encode"]:
        got = oracle.encode_e4m3(np.array([_golden_value(e["value"])]))[0]
        assert got == int(e["code"], 16), (e, hex(got))


def test_e4m3_encode_matches_torch_within_range():
    """Random fp32 values over the whole finite range (subnormals to 448, both signs), every
    midpoint between neighbouring codes and values just beside them, against torch's
    round-to-nearest-even cast to float8_e4m3fn.  (torch does not clamp above 448: that part
    is pinned by the hand table.)"""
    rng = np.random.default_rng(3)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000)).astype(np.float32)
    vals = mags * rng.choice([-1.0, 1.0], mags.size).astype(np.float32)
    grid = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    beside = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    vals = np.concatenate([vals, mids, -mids, beside, grid.astype(np.float32)])
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.encode_e4m3(vals)
    np.testing.assert_array_equal(got, want)


def test_e4m3_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    np.testing.assert_array_equal(oracle.encode_e4m3(oracle.decode_e4m3(codes)), codes)
    assert oracle.encode_e4m3(np.array([np.nan]))[0] == 0x7F


def test_quantize_fp8_hand_worked():
    g = json.load(open(GOLDEN_E4M3))["quantize"]
    row = synth.f32_to_bf16_bits(np.array([g["row"]], np.float32))
    codes, scales = oracle.quantize_fp8(row, 1)
    assert [int(c) for c in codes[0]] == [int(c, 16) for c in g["codes"]]
    assert scales[0] == np.float32(g["scale_numerator"]) / np.float32(g["scale_denominator"])


def test_quantize_fp8_group_properties():
    """Ragged groups of rows: each group's largest magnitude lands on +-448 (its scale is
    amax / 448); an all-zero group has scale 1 and zero codes; every dequantised value is
    within half a code step of the input (relative 2^-4 in the normal range, 2^-10 * scale
    absolute below it)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((23, 64)).astype(np.float32) * np.float32(3.0)
    x[10:15] = 0.0                      # group 2 (rows 10..14) all zero
    bits = synth.f32_to_bf16_bits(x)
    codes, scales = oracle.quantize_fp8(bits, 5)
    assert scales.shape == (5,) and scales.dtype == np.float32
    xv = oracle.widen_bf16(bits)
    for gi in range(5):
        rows = slice(5 * gi, min(23, 5 * gi + 5))
        dq = oracle.decode_e4m3(codes[rows])
        if gi == 2:
            assert scales[gi] == 1.0 and np.all(dq == 0)
            continue
        amax = np.max(np.abs(xv[rows]))
        assert scales[gi] == np.float32(np.float32(amax) / np.float32(448.0))
        assert np.max(np.abs(dq)) == 448.0
        err = np.abs(dq * float(scales[gi]) - xv[rows])
        bound = np.maximum(np.abs(xv[rows]) * 2.0 ** -4, 2.0 ** -10 * float(scales[gi]))
        assert np.all(err <= bound * (1 + 1e-6))


def test_projection_fp8_brute_force():
    """Pure-Python sums (math.fsum) on a non-square tiny shape with ragged scale groups: a
    dropped scale, a wrong group index or a transposed weight fails it."""
    rng = np.random.default_rng(9)
    T, K, H, G = 7, 5, 3, 3
    xq = rng.integers(0, 256, (T, K)).astype(np.uint8)
    wq = rng.integers(0, 256, (H, K)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x38   # no NaN codes
    wq[(wq & 0x7F) == 0x7F] = 0x40
    sx = np.array([0.5, 3.0, 0.25], np.float32)
    sw = np.float32(0.125)
    got = oracle.projection_fp8(xq, sx, G, wq, sw)
    xd, wd = oracle.decode_e4m3(xq), oracle.decode_e4m3(wq)
    for t in range(T):
        for h in range(H):
            s = math.fsum(float(xd[t, k]) * float(wd[h, k]) for k in range(K))
            want = s * float(sx[t // G]) * float(sw)
            assert got[t, h] == pytest.approx(want, rel=1e-12, abs=1e-300)


def test_fp8_region_exact_on_representable_integers():
    """Inputs whose every value is an E4M3 value and whose largest magnitude is 448 in every
    group quantise with scale exactly 1 and codes that decode to the inputs, so the FP8 region
    equals the bf16 region on the same values and the projection is an exact integer
    (checked against int64 arithmetic)."""
    rng = np.random.default_rng(12)
    T, K, H = 12, 64, 24
    vals = np.array([0, 1, 2, 3, 4, 6, 8, 12, 16], np.float32)
    x = rng.choice(vals, (T, K)) * rng.choice([-1.0, 1.0], (T, K)).astype(np.float32)
    W = rng.choice(vals, (H, K)) * rng.choice([-1.0, 1.0], (H, K)).astype(np.float32)
    x[:, 0] = 448.0
    W[:, 0] = -448.0
    xb, Wb = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(W)
    xq, sx = oracle.quantize_fp8(xb, 4)
    wq, sw = oracle.quantize_fp8(Wb, H)
    assert np.all(sx == 1.0) and np.all(sw == 1.0)
    np.testing.assert_array_equal(oracle.decode_e4m3(xq), x)
    y = oracle.projection_fp8(xq, sx, 4, wq, sw[0])
    np.testing.assert_array_equal(y, x.astype(np.int64) @ W.astype(np.int64).T)
    r = rng.standard_normal((T, H)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    a = oracle.proj_add_rmsnorm_fp8(xq, sx, 4, wq, sw[0], r, w, 1e-5)
    b = oracle.proj_add_rmsnorm(xb, Wb, r, w, 1e-5, oracle.NORM_STANDARD, "fused")
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
