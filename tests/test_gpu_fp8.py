"""GPU parity of the FP8 (OCP E4M3) projection path through the C ABI against the float64
oracle: the device's quantisation codes and scales equal the oracle's bit for bit (both take
the rounding decision on the fp32 quotient), the prepared weight has the documented layout,
and the fused region with the FP8 projection meets the same tolerances as the bf16 fused
region against oracle.proj_add_rmsnorm_fp8 on the same codes; representable integer inputs pin
the projection bitwise."""
import numpy as np
import pytest
import torch

import oracle
import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, bits, f32, i16


@pytest.fixture(autouse=True)
def _env(monkeypatch):
    for k in ("PR_FORCE_TILE", "PR_FORCE_SPLIT", "PR_FORCE_WAVES", "PR_FORCE_STAGES",
              "PR_FORCE_KGROUPS", "PR_FAULT_INJECT", "PR_SPIN_LIMIT"):
        monkeypatch.delenv(k, raising=False)
    pr.pr_clear_tuning()
    yield


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def _quantize_dev(bits16, group_rows):
    R, C = bits16.shape
    dst = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    scales = torch.empty(((R - 1) // group_rows + 1,), dtype=torch.float32, device=DEV)
    pr.pr_quantize_fp8(i16(bits16), dst, scales, R, C, group_rows)
    torch.cuda.synchronize()
    return dst, scales


@pytest.mark.parametrize("R,C,G", [(300, 512, 128), (64, 4096, 64), (1, 64, 1), (37, 1024, 5),
                                   (2048, 4096, 2048), (130, 1024, 4), (37, 8192, 2),
                                   (45, 16384, 4), (9, 16400, 1), (3, 4096, 1)])
def test_quantize_codes_and_scales_bitwise(R, C, G):
    """Several magnitude ranges per row (so groups differ), a ragged last group, an all-zero
    group and exact ties.  Groups of 1, 2 or 4 rows up to 8192 columns take the one-pass
    kernel (rows in registers, 8 or 16 vectors per lane), the others two passes."""
    rng = np.random.default_rng(R + C + G)
    x = rng.standard_normal((R, C)).astype(np.float32)
    x *= np.exp2(rng.integers(-12, 8, (R, 1))).astype(np.float32)
    if R >= 3 * G:
        x[G:2 * G] = 0.0
    x[0, :4] = [1.0625, -1.1875, 448.0, -0.0]
    xb = synth.f32_to_bf16_bits(x)
    dst, scales = _quantize_dev(xb, G)
    want_q, want_s = oracle.quantize_fp8(xb, G)
    np.testing.assert_array_equal(scales.cpu().numpy(), want_s)
    np.testing.assert_array_equal(dst.cpu().numpy(), want_q)


def _bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def _midpoints():
    """The values midway between neighbouring non-negative E4M3 codes (0 .. 448), and 464."""
    v = oracle.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))
    return np.append((v[:-1] + v[1:]) / 2, 464.0).astype(np.float32)


def _boundary_rows(cols=64):
    """Rows (one scale group each) whose fp32 quotients value / scale fall on an E4M3 rounding
    boundary or within 8 fp32 ulps of one: exact ties with scales that are powers of two, and,
    for 6000 drawn bf16 row maxima, the bf16 values next to boundary * scale whose quotient
    lands that close.  Column 0 holds the row maximum."""
    mids = _midpoints()
    rows = []

    def emit(amax_bits, xs_bits):
        xs_bits = np.concatenate([xs_bits, xs_bits | 0x8000]).astype(np.uint16)
        for i in range(0, len(xs_bits), cols - 1):
            r = np.zeros(cols, np.uint16)
            r[0] = amax_bits
            chunk = xs_bits[i:i + cols - 1]
            r[1:1 + len(chunk)] = chunk
            rows.append(r)

    # scale = 2^k: value / scale is exact, so every midpoint is an exact tie
    for k in range(-30, 9):
        amax = np.float32(448.0 * 2.0 ** k)
        xs = synth.f32_to_bf16_bits((mids[:-1].astype(np.float64) * 2.0 ** k).astype(np.float32))
        emit(synth.f32_to_bf16_bits(np.array([amax], np.float32))[0], xs)
    # drawn scales: bf16 candidates around boundary * scale
    rng = np.random.default_rng(1234)
    amax = synth.f32_to_bf16_bits(np.exp2(rng.uniform(-12, 13, 6000)).astype(np.float32))
    a32 = _bf16_bits_to_f32(amax)
    s = (a32 / np.float32(448.0)).astype(np.float32)
    target = (mids[None, :].astype(np.float64) * s[:, None].astype(np.float64)).astype(np.float32)
    base = (target.view(np.uint32) >> 16).astype(np.int64)
    for d in (-1, 0, 1, 2):
        cand = (base + d).astype(np.uint32)
        x = (cand << 16).view(np.float32)
        q = (x / s[:, None]).astype(np.float32)
        ulps = np.abs(q.view(np.int32).astype(np.int64) - mids[None, :].view(np.int32))
        ok = (ulps <= 8) & (x > 0) & (x <= a32[:, None])
        for i in np.nonzero(ok.any(axis=1))[0]:
            emit(amax[i], cand[i][ok[i]].astype(np.uint16))
    return np.stack(rows)


def test_quantize_rounding_boundaries_bitwise():
    """Quotients on or next to a rounding boundary decide the code by the last fp32 ulp: the
    device's codes equal the oracle's there too (ties to the even code, per-row scales)."""
    xb = _boundary_rows()
    q = (_bf16_bits_to_f32(xb[:, 1:]) / (_bf16_bits_to_f32(xb[:, :1]) / np.float32(448.0)))
    near = np.abs(q.astype(np.float32).view(np.int32)[..., None].astype(np.int64)
                  - np.abs(_midpoints()).view(np.int32)[None, None, :]).min(axis=-1)
    assert (near == 0).sum() > 1000 and ((near > 0) & (near <= 8)).sum() > 300
    dst, scales = _quantize_dev(xb, 1)
    want_q, want_s = oracle.quantize_fp8(xb, 1)
    np.testing.assert_array_equal(scales.cpu().numpy(), want_s)
    np.testing.assert_array_equal(dst.cpu().numpy(), want_q)


def test_quantize_every_bf16_value_unit_scale():
    """Every bf16 pattern of magnitude <= 448 with scale 1 (448 in every row): the codes are
    the nearest E4M3 values of the bf16 values themselves."""
    allb = np.arange(0, 0x10000, dtype=np.uint32)
    mag = _bf16_bits_to_f32(allb & 0x7FFF)
    xs = allb[mag <= 448.0].astype(np.uint16)
    cols = 512
    n = -(-len(xs) // (cols - 1))
    xb = np.zeros((n, cols), np.uint16)
    xb[:, 0] = 0x43E0  # 448
    flat = np.zeros(n * (cols - 1), np.uint16)
    flat[:len(xs)] = xs
    xb[:, 1:] = flat.reshape(n, cols - 1)
    dst, scales = _quantize_dev(xb, 1)
    want_q, want_s = oracle.quantize_fp8(xb, 1)
    assert np.all(want_s == 1.0)
    np.testing.assert_array_equal(scales.cpu().numpy(), want_s)
    np.testing.assert_array_equal(dst.cpu().numpy(), want_q)


def test_quantize_nonfinite_and_tiny_groups():
    """Groups holding a NaN, an infinity, only bf16 subnormals (a scale far below 2^-100) or
    only zeros get what the definition gives: the oracle's codes and scales."""
    rng = np.random.default_rng(7)
    G, C = 4, 256
    x = rng.standard_normal((6 * G, C)).astype(np.float32)
    x[1, 5] = np.nan
    x[G + 2, 9] = np.inf
    x[2 * G + 3, 0] = -np.inf
    x[2 * G, 1] = np.nan
    x[3 * G:4 * G] *= np.float32(1e-3)
    xb = synth.f32_to_bf16_bits(x)
    sub = rng.integers(1, 0x7F, (G, C)).astype(np.uint16) | (rng.integers(0, 2, (G, C)) << 15).astype(np.uint16)
    xb[4 * G:5 * G] = sub  # bf16 subnormals only
    xb[5 * G:6 * G] = 0
    dst, scales = _quantize_dev(xb, G)
    with np.errstate(invalid="ignore"):  # inf / inf in the definition
        want_q, want_s = oracle.quantize_fp8(xb, G)
    got_s = scales.cpu().numpy()
    assert np.isnan(want_s[0]) and np.isinf(want_s[1]) and np.isnan(want_s[2])
    assert 0 < want_s[4] < 2.0 ** -100 and want_s[5] == 1.0
    np.testing.assert_array_equal(got_s, want_s)
    np.testing.assert_array_equal(dst.cpu().numpy(), want_q)


@pytest.mark.parametrize("layout", [0, 1])
def test_prepare_weight_fp8_layout(layout):
    K, H = 256, 192
    rng = np.random.default_rng(3)
    W = rng.integers(0, 256, (H, K)).astype(np.uint8)
    src = W if layout == pr.PR_WEIGHT_OUT_IN else np.ascontiguousarray(W.T)
    dst = torch.empty(K * H, dtype=torch.uint8, device=DEV)
    pr.pr_prepare_weight_fp8(u8(src), layout, dst, K, H)
    got = dst.cpu().numpy().reshape(K // 16, H, 16)
    want = W.reshape(H, K // 16, 16).transpose(1, 0, 2)
    np.testing.assert_array_equal(got, want)


class Fp8Device:
    """Device FP8 inputs: x and W quantised on the device (codes checked against the oracle's),
    the prepared weight, residual, norm weight."""

    def __init__(self, d, scale_rows):
        self.d, self.G = d, scale_rows
        self.T, self.K, self.H = d["T"], d["K"], d["H"]
        self.xq, self.sx = _quantize_dev(d["x"], scale_rows)
        wq, sw = _quantize_dev(d["W"], self.H)
        self.xq_ref, self.sx_ref = oracle.quantize_fp8(d["x"], scale_rows)
        self.wq_ref, self.sw_ref = oracle.quantize_fp8(d["W"], self.H)
        np.testing.assert_array_equal(self.xq.cpu().numpy(), self.xq_ref)
        np.testing.assert_array_equal(wq.cpu().numpy(), self.wq_ref)
        np.testing.assert_array_equal(self.sx.cpu().numpy(), self.sx_ref)
        np.testing.assert_array_equal(sw.cpu().numpy(), self.sw_ref)
        self.sw = sw
        self.Wp = torch.empty(self.K * self.H, dtype=torch.uint8, device=DEV)
        pr.pr_prepare_weight_fp8(wq, pr.PR_WEIGHT_OUT_IN, self.Wp, self.K, self.H)
        self.w = f32(d["norm_w"])
        self.reset()

    def reset(self):
        self.r = f32(self.d["residual"])
        self.out = torch.full((self.T, self.H), 0x7BAD, dtype=torch.int16, device=DEV)

    def run(self):
        d = self.d
        pr.proj_add_rmsnorm_fp8(self.xq, self.sx, self.G, self.Wp, self.sw, self.r, self.w,
                                d["eps"], self.T, self.K, self.H, d["norm_kind"], self.out)
        assert pr.pr_device_status(torch.cuda.current_stream()) == 0
        torch.cuda.synchronize()
        return self.r.cpu().numpy(), bits(self.out)

    def check(self, r_dev, out_bits, rows=None):
        d = self.d
        r_ref, out_ref = oracle.proj_add_rmsnorm_fp8(self.xq_ref, self.sx_ref, self.G,
                                                     self.wq_ref, self.sw_ref[0], d["residual"],
                                                     d["norm_w"], d["eps"], d["norm_kind"])
        if rows is not None:
            r_dev, out_bits, r_ref, out_ref = r_dev[rows], out_bits[rows], r_ref[rows], out_ref[rows]
        err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
        assert oracle.within_tolerance(err), err
        return err


def _force_fp8_tile(monkeypatch, tile):
    """tile: "BMxBN", or "256x128kg2" for 8 waves in two K groups."""
    kg2 = tile.endswith("kg2")
    monkeypatch.setenv("PR_FORCE_TILE", tile[:-3] if kg2 else tile)
    monkeypatch.setenv("PR_FORCE_WAVES", "8")
    if kg2:
        monkeypatch.setenv("PR_FORCE_KGROUPS", "2")
    return (int(v) for v in (tile[:-3] if kg2 else tile).split("x"))


FP8_TILES = ["256x256", "256x128", "256x128kg2", "128x128"]


@pytest.mark.parametrize("tile", FP8_TILES)
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("T,K,H,G", [(300, 512, 768, 128), (64, 256, 512, 1), (513, 1024, 256, 77),
                                     (100, 320, 256, 16), (70, 128, 256, 70)])
def test_fp8_region_parity_small(monkeypatch, tile, kind, T, K, H, G):
    """Every FP8 tile and wave form, both norm forms, ragged tile rows, per-token and ragged
    scale groups; K = 320 is not a whole number of the two K groups' 128-deep stages, so the
    K-group request falls back to one group there."""
    bm, bn = _force_fp8_tile(monkeypatch, tile)
    if H % bn:
        pytest.skip(f"H={H} is not a multiple of the tile's {bn} columns")
    print(f"fp8 tile {tile} T={T} K={K} H={H} G={G} kind={kind}", flush=True)
    d = synth.make_custom(T, K, H, seed=T + K + kind, norm_kind=kind)
    dev = Fp8Device(d, G)
    r_dev, out_bits = dev.run()
    err = dev.check(r_dev, out_bits)
    print(err, flush=True)


@pytest.mark.parametrize("tile", FP8_TILES)
def test_fp8_integer_projection_is_exact(monkeypatch, tile):
    """E4M3-representable integer inputs with 448 in every scale group quantise with unit
    scales; with a zero residual the updated residual is the integer projection, bitwise."""
    _force_fp8_tile(monkeypatch, tile)
    T, K, H, G = 300, 1024, 512, 64
    rng = np.random.default_rng(17)
    vals = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.float32)
    x = rng.choice(vals, (T, K)) * rng.choice([-1.0, 1.0], (T, K)).astype(np.float32)
    W = rng.choice(vals, (H, K)) * rng.choice([-1.0, 1.0], (H, K)).astype(np.float32)
    x[:, 0], W[:, 0] = 448.0, 2.0
    W[0, 1] = 448.0
    d = {"x": synth.f32_to_bf16_bits(x), "W": synth.f32_to_bf16_bits(W),
         "residual": np.zeros((T, H), np.float32), "norm_w": np.ones(H, np.float32),
         "eps": float(np.float32(1e-5)), "norm_kind": 0, "T": T, "K": K, "H": H}
    dev = Fp8Device(d, G)
    assert np.all(dev.sx_ref == 1.0) and dev.sw_ref[0] == 1.0
    r_dev, out_bits = dev.run()
    want = x.astype(np.int64) @ W.astype(np.int64).T
    assert np.abs(want).max() < 2 ** 24
    np.testing.assert_array_equal(r_dev, want.astype(np.float32))
    dev.check(r_dev, out_bits)


@pytest.mark.parametrize("name,G", [("o_proj", 256), ("down_proj", 512), ("gemma", 1024),
                                    ("sweep_T8192", 2048)])
def test_fp8_workload_parity_full_size(name, G):
    """Full-size workloads with the chunk-size scale groups, on sampled rows (fixed seed) that
    include the last group's rows."""
    wl = synth.WORKLOADS[name]
    print(f"fp8 workload {name}: T={wl.T} K={wl.K} H={wl.H} G={G}", flush=True)
    d = synth.make_inputs(wl, seed=0)
    rng = np.random.default_rng(11)
    rows = np.array(sorted(set(rng.choice(wl.T, 48, replace=False).tolist()) |
                           {0, wl.T - 1, (wl.T - 1) // G * G}))
    # the device quantises the whole tensors; the oracle's codes are compared on the rows used
    xq, sx = _quantize_dev(d["x"], G)
    wq, sw = _quantize_dev(d["W"], wl.H)
    groups = {}  # the oracle's quantisation of each sampled row's group, once per group
    for g in sorted({int(t) // G for t in rows}):
        groups[g] = oracle.quantize_fp8(d["x"][g * G:min(wl.T, g * G + G)], G)
    xq_ref = np.stack([groups[t // G][0][t - (t // G) * G] for t in rows])
    sx_rows = np.array([groups[t // G][1][0] for t in rows], np.float32)
    wq_ref, sw_ref = oracle.quantize_fp8(d["W"], wl.H)
    np.testing.assert_array_equal(xq.cpu().numpy()[rows], xq_ref)
    np.testing.assert_array_equal(wq.cpu().numpy(), wq_ref)
    np.testing.assert_array_equal(sw.cpu().numpy(), sw_ref)
    sx_h = sx.cpu().numpy()
    Wp = torch.empty(wl.K * wl.H, dtype=torch.uint8, device=DEV)
    pr.pr_prepare_weight_fp8(wq, pr.PR_WEIGHT_OUT_IN, Wp, wl.K, wl.H)
    r = f32(d["residual"])
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=DEV)
    pr.proj_add_rmsnorm_fp8(xq, sx, G, Wp, sw, r, f32(d["norm_w"]), d["eps"], wl.T, wl.K, wl.H,
                            wl.norm_kind, out)
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sx_h[rows // G], sx_rows)
    r_ref, out_ref = oracle.proj_add_rmsnorm_fp8(xq_ref, sx_rows, 1, wq_ref, sw_ref[0],
                                                 d["residual"][rows], d["norm_w"], d["eps"],
                                                 wl.norm_kind)
    err = oracle.compare(r[rows].cpu().numpy(), bits(out[rows]), r_ref, out_ref)
    print(name, err, flush=True)
    assert oracle.within_tolerance(err), err


def test_fp8_invalid_arguments():
    T, K, H = 64, 256, 256
    xq = torch.zeros((T, K), dtype=torch.uint8, device=DEV)
    sx = torch.ones(T, dtype=torch.float32, device=DEV)
    Wp = torch.zeros(K * H, dtype=torch.uint8, device=DEV)
    sw = torch.ones(1, dtype=torch.float32, device=DEV)
    r = torch.zeros((T, H), dtype=torch.float32, device=DEV)
    w = torch.ones(H, dtype=torch.float32, device=DEV)
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm_fp8(xq, sx, 0, Wp, sw, r, w, 1e-5, T, K, H, 0, out)
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm_fp8(xq, sx, 1, Wp, sw, r, w, 1e-5, T, 96, H, 0, out)
    assert e.value.code == pr.PR_ERR_SHAPE
    with pytest.raises(pr.PRError) as e:  # out on top of the activation scales
        pr.proj_add_rmsnorm_fp8(xq, sx, 1, Wp, sw, r, w, 1e-5, T, K, H, 0, sx.data_ptr())
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    pr.proj_add_rmsnorm_fp8(xq, sx, 1, Wp, sw, r, w, 1e-5, 0, K, H, 0, out)  # T = 0: no-op
    with pytest.raises(pr.PRError) as e:
        pr.pr_quantize_fp8(i16(np.zeros((4, 40), np.uint16)), xq, sx, 4, 40, 1)
    assert e.value.code == pr.PR_ERR_SHAPE
