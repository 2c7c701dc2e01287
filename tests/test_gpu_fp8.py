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
                                   (2048, 4096, 2048)])
def test_quantize_codes_and_scales_bitwise(R, C, G):
    """Several magnitude ranges per row (so groups differ), a ragged last group, an all-zero
    group and exact ties."""
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


@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128"])
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("T,K,H,G", [(300, 512, 768, 128), (64, 256, 512, 1), (513, 1024, 256, 77)])
def test_fp8_region_parity_small(monkeypatch, tile, kind, T, K, H, G):
    """Every FP8 tile, both norm forms, ragged tile rows, per-token and ragged scale groups."""
    bm, bn = (int(v) for v in tile.split("x"))
    if H % bn:
        pytest.skip(f"H={H} is not a multiple of the tile's {bn} columns")
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_WAVES", "8")
    print(f"fp8 tile {tile} T={T} K={K} H={H} G={G} kind={kind}", flush=True)
    d = synth.make_custom(T, K, H, seed=T + K + kind, norm_kind=kind)
    dev = Fp8Device(d, G)
    r_dev, out_bits = dev.run()
    err = dev.check(r_dev, out_bits)
    print(err, flush=True)


@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128"])
def test_fp8_integer_projection_is_exact(monkeypatch, tile):
    """E4M3-representable integer inputs with 448 in every scale group quantise with unit
    scales; with a zero residual the updated residual is the integer projection, bitwise."""
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_WAVES", "8")
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
