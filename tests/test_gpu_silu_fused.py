"""The down_proj region taken from the merged gate/up output in one launch, with SiluAndMul
formed inside the projection's main loop (proj_add_rmsnorm_silu).  Its conversion is the fp32
arithmetic of pr_silu_mul, so on the same tile configuration it equals pr_silu_mul followed by
the single launch bit for bit; against the oracle it is SiluAndMul in float64 followed by the
fused region."""
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


class SiluDevice:
    def __init__(self, d):
        self.d = d
        self.T, self.K, self.H = d["T"], d["K"], d["H"]
        self.gu = i16(d["gate_up"])
        self.Wp = torch.empty(self.K * self.H, dtype=torch.int16, device=DEV)
        pr.pr_prepare_weight(i16(d["W"]), pr.PR_WEIGHT_OUT_IN, self.Wp, self.K, self.H)
        self.w = f32(d["norm_w"])
        self.x = torch.empty((self.T, self.K), dtype=torch.int16, device=DEV)
        self.reset()

    def reset(self):
        self.r = f32(self.d["residual"])
        self.out = torch.full((self.T, self.H), 0x7BAD, dtype=torch.int16, device=DEV)

    def fused(self):
        d = self.d
        pr.proj_add_rmsnorm_silu(self.gu, self.Wp, self.r, self.w, d["eps"], self.T, self.K,
                                 self.H, d["norm_kind"], self.out)
        assert pr.pr_device_status(torch.cuda.current_stream()) == 0
        torch.cuda.synchronize()
        return self.r.cpu().numpy(), bits(self.out)

    def separate(self):
        d = self.d
        pr.pr_silu_mul(self.gu, self.x, self.T, self.K)
        pr.proj_add_rmsnorm_single_launch(self.x, self.Wp, self.r, self.w, d["eps"], self.T,
                                          self.K, self.H, d["norm_kind"], self.out)
        assert pr.pr_device_status(torch.cuda.current_stream()) == 0
        torch.cuda.synchronize()
        return self.r.cpu().numpy(), bits(self.out)

    def check(self, r_dev, out_bits, rows=None):
        d = self.d
        gu = d["gate_up"] if rows is None else d["gate_up"][rows]
        res = d["residual"] if rows is None else d["residual"][rows]
        x = oracle.silu_mul(gu, self.K)
        r_ref, out_ref = oracle.proj_add_rmsnorm(x, d["W"], res, d["norm_w"], d["eps"],
                                                 d["norm_kind"], "fused")
        if rows is not None:
            r_dev, out_bits = r_dev[rows], out_bits[rows]
        err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
        assert oracle.within_tolerance(err), err
        return err


@pytest.mark.parametrize("tile", ["256x256", "256x128", "128x128"])
@pytest.mark.parametrize("T,K,H,K_real,kind", [(300, 1024, 512, 1000, 0), (700, 512, 1024, 512, 1),
                                               (64, 2048, 256, 2048, 0)])
def test_fused_silu_equals_separate_block_bitwise(monkeypatch, tile, T, K, H, K_real, kind):
    bn = int(tile.split("x")[1])
    if H % bn:
        pytest.skip(f"H={H} is not a multiple of {bn}")
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_WAVES", "8")
    print(f"fused SiluAndMul tile {tile} T={T} K={K} H={H} kind={kind}", flush=True)
    d = synth.gate_up_inputs(T, K, H, seed=T + K, K_real=K_real)
    d["norm_kind"] = kind
    if kind == 1:  # the Gemma recipe: offset weight w ~ N(0, 0.1), gain 1 + w
        d["norm_w"] = (d["norm_w"] - np.float32(1.0)).astype(np.float32)
    dev = SiluDevice(d)
    r_f, o_f = dev.fused()
    dev.check(r_f, o_f)
    dev.reset()
    r_s, o_s = dev.separate()
    np.testing.assert_array_equal(r_f, r_s)
    np.testing.assert_array_equal(o_f, o_s)


@pytest.mark.parametrize("T,K,H,K_real", [(4096, 14336, 4096, 14336), (3000, 16384, 3072, 16360)])
def test_fused_silu_full_size(T, K, H, K_real):
    """down_proj and Gemma at full size from gate_up, on sampled rows (the tile the library
    picks)."""
    print(f"fused SiluAndMul full size T={T} K={K} H={H}", flush=True)
    d = synth.gate_up_inputs(T, K, H, seed=0, K_real=K_real)
    dev = SiluDevice(d)
    r_f, o_f = dev.fused()
    rng = np.random.default_rng(21)
    rows = np.array(sorted(set(rng.choice(T, 40, replace=False).tolist()) | {0, T - 1}))
    print(dev.check(r_f, o_f, rows), flush=True)


def test_fused_silu_rejects_bad_arguments():
    gu = torch.zeros((64, 256), dtype=torch.int16, device=DEV)
    Wp = torch.zeros(128 * 256, dtype=torch.int16, device=DEV)
    r = torch.zeros((64, 256), dtype=torch.float32, device=DEV)
    w = torch.ones(256, dtype=torch.float32, device=DEV)
    out = torch.empty((64, 256), dtype=torch.int16, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm_silu(gu, Wp, r, w, 1e-5, 64, 96, 256, 0, out)
    assert e.value.code == pr.PR_ERR_SHAPE
    with pytest.raises(pr.PRError) as e:  # out inside gate_up
        pr.proj_add_rmsnorm_silu(gu, Wp, r, w, 1e-5, 64, 128, 256, 0, gu.data_ptr())
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    assert pr.pr_validate_silu(gu.data_ptr(), Wp.data_ptr(), r.data_ptr(), w.data_ptr(), 1e-5,
                               64, 128, 256, 0, out.data_ptr()) == 0
