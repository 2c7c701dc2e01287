"""Seeded random shapes through every path with the library's own configuration choice (no
forced tile, split or wave count): the conventional path, the microchunk pipeline at a random
chunk size, the single launch, and the FP8 single launch with a random scale group, each
against the float64 oracle.  The shapes cover ragged tile rows and chunks, K from one to many
64-deep steps, and H from one to many tile columns, so the tile and split the library picks
varies from case to case."""
import numpy as np
import pytest
import torch

import oracle
import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, Device, bits, f32, i16


def _cases(n=32, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 1201))
        K = 64 * int(rng.integers(1, 33))
        H = 128 * int(rng.integers(1, 17))
        kind = int(rng.integers(0, 2))
        mc = int(rng.choice([16, 77, 128, 256, 512, 1024]))
        G = int(rng.choice([1, 2, 7, 64, 256]))
        out.append((i, T, K, H, kind, mc, G))
    return out


CASES = _cases()


@pytest.fixture(autouse=True)
def _env(monkeypatch):
    for k in ("PR_FORCE_TILE", "PR_FORCE_SPLIT", "PR_FORCE_WAVES", "PR_FORCE_STAGES",
              "PR_FORCE_KGROUPS", "PR_FORCE_CU_SPLIT", "PR_FAULT_INJECT", "PR_SPIN_LIMIT",
              "PR_MICROCHUNK_TOKENS", "PR_THRESHOLD_TOKENS"):
        monkeypatch.delenv(k, raising=False)
    pr.pr_clear_tuning()
    yield


@pytest.mark.parametrize("i,T,K,H,kind,mc,G", CASES)
def test_random_shape_every_path(i, T, K, H, kind, mc, G):
    print(f"random case {i}: T={T} K={K} H={H} kind={kind} mc={mc} G={G}", flush=True)
    d = synth.make_custom(T, K, H, seed=1000 + i, norm_kind=kind, eps=1e-5 if i % 2 else 1e-6)
    dev = Device(d)
    fused_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"], d["eps"],
                                        kind, "fused")
    for path in ("conventional", "pipeline", "single"):
        dev.reset()
        r_dev, out_bits = dev.run({"conventional": None, "pipeline": mc,
                                   "single": "single"}[path])
        if path == "conventional":
            # the device's bf16 rounding of y, where it is a correct one
            ref = oracle.proj_add_rmsnorm_conventional_taken(d["x"], d["W"], d["residual"],
                                                             d["norm_w"], d["eps"], kind, r_dev)
        else:
            ref = fused_ref
        err = oracle.compare(r_dev, out_bits, *ref)
        assert oracle.within_tolerance(err), (path, err)

    # FP8: the device's codes and scales equal the oracle's, then the region against the
    # oracle's FP8 region on those codes.
    xq = torch.empty((T, K), dtype=torch.uint8, device=DEV)
    sx = torch.empty(((T - 1) // G + 1,), dtype=torch.float32, device=DEV)
    pr.pr_quantize_fp8(i16(d["x"]), xq, sx, T, K, G)
    wq = torch.empty((H, K), dtype=torch.uint8, device=DEV)
    sw = torch.empty(1, dtype=torch.float32, device=DEV)
    pr.pr_quantize_fp8(i16(d["W"]), wq, sw, H, K, H)
    xq_ref, sx_ref = oracle.quantize_fp8(d["x"], G)
    wq_ref, sw_ref = oracle.quantize_fp8(d["W"], H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), sx_ref)
    np.testing.assert_array_equal(wq.cpu().numpy(), wq_ref)
    Wp = torch.empty(K * H, dtype=torch.uint8, device=DEV)
    pr.pr_prepare_weight_fp8(wq, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    r = f32(d["residual"])
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    pr.proj_add_rmsnorm_fp8(xq, sx, G, Wp, sw, r, f32(d["norm_w"]), d["eps"], T, K, H, kind, out)
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()
    r_ref, out_ref = oracle.proj_add_rmsnorm_fp8(xq_ref, sx_ref, G, wq_ref, sw_ref[0],
                                                 d["residual"], d["norm_w"], d["eps"], kind)
    err = oracle.compare(r.cpu().numpy(), bits(out), r_ref, out_ref)
    assert oracle.within_tolerance(err), ("fp8", err)


def _hard_inputs(i, T, K, H, kind, mix):
    d = synth.make_custom(T, K, H, seed=3000 + i, norm_kind=kind, eps=1e-6)
    rng = np.random.default_rng(4000 + i)
    if mix == "wide":      # x spread over 2^-8 .. 2^8
        xf = (rng.standard_normal((T, K)) * np.exp2(rng.integers(-8, 9, (T, K)))).astype(np.float32)
        d["x"] = synth.f32_to_bf16_bits(xf)
    elif mix == "large_residual":
        d["residual"] = (d["residual"] * np.float32(1000.0)).astype(np.float32)
    elif mix == "zero_rows":  # all-zero x rows, and all-zero residual rows
        d["x"][rng.random(T) < 0.2] = 0
        d["residual"][rng.random(T) < 0.1] = 0.0
    return d


HARD = [(0, 700, 1024, 1536, 0, "wide"), (1, 1300, 512, 2048, 1, "wide"),
        (2, 513, 2048, 768, 0, "large_residual"), (3, 2048, 1024, 1024, 1, "large_residual"),
        (4, 999, 768, 1280, 0, "zero_rows"), (5, 257, 4096, 512, 1, "zero_rows")]


@pytest.mark.parametrize("i,T,K,H,kind,mix", HARD)
def test_hard_value_mixes(i, T, K, H, kind, mix):
    """Every path against the oracle on value mixes beyond the workloads' normal draws: x spread
    over sixteen binades, a residual a thousand times larger, and all-zero x and residual rows
    (a zero row of x leaves y = 0; a zero residual row too gives r' = 0 and the norm's output
    0 through eps)."""
    print(f"hard case {i}: T={T} K={K} H={H} kind={kind} mix={mix}", flush=True)
    d = _hard_inputs(i, T, K, H, kind, mix)
    dev = Device(d)
    fused_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"], d["eps"],
                                        kind, "fused")
    for path, mc in (("conventional", None), ("pipeline", 256), ("pipeline", 1000),
                     ("single", "single")):
        dev.reset()
        r_dev, out_bits = dev.run(mc)
        if path == "conventional":
            ref = oracle.proj_add_rmsnorm_conventional_taken(d["x"], d["W"], d["residual"],
                                                             d["norm_w"], d["eps"], kind, r_dev)
        else:
            ref = fused_ref
        err = oracle.compare(r_dev, out_bits, *ref)
        assert oracle.within_tolerance(err), (path, mc, err)
