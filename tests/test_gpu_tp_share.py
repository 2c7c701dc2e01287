"""One rank's share of the tensor-parallel region, at real share shapes on one GPU, against the
float64 oracle.  With P ranks and a row-parallel projection, rank p holds input columns
[p K/P, (p+1) K/P) of x and of the weight; its projection share is a partial sum of y
(pr_project_partial), the reduce-scatter hands the owner of token shard q the P partials of its
rows, and the owner adds them in rank order to its residual rows and normalises them
(pr_add_rmsnorm_partials).  The reduce-scatter is emulated by the owner reading its rows of
every rank's partial (the planes' row slice q), so the chain computes the whole region: the
owners' results must match the oracle's fused region on the full x and W."""
import numpy as np
import pytest
import torch

import oracle
import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, bits, f32, i16


@pytest.mark.parametrize("name,P,mc", [("o_proj", 8, 2048), ("o_proj", 8, 512), ("o_proj", 4, 512),
                                       ("down_proj", 8, 4096), ("down_proj", 8, 512),
                                       ("down_proj", 2, 1024), ("gemma", 8, 1024)])
def test_tp_share_chain_matches_oracle(name, P, mc):
    """A microchunk of mc tokens (the batch's last, so a ragged one for Gemma's T = 3000): every
    rank's K/P projection share against the oracle's projection of the column slices on sampled
    rows, then every owner's add/norm of its mc/P rows against the oracle's fused region."""
    wl = synth.WORKLOADS[name]
    T, K, H = wl.T, wl.K, wl.H
    kp = K // P
    print(f"tp share {name}: P={P} mc={mc} K/P={kp} H={H}", flush=True)
    d = synth.make_inputs(wl, seed=0)
    c0 = (T - 1) // mc * mc  # the last chunk
    rows = min(mc, T - c0)
    shard = rows // P
    assert shard * P == rows or name == "gemma"
    x_c = d["x"][c0:c0 + rows]
    x_dev = i16(x_c)
    partials = torch.empty((P, rows, H), dtype=torch.float32, device=DEV)
    rng = np.random.default_rng(P * 1000 + mc)
    check_rows = np.array(sorted(set(rng.choice(rows, 16, replace=False).tolist()) |
                                 {0, rows - 1}))
    for p in range(P):
        cols = slice(p * kp, (p + 1) * kp)
        W_p = np.ascontiguousarray(d["W"][:, cols])
        Wp = torch.empty(kp * H, dtype=torch.int16, device=DEV)
        pr.pr_prepare_weight(i16(W_p), pr.PR_WEIGHT_OUT_IN, Wp, kp, H)
        xp = x_dev[:, cols].contiguous()
        pr.pr_project_partial(xp, Wp, partials[p], rows, kp, H)
        torch.cuda.synchronize()
        got = partials[p][check_rows].cpu().numpy().astype(np.float64)
        want = oracle.projection(oracle.widen_bf16(x_c[check_rows][:, cols]),
                                 oracle.widen_bf16(W_p))
        # fp32 accumulation over K/P products of bf16 values
        assert np.max(np.abs(got - want)) <= 2e-6 * max(np.max(np.abs(want)), 1.0) * np.sqrt(kp), p
    # owners: shard q takes rows [q shard, (q+1) shard) of every partial (the last owner takes
    # the remainder when P does not divide the chunk)
    r_dev = f32(d["residual"][c0:c0 + rows])
    w = f32(d["norm_w"])
    out = torch.full((rows, H), 0x7BAD, dtype=torch.int16, device=DEV)
    for q in range(P):
        lo = q * shard
        n = shard if q < P - 1 else rows - lo
        pr.pr_add_rmsnorm_partials(partials.data_ptr() + 4 * lo * H, P, rows * H,
                                   r_dev.data_ptr() + 4 * lo * H, w, d["eps"], n, H,
                                   wl.norm_kind, out.data_ptr() + 2 * lo * H)
    torch.cuda.synchronize()
    check = np.array(sorted(set(rng.choice(rows, 32, replace=False).tolist()) |
                            {0, shard - 1, shard, rows - 1}))
    r_ref, out_ref = oracle.proj_add_rmsnorm(x_c[check], d["W"], d["residual"][c0 + check],
                                             d["norm_w"], d["eps"], wl.norm_kind, "fused")
    err = oracle.compare(r_dev.cpu().numpy()[check], bits(out)[check], r_ref, out_ref)
    print(err, flush=True)
    assert oracle.within_tolerance(err), err


def test_partials_add_in_rank_order_bitwise():
    """Small-integer partials (every fp32 sum exact) and a zero residual: the owner's residual
    is the exact integer sum of the P planes, and one plane equals the single-plane call."""
    P, rows, H = 5, 37, 512
    rng = np.random.default_rng(4)
    planes = rng.integers(-1000, 1000, (P, rows, H)).astype(np.float32)
    part = f32(planes)
    r = torch.zeros((rows, H), dtype=torch.float32, device=DEV)
    w = torch.ones(H, dtype=torch.float32, device=DEV)
    out = torch.empty((rows, H), dtype=torch.int16, device=DEV)
    pr.pr_add_rmsnorm_partials(part, P, rows * H, r, w, 1e-5, rows, H, 0, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r.cpu().numpy(), planes.sum(axis=0))
    rr, oo = oracle.proj_add_rmsnorm(np.zeros((rows, 64), np.uint16), np.zeros((H, 64), np.uint16),
                                     planes.sum(axis=0), np.ones(H, np.float32), 1e-5)
    err = oracle.compare(r.cpu().numpy(), bits(out), rr, oo)
    assert oracle.within_tolerance(err), err


def test_share_entry_points_reject_bad_arguments():
    x = torch.zeros((64, 128), dtype=torch.int16, device=DEV)
    W = torch.zeros(128 * 256, dtype=torch.int16, device=DEV)
    y = torch.zeros((64, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.pr_project_partial(x, W, y, 64, 96, 256)
    assert e.value.code == pr.PR_ERR_SHAPE
    with pytest.raises(pr.PRError) as e:
        pr.pr_project_partial(x, W, x.data_ptr(), 64, 128, 256)  # output on top of x
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    r = torch.zeros((64, 256), dtype=torch.float32, device=DEV)
    w = torch.ones(256, dtype=torch.float32, device=DEV)
    out = torch.empty((64, 256), dtype=torch.int16, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.pr_add_rmsnorm_partials(y.data_ptr(), 2, 64 * 256 - 4, r, w, 1e-5, 64, 256, 0, out)
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    with pytest.raises(pr.PRError) as e:
        pr.pr_add_rmsnorm_partials(y, 1, 64 * 256, y.data_ptr(), w, 1e-5, 64, 256, 0, out)
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    pr.pr_project_partial(x, W, y, 0, 128, 256)  # T = 0: no-op
