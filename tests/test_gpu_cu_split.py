"""The CU-partitioned pipeline on the GPU: projections on a library stream masked to all but
`n` CUs, add/norms on one masked to those n, three slots with ready and done events.  It runs
the same kernels with the same configurations as the ping-pong schedule, so its results must
be bitwise equal to it for every split, and within the oracle's tolerances."""
import numpy as np
import pytest
import torch

import oracle
import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import Device


@pytest.fixture(autouse=True)
def _env(monkeypatch):
    for k in ("PR_FORCE_TILE", "PR_FORCE_SPLIT", "PR_FORCE_WAVES", "PR_FORCE_STAGES",
              "PR_FORCE_KGROUPS", "PR_FORCE_CU_SPLIT", "PR_DEBUG_POISON", "PR_DEBUG_DELAY",
              "PR_MICROCHUNK_TOKENS", "PR_THRESHOLD_TOKENS", "PR_FAULT_INJECT"):
        monkeypatch.delenv(k, raising=False)
    pr.pr_clear_tuning()
    yield
    pr.pr_clear_tuning()


def _pin_chunk_config(T, K, H, mc):
    """Installs the chunk size's projection configuration, so that a CU split changes only the
    schedule (untuned, each split would take the time model's configuration for its CUs)."""
    c = pr.pr_select(T, K, H, mc)
    pr.pr_set_chunk_config(K, H, mc, c["gemm_bm"], c["gemm_bn"], c["split_k"], c["gemm_waves"])


@pytest.mark.parametrize("T,K,H,mc", [(1000, 512, 1024, 128), (3000, 1024, 3072, 1024),
                                      (70, 512, 512, 16), (2048, 4096, 4096, 512)])
def test_partitioned_equals_ping_pong_bitwise(monkeypatch, T, K, H, mc):
    d = synth.make_custom(T, K, H, seed=T + mc)
    dev = Device(d)
    _pin_chunk_config(T, K, H, mc)
    r0, o0 = dev.run(mc)
    _check = oracle.compare(r0, o0, *oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"],
                                                             d["norm_w"], d["eps"], 0, "fused"))
    assert oracle.within_tolerance(_check), _check
    for n in (8, 32, 64, 128):
        monkeypatch.setenv("PR_FORCE_CU_SPLIT", str(n))
        assert pr.pr_select(T, K, H, mc)["addnorm_cus"] == n
        print(f"T={T} K={K} H={H} mc={mc} split {n}", flush=True)
        dev.reset()
        r1, o1 = dev.run(mc)
        np.testing.assert_array_equal(r1, r0)
        np.testing.assert_array_equal(o1, o0)


@pytest.mark.parametrize("var,val", [("PR_DEBUG_POISON", "1"), ("PR_DEBUG_DELAY", "20")])
def test_partitioned_race_aids(monkeypatch, var, val):
    """Slots NaN-filled after each add/norm, or every launch delayed: still bitwise equal, so
    no add/norm reads a slot before its projection landed and no projection rewrites a slot
    before the add/norm three chunks earlier read it."""
    d = synth.make_custom(1100, 512, 512, seed=9)
    dev = Device(d)
    _pin_chunk_config(1100, 512, 512, 128)
    r0, o0 = dev.run(128)
    monkeypatch.setenv("PR_FORCE_CU_SPLIT", "32")
    monkeypatch.setenv(var, val)
    dev.reset()
    r1, o1 = dev.run(128)
    np.testing.assert_array_equal(r1, r0)
    np.testing.assert_array_equal(o1, o0)


def test_partitioned_caller_join_and_alternating_schedules(monkeypatch):
    """On a side stream, a partitioned call, a ping-pong call and a partitioned call again on
    the same residual, each followed at once by a torch copy on the caller's stream with no
    synchronisation, and every library launch delayed: each copy holds its call's result."""
    d = synth.make_custom(1000, 512, 1024, seed=29)
    dev = Device(d)
    want = []
    r = d["residual"]
    for _ in range(3):
        rr, oo = oracle.proj_add_rmsnorm(d["x"], d["W"], r, d["norm_w"], d["eps"], 0, "fused")
        want.append((rr, oo))
        r = rr.astype(np.float32)
    monkeypatch.setenv("PR_DEBUG_DELAY", "100")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    copies = []
    with torch.cuda.stream(s):
        for split in ("32", "0", "64"):
            monkeypatch.setenv("PR_FORCE_CU_SPLIT", split)
            pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K, dev.H, 128,
                                0, dev.out, s)
            copies.append((dev.r.clone(), dev.out.clone()))
    torch.cuda.synchronize()
    for (rc, oc), (rr, oo) in zip(copies, want):
        err = oracle.compare(rc.cpu().numpy(), oc.cpu().numpy().view(np.uint16), rr, oo)
        # the residual accumulates three projections: the tolerance is the oracle's per call
        assert oracle.within_tolerance(err), err


@pytest.mark.parametrize("name,mc,n", [("o_proj", 512, 32), ("down_proj", 1024, 64),
                                       ("gemma", 1024, 32)])
def test_partitioned_full_size(monkeypatch, name, mc, n):
    wl = synth.WORKLOADS[name]
    print(f"partitioned {name} mc={mc} split {n}", flush=True)
    d = synth.make_inputs(wl, seed=0)
    dev = Device(d)
    monkeypatch.setenv("PR_FORCE_CU_SPLIT", str(n))
    r_dev, out_bits = dev.run(mc)
    rng = np.random.default_rng(7)
    rows = np.array(sorted(set(rng.choice(wl.T, 48, replace=False).tolist()) |
                           {0, wl.T - 1, (wl.T - 1) // mc * mc}))
    r_ref, out_ref = oracle.proj_add_rmsnorm(d["x"][rows], d["W"], d["residual"][rows],
                                             d["norm_w"], d["eps"], wl.norm_kind, "fused")
    err = oracle.compare(r_dev[rows], out_bits[rows], r_ref, out_ref)
    print(err, flush=True)
    assert oracle.within_tolerance(err), err


def test_tuner_chooses_a_cu_split_and_auto_mode_runs_it():
    """pr_tune on a small grid picks a split per chunk size (0 or a partition); auto mode then
    runs whatever was chosen, with oracle parity."""
    rep = pr.pr_tune([1024], [2048], 0, [512, 2048], [256, 512], reps=3)
    print(rep["threshold_tokens"], rep["n_checked"], rep["n_rejected"], flush=True)
    for mc in (256, 512):
        n = pr.pr_select(2048, 1024, 2048, mc)["addnorm_cus"]
        assert n in (0, 32, 64), n
        print("chunk", mc, "split", n, flush=True)
    d = synth.make_custom(2048, 1024, 2048, seed=33)
    dev = Device(d)
    for mc in (256, 512):
        dev.reset()
        r_dev, out_bits = dev.run(mc)
        err = oracle.compare(r_dev, out_bits, *oracle.proj_add_rmsnorm(
            d["x"], d["W"], d["residual"], d["norm_w"], d["eps"], 0, "fused"))
        assert oracle.within_tolerance(err), err
