"""The single-launch entry point that allocates nothing, for callers that cannot allocate: its
workspace is a fixed device array of the library set up by pr_init.  It must give the result of
the single-launch entry point it mirrors (same kernels, same configuration: bitwise equal) and
meet the oracle's tolerances, over consecutive calls that share the array."""
import numpy as np
import pytest
import torch

import oracle
import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, Device, bits


@pytest.fixture(autouse=True)
def _env(monkeypatch):
    for k in ("PR_MICROCHUNK_TOKENS", "PR_THRESHOLD_TOKENS", "PR_FORCE_TILE", "PR_FORCE_SPLIT",
              "PR_FORCE_WAVES", "PR_FORCE_STAGES", "PR_FORCE_KGROUPS", "PR_FORCE_ADDNORM_WGS",
              "PR_DEBUG_POISON", "PR_DEBUG_DELAY", "PR_SPIN_LIMIT", "PR_DEBUG_EPOCH",
              "PR_FAULT_INJECT"):
        monkeypatch.delenv(k, raising=False)
    pr.pr_clear_tuning()
    yield


def _noalloc(dev, out="own", stream=None):
    d = dev.d
    pr.proj_add_rmsnorm_single_launch_noalloc(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T,
                                              dev.K, dev.H, d["norm_kind"],
                                              dev.out if out == "own" else out, stream)


def test_noalloc_matches_single_launch_on_consecutive_calls():
    """Two calls in a row on one stream with no synchronisation between them, the second with
    a smaller input (fewer tokens, another width and the Gemma norm), each against the
    single-launch entry point's result on the same inputs (bitwise) and the oracle."""
    pr.pr_init()
    cases = [synth.make_custom(1000, 512, 1024, seed=51),
             synth.make_custom(300, 512, 768, seed=52, norm_kind=1)]
    devs = [Device(d) for d in cases]
    refs = []
    for dev in devs:
        refs.append(dev.run("single"))  # the entry point with the grown workspace
        dev.reset()
    torch.cuda.synchronize()
    for dev in devs:
        print(f"no-allocation call T={dev.T} K={dev.K} H={dev.H}", flush=True)
        _noalloc(dev)
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0
    for dev, (r_ref, o_ref) in zip(devs, refs):
        r_dev, out_bits = dev.r[:dev.T].cpu().numpy(), bits(dev.out[:dev.T])
        np.testing.assert_array_equal(r_dev, r_ref)
        np.testing.assert_array_equal(out_bits, o_ref)
        d = dev.d
        r_or, o_or = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"],
                                             d["eps"], d["norm_kind"], "fused")
        err = oracle.compare(r_dev, out_bits, r_or, o_or)
        assert oracle.within_tolerance(err), err


def test_noalloc_graph_replay():
    """Captured on a side stream (the call allocates and fills nothing) and replayed three
    times with the program's own work between replays: every replay equals the eager call."""
    pr.pr_init()
    d = synth.make_custom(700, 512, 1024, seed=53)
    dev = Device(d)
    T = dev.T
    _noalloc(dev)
    torch.cuda.synchronize()
    r_eager, o_eager = dev.r[:T].cpu().numpy(), bits(dev.out[:T])
    r0 = torch.from_numpy(d["residual"]).to(DEV)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    dev.r.copy_(r0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        _noalloc(dev)
    for rep in range(3):
        dev.r.copy_(r0)
        dev.out.fill_(0x7BAD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("replay", rep, flush=True)
        np.testing.assert_array_equal(dev.r[:T].cpu().numpy(), r_eager)
        np.testing.assert_array_equal(bits(dev.out[:T]), o_eager)
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0


def test_noalloc_refuses_what_it_cannot_hold():
    """A call whose slots exceed the fixed array (T * H = 2^29) and a call without an output
    buffer are refused before anything is enqueued."""
    pr.pr_init()
    T, K, H = 65536, 64, 8192
    x = torch.zeros((T, K), dtype=torch.int16, device=DEV)
    Wp = torch.zeros(K * H, dtype=torch.int16, device=DEV)
    r = torch.zeros((T, H), dtype=torch.float32, device=DEV)
    w = torch.ones(H, dtype=torch.float32, device=DEV)
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm_single_launch_noalloc(x, Wp, r, w, 1e-5, T, K, H, 0, out)
    assert e.value.code == pr.PR_ERR_SHAPE, str(e.value)
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm_single_launch_noalloc(x, Wp, r, w, 1e-5, 64, K, H, 0, None)
    assert e.value.code == pr.PR_ERR_INVALID_ARG, str(e.value)
    torch.cuda.synchronize()
    assert float(r.abs().sum()) == 0.0
    del x, Wp, r, w, out
    torch.cuda.empty_cache()
