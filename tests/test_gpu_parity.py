"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Tolerances: bf16 output max |delta| <= 2e-2 and relative L2 <= 5e-3; fp32 residual relative
L2 <= 1e-3 (oracle.within_tolerance).  The fused path is compared with the oracle's fused
mode (unrounded projection), the conventional path with its conventional mode (projection
rounded to bf16).  Integer-valued inputs pin the projection bitwise.  Full-size workloads are
checked on sampled rows (rows are independent, so a row subset is an exact check of those
rows), always including the last chunk's rows.
"""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, Device, bits, f32, i16


@pytest.fixture(autouse=True)
def _env(monkeypatch):
    for k in ("PR_MICROCHUNK_TOKENS", "PR_THRESHOLD_TOKENS", "PR_FORCE_TILE", "PR_FORCE_SPLIT",
              "PR_FORCE_WAVES", "PR_FORCE_STAGES", "PR_FORCE_KGROUPS", "PR_FORCE_ADDNORM_WGS",
              "PR_DEBUG_POISON",
              "PR_DEBUG_DELAY", "PR_SPIN_LIMIT", "PR_DEBUG_EPOCH",
              "PR_FAULT_INJECT"):
        monkeypatch.delenv(k, raising=False)
    pr.pr_clear_tuning()
    yield
    pr.pr_clear_tuning()


def _check(d, r_dev, out_bits, mode, rows=None):
    """Against the oracle's mode; the conventional path's bf16 rounding of y is taken as the
    device took it where that rounding is a correct one (its fp32 sum may land on the other
    side of a rounding midpoint than the exact y)."""
    x, r = d["x"], d["residual"]
    if rows is not None:
        x, r = x[rows], r[rows]
        r_dev, out_bits = r_dev[rows], out_bits[rows]
    if mode == "conventional":
        r_ref, out_ref = oracle.proj_add_rmsnorm_conventional_taken(
            x, d["W"], r, d["norm_w"], d["eps"], d["norm_kind"], r_dev)
    else:
        r_ref, out_ref = oracle.proj_add_rmsnorm(x, d["W"], r, d["norm_w"], d["eps"],
                                                 d["norm_kind"], mode)
    err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
    assert oracle.within_tolerance(err), err
    return err


# (tile, K split, waves per workgroup, LDS ring depth; 0 = the tile's deepest).  Together these
# reach every instantiated kernel: 256x256 at depths 5 and 4, 256x128 at 6, 5, 4 and 128x128 at
# 8, 6, 4, each with 4 and 8 waves.  K = 1024 gives 32 k-steps per split of 1, so most depths
# end in a partial ring trip; split 8 leaves fewer k-steps than stages.
TILES = [("256x256", 1, 8, 0), ("256x256", 1, 4, 0), ("256x256", 2, 8, 4), ("256x256", 1, 4, 4),
         ("256x128", 1, 8, 0), ("256x128", 8, 4, 0), ("256x128", 1, 8, 5), ("256x128", 2, 4, 5),
         ("256x128", 1, 8, 4), ("256x128", 1, 4, 4),
         ("128x128", 1, 8, 0), ("128x128", 4, 4, 0), ("128x128", 2, 8, 0), ("128x128", 1, 8, 6),
         ("128x128", 1, 4, 6), ("128x128", 1, 4, 4), ("128x128", 2, 8, 4)]


# ------------------------------------------------------------------------ bitwise projection
@pytest.mark.parametrize("tile,split,waves,stages", TILES)
def test_integer_projection_is_exact(monkeypatch, tile, split, waves, stages):
    """Small integers: every partial sum is exact in fp32, so the residual must match bitwise.

    T=300 spans two 256-row tiles with a ragged tail; H=768 spans 3-6 column tiles."""
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_SPLIT", str(split))
    monkeypatch.setenv("PR_FORCE_WAVES", str(waves))
    if stages:
        monkeypatch.setenv("PR_FORCE_STAGES", str(stages))
    d = synth.integer_inputs(300, 1024, 768, seed=3)
    dev = Device(d)
    for mc, mode in ((None, "conventional"), (128, "fused"), (300, "fused"), (77, "fused")):
        dev.reset()
        r_dev, out_bits = dev.run(mc)
        r_ref, out_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"],
                                                 d["eps"], 0, mode)
        np.testing.assert_array_equal(r_dev.astype(np.float64), r_ref)
        err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
        assert oracle.within_tolerance(err), (mc, err)


# ------------------------------------------------------------------------- random parity
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("T,K,H", [(300, 512, 768), (64, 512, 512), (1, 256, 320),
                                   (513, 1024, 256)])
def test_random_parity_small(T, K, H, kind):
    d = synth.make_custom(T, K, H, seed=T + K, norm_kind=kind, eps=1e-5)
    dev = Device(d)
    for mc in (None, 16, 128, 256, 4096):
        dev.reset()
        r_dev, out_bits = dev.run(mc)
        _check(d, r_dev, out_bits, "conventional" if mc is None else "fused")


# ------------------------------------------------------------- single-launch fused path
# (tile, waves per workgroup, K groups, K split) of every single-launch instantiation; split 2
# is the pair form (each 256x256 tile's K halves on two workgroups)
SINGLE_CFGS = [("256x256", 8, 1, 1), ("256x128", 8, 1, 1), ("256x128", 4, 1, 1),
               ("256x128", 8, 2, 1), ("128x128", 8, 1, 1), ("256x256", 8, 1, 2),
               ("192x192", 12, 1, 1)]


def _force_single(monkeypatch, tile, waves, kgroups, split):
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_WAVES", str(waves))
    monkeypatch.setenv("PR_FORCE_KGROUPS", str(kgroups))
    monkeypatch.setenv("PR_FORCE_SPLIT", str(split))
    print(f"single launch {tile} {waves} waves {kgroups} K groups split {split}", flush=True)


@pytest.mark.parametrize("tile,waves,kgroups,split", SINGLE_CFGS)
def test_single_launch_integer_projection_is_exact(monkeypatch, tile, waves, kgroups, split):
    """Small integers: the fp32 residual is exact, so it must match bitwise.  T=300 leaves a
    ragged last tile row; H=768 is 3 or 6 tile columns."""
    _force_single(monkeypatch, tile, waves, kgroups, split)
    d = synth.integer_inputs(300, 1024, 768, seed=3)
    dev = Device(d)
    r_dev, out_bits = dev.run("single")
    r_ref, out_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"],
                                             d["eps"], 0, "fused")
    np.testing.assert_array_equal(r_dev.astype(np.float64), r_ref)
    err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
    assert oracle.within_tolerance(err), err


@pytest.mark.parametrize("tile,waves,kgroups,split", [c for c in SINGLE_CFGS if c[3] == 1])
@pytest.mark.parametrize("K", [64, 128, 192])
def test_single_launch_short_k_is_exact(monkeypatch, tile, waves, kgroups, split, K):
    """K of one to three 64-deep stages: the main loop is all prologue and tail refills (two K
    groups: one stage at K = 64, the whole loop in the thin tail), and the residual must still
    be exact on small integers."""
    _force_single(monkeypatch, tile, waves, kgroups, split)
    d = synth.integer_inputs(300, K, 768, seed=K)
    dev = Device(d)
    r_dev, out_bits = dev.run("single")
    r_ref, out_ref = oracle.proj_add_rmsnorm(d["x"], d["W"], d["residual"], d["norm_w"],
                                             d["eps"], 0, "fused")
    np.testing.assert_array_equal(r_dev.astype(np.float64), r_ref)
    err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
    assert oracle.within_tolerance(err), err


def _identity_inputs(T, H, kind):
    rng = np.random.default_rng(11)
    w = (0.1 * rng.standard_normal(H)).astype(np.float32)
    return {"x": synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
            "W": synth.f32_to_bf16_bits(np.eye(H, dtype=np.float32)),
            "residual": np.zeros((T, H), dtype=np.float32),
            "norm_w": w + np.float32(1.0) if kind == 0 else w, "eps": float(np.float32(1e-5)),
            "norm_kind": kind, "T": T, "K": H, "H": H, "K_real": H}


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("path", ["conventional", "pipeline", "single"] +
                         [f"single {c[0]} {c[1]}w kg{c[2]} split{c[3]}" for c in SINGLE_CFGS])
def test_identity_weight_residual_is_x_bitwise(monkeypatch, path, kind):
    """W = I and r = 0: each output's projection has one nonzero product, so every path (any
    tile, K split or chunking) returns x exactly and the updated residual equals x bitwise;
    the output is RMSNorm(x).  T = 300 leaves ragged tile rows and chunks; H = 768 is a whole
    number of tile columns for every tile."""
    T, H = 300, 768
    if path.startswith("single "):
        _force_single(monkeypatch, *SINGLE_CFGS[[f"single {c[0]} {c[1]}w kg{c[2]} split{c[3]}"
                                                 for c in SINGLE_CFGS].index(path)])
    d = _identity_inputs(T, H, kind)
    dev = Device(d)
    mc = {"conventional": None, "pipeline": 128}.get(path, "single")
    r_dev, out_bits = dev.run(mc)
    np.testing.assert_array_equal(r_dev, synth.bf16_bits_to_f32(d["x"]))
    _check(d, r_dev, out_bits, "conventional" if mc is None else "fused")


@pytest.mark.parametrize("tile,waves,kgroups,split", SINGLE_CFGS)
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("T,K,H", [(300, 512, 768), (64, 512, 512), (1, 256, 512),
                                   (513, 1024, 256)])
def test_single_launch_random_parity_small(monkeypatch, tile, waves, kgroups, split, kind, T, K,
                                           H):
    if H % int(tile.split("x")[1]):
        pytest.skip("tile columns do not divide H")
    _force_single(monkeypatch, tile, waves, kgroups, split)
    d = synth.make_custom(T, K, H, seed=T + K, norm_kind=kind, eps=1e-5)
    dev = Device(d)
    r_dev, out_bits = dev.run("single")
    _check(d, r_dev, out_bits, "fused")


@pytest.mark.parametrize("tile,waves,kgroups,split,T,H", [("256x128", 8, 1, 1, 4096, 4096),
                                                          ("256x128", 4, 1, 1, 4096, 4096),
                                                          ("256x128", 8, 2, 1, 4096, 4096),
                                                          ("128x128", 8, 1, 1, 8192, 2048),
                                                          ("256x256", 8, 1, 1, 4100, 8192),
                                                          ("256x256", 8, 1, 2, 4100, 8192),
                                                          ("256x256", 8, 1, 2, 1000, 1280),
                                                          ("256x256", 8, 1, 2, 2048, 4096),
                                                          ("192x192", 12, 1, 1, 4000, 3072)])
def test_single_launch_several_rounds(monkeypatch, tile, waves, kgroups, split, T, H):
    """More tiles than resident workgroups: the launch runs several rounds of whole tile rows
    (256x128: 512 tiles in 2 rounds; 128x128: 1024 tiles in 2; 256x256: 17 x 32 tiles, the
    last round one ragged tile row).  Pairs: 17 x 32 tiles in 5 rounds of 4 tile rows (both
    exchange-region parities); 4 x 5 tiles in one round with 32 workgroups in same-XCD pairs and
    8 in neighbour pairs; the o_proj shape in one full round.  192x192: 21 x 16 tiles, a round
    of 16 tile rows and one of 5."""
    _force_single(monkeypatch, tile, waves, kgroups, split)
    print(f"T={T} H={H}", flush=True)
    d = synth.make_custom(T, 256, H, seed=11)
    dev = Device(d)
    r_dev, out_bits = dev.run("single")
    rows = _sample_rows(T, 256, n=96, seed=2)
    _check(d, r_dev, out_bits, "fused", rows)


def test_largest_workload_every_path():
    """The largest configuration (K=H=8192, T=32768) on every path: the single launch (128 tile
    rows in rounds of whole tile rows per XCD pair), the microchunk pipeline at each chunk size
    of the threshold sweep (512, 1024, 2048: 64, 32 and 16 chunks over two streams and three
    slots) and the conventional path; sampled rows (each chunk size's last-chunk rows among
    them) against the oracle."""
    wl = synth.WORKLOADS["sweep_T32768"]
    print(f"largest workload T={wl.T} K={wl.K} H={wl.H}", flush=True)
    d = synth.make_inputs(wl, seed=0)
    dev = Device(d)
    for mc in ("single",) + wl.microchunks + (None,):
        rows = _sample_rows(wl.T, mc if isinstance(mc, int) else 256, n=64, seed=5)
        dev.reset()
        print("path", mc, flush=True)
        r_dev, out_bits = dev.run(mc)
        err = _check(d, r_dev, out_bits, "conventional" if mc is None else "fused", rows)
        print(mc, err, flush=True)
        assert np.all(np.isfinite(r_dev[rows]))


@pytest.mark.parametrize("cfg", [None] + SINGLE_CFGS, ids=lambda c: "auto" if c is None else
                         f"{c[0]}-{c[1]}w-{c[2]}kg-s{c[3]}")
def test_single_launch_padded_rows_untouched(monkeypatch, cfg):
    """Rows past T (sentinel-filled, NaN in x) stay untouched in every tile configuration: T =
    300 leaves a ragged last tile row for 256- and 192-row tiles, whose residual and output
    stores are bounded by the tile row's valid rows."""
    T = 300
    H = 384 if cfg is None else 768
    if cfg is not None:
        _force_single(monkeypatch, *cfg)
    d = synth.make_custom(T, 512, H, seed=5)
    dev = Device(d, extra_rows=212, pad_x_nan=True)
    dev.reset(sentinel=12345.0)
    r_dev, out_bits = dev.run("single")
    _check(d, r_dev, out_bits, "fused")
    assert np.all(dev.r.cpu().numpy()[T:] == 12345.0)
    assert np.all(bits(dev.out)[T:] == 0x7BAD)


@pytest.mark.parametrize("split", [1, 2])
def test_single_launch_back_to_back_calls(monkeypatch, split):
    """The completion counters return to zero at the end of every launch: calls of different
    sizes in a row (on one stream, no host synchronisation between them) are all correct.
    Split 2: the pair form, whose flags are epoch-tagged per launch."""
    if split == 2:
        _force_single(monkeypatch, "256x256", 8, 1, 2)
    cases = [synth.make_custom(T, 512, 1024, seed=T) for T in (1000, 300, 1000, 17)]
    devs = [Device(d) for d in cases]
    for dev in devs:
        dev.reset()
    for dev in devs:
        d = dev.d
        pr.proj_add_rmsnorm_single_launch(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K,
                                          dev.H, d["norm_kind"], dev.out)
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0
    for dev in devs:
        _check(dev.d, dev.r[:dev.T].cpu().numpy(), bits(dev.out[:dev.T]), "fused")


def test_single_launch_agrees_with_pipeline():
    """Same fused semantics as the microchunk pipeline: the residuals agree to fp32 rounding of
    the projection's summation order, the outputs within one bf16 step."""
    d = synth.make_custom(700, 1024, 2048, seed=9)
    dev = Device(d)
    r_s, o_s = dev.run("single")
    dev.reset()
    r_p, o_p = dev.run(256)
    assert np.max(np.abs(r_s - r_p)) <= 1e-5 * np.max(np.abs(r_p))
    a = o_s.astype(np.uint32) << 16
    b = o_p.astype(np.uint32) << 16
    diff = np.abs(a.view(np.float32) - b.view(np.float32))
    assert np.max(diff) <= 2 ** -7 * np.max(np.abs(b.view(np.float32)))


@pytest.mark.parametrize("tile,waves,split", [("256x128", 4, 1), ("256x256", 8, 1),
                                              ("256x256", 8, 2), ("192x192", 12, 1)])
def test_single_launch_wait_limit_reports(monkeypatch, tile, waves, split):
    """Row reads that look for an epoch no slot carries (set from the host) give up after 64
    polls each; every kernel still ends.  The call leaves no state behind: no output row is
    written and the residual keeps its value before the call (every tile stores it only after
    its wait; the 256x128 tile with 4 waves is the one that prefetches the residual).  The next
    call on the device, of any entry point, returns PR_ERR_HIP without the caller polling
    anything and enqueues nothing; the status bit still reads set, and reading clears it.  A
    later call without the fault is correct.  Split 2: the pair form's partner wait gives up
    first, and neither half writes anything."""
    _force_single(monkeypatch, tile, waves, 1, split)
    monkeypatch.setenv("PR_FAULT_INJECT", "wait")
    monkeypatch.setenv("PR_SPIN_LIMIT", "64")
    d = synth.make_custom(600, 256, 1536, seed=4)
    dev = Device(d)
    print(f"forced give-up: tile {tile}, {waves} waves, split {split}", flush=True)
    pr.proj_add_rmsnorm_single_launch(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K, dev.H,
                                      d["norm_kind"], dev.out)
    torch.cuda.synchronize()
    assert np.all(bits(dev.out) == 0x7BAD)  # no tile wrote output
    np.testing.assert_array_equal(dev.r.cpu().numpy(), d["residual"])  # nor the residual
    monkeypatch.delenv("PR_FAULT_INJECT")
    monkeypatch.delenv("PR_SPIN_LIMIT")
    for k in ("PR_FORCE_TILE", "PR_FORCE_WAVES", "PR_FORCE_KGROUPS", "PR_FORCE_SPLIT"):
        monkeypatch.delenv(k, raising=False)
    with pytest.raises(pr.PRError) as e:
        dev.run(None)  # the next call on the device: the conventional entry point
    assert e.value.code == pr.PR_ERR_HIP and "gave up" in str(e.value), str(e.value)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.r.cpu().numpy(), d["residual"])  # it enqueued nothing
    assert pr.pr_device_status(torch.cuda.current_stream()) & 1
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0
    dev.reset()
    r_dev, out_bits = dev.run(None)  # reported once: calls work again
    _check(d, r_dev, out_bits, "conventional")
    _force_single(monkeypatch, tile, waves, 1, split)
    dev.reset()
    r_dev, out_bits = dev.run("single")
    _check(d, r_dev, out_bits, "fused")


def test_give_up_status_read_clears_host_flag(monkeypatch):
    """pr_device_status consumes the report: after it, the next call is not failed."""
    monkeypatch.setenv("PR_FAULT_INJECT", "wait")
    monkeypatch.setenv("PR_SPIN_LIMIT", "64")
    d = synth.make_custom(300, 256, 512, seed=6)
    dev = Device(d)
    pr.proj_add_rmsnorm_single_launch(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K, dev.H,
                                      d["norm_kind"], dev.out)
    assert pr.pr_device_status(torch.cuda.current_stream()) & 1
    monkeypatch.delenv("PR_FAULT_INJECT")
    monkeypatch.delenv("PR_SPIN_LIMIT")
    dev.reset()
    r_dev, out_bits = dev.run("single")
    _check(d, r_dev, out_bits, "fused")


def test_single_launch_rejects_unsupported_width():
    d = synth.make_custom(64, 256, 320, seed=1)
    dev = Device(d)
    with pytest.raises(pr.PRError) as e:
        dev.run("single")
    assert e.value.code == pr.PR_ERR_SHAPE


def test_borrowed_output_workspace():
    d = synth.make_custom(200, 512, 512, seed=1)
    dev = Device(d)
    for mc in (None, 64):
        dev.reset()
        r_dev, out_bits = dev.run(mc, out=None)
        _check(d, r_dev, out_bits, "conventional" if mc is None else "fused")


# ------------------------------------------------------------------------- padded rows
@pytest.mark.parametrize("T,mc", [(300, 128), (3000 // 8, 64), (70, 16)])
def test_padded_rows_untouched(T, mc):
    """Rows past T (allocated, sentinel-filled, NaN in x) are never written or read into
    valid rows."""
    d = synth.make_custom(T, 512, 384, seed=5)
    dev = Device(d, extra_rows=mc, pad_x_nan=True)
    for m in (None, mc):
        dev.reset(sentinel=12345.0)
        r_dev, out_bits = dev.run(m)
        _check(d, r_dev, out_bits, "conventional" if m is None else "fused")
        r_all = dev.r.cpu().numpy()
        out_all = bits(dev.out)
        assert np.all(r_all[T:] == 12345.0)
        assert np.all(out_all[T:] == 0x7BAD)


# ------------------------------------------------------- add/norm workgroup cap is inert
@pytest.mark.parametrize("T,K,H", [(700, 512, 4096), (301, 512, 320)])
def test_addnorm_workgroup_cap_is_bitwise_inert(monkeypatch, T, K, H):
    """The pipeline's add/norm may run on fewer workgroups than row groups (each strides over
    row groups); results are bitwise those of the uncapped launch, for the register-resident
    kernel (H = 4096) and the generic one (H = 320), including a partial last row group."""
    d = synth.make_custom(T, K, H, seed=15)
    dev = Device(d)
    dev.reset()
    r1, o1 = dev.run(128)
    for cap in ("1", "7", "64"):
        monkeypatch.setenv("PR_FORCE_ADDNORM_WGS", cap)
        dev.reset()
        r2, o2 = dev.run(128)
        np.testing.assert_array_equal(r1, r2)
        np.testing.assert_array_equal(o1, o2)
    _check(d, r1, o1, "fused")


# ------------------------------------------------------------ installed chunk configuration
def test_installed_chunk_config_matches_forced(monkeypatch):
    """A chunk configuration installed for (K, H, microchunk) runs exactly that configuration:
    bitwise equal to the same configuration forced through the debug overrides."""
    d = synth.make_custom(600, 1024, 768, seed=16)
    dev = Device(d)
    pr.pr_set_chunk_config(1024, 768, 256, 256, 128, 2, 4)
    dev.reset()
    r1, o1 = dev.run(256)
    pr.pr_clear_tuning()
    monkeypatch.setenv("PR_FORCE_TILE", "256x128")
    monkeypatch.setenv("PR_FORCE_SPLIT", "2")
    monkeypatch.setenv("PR_FORCE_WAVES", "4")
    dev.reset()
    r2, o2 = dev.run(256)
    np.testing.assert_array_equal(r1, r2)
    np.testing.assert_array_equal(o1, o2)
    _check(d, r1, o1, "fused")


# --------------------------------------------------------------- zero-padded K is inert
@pytest.mark.parametrize("tile", ["256x256", "128x128"])
def test_zero_padded_k_is_bitwise_inert(monkeypatch, tile):
    """K = 448 real columns zero-padded to 512: with the K split pinned to 1, the padded run
    adds two k-stages of exact zeros to the same accumulation, so residual and output match
    the unpadded run bitwise (fused and conventional), and both match the oracle."""
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_SPLIT", "1")
    d = synth.make_custom(300, 512, 384, seed=12, norm_kind=1, eps=1e-6, K_real=448)
    cut = dict(d, x=np.ascontiguousarray(d["x"][:, :448]),
               W=np.ascontiguousarray(d["W"][:, :448]), K=448)
    pad_dev, cut_dev = Device(d), Device(cut)
    for mc in (None, 128):
        pad_dev.reset()
        cut_dev.reset()
        r1, o1 = pad_dev.run(mc)
        r2, o2 = cut_dev.run(mc)
        np.testing.assert_array_equal(r1, r2)
        np.testing.assert_array_equal(o1, o2)
        _check(cut, r2, o2, "conventional" if mc is None else "fused")


# ---------------------------------------------------------------- chunked == unchunked
@pytest.mark.parametrize("tile,split,T,K,H", [("256x256", 1, 1000, 1024, 512),
                                               ("128x128", 2, 1000, 1024, 512),
                                               ("256x128", 1, 1100, 512, 4096)])
def test_microchunked_equals_unchunked_bitwise(monkeypatch, tile, split, T, K, H):
    """With the projection configuration pinned, every row's arithmetic is the same whatever
    the chunk size (the add/norm's row split depends on H only)."""
    monkeypatch.setenv("PR_FORCE_TILE", tile)
    monkeypatch.setenv("PR_FORCE_SPLIT", str(split))
    d = synth.make_custom(T, K, H, seed=7)
    dev = Device(d)
    dev.reset()
    r1, o1 = dev.run(T)
    for mc in (100, 256, 333, 512):
        dev.reset()
        r2, o2 = dev.run(mc)
        np.testing.assert_array_equal(r1, r2)
        np.testing.assert_array_equal(o1, o2)


@pytest.mark.parametrize("mc", [128, 200, 256, "single", None])
def test_caller_stream_join_before_any_sync(monkeypatch, mc):
    """The join (the caller's stream waits for the library stream's last chunk) checked on the
    GPU: on a side stream, the call is followed at once by torch copies of the residual and the
    output on that same stream, with no synchronisation in between, and every library launch
    is delayed (PR_DEBUG_DELAY) so that the library stream runs late.  The copies must hold the
    finished result.  T = 1000: mc = 128 and 256 end on a library-stream chunk, mc = 200 on a
    caller-stream chunk after a library-stream one; the single launch and the conventional
    path run on the caller's stream."""
    d = synth.make_custom(1000, 512, 1024, seed=23)
    dev = Device(d)
    monkeypatch.setenv("PR_DEBUG_DELAY", "150")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        if mc is None:
            pr.proj_add_rmsnorm_unfused(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K,
                                        dev.H, d["norm_kind"], dev.out, s)
        elif mc == "single":
            pr.proj_add_rmsnorm_single_launch(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K,
                                              dev.H, d["norm_kind"], dev.out, s)
        else:
            pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, d["eps"], dev.T, dev.K, dev.H, mc,
                                d["norm_kind"], dev.out, s)
        r_copy = dev.r.clone()
        o_copy = dev.out.clone()
    torch.cuda.synchronize()
    _check(d, r_copy[:dev.T].cpu().numpy(), bits(o_copy[:dev.T]),
           "conventional" if mc is None else "fused")


def test_pipeline_refuses_graph_capture():
    """Capture of the microchunk pipeline is refused before anything is enqueued (it records
    events and waits across a library stream); the conventional path is captured once its
    workspace exists, and a call whose workspace would have to grow under capture is refused.
    Every refusal leaves the capture valid: the graph replays the calls that were accepted."""
    d = synth.make_custom(300, 512, 512, seed=3)
    dev = Device(d)
    pr.pr_release_workspace()  # earlier calls may have grown it past the larger call below
    r_eager, o_eager = dev.run(None)  # sizes the conventional workspace
    big = synth.make_custom(600, 512, 512, seed=4)
    dbig = Device(big)
    r0 = torch.from_numpy(d["residual"]).to(DEV)
    T = dev.T
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    dev.r.copy_(r0)
    torch.cuda.synchronize()
    codes = []
    with torch.cuda.graph(graph, stream=side):
        for call in (lambda: pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, d["eps"], T,
                                                 dev.K, dev.H, 64, d["norm_kind"], dev.out),
                     lambda: pr.proj_add_rmsnorm_unfused(dbig.x, dbig.Wp, dbig.r, dbig.w,
                                                         big["eps"], dbig.T, dbig.K, dbig.H,
                                                         big["norm_kind"], dbig.out)):
            try:
                call()
                codes.append(0)
            except pr.PRError as e:
                codes.append(e.code)
        pr.proj_add_rmsnorm_unfused(dev.x, dev.Wp, dev.r, dev.w, d["eps"], T, dev.K, dev.H,
                                    d["norm_kind"], dev.out)
    assert codes == [pr.PR_ERR_UNSUPPORTED, pr.PR_ERR_UNSUPPORTED], codes
    for rep in range(3):
        dev.r.copy_(r0)
        dev.out.fill_(0x7BAD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("replay", rep, flush=True)
        np.testing.assert_array_equal(dev.r[:T].cpu().numpy(), r_eager)
        np.testing.assert_array_equal(bits(dev.out[:T]), o_eager)
    dev.reset()
    r_dev, out_bits = dev.run(64)  # the pipeline still works outside a capture
    _check(d, r_dev, out_bits, "fused")


def test_deterministic_and_stream_ordered():
    d = synth.make_custom(700, 1024, 1024, seed=8)
    dev = Device(d)
    s = torch.cuda.Stream()
    results = []
    for _ in range(2):
        dev.reset()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            r, o = dev.run(128, stream=s)
        results.append((r, o))
    np.testing.assert_array_equal(results[0][0], results[1][0])
    np.testing.assert_array_equal(results[0][1], results[1][1])
    _check(d, results[0][0], results[0][1], "fused")


# ------------------------------------------------------------------ race detection aids
@pytest.mark.parametrize("var,val", [("PR_DEBUG_POISON", "1"), ("PR_DEBUG_DELAY", "20")])
def test_poison_and_delay_do_not_change_results(monkeypatch, var, val):
    """Slots are NaN-filled after use / streams are delayed: results must stay bitwise equal,
    so no chunk reads a slot before its projection landed or after it was reused."""
    d = synth.make_custom(1100, 512, 512, seed=9)
    dev = Device(d)
    dev.reset()
    r1, o1 = dev.run(128)
    monkeypatch.setenv(var, val)
    dev.reset()
    r2, o2 = dev.run(128)
    np.testing.assert_array_equal(r1, r2)
    np.testing.assert_array_equal(o1, o2)


def test_fault_injection_propagates(monkeypatch):
    d = synth.make_custom(64, 512, 512, seed=10)
    dev = Device(d)
    monkeypatch.setenv("PR_FAULT_INJECT", "launch")
    for mc in (None, 16):
        with pytest.raises(pr.PRError) as e:
            dev.run(mc)
        assert e.value.code == pr.PR_ERR_HIP
    monkeypatch.delenv("PR_FAULT_INJECT")
    dev.reset()
    r_dev, out_bits = dev.run(16)
    _check(d, r_dev, out_bits, "fused")


def test_invalid_arguments_raise():
    d = synth.make_custom(64, 512, 512, seed=11)
    dev = Device(d)
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 64, 500, 512, 16)
    assert e.value.code == pr.PR_ERR_SHAPE
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 64, 512, 512, 5000)
    assert e.value.code == pr.PR_ERR_MICROCHUNK
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 64, 512, 512, -1)
    assert e.value.code == pr.PR_ERR_MICROCHUNK
    # T == 0 is a successful no-op on every entry point: nothing is written
    r_before, out_before = dev.r.clone(), dev.out.clone()
    pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 0, 512, 512, 16)
    pr.proj_add_rmsnorm(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 0, 512, 512, 0, 0, dev.out)
    pr.proj_add_rmsnorm_unfused(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 0, 512, 512, 0, dev.out)
    pr.proj_add_rmsnorm_single_launch(dev.x, dev.Wp, dev.r, dev.w, 1e-5, 0, 512, 512, 0, dev.out)
    torch.cuda.synchronize()
    assert torch.equal(dev.r, r_before) and torch.equal(dev.out, out_before)


# --------------------------------------------------------------------- weight preparation
def test_prepared_weight_layout_and_sources():
    K, H = 128, 192
    rng = np.random.default_rng(12)
    W = synth.f32_to_bf16_bits(rng.standard_normal((H, K)).astype(np.float32))
    Wp1 = torch.empty(K * H, dtype=torch.int16, device=DEV)
    Wp2 = torch.empty(K * H, dtype=torch.int16, device=DEV)
    pr.pr_prepare_weight(i16(W), pr.PR_WEIGHT_OUT_IN, Wp1, K, H)
    pr.pr_prepare_weight(i16(np.ascontiguousarray(W.T)), pr.PR_WEIGHT_IN_OUT, Wp2, K, H)
    torch.cuda.synchronize()
    want = W.reshape(H, K // 8, 8).transpose(1, 0, 2).reshape(-1)  # [(k/8)][h][k%8]
    np.testing.assert_array_equal(bits(Wp1), want)
    np.testing.assert_array_equal(bits(Wp2), want)


def test_pretransposed_source_gives_same_result():
    d = synth.make_custom(256, 512, 512, seed=13)
    a = Device(d, weight_layout=pr.PR_WEIGHT_OUT_IN)
    b = Device(d, weight_layout=pr.PR_WEIGHT_IN_OUT)
    ra, oa = a.run(128)
    rb, ob = b.run(128)
    np.testing.assert_array_equal(ra, rb)
    np.testing.assert_array_equal(oa, ob)


# ------------------------------------------------------------------------ automatic mode
def test_auto_mode_overrides_and_tuning(monkeypatch):
    d = synth.make_custom(512, 512, 512, seed=14)
    dev = Device(d)
    dev.reset()
    r0, o0 = dev.run(0)          # untuned: conventional
    _check(d, r0, o0, "conventional")
    monkeypatch.setenv("PR_MICROCHUNK_TOKENS", "128")
    monkeypatch.setenv("PR_THRESHOLD_TOKENS", "256")
    dev.reset()
    r1, o1 = dev.run(0)          # both overrides: fused
    _check(d, r1, o1, "fused")
    dev.reset()
    r2, o2 = dev.run(128)
    np.testing.assert_array_equal(r1, r2)
    monkeypatch.delenv("PR_MICROCHUNK_TOKENS")
    monkeypatch.delenv("PR_THRESHOLD_TOKENS")
    rep = pr.pr_tune([512], [512], 0, [128, 512], [64, 128, 256], reps=3)
    # T=128: chunks 64 and 128 and the single launch; T=512: three chunk sizes and the single
    assert rep["n_checked"] == 7 and rep["n_rejected"] == 0
    assert rep["max_tokens"] == 512
    for row in rep["timings"][0]:  # conventional, best fused, chunks 64/128/256, single
        assert len(row) == 6 and row[0] > 0 and row[1] > 0 and row[5] > 0
        assert row[1] == min(v for v in row[2:] if v > 0)
    for mc in (64, 128, 256):  # a chunk configuration was tuned and installed per chunk size
        cfg = pr.pr_select(512, 512, 512, mc)
        assert (cfg["gemm_bm"], cfg["gemm_bn"]) in ((256, 256), (256, 128), (128, 128))
        assert 512 % (64 * cfg["split_k"]) == 0 and cfg["gemm_waves"] in (4, 8)
    sel = pr.pr_select(512, 512, 512, 0)
    thr = rep["threshold_tokens"]
    if 512 >= thr:
        assert sel["path"] in (pr.PR_PATH_FUSED, pr.PR_PATH_SINGLE)
    else:
        assert sel["path"] == pr.PR_PATH_CONVENTIONAL
    dev.reset()
    r3, o3 = dev.run(0)          # tuned auto mode, whichever path it chose
    _check(d, r3, o3, "conventional" if sel["path"] == pr.PR_PATH_CONVENTIONAL else "fused")
    # T above the largest tuned token count is refused before anything runs
    x600 = torch.zeros((600, 512), dtype=torch.int16, device=DEV)
    r600 = torch.zeros((600, 512), dtype=torch.float32, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.proj_add_rmsnorm(x600, dev.Wp, r600, dev.w, 1e-5, 600, 512, 512, 0)
    assert e.value.code == pr.PR_ERR_UNSUPPORTED


def test_tuner_accepts_large_hidden_sizes():
    """At H = 8192 two correct bf16 outputs differ by an ulp at |out| >= 4 (0.031 > 2e-2):
    the candidate check must still accept the fused candidates (every one checked, none
    rejected: two chunk sizes and the single launch at each of the two token counts)."""
    rep = pr.pr_tune([1024], [8192], 0, [512, 1024], [256, 512], reps=2)
    assert rep["n_rejected"] == 0 and rep["n_checked"] == 6, rep


# -------------------------------------------------------------------- full-size workloads
def _sample_rows(T, mc, n=48, seed=0):
    rng = np.random.default_rng(seed)
    last = (T - 1) // mc * mc if mc else 0
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows |= {0, T - 1, last, min(T - 1, last + 1)}
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["tiny", "o_proj", "down_proj", "gemma", "sweep_T128",
                                  "sweep_T512", "sweep_T2048", "sweep_T8192"])
def test_workload_parity_full_size(name):
    """Every workload at its full size on every path: the conventional path, the pipeline at
    each of the workload's chunk sizes (for the threshold sweep, 512, 1024 and 2048 where they
    do not exceed T) and the single launch, on sampled rows (a fixed per-workload seed, so a
    failure replays) that always include each chunk size's last-chunk rows."""
    wl = synth.WORKLOADS[name]
    print(f"workload {name}: T={wl.T} K={wl.K} H={wl.H}", flush=True)
    d = synth.make_inputs(wl, seed=0)
    dev = Device(d)
    seed = zlib.crc32(name.encode()) % 1000
    for mc in (None,) + wl.microchunks + ("single",):
        dev.reset()
        print("path", mc, flush=True)
        r_dev, out_bits = dev.run(mc)
        rows = _sample_rows(wl.T, mc if isinstance(mc, int) else wl.T, seed=seed)
        err = _check(d, r_dev, out_bits, "conventional" if mc is None else "fused", rows)
        print(name, mc, err, flush=True)
        assert np.all(np.isfinite(r_dev))


def test_launch_split_past_2_30_elements_of_x():
    """x with more than 2^30 elements (T = 65600, K = 16384) is projected in two launches,
    since offsets inside a launch are 32-bit: rows on both sides of the boundary at row 65536
    and the last rows match the oracle on the conventional path and the single launch.  x is a
    4099-row block tiled down the rows (4099 does not divide 65536, so a row offset error across
    the boundary reads other data)."""
    T, K, H, P = 65600, 16384, 256, 4099
    print(f"launch split: T={T} K={K} H={H}", flush=True)
    d = synth.tiled_inputs(T, K, H, period=P, seed=13)
    x = i16(d["x_block"]).repeat((T + P - 1) // P, 1)[:T].contiguous()
    assert x.numel() > 2 ** 30
    W_src = i16(d["W"])
    Wp = torch.empty(K * H, dtype=torch.int16, device=DEV)
    pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    w = f32(d["norm_w"])
    rng = np.random.default_rng(5)
    rows = np.array(sorted(set(rng.choice(T, 40, replace=False).tolist()) |
                           {0, 1, 65535, 65536, 65537, T - 2, T - 1}))
    for path in ("conventional", "single"):
        r = f32(d["residual"])
        out = torch.full((T, H), 0x7BAD, dtype=torch.int16, device=DEV)
        if path == "conventional":
            pr.proj_add_rmsnorm_unfused(x, Wp, r, w, d["eps"], T, K, H, 0, out)
        else:
            pr.proj_add_rmsnorm_single_launch(x, Wp, r, w, d["eps"], T, K, H, 0, out)
            assert pr.pr_device_status(torch.cuda.current_stream()) == 0
        torch.cuda.synchronize()
        r_dev, out_bits = r[rows].cpu().numpy(), bits(out[rows])
        if path == "conventional":
            r_ref, out_ref = oracle.proj_add_rmsnorm_conventional_taken(
                d["x_block"][rows % P], d["W"], d["residual"][rows], d["norm_w"], d["eps"], 0,
                r_dev)
        else:
            r_ref, out_ref = oracle.proj_add_rmsnorm(d["x_block"][rows % P], d["W"],
                                                     d["residual"][rows], d["norm_w"], d["eps"],
                                                     0, "fused")
        err = oracle.compare(r_dev, out_bits, r_ref, out_ref)
        print(path, err, flush=True)
        assert oracle.within_tolerance(err), (path, err)
    del x


# ---------------------------------------------------------------------------------- SiluAndMul
def _bf16_ordered(b):
    """bf16 bit patterns as integers in value order (one step per ulp; +0 and -0 both 0)."""
    b = np.asarray(b, dtype=np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _silu_mul_check(gu_bits, x_bits, K, K_real):
    """x against the oracle: the kernel computes in fp32, the oracle in float64, and each
    rounds once to bf16, so an element may land one bf16 ulp apart when the exact value sits
    next to a rounding boundary.  Distances are counted in ulps on the value line, where the
    two zeros coincide (a zero gate or up drawn with a sign gives -0 on the device, +0 in the
    oracle).  Padded columns must be exactly zero."""
    want = _bf16_ordered(oracle.silu_mul(gu_bits, K))
    got = _bf16_ordered(x_bits)
    assert np.all(np.abs(got - want) <= 1), np.abs(got - want).max()
    assert np.mean(got != want) < 1e-3, np.mean(got != want)
    assert np.all(x_bits[:, K_real:] == 0)


@pytest.mark.parametrize("T,K,K_real", [(300, 512, 512), (1, 64, 64), (777, 2048, 2000),
                                        (3000, 16384, 16360)])
def test_silu_mul_matches_oracle(T, K, K_real):
    """Ragged token counts, padded intermediate sizes (Gemma's 16360 padded to 16384), and a
    sentinel row past T that must stay untouched."""
    d = synth.gate_up_inputs(T, K, 64, seed=T + K, K_real=K_real)
    gu = i16(d["gate_up"])
    x = torch.full((T + 1, K), 0x7BAD, dtype=torch.int16, device=DEV)
    pr.pr_silu_mul(gu, x, T, K)
    torch.cuda.synchronize()
    xb = bits(x)
    _silu_mul_check(d["gate_up"], xb[:T], K, K_real)
    assert np.all(xb[T] == 0x7BAD)


def test_silu_mul_large_and_special_gates():
    """Gates far out in both tails and at infinity: silu(g) tends to g for large g and to 0
    for large -g.  The device's native exponential overflows to infinity for -g above about
    88.7, where the quotient becomes a signed zero; the float64 oracle's value there is below
    half the smallest bf16 subnormal, so both round to zero.  An infinite gate gives a NaN
    where the oracle gives one (-inf / inf, or inf * 0), and +-inf otherwise."""
    gates = [0.0, -0.0, 1.0, -1.0, 20.0, -20.0, 60.0, -60.0, 88.0, -88.0, 100.0, -100.0,
             np.inf, -np.inf]
    K = 64
    rng = np.random.default_rng(77)
    T = len(gates) * 3
    g = np.repeat(np.array(gates, dtype=np.float32), 3)[:, None] * np.ones((1, K), np.float32)
    u = rng.standard_normal((T, K), dtype=np.float32)
    u[::7, ::5] = 0.0
    gu = np.concatenate([synth.f32_to_bf16_bits(g), synth.f32_to_bf16_bits(u)], axis=1)
    x = torch.empty((T, K), dtype=torch.int16, device=DEV)
    pr.pr_silu_mul(i16(gu), x, T, K)
    torch.cuda.synchronize()
    got = bits(x)
    want = oracle.silu_mul(gu, K)
    is_nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    assert np.array_equal(is_nan(got), is_nan(want))
    keep = ~is_nan(want)
    d_ulp = np.abs(_bf16_ordered(got[keep]) - _bf16_ordered(want[keep]))
    assert d_ulp.max() <= 1, d_ulp.max()
    assert np.all(np.isinf(oracle.widen_bf16(got[keep])) == np.isinf(oracle.widen_bf16(want[keep])))


@pytest.mark.parametrize("path", ["single", 128, None])
def test_silu_mul_then_down_proj_parity(path):
    """The down_proj block from the merged gate/up output: SiluAndMul, then the projection,
    residual add and RMSNorm, against the oracle's SiluAndMul followed by its fused (or
    conventional) region."""
    T, K, H = 300, 1024, 512
    d = synth.gate_up_inputs(T, K, H, seed=31, K_real=1000)
    x = torch.empty((T, K), dtype=torch.int16, device=DEV)
    pr.pr_silu_mul(i16(d["gate_up"]), x, T, K)
    torch.cuda.synchronize()
    dd = dict(d, x=oracle.silu_mul(d["gate_up"], K))
    dev = Device(dd)
    dev.x = x  # the device's own SiluAndMul output feeds the projection
    r_dev, out_bits = dev.run(path)
    _check(dd, r_dev, out_bits, "conventional" if path is None else "fused")


def test_silu_mul_down_proj_full_size():
    """down_proj at full size (T = 4096, intermediate 14336, H = 4096) from gate_up: x on
    sampled rows, then the single launch on those rows."""
    T, K, H = 4096, 14336, 4096
    print(f"silu_mul down_proj: T={T} K={K} H={H}", flush=True)
    d = synth.gate_up_inputs(T, K, H, seed=0)
    gu = i16(d["gate_up"])
    x = torch.empty((T, K), dtype=torch.int16, device=DEV)
    pr.pr_silu_mul(gu, x, T, K)
    torch.cuda.synchronize()
    rows = _sample_rows(T, T, seed=3)
    _silu_mul_check(d["gate_up"][rows], bits(x[rows]), K, K)
    W_src = i16(d["W"])
    Wp = torch.empty(K * H, dtype=torch.int16, device=DEV)
    pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    r = f32(d["residual"])
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    pr.proj_add_rmsnorm_single_launch(x, Wp, r, f32(d["norm_w"]), d["eps"], T, K, H, 0, out)
    assert pr.pr_device_status(torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()
    x_ref = oracle.silu_mul(d["gate_up"][rows], K)
    r_ref, out_ref = oracle.proj_add_rmsnorm(x_ref, d["W"], d["residual"][rows], d["norm_w"],
                                             d["eps"], 0, "fused")
    err = oracle.compare(r[rows].cpu().numpy(), bits(out[rows]), r_ref, out_ref)
    print(err, flush=True)
    assert oracle.within_tolerance(err), err


def test_silu_mul_invalid_arguments():
    gu = torch.zeros((4, 256), dtype=torch.int16, device=DEV)
    x = torch.zeros((4, 128), dtype=torch.int16, device=DEV)
    with pytest.raises(pr.PRError) as e:
        pr.pr_silu_mul(gu, x, 4, 96)
    assert e.value.code == pr.PR_ERR_SHAPE
    with pytest.raises(pr.PRError) as e:
        pr.pr_silu_mul(gu, gu, 4, 64)   # x inside gate_up
    assert e.value.code == pr.PR_ERR_INVALID_ARG
    pr.pr_silu_mul(gu, x, 0, 128)        # T = 0: no-op
    torch.cuda.synchronize()
    assert int(x.abs().sum()) == 0


def test_tuning_file_on_the_device(tmp_path):
    """A tuning file saved on this device carries its key (architecture and CU count);
    reloaded after a clear it restores every decision, and an auto-mode call then runs the
    restored choice (the single launch at T=2048) with oracle parity."""
    pr.pr_clear_tuning()
    pr.pr_set_tuning(1024, 2048, 1024, 8192, [128, 1024], [128, pr.PR_SINGLE_LAUNCH])
    pr.pr_set_chunk_config(1024, 2048, 128, 128, 128, 2, 8)
    before = [pr.pr_select(T, 1024, 2048, 0) for T in (64, 512, 2048)]
    path = tmp_path / "tune.txt"
    pr.pr_tuning_save(str(path))
    key = path.read_text().split("\n")[0].split()[3]
    print("device key", key, flush=True)
    assert key.startswith("gfx950") and key.rsplit(":", 1)[1].isdigit()
    pr.pr_clear_tuning()
    pr.pr_tuning_load(str(path))
    assert [pr.pr_select(T, 1024, 2048, 0) for T in (64, 512, 2048)] == before
    assert before[2]["path"] == pr.PR_PATH_SINGLE
    d = synth.make_custom(2048, 1024, 2048, seed=21)
    dev = Device(d)
    r_dev, out_bits = dev.run(0)
    _check(d, r_dev, out_bits, "fused")
    pr.pr_clear_tuning()


@pytest.mark.parametrize("split", [1, 2])
def test_single_launch_graph_replay(monkeypatch, split):
    """The single launch keeps its epoch on the device, so a captured call replays correctly:
    replays with the program's own work between them (residual restore, output reset,
    synchronisation) all equal the eager call bitwise.  Split 2: the pair form."""
    if split == 2:
        _force_single(monkeypatch, "256x256", 8, 1, 2)
    d = synth.make_custom(1000, 512, 1024, seed=31)
    dev = Device(d)
    r_eager, o_eager = dev.run("single")  # also sizes the workspace (not capturable)
    r0 = torch.from_numpy(d["residual"]).to(DEV)
    T = dev.T
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    dev.r.copy_(r0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        pr.proj_add_rmsnorm_single_launch(dev.x, dev.Wp, dev.r, dev.w, d["eps"], T, dev.K, dev.H,
                                          d["norm_kind"], dev.out)
    for rep in range(5):
        dev.r.copy_(r0)
        dev.out.fill_(0x7BAD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("replay", rep, flush=True)
        assert pr.pr_device_status(torch.cuda.current_stream()) == 0
        np.testing.assert_array_equal(dev.r[:T].cpu().numpy(), r_eager)
        np.testing.assert_array_equal(bits(dev.out[:T]), o_eager)
    dev.reset()
    r_dev, out_bits = dev.run("single")  # eager again after the replays
    np.testing.assert_array_equal(r_dev, r_eager)
    np.testing.assert_array_equal(out_bits, o_eager)


@pytest.mark.parametrize("split", [1, 2])
def test_single_launch_epoch_wrap(monkeypatch, split):
    """The launch that takes the last 32-bit epoch clears every epoch-tagged word and restarts
    the count: that call and the two after it (epochs 1 and 2, whose tags stale words from
    before the wrap could otherwise carry) are correct."""
    if split == 2:
        _force_single(monkeypatch, "256x256", 8, 1, 2)
    d = synth.make_custom(600, 512, 1024, seed=41)
    dev = Device(d)
    dev.run("single")
    for k in range(3):
        if k == 0:
            monkeypatch.setenv("PR_DEBUG_EPOCH", str(2 ** 32 - 2))
        dev.reset()
        r_dev, out_bits = dev.run("single")
        _check(d, r_dev, out_bits, "fused")
        monkeypatch.delenv("PR_DEBUG_EPOCH", raising=False)
