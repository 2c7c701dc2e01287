"""CPU tests of the C ABI's host side: the library loads, exports every declared entry point,
validates arguments, decides the path per call, plans a race-free pipeline schedule, and
computes the token threshold.  No GPU is touched (only host-only entry points are called)."""
import ctypes
import json
import os
import re

import pytest

import projection_residual_rmsnorm_amd as pr

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "proj_add_rmsnorm.h")
A = 1 << 20  # a fake, 16-byte aligned address for pointer arguments


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    for k in ("PR_MICROCHUNK_TOKENS", "PR_THRESHOLD_TOKENS", "PR_LOG", "PR_FORCE_TILE",
              "PR_FORCE_SPLIT", "PR_FORCE_WAVES", "PR_FORCE_STAGES", "PR_FORCE_KGROUPS",
              "PR_FORCE_CU_SPLIT"):
        monkeypatch.delenv(k, raising=False)
    pr.pr_clear_tuning()
    yield
    pr.pr_clear_tuning()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(
        r"^(?:int|void|const char\s*\*|const uint16_t\s*\*)\s*(\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "proj_add_rmsnorm" in names and "pr_tune" in names and len(names) >= 14
    lib = pr.library()
    for n in names:
        assert hasattr(lib, n), n
        assert n in pr.SIGNATURES, f"binding lacks {n}"
    assert pr.pr_version() == 1
    assert pr.pr_strerror(pr.PR_ERR_SHAPE) == "unsupported shape"


def test_phase_stamp_library_exports_the_same_abi():
    """The diagnostic build (in-kernel phase stamps) exports every declared entry point and the
    three stamp functions; the default library exports none of the latter.  Loaded in its own
    handle, without touching a GPU."""
    assert os.path.exists(pr.STAMPS_LIB_PATH), "build() makes both libraries"
    lib = ctypes.CDLL(pr.STAMPS_LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    layout = lib.pr_phase_stamps_layout
    layout.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    g, w = ctypes.c_int(), ctypes.c_int()
    assert layout(ctypes.byref(g), ctypes.byref(w)) == 0 and (g.value, w.value) == (4096, 12)
    for n in ("pr_phase_stamps_read", "pr_phase_stamps_clear"):
        assert hasattr(lib, n), n
    default = ctypes.CDLL(pr.LIB_PATH)
    for n in ("pr_phase_stamps_layout", "pr_phase_stamps_read", "pr_phase_stamps_clear"):
        assert not hasattr(default, n), n


def test_phase_summary_from_synthetic_stamps():
    """The phase table's arithmetic on stamps whose phases, clocks and XCDs are known."""
    import numpy as np
    from projection_residual_rmsnorm_amd import profiling
    n = 16
    a = np.zeros((n, 12), dtype=np.uint64)
    base = 10_000
    steps = [5000, 170, 340, 20, 450, 210, 480]  # 10 ns ticks: 50, 1.7, 3.4, ... µs
    for g in range(n):
        a[g, 0] = g % 8
        t = base + g  # starts 10 ns apart
        a[g, 1] = t
        for p, dt in enumerate(steps):
            t += dt + (g if p == 0 else 0)  # main loops differ by g ticks
            a[g, 2 + p] = t
        a[g, 10] = 1_000_000
        a[g, 11] = 1_000_000 + int(round(1650.0 * (steps[0] + g) / 100.0))  # 1650 MHz
    st = profiling.phase_stats(a, flops_per_group=2.0 * 256 * 128 * 4096)
    assert st["workgroups"] == n
    assert abs(st["phases_us"][0] - (5000 + 7.5) / 100) < 1e-9
    assert [round(v, 6) for v in st["phases_us"][1:]] == [d / 100 for d in steps[1:]]
    assert abs(st["clock_mhz"] - 1650.0) < 0.1
    assert abs(st["main_loop_end_spread_us"] - 2 * (n - 1) / 100) < 1e-9
    busy = 2.0 * 256 * 128 * 4096 / (4096 * 1650e6 * 50.075e-6)
    assert abs(st["mfma_busy_main_loop"] - busy) < 1e-3
    assert sorted(st["xcd"]) == list(range(8))
    text = profiling.phases_summary({"o_proj": {"shape": "T=2048, K=4096, H=4096",
                                                "config": "256x128 tiles", "trials": [st, st]}},
                                    "python bench.py --phases o_proj")
    assert "| main loop | 50.1 [50.1–50.1] |" in text and "1650" in text


def test_validate():
    ok = dict(x=A, W=A * 2, residual_inout=A * 3, norm_w=A * 4, eps=1e-5, T=64, K=512, H=512,
              microchunk=16, norm_kind=0, out=A * 5)
    assert pr.pr_validate(**ok) == 0
    bad = [
        (dict(K=100), pr.PR_ERR_SHAPE), (dict(H=96), pr.PR_ERR_SHAPE),
        (dict(T=-1), pr.PR_ERR_INVALID_ARG), (dict(K=0), pr.PR_ERR_INVALID_ARG),
        (dict(microchunk=4097), pr.PR_ERR_MICROCHUNK), (dict(microchunk=-5), pr.PR_ERR_MICROCHUNK),
        (dict(norm_kind=2), pr.PR_ERR_INVALID_ARG), (dict(eps=-1.0), pr.PR_ERR_INVALID_ARG),
        (dict(eps=float("nan")), pr.PR_ERR_INVALID_ARG), (dict(x=None), pr.PR_ERR_INVALID_ARG),
        (dict(out=A), pr.PR_ERR_INVALID_ARG), (dict(out=A * 3), pr.PR_ERR_INVALID_ARG),
        (dict(x=A + 2), pr.PR_ERR_INVALID_ARG), (dict(K=1 << 16, H=1 << 16), pr.PR_ERR_SHAPE),
        # partial overlaps (16-byte aligned): out inside the residual, residual inside x,
        # residual reaching into the weight, out covering the norm weight
        (dict(out=A * 3 + 64), pr.PR_ERR_INVALID_ARG),
        (dict(residual_inout=A + 1024), pr.PR_ERR_INVALID_ARG),
        (dict(residual_inout=A * 2 - 1024), pr.PR_ERR_INVALID_ARG),
        (dict(out=A * 4 - 1024), pr.PR_ERR_INVALID_ARG),
    ]
    for change, code in bad:
        args = dict(ok, **change)
        assert pr.pr_validate(**args) == code, change
    # T == 0 is a no-op: null pointers are accepted
    assert pr.pr_validate(None, None, None, None, 1e-5, 0, 512, 512, 16, 0, None) == 0
    # microchunk >= T is allowed (one chunk); out == NULL borrows the workspace
    assert pr.pr_validate(**dict(ok, microchunk=4096, out=None)) == 0


def test_validate_silu():
    """The fused SiluAndMul region reads gate_up, twice the bytes of x (4 T K): a residual
    placed in gate_up's upper half overlaps it, one placed beyond it does not."""
    T, K, H = 64, 512, 512
    ok = dict(gate_up=A, W=A * 2, residual_inout=A * 3, norm_w=A * 4, eps=1e-5, T=T, K=K, H=H,
              norm_kind=0, out=A * 5)
    assert pr.pr_validate_silu(**ok) == 0
    bad = [
        (dict(K=100), pr.PR_ERR_SHAPE), (dict(norm_kind=2), pr.PR_ERR_INVALID_ARG),
        (dict(gate_up=None), pr.PR_ERR_INVALID_ARG), (dict(gate_up=A + 8), pr.PR_ERR_INVALID_ARG),
        (dict(residual_inout=A + 2 * T * K), pr.PR_ERR_INVALID_ARG),   # inside the up half
        (dict(out=A * 2 + 1024), pr.PR_ERR_INVALID_ARG),               # inside the weight
        (dict(eps=float("inf")), pr.PR_ERR_INVALID_ARG),
    ]
    for change, code in bad:
        assert pr.pr_validate_silu(**dict(ok, **change)) == code, change
    assert pr.pr_validate_silu(**dict(ok, residual_inout=A + 4 * T * K)) == 0  # just past it
    assert pr.pr_validate_silu(None, None, None, None, 1e-5, 0, K, H, 0, None) == 0


def test_validate_fp8():
    """One byte per element for x_q and W_q; the scale pointers are checked for NULL, 4-byte
    alignment and overlap with the written buffers; scale_rows >= 1."""
    T, K, H = 64, 512, 512
    ok = dict(x_q=A, x_scales=A * 6, scale_rows=16, W_q=A * 2, w_scale=A * 7,
              residual_inout=A * 3, norm_w=A * 4, eps=1e-5, T=T, K=K, H=H, norm_kind=0,
              out=A * 5)
    assert pr.pr_validate_fp8(**ok) == 0
    bad = [
        (dict(scale_rows=0), pr.PR_ERR_INVALID_ARG), (dict(x_scales=None), pr.PR_ERR_INVALID_ARG),
        (dict(w_scale=None), pr.PR_ERR_INVALID_ARG), (dict(x_scales=A * 6 + 2), pr.PR_ERR_INVALID_ARG),
        (dict(w_scale=A * 3 + 8), pr.PR_ERR_INVALID_ARG),      # scale inside the residual
        (dict(x_scales=A * 5 + 16), pr.PR_ERR_INVALID_ARG),    # scales inside the output
        (dict(residual_inout=A + T * K // 2), pr.PR_ERR_INVALID_ARG),  # inside x_q
        (dict(out=A * 2 + K * H // 2), pr.PR_ERR_INVALID_ARG),          # inside W_q
        (dict(K=96), pr.PR_ERR_SHAPE), (dict(T=-1), pr.PR_ERR_INVALID_ARG),
    ]
    for change, code in bad:
        assert pr.pr_validate_fp8(**dict(ok, **change)) == code, change
    # byte operands: a residual right after x_q's T*K bytes and an output right after W_q's
    # K*H bytes do not overlap them
    assert pr.pr_validate_fp8(**dict(ok, residual_inout=A + T * K)) == 0
    assert pr.pr_validate_fp8(**dict(ok, out=A * 2 + K * H)) == 0
    # the last of ceil(T / scale_rows) scales may not reach into the residual
    assert pr.pr_validate_fp8(**dict(ok, x_scales=A * 3 - 4 * (T // 16))) == 0
    assert pr.pr_validate_fp8(**dict(ok, x_scales=A * 3 - 4 * (T // 16) + 4)) == pr.PR_ERR_INVALID_ARG
    assert pr.pr_validate_fp8(None, None, 16, None, None, None, None, 1e-5, 0, K, H, 0, None) == 0


def test_select_explicit_and_unfused():
    d = pr.pr_select(3000, 16384, 3072, 256)
    assert d["path"] == pr.PR_PATH_FUSED and d["microchunk"] == 256
    assert d["n_chunks"] == 12 and d["last_valid"] == 184 and d["reason"] == 0
    d = pr.pr_select(3000, 16384, 3072, 1024)
    assert d["n_chunks"] == 3 and d["last_valid"] == 952
    d = pr.pr_select(64, 512, 512, 4096)  # microchunk >= T: one chunk
    assert d["n_chunks"] == 1 and d["last_valid"] == 64
    d = pr.pr_select(2048, 4096, 4096, -1)
    assert d["path"] == pr.PR_PATH_CONVENTIONAL and d["reason"] == 5
    with pytest.raises(pr.PRError):
        pr.pr_select(10, 64, 64, 5000)


@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (512, 4096, 4096), (2048, 4096, 4096),
                                   (4096, 4096, 14336), (3000, 3072, 16384), (128, 8192, 8192),
                                   (32768, 8192, 8192), (184, 3072, 16384)])
def test_tile_choice_is_valid(M, N, K):
    for mc in (-1, min(M, 4096)):
        d = pr.pr_select(M, K, N, mc if mc > 0 else -1)
        assert (d["gemm_bm"], d["gemm_bn"]) in ((256, 256), (256, 128), (128, 128))
        assert K % (64 * d["split_k"]) == 0 and d["split_k"] >= 1


def test_forced_projection_config(monkeypatch):
    """Debug overrides of the projection configuration are validated on the host."""
    monkeypatch.setenv("PR_FORCE_TILE", "128x128")
    monkeypatch.setenv("PR_FORCE_SPLIT", "2")
    monkeypatch.setenv("PR_FORCE_WAVES", "4")
    d = pr.pr_select(512, 4096, 4096, 512)
    assert (d["gemm_bm"], d["gemm_bn"], d["split_k"], d["gemm_waves"]) == (128, 128, 2, 4)
    for name, bad in (("PR_FORCE_TILE", "64x64"), ("PR_FORCE_SPLIT", "3"),
                      ("PR_FORCE_WAVES", "6"), ("PR_FORCE_STAGES", "1"),
                      ("PR_FORCE_STAGES", "9")):
        monkeypatch.setenv(name, bad)
        with pytest.raises(pr.PRError):
            pr.pr_select(512, 4096, 4096, 512)
        monkeypatch.delenv(name)
        if name != "PR_FORCE_STAGES":
            monkeypatch.setenv(name, {"PR_FORCE_TILE": "128x128", "PR_FORCE_SPLIT": "2",
                                      "PR_FORCE_WAVES": "4"}[name])
    monkeypatch.setenv("PR_FORCE_STAGES", "6")  # an instantiated depth of the 128x128 tile
    d = pr.pr_select(512, 4096, 4096, 512)
    assert d["gemm_bm"] == 128 and d["gemm_stages"] == 6


def test_chunk_config_table(monkeypatch):
    """A tuned chunk configuration applies to fused calls of its group and chunk size only;
    clearing the tuning removes it; forced overrides still win."""
    base = pr.pr_select(2048, 4096, 4096, 512)
    pr.pr_set_chunk_config(4096, 4096, 512, 256, 256, 4, 4)
    d = pr.pr_select(2048, 4096, 4096, 512)
    assert (d["gemm_bm"], d["gemm_bn"], d["split_k"], d["gemm_waves"]) == (256, 256, 4, 4)
    assert pr.pr_select(2048, 4096, 4096, 256)["gemm_waves"] == 8  # another chunk size: model
    conv = pr.pr_select(2048, 4096, 4096, -1)        # conventional: the model
    assert conv["gemm_waves"] == 8
    assert pr.pr_select(2048, 4096, 8192, 512)["gemm_waves"] == 8   # another group
    monkeypatch.setenv("PR_FORCE_WAVES", "8")
    assert pr.pr_select(2048, 4096, 4096, 512)["gemm_waves"] == 8
    monkeypatch.delenv("PR_FORCE_WAVES")
    pr.pr_clear_tuning()
    assert pr.pr_select(2048, 4096, 4096, 512) == base
    for args, code in (((4096, 4096, 512, 64, 64, 1, 8), pr.PR_ERR_INVALID_ARG),
                       ((4096, 4096, 512, 256, 256, 3, 8), pr.PR_ERR_INVALID_ARG),
                       ((4096, 4096, 512, 256, 256, 1, 6), pr.PR_ERR_INVALID_ARG),
                       ((4096, 4096, 5000, 256, 256, 1, 8), pr.PR_ERR_MICROCHUNK),
                       ((4000, 4096, 512, 256, 256, 1, 8), pr.PR_ERR_SHAPE)):
        with pytest.raises(pr.PRError) as e:
            pr.pr_set_chunk_config(*args)
        assert e.value.code == code, args


def test_select_single_launch():
    d = pr.pr_select(2048, 4096, 4096, pr.PR_SINGLE_LAUNCH)
    assert d["path"] == pr.PR_PATH_SINGLE and d["reason"] == 6
    assert (d["microchunk"], d["n_chunks"], d["last_valid"]) == (2048, 1, 2048)
    assert d["split_k"] == 1 and 4096 % d["gemm_bn"] == 0
    # one round of 256 x 128 tiles (8 x 32 = 256 workgroups) runs with 8 waves in 2 K groups
    assert (d["gemm_bm"], d["gemm_bn"], d["gemm_waves"], d["gemm_kgroups"]) == (256, 128, 8, 2)
    # a forced tile or wave count takes the one-group form unless K groups are forced too
    for T, K, H in [(4096, 14336, 4096), (3000, 16384, 3072), (32768, 8192, 8192), (1, 512, 512)]:
        d = pr.pr_select(T, K, H, pr.PR_SINGLE_LAUNCH)
        assert d["path"] == pr.PR_PATH_SINGLE
        assert H % d["gemm_bn"] == 0 and H // d["gemm_bn"] <= 64
        assert d["gemm_waves"] in (4, 8) or (d["gemm_bm"], d["gemm_bn"], d["gemm_waves"]) == (
            192, 192, 12)
    # 3000 x 3072: 144 tiles of 256 x 256 would leave 112 CUs idle; 16 x 16 tiles of 192 x 192
    # with 12 waves fill the GPU in one round
    d = pr.pr_select(3000, 16384, 3072, pr.PR_SINGLE_LAUNCH)
    assert (d["gemm_bm"], d["gemm_bn"], d["gemm_waves"], d["gemm_kgroups"]) == (192, 192, 12, 1)
    # a width only the 192-column tile divides (H = 576) is accepted
    assert pr.pr_select(1000, 4096, 576, pr.PR_SINGLE_LAUNCH)["gemm_bn"] == 192
    with pytest.MonkeyPatch.context() as mp:
        mp.setenv("PR_FORCE_WAVES", "4")
        d = pr.pr_select(2048, 4096, 4096, pr.PR_SINGLE_LAUNCH)
        assert (d["gemm_waves"], d["gemm_kgroups"]) == (4, 1)
        mp.setenv("PR_FORCE_WAVES", "8")
        mp.setenv("PR_FORCE_KGROUPS", "2")
        assert pr.pr_select(2048, 4096, 4096, pr.PR_SINGLE_LAUNCH)["gemm_kgroups"] == 2
    with pytest.raises(pr.PRError) as e:  # no tile's columns divide H = 320
        pr.pr_select(64, 256, 320, pr.PR_SINGLE_LAUNCH)
    assert e.value.code == pr.PR_ERR_SHAPE
    with pytest.raises(pr.PRError) as e:
        pr.pr_select(64, 256, 256, -3)
    assert e.value.code == pr.PR_ERR_MICROCHUNK


def test_auto_untuned_and_overrides(monkeypatch):
    d = pr.pr_select(2048, 4096, 4096, 0)
    assert d["path"] == pr.PR_PATH_CONVENTIONAL and pr.REASON_NAMES[d["reason"]] == "untuned"
    monkeypatch.setenv("PR_MICROCHUNK_TOKENS", "512")
    monkeypatch.setenv("PR_THRESHOLD_TOKENS", "1024")
    d = pr.pr_select(2048, 4096, 4096, 0)
    assert d["path"] == pr.PR_PATH_FUSED and d["microchunk"] == 512
    d = pr.pr_select(1000, 4096, 4096, 0)
    assert d["path"] == pr.PR_PATH_CONVENTIONAL and d["reason"] == 2
    monkeypatch.setenv("PR_MICROCHUNK_TOKENS", "9000")
    with pytest.raises(pr.PRError) as e:
        pr.pr_select(2048, 4096, 4096, 0)
    assert e.value.code == pr.PR_ERR_MICROCHUNK
    monkeypatch.setenv("PR_MICROCHUNK_TOKENS", "abc")
    with pytest.raises(pr.PRError):
        pr.pr_select(2048, 4096, 4096, 0)


def test_auto_tuned(monkeypatch):
    pr.pr_set_tuning(4096, 4096, 2048, 32768, [128, 512, 2048, 8192, 32768],
                     [128, 512, 512, 1024, 2048])
    d = pr.pr_select(1024, 4096, 4096, 0)
    assert d["path"] == pr.PR_PATH_CONVENTIONAL and d["reason"] == 2
    d = pr.pr_select(2048, 4096, 4096, 0)
    assert d["path"] == pr.PR_PATH_FUSED and d["microchunk"] == 512
    d = pr.pr_select(9000, 4096, 4096, 0)  # between grid points: lower grid point's choice
    assert d["microchunk"] == 1024
    with pytest.raises(pr.PRError) as e:  # above the profiled token maximum
        pr.pr_select(40000, 4096, 4096, 0)
    assert e.value.code == pr.PR_ERR_UNSUPPORTED
    # an explicit microchunk ignores the tuning entirely
    assert pr.pr_select(40000, 4096, 4096, 256)["path"] == pr.PR_PATH_FUSED
    # a single override replaces its tuned value
    monkeypatch.setenv("PR_THRESHOLD_TOKENS", "100")
    assert pr.pr_select(1024, 4096, 4096, 0)["path"] == pr.PR_PATH_FUSED
    monkeypatch.delenv("PR_THRESHOLD_TOKENS")
    monkeypatch.setenv("PR_MICROCHUNK_TOKENS", "256")
    assert pr.pr_select(8192, 4096, 4096, 0)["microchunk"] == 256
    monkeypatch.delenv("PR_MICROCHUNK_TOKENS")
    # inconclusive tuning keeps the conventional path
    # the single launch as the tuned fused form of a grid range
    pr.pr_set_tuning(4096, 4096, 512, 32768, [128, 512, 2048], [128, 256, pr.PR_SINGLE_LAUNCH])
    assert pr.pr_select(1024, 4096, 4096, 0)["microchunk"] == 256
    d = pr.pr_select(2048, 4096, 4096, 0)
    assert d["path"] == pr.PR_PATH_SINGLE and d["reason"] == 1  # above threshold
    assert pr.pr_select(256, 4096, 4096, 0)["path"] == pr.PR_PATH_CONVENTIONAL
    with pytest.raises(pr.PRError):
        pr.pr_set_tuning(64, 64, 1, 10, [4], [-3])
    pr.pr_set_tuning(8192, 8192, pr.INT32_MAX, 32768, [128], [128])
    d = pr.pr_select(4096, 8192, 8192, 0)
    assert d["path"] == pr.PR_PATH_CONVENTIONAL and pr.REASON_NAMES[d["reason"]] == "inconclusive"
    with pytest.raises(pr.PRError):
        pr.pr_set_tuning(64, 64, 1, 10, [4, 2], [1, 1])  # grid must ascend


def _simulate(calls):
    """Vector-clock happens-before over the planned enqueue order of one or more calls.

    `calls` is a list of (plan, caller_stream_name).  Streams execute in order; a record
    snapshots the stream's clock into the event; a wait joins the most recent record of that
    event at enqueue time (HIP semantics).  WAIT_PREV, for a call on a different caller stream,
    joins the previous call's last done record on each stream.  Returns per call the clock of
    every GEMM / ADDNORM, keyed by (kind, chunk), and the caller's clock after the call.
    """
    clocks = {}
    events = {}
    counter = [0]
    out = []
    prev = None  # (caller name, {stream id: last done event key})

    def tick(s, label):
        counter[0] += 1
        c = dict(clocks.get(s, {}))
        c[label] = counter[0]
        clocks[s] = c
        return c

    for k, (ops, caller) in enumerate(calls):
        names = {0: caller, 1: "library", 2: "library_addnorm"}
        tick(caller, ("caller_pre", k))
        stamps = {}
        last_done = {}
        for name, stream, chunk, slot, rows in ops:
            sn = names[stream]
            if name == "WAIT_PREV":
                if prev is not None and prev[0] != caller:
                    for ev in prev[1].values():
                        clocks[caller] = {**clocks.get(caller, {}), **events[ev]}
            elif name == "RECORD_ENTRY":
                events["entry"] = dict(clocks.get(sn, {}))
            elif name == "WAIT_ENTRY":
                clocks[sn] = {**clocks.get(sn, {}), **events["entry"]}
            elif name in ("GEMM", "ADDNORM"):
                stamps[(name, chunk)] = (tick(sn, (name, chunk, k)), slot, rows, stream)
            elif name == "RECORD_DONE":
                events[("done", slot)] = dict(clocks.get(sn, {}))
                last_done[stream] = ("done", slot)
            elif name == "WAIT_DONE":
                clocks[sn] = {**clocks.get(sn, {}), **events[("done", slot)]}
            elif name == "RECORD_READY":
                events[("ready", slot)] = dict(clocks.get(sn, {}))
            elif name == "WAIT_READY":
                clocks[sn] = {**clocks.get(sn, {}), **events[("ready", slot)]}
            elif name == "JOIN":
                clocks[sn] = {**clocks.get(sn, {}), **events[("done", slot)]}
            else:
                raise AssertionError(name)
        out.append((stamps, dict(clocks.get(caller, {}))))
        prev = (caller, last_done)
    return out


@pytest.mark.parametrize("T,mc", [(64, 16), (3000, 256), (3000, 1024), (2048, 512), (7, 7),
                                  (1, 4096), (10, 3), (4096, 4096), (5000, 512)])
def test_plan_is_race_free(T, mc):
    ops = pr.pr_plan(T, mc)
    nc = -(-T // mc)
    gemms = [o for o in ops if o[0] == "GEMM"]
    norms = [o for o in ops if o[0] == "ADDNORM"]
    assert len(gemms) == nc and len(norms) == nc
    assert sum(o[4] for o in norms) == T                 # valid rows only, each once
    assert all(o[4] == mc for o in norms[:-1]) and norms[-1][4] == T - (nc - 1) * mc
    assert {o[3] for o in ops if o[3] >= 0} <= {0, 1, 2}  # three reusable slots
    (st, caller_end), = _simulate([(ops, "caller")])
    for c in range(nc):
        g, a = ("GEMM", c, 0), ("ADDNORM", c, 0)
        assert g in st[("ADDNORM", c)][0]                    # slot written before it is read
        if c + 3 < nc:                                       # slot reused only after its read
            assert a in st[("GEMM", c + 3)][0]
        assert a in caller_end                               # caller waits for every chunk
        assert ("caller_pre", 0) in st[("GEMM", c)][0]       # nothing starts before entry
        assert st[("GEMM", c)][1] == c % 3
    # overlap is possible: chunk c+1's projection does not wait for chunk c's add/norm
    for c in range(nc - 1):
        assert ("ADDNORM", c, 0) not in st[("GEMM", c + 1)][0]


@pytest.mark.parametrize("T1,mc1,T2,mc2", [(2048, 512, 2048, 512), (3000, 256, 700, 128),
                                           (10, 3, 7, 2), (512, 512, 2048, 256)])
@pytest.mark.parametrize("same_stream", [True, False])
def test_consecutive_calls_are_ordered(T1, mc1, T2, mc2, same_stream):
    """A second call, on the same or on another caller stream, starts each chunk only after
    every chunk of the first call has finished (they share slots, rows and the residual)."""
    first, second = pr.pr_plan(T1, mc1), pr.pr_plan(T2, mc2)
    (st1, end1), (st2, _) = _simulate([(first, "s1"), (second, "s1" if same_stream else "s2")])
    nc1, nc2 = -(-T1 // mc1), -(-T2 // mc2)
    for c2 in range(nc2):
        for c1 in range(nc1):
            assert ("ADDNORM", c1, 0) in st2[("GEMM", c2)][0], (c1, c2)


@pytest.mark.parametrize("T,mc", [(64, 16), (3000, 256), (2048, 512), (7, 7), (1, 4096),
                                  (10, 3), (4096, 1024), (5000, 512)])
def test_cu_split_plan_is_race_free(T, mc):
    """The CU-partitioned schedule: every projection on stream 1, every add/norm on stream 2;
    a chunk's add/norm reads its slot only after the projection wrote it, a slot is rewritten
    only after the add/norm three chunks earlier read it, the caller waits for every chunk,
    nothing starts before the call's entry, and the next chunk's projection does not wait for
    the previous chunk's add/norm (they can co-run on their disjoint CUs)."""
    ops = pr.pr_plan_cu_split(T, mc)
    nc = -(-T // mc)
    gemms = [o for o in ops if o[0] == "GEMM"]
    norms = [o for o in ops if o[0] == "ADDNORM"]
    assert len(gemms) == nc and len(norms) == nc
    assert all(o[1] == 1 for o in gemms) and all(o[1] == 2 for o in norms)
    assert sum(o[4] for o in norms) == T and norms[-1][4] == T - (nc - 1) * mc
    (st, caller_end), = _simulate([(ops, "caller")])
    for c in range(nc):
        assert ("GEMM", c, 0) in st[("ADDNORM", c)][0]
        if c + 3 < nc:
            assert ("ADDNORM", c, 0) in st[("GEMM", c + 3)][0]
        assert ("ADDNORM", c, 0) in caller_end
        assert ("caller_pre", 0) in st[("GEMM", c)][0]
        assert ("caller_pre", 0) in st[("ADDNORM", c)][0]
    for c in range(nc - 1):
        assert ("ADDNORM", c, 0) not in st[("GEMM", c + 1)][0]


@pytest.mark.parametrize("first,second", [("split", "split"), ("split", "pingpong"),
                                          ("pingpong", "split")])
@pytest.mark.parametrize("same_stream", [True, False])
def test_consecutive_calls_across_schedules_are_ordered(first, second, same_stream):
    """Calls alternating between the two schedules share slots, rows and the residual: every
    chunk of the second starts after every chunk of the first."""
    plan = {"split": pr.pr_plan_cu_split, "pingpong": pr.pr_plan}
    a, b = plan[first](3000, 256), plan[second](700, 128)
    (st1, _), (st2, _) = _simulate([(a, "s1"), (b, "s1" if same_stream else "s2")])
    for c2 in range(-(-700 // 128)):
        for c1 in range(-(-3000 // 256)):
            assert ("ADDNORM", c1, 0) in st2[("GEMM", c2)][0], (c1, c2)


def test_cu_split_plan_detects_a_missing_ready_wait():
    ops = [o for o in pr.pr_plan_cu_split(2048, 256) if o[0] != "WAIT_READY"]
    (st, _), = _simulate([(ops, "caller")])
    assert not all(("GEMM", c, 0) in st[("ADDNORM", c)][0] for c in range(8))


def test_cu_split_setting_and_decision(monkeypatch):
    monkeypatch.delenv("PR_FORCE_CU_SPLIT", raising=False)
    assert pr.pr_select(2048, 4096, 4096, 512)["addnorm_cus"] == 0
    pr.pr_set_cu_split(4096, 4096, 512, 32)
    d = pr.pr_select(2048, 4096, 4096, 512)
    assert d["addnorm_cus"] == 32 and d["path"] == pr.PR_PATH_FUSED
    before = (d["gemm_bm"], d["gemm_bn"], d["split_k"])
    pr.pr_set_chunk_config(4096, 4096, 512, 128, 128, 2, 8)   # keeps the split
    d = pr.pr_select(2048, 4096, 4096, 512)
    assert d["addnorm_cus"] == 32 and (d["gemm_bm"], d["split_k"]) == (128, 2)
    assert pr.pr_select(2048, 4096, 4096, 256)["addnorm_cus"] == 0   # other chunk sizes
    assert pr.pr_select(2048, 4096, 4096, pr.PR_SELECT_UNFUSED)["addnorm_cus"] == 0
    for bad in (4, 7, 136, -8):
        with pytest.raises(pr.PRError):
            pr.pr_set_cu_split(4096, 4096, 512, bad)
    monkeypatch.setenv("PR_FORCE_CU_SPLIT", "64")
    assert pr.pr_select(2048, 4096, 4096, 256)["addnorm_cus"] == 64
    monkeypatch.setenv("PR_FORCE_CU_SPLIT", "12")
    with pytest.raises(pr.PRError):
        pr.pr_select(2048, 4096, 4096, 256)
    assert before[0] in (128, 256)


def test_cu_split_in_tuning_file(tmp_path):
    pr.pr_set_chunk_config(1024, 2048, 256, 128, 128, 2, 8)
    pr.pr_set_cu_split(1024, 2048, 256, 64)
    pr.pr_set_cu_split(1024, 2048, 512, 16)   # no chunk record: the model's tile
    path = tmp_path / "t.txt"
    pr.pr_tuning_save(str(path), "dev:1")
    text = path.read_text()
    assert "cusplit 1024 2048 256 64" in text and "cusplit 1024 2048 512 16" in text
    pr.pr_clear_tuning()
    pr.pr_tuning_load(str(path), "dev:1")
    assert pr.pr_select(4096, 1024, 2048, 256)["addnorm_cus"] == 64
    assert pr.pr_select(4096, 1024, 2048, 256)["split_k"] == 2
    assert pr.pr_select(4096, 1024, 2048, 512)["addnorm_cus"] == 16
    path.write_text(text + "cusplit 1024 2048 256 12\n")
    with pytest.raises(pr.PRError):
        pr.pr_tuning_load(str(path), "dev:1")
    assert pr.pr_select(4096, 1024, 2048, 256)["addnorm_cus"] == 64   # load is all-or-nothing


def test_plan_detects_a_missing_wait():
    """The simulator itself catches a schedule without the slot-reuse wait."""
    full = pr.pr_plan(3000, 256)
    ops = [o for o in full if o[0] != "WAIT_DONE"]
    (st, _), = _simulate([(ops, "caller")])
    assert not all(("ADDNORM", c, 0) in st[("GEMM", c + 3)][0] for c in range(9))
    # done records: 9 for reuse (chunks 0..8), plus the last chunk on each stream (10, 11)
    assert sum(o[0] == "RECORD_DONE" for o in full) == 11


def test_plan_edge_cases():
    assert pr.pr_plan(0, 16) == []
    with pytest.raises(pr.PRError):
        pr.pr_plan(10, 0)
    with pytest.raises(pr.PRError):
        pr.pr_plan(10, 4097)


def test_threshold_from_timings():
    T = [128, 512, 2048, 8192, 32768]
    conv = [[1.0, 2.0, 4.0, 8.0, 16.0]]
    # fused wins from 2048 upward by more than 2 %
    fused = [[1.5, 2.5, 3.5, 7.0, 14.0]]
    assert pr.pr_threshold_from_timings(T, conv, fused) == 2048
    # a win inside the noise margin does not count
    fused2 = [[1.5, 2.5, 3.95, 7.0, 14.0]]
    assert pr.pr_threshold_from_timings(T, conv, fused2) == 8192
    # large spread suppresses a small win
    assert pr.pr_threshold_from_timings(T, conv, fused, spread=[[0, 0, 0, 0, 3.0]]) \
        == pr.INT32_MAX
    # a loss at the top of the grid: no range where fused keeps winning -> inconclusive
    fused3 = [[0.5, 0.5, 0.5, 0.5, 20.0]]
    assert pr.pr_threshold_from_timings(T, conv, fused3) == pr.INT32_MAX
    # groups are summed: one group's loss can outweigh the other's win
    conv2 = [[1, 1, 1, 1, 1], [1, 1, 1, 1, 1]]
    fused4 = [[0.5, 0.5, 0.5, 0.5, 0.5], [2, 2, 1.6, 1.6, 1.6]]
    assert pr.pr_threshold_from_timings(T, conv2, fused4) == pr.INT32_MAX
    fused5 = [[0.5, 0.5, 0.5, 0.5, 0.5], [2, 2, 1.2, 1.2, 1.0]]
    assert pr.pr_threshold_from_timings(T, conv2, fused5) == 2048
    # a rejected candidate (no fused time) is never profitable
    assert pr.pr_threshold_from_timings([1, 2], [[1, 1]], [[0.1, -1]]) == pr.INT32_MAX
    with pytest.raises(pr.PRError):
        pr.pr_threshold_from_timings([2, 1], [[1, 1]], [[1, 1]])


def test_calls_without_gpu_fail_cleanly():
    """On a machine without a GPU the device entry points report an error, never crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = pr.library().proj_add_rmsnorm(A, A * 2, A * 3, A * 4, 1e-5, 64, 512, 512, 16, 0,
                                       A * 5, None)
    assert rc in (pr.PR_ERR_HIP, pr.PR_ERR_UNSUPPORTED)
    assert pr.pr_last_error() != ""
    # a T == 0 call is a no-op that still needs a device context
    rc = pr.library().proj_add_rmsnorm(None, None, None, None, 1e-5, 0, 512, 512, 16, 0, None,
                                       None)
    assert rc in (0, pr.PR_ERR_HIP, pr.PR_ERR_UNSUPPORTED)


def test_silu_mul_validates_before_touching_a_device():
    """pr_silu_mul checks shape, alignment and overlap on the host, before any device call;
    valid arguments without a GPU report an error rather than crash."""
    lib = pr.library()
    g, x = A, A + (1 << 24)
    assert lib.pr_silu_mul(g, x, 4, 96, None) == pr.PR_ERR_SHAPE       # K % 64 != 0
    assert lib.pr_silu_mul(g, x, -1, 64, None) == pr.PR_ERR_SHAPE      # T < 0
    assert lib.pr_silu_mul(g, x, 4, 0, None) == pr.PR_ERR_SHAPE        # K == 0
    assert lib.pr_silu_mul(None, x, 4, 64, None) == pr.PR_ERR_INVALID_ARG
    assert lib.pr_silu_mul(g + 8, x, 4, 64, None) == pr.PR_ERR_INVALID_ARG  # misaligned
    assert lib.pr_silu_mul(g, g + 256, 4, 64, None) == pr.PR_ERR_INVALID_ARG  # x in gate_up
    assert lib.pr_silu_mul(None, None, 0, 64, None) == 0                # T == 0: no-op
    import torch
    if torch.cuda.is_available():
        return  # the calls below pass validation and would launch on the fake addresses
    # adjacent buffers pass the overlap check; with no device the call then fails cleanly
    assert lib.pr_silu_mul(g, g + 1024, 4, 64, None) in (pr.PR_ERR_HIP, pr.PR_ERR_UNSUPPORTED)
    assert lib.pr_silu_mul(g, x, 4, 64, None) in (pr.PR_ERR_HIP, pr.PR_ERR_UNSUPPORTED)


def test_binding_rejects_strided_or_short_tensors():
    """The binding hands the library raw addresses: tensors must be contiguous and hold the
    extent the shape arguments describe (checked before the library is reached)."""
    import torch
    T, K, H = 8, 64, 64
    x = torch.zeros((T, K), dtype=torch.int16)
    W = torch.zeros(K * H, dtype=torch.int16)
    r = torch.zeros((T, H), dtype=torch.float32)
    w = torch.zeros(H, dtype=torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        pr.proj_add_rmsnorm(x.t(), W, r, w, 1e-5, T, K, H, 4)
    with pytest.raises(ValueError, match="residual_inout"):
        pr.proj_add_rmsnorm(x, W, r[: T - 1], w, 1e-5, T, K, H, 4)
    with pytest.raises(ValueError, match="W"):
        pr.proj_add_rmsnorm_unfused(x, W[:-1], r, w, 1e-5, T, K, H)
    with pytest.raises(ValueError, match="W_prep"):
        pr.pr_prepare_weight(W, pr.PR_WEIGHT_OUT_IN, W[: K * H // 2], K, H)


def test_traffic_digest_ignores_comments_only(tmp_path):
    """Counter summaries stay valid across comment edits of the kernel source and are void
    after any code change."""
    from projection_residual_rmsnorm_amd.profiling import source_digest
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text('int f(int x) {  // add one\n  return x + 1; /* done */ }\nconst char* s = "//";\n')
    b.write_text('// header\nint f(int x) {\n  return x + 1;\n}\nconst char* s = "//";\n')
    c.write_text('int f(int x) { return x + 2; }\nconst char* s = "//";\n')
    assert source_digest(str(a)) == source_digest(str(b))
    assert source_digest(str(a)) != source_digest(str(c))


def test_traffic_digest_ignores_phase_stamps(tmp_path):
    """The diagnostic phase stamps (PR_PHASE_STAMPS blocks, nested #ifs included, and the
    PR_PHASE(n) statements), which the default library does not compile, leave the digest
    unchanged; code outside them still counts."""
    from projection_residual_rmsnorm_amd.profiling import source_digest
    plain = "int f(int x) {\n  int y = x + 1;\n  return y;\n}\n"
    stamped = ("#ifdef PR_PHASE_STAMPS\n__device__ int s[4];\n#if 1\nint g();\n#endif\n"
               "#define PR_PHASE(p) g()\n#else\n#define PR_PHASE(p) ((void)0)\n#endif\n"
               "int f(int x) {\n  PR_PHASE(0);\n  int y = x + 1;\n  PR_PHASE(12);\n"
               "  return y;\n}\n")
    changed = stamped.replace("x + 1", "x + 2")
    paths = []
    for i, text in enumerate((plain, stamped, changed)):
        paths.append(tmp_path / f"{i}.hip")
        paths[-1].write_text(text)
    assert source_digest(str(paths[0])) == source_digest(str(paths[1]))
    assert source_digest(str(paths[0])) != source_digest(str(paths[2]))


def test_counter_summary_derivations(tmp_path):
    """Per-dispatch means and the derived MFMA / LDS ratios of a counter file (rocprofv3's
    counter_collection.csv layout: one row per dispatch and counter)."""
    from projection_residual_rmsnorm_amd.profiling import counter_table, derived
    path = tmp_path / "c.csv"
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
    lines = [",".join(cols)]
    # two dispatches of one kernel, 100 us each; busy = half of 1024 SIMDs x 100 us x 2.4 GHz
    for disp in (1, 2):
        for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * 100e3 * 2.4),
                     ("GRBM_GUI_ACTIVE", 8 * 100e3 * 2.0),
                     ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6),
                     ("SQ_LDS_IDX_ACTIVE", 256 * 1000.0), ("SQ_LDS_BANK_CONFLICT", 256 * 250.0)):
            lines.append(f'{disp},65536,"void pr::gemm_add_rmsnorm_kernel<256, 128, 4, 2, 2, 1>(x)",'
                         f'{c},{v},1000,{1000 + 100_000}')
    lines.append('3,256,"void pr::fill_nan_kernel(x)",GRBM_GUI_ACTIVE,5,0,10')
    path.write_text("\n".join(lines) + "\n")
    tab = counter_table(str(path), ["gemm_add_rmsnorm_kernel"])
    t = tab["gemm_add_rmsnorm_kernel"]
    assert t["dispatches"] == 2
    dv = derived(t["mean"])
    assert abs(dv["duration_us"] - 100.0) < 1e-9
    # GRBM_GUI_ACTIVE spans the counter window, not the dispatch: no clock is derived from it,
    # and the MFMA busy sum (flops / 1024 for bf16) is not restated as a utilisation
    assert not any("gui" in k or "nameplate" in k for k in dv), dv
    assert dv["mfma_bf16_flops"] == 512e6
    assert abs(dv["lds_bank_conflict_frac"] - 0.25) < 1e-12
    assert counter_table(str(path), ["gemm_add_rmsnorm_kernel"], grid=256) == {}
    # shader clock bounds over the 32 shader engines: SQ_BUSY_CYCLES (cycles with waves
    # present) 1.5 GHz for 100 us, SQ_CYCLES (the counter window) 2.0 GHz
    dv = derived({**t["mean"], "SQ_BUSY_CYCLES": 32 * 100e3 * 1.5,
                  "SQ_CYCLES": 32 * 100e3 * 2.0})
    assert abs(dv["shader_clock_GHz_busy"] - 1.5) < 1e-9
    assert abs(dv["shader_clock_GHz_cycles"] - 2.0) < 1e-9
    assert abs(dv["mfma_util_at_busy_clock"] - 0.8) < 1e-9  # 0.5 of 2.4 GHz = 0.8 of 1.5
    # L1 -> L2 reads: 64-byte requests, mean latency, pending-stall cycles per CU
    dv = derived({**t["mean"], "TCP_TCC_READ_REQ_sum": 1e6, "TCP_TCC_READ_REQ_LATENCY_sum": 5e8,
                  "TCP_PENDING_STALL_CYCLES_sum": 256 * 7e4})
    assert dv["l1_l2_read_MB_at_64B"] == 64.0
    assert dv["l1_l2_read_latency_cycles"] == 500.0
    assert dv["l1_pending_stall_cycles_per_cu"] == 7e4


def test_last_pass_and_bench_line(tmp_path):
    """The last-pass figure takes the last n dispatches of the kernel in dispatch order (not
    file order), and the bench figure comes from the JSON line of the profiled program."""
    from projection_residual_rmsnorm_amd.profiling import bench_line_lines, last_dispatches
    trace = tmp_path / "t.csv"
    lines = ["Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp"]
    durs = {1: 50, 2: 90, 5: 80, 3: 70, 4: 60, 6: 10}   # microseconds; 6 is another kernel
    for d, us in durs.items():
        k = "fill_nan_kernel" if d == 6 else "gemm_add_rmsnorm_kernel<256, 128, 4, 2, 2, 1>"
        lines.append(f'{d},"void pr::{k}(x)",1000,{1000 + us * 1000}')
    trace.write_text("\n".join(lines) + "\n")
    res = last_dispatches(str(trace), "gemm_add_rmsnorm_kernel<256, 128", 3)
    assert (res["mean_us"], res["min_us"], res["max_us"]) == (70.0, 60.0, 80.0)
    with pytest.raises(SystemExit):
        last_dispatches(str(trace), "gemm_add_rmsnorm_kernel", 6)
    log = tmp_path / "b.log"
    roof = {"kernel": "gemm_add_rmsnorm_kernel", "avg_launch_us": 81.25, "launches": 20,
            "achieved": 845.0, "unit": "TFLOP/s"}
    log.write_text("[bench] x\n" + json.dumps({"roofline": roof}) + "\n")
    text = "\n".join(bench_line_lines(str(log)))
    assert "81.25 us over 20" in text and "845.0 TFLOP/s" in text


def test_dispatch_runs(tmp_path):
    """Runs are consecutive dispatches in dispatch order; a count that does not match the
    labels is refused rather than silently regrouped."""
    from projection_residual_rmsnorm_amd.profiling import dispatch_runs
    trace = tmp_path / "t.csv"
    lines = ["Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp"]
    us = [10, 12, 11, 30, 31, 29]
    for d in (6, 5, 4, 3, 2, 1):   # file order reversed
        lines.append(f'{d},"void pr::add_rmsnorm_kernel<8, 2, true>(x)",0,{us[d - 1] * 1000}')
    lines.append('7,"void pr::fill_nan_kernel(x)",0,5000')
    trace.write_text("\n".join(lines) + "\n")
    runs = dispatch_runs(str(trace), "add_rmsnorm_kernel", 3, ["warm", "flushed"])
    assert [(r["label"], r["median_us"], r["min_us"], r["max_us"]) for r in runs] == [
        ("warm", 11.0, 10.0, 12.0), ("flushed", 30.0, 29.0, 31.0)]
    with pytest.raises(SystemExit):
        dispatch_runs(str(trace), "add_rmsnorm_kernel", 2, ["a", "b"])
    runs = dispatch_runs(str(trace), "add_rmsnorm_kernel", [2, 4], ["a", "b"])
    assert [(r["n"], r["median_us"]) for r in runs] == [(2, 11.0), (4, 29.5)]


# ------------------------------------------------------------------ tuning files
TUNE_KEY = "gfx950-test:256"


def _install_example_tuning():
    pr.pr_set_tuning(4096, 4096, 1024, 8192, [128, 1024, 4096], [128, 512, pr.PR_SINGLE_LAUNCH])
    pr.pr_set_tuning(8192, 8192, pr.INT32_MAX, 32768, [128, 32768], [512, 2048])  # inconclusive
    pr.pr_set_chunk_config(4096, 4096, 512, 128, 128, 2, 8)
    pr.pr_set_chunk_config(8192, 8192, 2048, 256, 256, 1, 4)


def _decisions():
    out = []
    for K, H in ((4096, 4096), (8192, 8192)):
        for T in (64, 128, 1000, 1024, 4000, 8192):
            for mc in (0, 512, 2048):
                out.append(pr.pr_select(T, K, H, mc))
    return out


def test_tuning_file_round_trip(tmp_path):
    """Saved tuning results and chunk configurations, reloaded after a clear, give the same
    decision for every call; a second save writes the same bytes."""
    pr.pr_clear_tuning()
    _install_example_tuning()
    before = _decisions()
    path = tmp_path / "tune.txt"
    pr.pr_tuning_save(str(path), TUNE_KEY)
    pr.pr_clear_tuning()
    assert pr.pr_select(2048, 4096, 4096, 0)["reason"] == pr.REASON_NAMES.index("untuned")
    pr.pr_tuning_load(str(path), TUNE_KEY)
    assert _decisions() == before
    again = tmp_path / "again.txt"
    pr.pr_tuning_save(str(again), TUNE_KEY)
    assert again.read_bytes() == path.read_bytes()
    pr.pr_clear_tuning()


@pytest.mark.parametrize("edit,code", [
    (lambda t: t.replace(f" {TUNE_KEY}", " gfx942:304"), pr.PR_ERR_UNSUPPORTED),   # device
    (lambda t: t.replace("pr_tuning 1 1 ", "pr_tuning 1 99 "), pr.PR_ERR_UNSUPPORTED),  # version
    (lambda t: t.replace("pr_tuning 1", "pr_tuning 2"), pr.PR_ERR_INVALID_ARG),      # format
    (lambda t: t + "chunk 4096 4096 256 100 128 1 8\n", pr.PR_ERR_INVALID_ARG),     # no such tile
    (lambda t: t + "chunk 4096 4096 256 128 128 3 8\n", pr.PR_ERR_INVALID_ARG),     # split
    (lambda t: t + "tuning 1024 1024 64 4096 1 64 5000\n", pr.PR_ERR_MICROCHUNK),   # chunk size
    (lambda t: t + "tuning 1024 1024 64 4096 2 64 64\n", pr.PR_ERR_INVALID_ARG),    # pair count
    (lambda t: t + "tuning 1024 1024 64 4096 2 512 64 64 64\n", pr.PR_ERR_INVALID_ARG),  # order
    (lambda t: t + "chunk 4096 4096 x 128 128 1 8\n", pr.PR_ERR_INVALID_ARG),       # not a number
    (lambda t: t + "grid 1 2 3\n", pr.PR_ERR_INVALID_ARG),                          # record kind
])
def test_tuning_file_refusals(tmp_path, edit, code):
    """A file of another device or library version is refused; a malformed or invalid record
    fails the whole load and leaves the installed tables as they were (its valid records,
    read before the bad one, are rolled back)."""
    pr.pr_clear_tuning()
    _install_example_tuning()
    path = tmp_path / "tune.txt"
    pr.pr_tuning_save(str(path), TUNE_KEY)
    pr.pr_clear_tuning()
    pr.pr_set_tuning(2048, 2048, 256, 4096, [256], [256])  # installed before the load
    kept = pr.pr_select(1000, 2048, 2048, 0)
    path.write_text(edit(path.read_text()))
    with pytest.raises(pr.PRError) as e:
        pr.pr_tuning_load(str(path), TUNE_KEY)
    assert e.value.code == code, pr.pr_last_error()
    assert pr.pr_select(2048, 4096, 4096, 0)["reason"] == pr.REASON_NAMES.index("untuned")
    assert pr.pr_select(1000, 2048, 2048, 0) == kept
    pr.pr_clear_tuning()


def test_tuning_file_needs_a_key_without_a_device(tmp_path):
    """Without a device the current-device key cannot be formed: the call fails cleanly (a
    caller-supplied key works, as above)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(pr.PRError):
        pr.pr_tuning_save(str(tmp_path / "t.txt"))
    with pytest.raises(pr.PRError):
        pr.pr_tuning_save(str(tmp_path / "t.txt"), "has space")
    with pytest.raises(pr.PRError):
        pr.pr_tuning_load(str(tmp_path / "missing.txt"), TUNE_KEY)
