"""The diagnostic library with in-kernel phase stamps (libprojaddnorm_stamps.so, the same sources
compiled with PR_PHASE_STAMPS): its single launch gives the default library's results bitwise,
and its stamps are ordered and give a shader clock within the chip's range.  The diagnostic
library is loaded through a ctypes handle of its own beside the default one; each keeps its own
workspaces and state."""
import ctypes

import numpy as np
import pytest
import torch

import projection_residual_rmsnorm_amd as pr
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import DEV, bits, f32, i16


@pytest.fixture(scope="module")
def stamps_lib():
    lib = ctypes.CDLL(pr.STAMPS_LIB_PATH)
    for name, (res, args) in pr.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    lib.pr_phase_stamps_read.restype = ctypes.c_int
    lib.pr_phase_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.pr_phase_stamps_clear.restype = ctypes.c_int
    lib.pr_phase_stamps_clear.argtypes = []
    assert lib.pr_init() == 0
    return lib


# o_proj's shape (one round of 256 x 128 tiles in two K groups), a ragged Gemma-norm shape, and
# a shape of four rounds of 256 x 256 tiles (only round 0 is stamped)
@pytest.mark.parametrize("T,K,H,kind", [(2048, 4096, 4096, 0), (700, 512, 1024, 1),
                                        (8192, 512, 8192, 0)])
def test_stamped_single_launch_matches_default(stamps_lib, T, K, H, kind):
    print(f"phase stamps: T={T} K={K} H={H} kind={kind}", flush=True)
    d = synth.make_custom(T, K, H, seed=31, norm_kind=kind, eps=1e-5)
    x = i16(d["x"])
    Wp = torch.empty(K * H, dtype=torch.int16, device=DEV)
    pr.pr_prepare_weight(i16(d["W"]), pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    w = f32(d["norm_w"])
    stream = torch.cuda.current_stream()

    r_def = f32(d["residual"])
    out_def = torch.empty((T, H), dtype=torch.int16, device=DEV)
    pr.proj_add_rmsnorm_single_launch(x, Wp, r_def, w, d["eps"], T, K, H, kind, out_def)
    assert pr.pr_device_status(stream) == 0

    assert stamps_lib.pr_phase_stamps_clear() == 0
    r_st = f32(d["residual"])
    out_st = torch.empty((T, H), dtype=torch.int16, device=DEV)
    torch.cuda.synchronize()
    rc = stamps_lib.proj_add_rmsnorm_single_launch(
        x.data_ptr(), Wp.data_ptr(), r_st.data_ptr(), w.data_ptr(), d["eps"], T, K, H, kind,
        out_st.data_ptr(), stream.cuda_stream)
    assert rc == 0
    status = ctypes.c_uint(0xFFFF)
    assert stamps_lib.pr_device_status(stream.cuda_stream, ctypes.byref(status)) == 0
    assert status.value == 0, f"status bits {status.value:#x}"
    a = np.zeros(4096 * 12, dtype=np.uint64)
    assert stamps_lib.pr_phase_stamps_read(a.ctypes.data, a.size) == 0  # synchronises
    torch.cuda.synchronize()

    np.testing.assert_array_equal(bits(out_st), bits(out_def))
    np.testing.assert_array_equal(r_st.cpu().numpy().view(np.uint32),
                                  r_def.cpu().numpy().view(np.uint32))

    a = a.reshape(4096, 12)
    stamped = a[a[:, 1] != 0]
    c = pr.pr_select(T, K, H, pr.PR_SINGLE_LAUNCH)
    tiles = -(-T // c["gemm_bm"]) * (H // c["gemm_bn"])
    assert 0 < stamped.shape[0] <= tiles
    assert np.all(stamped[:, 0] < 8)  # XCC ids
    rt = stamped[:, 1:9].astype(np.int64)
    assert np.all(rt > 0) and np.all(np.diff(rt, axis=1) >= 0), "phases out of order"
    main = (rt[:, 1] - rt[:, 0]) / 100.0  # µs
    clock = (stamped[:, 11].astype(np.int64) - stamped[:, 10].astype(np.int64)) / main
    assert np.all(main > 0)
    med = float(np.median(clock))
    print(f"  {stamped.shape[0]} workgroups, main loop {np.median(main):.1f} us at {med:.0f} MHz")
    assert 300.0 < med < 3000.0, med
