"""Thin Python binding of the MI355X projection -> residual add -> RMSNorm library.

Every function here marshals arguments and calls the C ABI declared in
include/proj_add_rmsnorm.h (same names); all computation runs in the HIP library.  Tensors may
be torch tensors (their device pointers are passed) or raw integer addresses.  A non-zero return
code raises PRError with the library's message.  The library must have been built
(``python -m projection_residual_rmsnorm_amd.build``); importing the binding without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libprojaddnorm.so")
# The diagnostic build: the same sources and ABI, with in-kernel phase and clock stamps of the
# single launch (and pr_phase_stamps_{layout,read,clear} to read them).  PR_PHASE_STAMPS=1 in
# the environment when the library is first used selects it.
STAMPS_LIB_PATH = os.path.join(_PKG_DIR, "libprojaddnorm_stamps.so")

PR_OK = 0
PR_ERR_INVALID_ARG = -1
PR_ERR_SHAPE = -2
PR_ERR_MICROCHUNK = -3
PR_ERR_UNSUPPORTED = -4
PR_ERR_NOMEM = -5
PR_ERR_HIP = -6

PR_NORM_STANDARD = 0
PR_NORM_GEMMA = 1
PR_WEIGHT_OUT_IN = 0
PR_WEIGHT_IN_OUT = 1
PR_MAX_MICROCHUNK = 4096
PR_PATH_CONVENTIONAL = 0
PR_PATH_FUSED = 1
PR_PATH_SINGLE = 2
PR_SELECT_UNFUSED = -1  # pr_select: the decision of proj_add_rmsnorm_unfused
PR_SINGLE_LAUNCH = -2   # chunk value of the single-launch path (pr_select, pr_set_tuning)
PR_NUM_SLOTS = 3
INT32_MAX = 2**31 - 1

OP_NAMES = ["RECORD_ENTRY", "WAIT_ENTRY", "WAIT_DONE", "GEMM", "ADDNORM", "RECORD_DONE", "JOIN",
            "WAIT_PREV", "RECORD_READY", "WAIT_READY"]
REASON_NAMES = ["explicit", "above_threshold", "below_threshold", "untuned", "inconclusive",
                "unfused_call", "single_call"]

# C signatures of every exported entry point (the header's declarations).
_c = ctypes
_vp, _i, _f, _d = _c.c_void_p, _c.c_int, _c.c_float, _c.c_double


class pr_decision(_c.Structure):
    _fields_ = [("path", _i), ("microchunk", _i), ("n_chunks", _i), ("last_valid", _i),
                ("gemm_bm", _i), ("gemm_bn", _i), ("split_k", _i), ("gemm_waves", _i),
                ("reason", _i), ("gemm_stages", _i), ("gemm_kgroups", _i),
                ("addnorm_cus", _i)]


class pr_plan_op(_c.Structure):
    _fields_ = [("op", _i), ("stream", _i), ("chunk", _i), ("slot", _i), ("rows", _i)]


class pr_tune_report(_c.Structure):
    _fields_ = [("threshold_tokens", _i), ("max_tokens", _i), ("n_checked", _i),
                ("n_rejected", _i)]


class pr_profile(_c.Structure):
    _fields_ = [("gemm_ms", _d), ("gemm_launches", _i), ("addnorm_ms", _d),
                ("addnorm_launches", _i)]


SIGNATURES = {
    "pr_profile_enable": (_i, [_i]),
    "pr_profile_read": (_i, [_c.POINTER(pr_profile)]),
    "pr_prepare_weight": (_i, [_vp, _i, _vp, _i, _i, _vp]),
    "pr_silu_mul": (_i, [_vp, _vp, _i, _i, _vp]),
    "proj_add_rmsnorm": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _i, _vp, _vp]),
    "proj_add_rmsnorm_unfused": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp, _vp]),
    "proj_add_rmsnorm_single_launch": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp, _vp]),
    "proj_add_rmsnorm_single_launch_noalloc": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp,
                                                   _vp]),
    "pr_init": (_i, []),
    "proj_add_rmsnorm_silu": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp, _vp]),
    "pr_validate_silu": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp]),
    "pr_project_partial": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "pr_add_rmsnorm_partials": (_i, [_vp, _i, _c.c_longlong, _vp, _vp, _f, _i, _i, _i, _vp,
                                     _vp]),
    "pr_quantize_fp8": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "pr_prepare_weight_fp8": (_i, [_vp, _i, _vp, _i, _i, _vp]),
    "proj_add_rmsnorm_fp8": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp,
                                  _vp]),
    "pr_validate_fp8": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _vp]),
    "pr_device_status": (_i, [_vp, _c.POINTER(_c.c_uint)]),
    "pr_workspace_output": (_vp, []),
    "pr_release_workspace": (_i, []),
    "pr_validate": (_i, [_vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _i, _vp]),
    "pr_select": (_i, [_i, _i, _i, _i, _c.POINTER(pr_decision)]),
    "pr_plan": (_i, [_i, _i, _c.POINTER(pr_plan_op), _i]),
    "pr_plan_cu_split": (_i, [_i, _i, _c.POINTER(pr_plan_op), _i]),
    "pr_set_cu_split": (_i, [_i, _i, _i, _i]),
    "pr_threshold_from_timings": (_i, [_i, _i, _c.POINTER(_i), _c.POINTER(_d), _c.POINTER(_d),
                                       _c.POINTER(_d), _c.POINTER(_i)]),
    "pr_set_tuning": (_i, [_i, _i, _i, _i, _c.POINTER(_i), _c.POINTER(_i), _i]),
    "pr_set_chunk_config": (_i, [_i, _i, _i, _i, _i, _i, _i]),
    "pr_clear_tuning": (None, []),
    "pr_tuning_save": (_i, [_c.c_char_p, _c.c_char_p]),
    "pr_tuning_load": (_i, [_c.c_char_p, _c.c_char_p]),
    "pr_tune": (_i, [_c.POINTER(_i), _c.POINTER(_i), _i, _i, _c.POINTER(_i), _i, _c.POINTER(_i),
                     _i, _i, _c.POINTER(pr_tune_report), _c.POINTER(_d), _vp]),
    "pr_strerror": (_c.c_char_p, [_i]),
    "pr_last_error": (_c.c_char_p, []),
    "pr_version": (_i, []),
}


class PRError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{code} ({_lib().pr_strerror(code).decode()}): {message}")
        self.code = code


_LIB = None
_LIB_LOADED = None
_STAMP_SIGNATURES = {
    "pr_phase_stamps_layout": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(ctypes.c_int)]),
    "pr_phase_stamps_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "pr_phase_stamps_clear": (ctypes.c_int, []),
}


def _lib():
    global _LIB, _LIB_LOADED
    if _LIB is None:
        stamps = os.environ.get("PR_PHASE_STAMPS") == "1"
        path = STAMPS_LIB_PATH if stamps else LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is missing; build it with "
                "`python -m projection_residual_rmsnorm_amd.build`")
        # torch ships its own HIP runtime; importing it first makes the library bind to that one
        # runtime (same soname) instead of loading a second copy from /opt/rocm.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(path)
        for name, (res, args) in {**SIGNATURES, **(_STAMP_SIGNATURES if stamps else {})}.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
        _LIB_LOADED = path
    return _LIB


def loaded_library_path() -> Optional[str]:
    """Path of the library this process loaded (None before the first call)."""
    return _LIB_LOADED


def pr_phase_stamps(clear: bool = False):
    """The diagnostic library's phase stamps as a (workgroups, words) uint64 array (after
    synchronising the device), or, with clear=True, zero them and return None.  Raises unless
    the process loaded libprojaddnorm_stamps.so (PR_PHASE_STAMPS=1)."""
    lib = _lib()
    if _LIB_LOADED != STAMPS_LIB_PATH:
        raise RuntimeError("phase stamps need the diagnostic library: set PR_PHASE_STAMPS=1 "
                           "before the first library call")
    def check(rc: int, name: str) -> None:
        if rc != PR_OK:
            raise PRError(rc, f"{name} failed")
    if clear:
        check(lib.pr_phase_stamps_clear(), "pr_phase_stamps_clear")
        return None
    import numpy as np
    groups, words = ctypes.c_int(), ctypes.c_int()
    check(lib.pr_phase_stamps_layout(ctypes.byref(groups), ctypes.byref(words)),
          "pr_phase_stamps_layout")
    buf = np.zeros(groups.value * words.value, dtype=np.uint64)
    check(lib.pr_phase_stamps_read(buf.ctypes.data, buf.size), "pr_phase_stamps_read")
    return buf.reshape(groups.value, words.value)


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _ptr(t, nbytes: int = 0, name: str = "buffer") -> Optional[int]:
    """Device address of a tensor (or a raw integer address, passed through unchecked).

    A tensor must be contiguous and hold at least `nbytes` bytes: the library reads and writes
    the dense row-major extent the shape arguments describe."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; the call needs "
                         f"{nbytes}")
    return t.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(rc: int) -> int:
    if rc != PR_OK:
        raise PRError(rc, _lib().pr_last_error().decode())
    return rc


def pr_prepare_weight(W_src, src_layout: int, W_prep, K: int, H: int, stream=None) -> None:
    n = 2 * max(K, 0) * max(H, 0)
    _check(_lib().pr_prepare_weight(_ptr(W_src, n, "W_src"), src_layout,
                                    _ptr(W_prep, n, "W_prep"), K, H, _stream(stream, W_src)))


def pr_silu_mul(gate_up, x, T: int, K: int, stream=None) -> None:
    """x[T][K] = bf16(silu(gate) * up) from the merged gate_up[T][2K] (gate first)."""
    n = 2 * max(T, 0) * max(K, 0)
    _check(_lib().pr_silu_mul(_ptr(gate_up, 2 * n, "gate_up"), _ptr(x, n, "x"), T, K,
                              _stream(stream, gate_up)))


def _call_ptrs(x, W, residual_inout, norm_w, out, T: int, K: int, H: int):
    T, K, H = max(T, 0), max(K, 0), max(H, 0)
    return (_ptr(x, 2 * T * K, "x"), _ptr(W, 2 * K * H, "W"),
            _ptr(residual_inout, 4 * T * H, "residual_inout"), _ptr(norm_w, 4 * H, "norm_w"),
            _ptr(out, 2 * T * H, "out"))


def proj_add_rmsnorm(x, W, residual_inout, norm_w, eps: float, T: int, K: int, H: int,
                     microchunk: int, norm_kind: int = PR_NORM_STANDARD, out=None,
                     stream=None) -> None:
    px, pw, pr_, pn, po = _call_ptrs(x, W, residual_inout, norm_w, out, T, K, H)
    _check(_lib().proj_add_rmsnorm(px, pw, pr_, pn, eps, T, K, H, microchunk, norm_kind, po,
                                   _stream(stream, x, residual_inout)))


def proj_add_rmsnorm_unfused(x, W, residual_inout, norm_w, eps: float, T: int, K: int, H: int,
                             norm_kind: int = PR_NORM_STANDARD, out=None, stream=None) -> None:
    px, pw, pr_, pn, po = _call_ptrs(x, W, residual_inout, norm_w, out, T, K, H)
    _check(_lib().proj_add_rmsnorm_unfused(px, pw, pr_, pn, eps, T, K, H, norm_kind, po,
                                           _stream(stream, x, residual_inout)))


def proj_add_rmsnorm_single_launch(x, W, residual_inout, norm_w, eps: float, T: int, K: int,
                                   H: int, norm_kind: int = PR_NORM_STANDARD, out=None,
                                   stream=None) -> None:
    px, pw, pr_, pn, po = _call_ptrs(x, W, residual_inout, norm_w, out, T, K, H)
    _check(_lib().proj_add_rmsnorm_single_launch(px, pw, pr_, pn, eps, T, K, H, norm_kind, po,
                                                 _stream(stream, x, residual_inout)))


def pr_init() -> None:
    """Sets the library up on the current device (needed before the no-allocation call)."""
    _check(_lib().pr_init())


def proj_add_rmsnorm_single_launch_noalloc(x, W, residual_inout, norm_w, eps: float, T: int,
                                           K: int, H: int, norm_kind: int = PR_NORM_STANDARD,
                                           out=None, stream=None) -> None:
    px, pw, pr_, pn, po = _call_ptrs(x, W, residual_inout, norm_w, out, T, K, H)
    _check(_lib().proj_add_rmsnorm_single_launch_noalloc(px, pw, pr_, pn, eps, T, K, H,
                                                         norm_kind, po,
                                                         _stream(stream, x, residual_inout)))


def proj_add_rmsnorm_silu(gate_up, W, residual_inout, norm_w, eps: float, T: int, K: int,
                          H: int, norm_kind: int = PR_NORM_STANDARD, out=None,
                          stream=None) -> None:
    """The down_proj region from the merged gate/up output, SiluAndMul inside the launch."""
    T_, K_, H_ = max(T, 0), max(K, 0), max(H, 0)
    _check(_lib().proj_add_rmsnorm_silu(
        _ptr(gate_up, 4 * T_ * K_, "gate_up"), _ptr(W, 2 * K_ * H_, "W"),
        _ptr(residual_inout, 4 * T_ * H_, "residual_inout"), _ptr(norm_w, 4 * H_, "norm_w"), eps,
        T, K, H, norm_kind, _ptr(out, 2 * T_ * H_, "out"), _stream(stream, gate_up, residual_inout)))


def pr_validate_silu(gate_up, W, residual_inout, norm_w, eps, T, K, H, norm_kind, out) -> int:
    """Returns the code (does not raise)."""
    return _lib().pr_validate_silu(_ptr(gate_up), _ptr(W), _ptr(residual_inout), _ptr(norm_w), eps,
                                   T, K, H, norm_kind, _ptr(out))


def pr_project_partial(x, W, y_partial, T: int, K: int, H: int, stream=None) -> None:
    """One rank's projection share: y_partial [T][H] fp32 = x [T][K] . W_slice^T."""
    T_, K_, H_ = max(T, 0), max(K, 0), max(H, 0)
    _check(_lib().pr_project_partial(_ptr(x, 2 * T_ * K_, "x"), _ptr(W, 2 * K_ * H_, "W"),
                                     _ptr(y_partial, 4 * T_ * H_, "y_partial"), T, K, H,
                                     _stream(stream, x)))


def pr_add_rmsnorm_partials(partials, P: int, plane_stride: int, residual_inout, norm_w,
                            eps: float, rows: int, H: int, norm_kind: int = PR_NORM_STANDARD,
                            out=None, stream=None) -> None:
    """The owner's add/norm after a reduce-scatter: r += sum of P fp32 partials (rank order)."""
    rows_, H_ = max(rows, 0), max(H, 0)
    need = 4 * ((max(P, 1) - 1) * plane_stride + rows_ * H_) if rows_ else 0
    _check(_lib().pr_add_rmsnorm_partials(
        _ptr(partials, need, "partials"), P, plane_stride,
        _ptr(residual_inout, 4 * rows_ * H_, "residual_inout"), _ptr(norm_w, 4 * H_, "norm_w"),
        eps, rows, H, norm_kind, _ptr(out, 2 * rows_ * H_, "out"),
        _stream(stream, partials, residual_inout)))


def pr_quantize_fp8(src, dst, scales, rows: int, cols: int, group_rows: int,
                    stream=None) -> None:
    """E4M3 codes of the bf16 src [rows][cols] by groups of group_rows rows; scales per group."""
    rows_, cols_ = max(rows, 0), max(cols, 0)
    groups = (rows_ - 1) // group_rows + 1 if rows_ > 0 and group_rows > 0 else 0
    _check(_lib().pr_quantize_fp8(_ptr(src, 2 * rows_ * cols_, "src"),
                                  _ptr(dst, rows_ * cols_, "dst"),
                                  _ptr(scales, 4 * groups, "scales"), rows, cols, group_rows,
                                  _stream(stream, src)))


def pr_prepare_weight_fp8(W_src, src_layout: int, W_prep, K: int, H: int, stream=None) -> None:
    n = max(K, 0) * max(H, 0)
    _check(_lib().pr_prepare_weight_fp8(_ptr(W_src, n, "W_src"), src_layout,
                                        _ptr(W_prep, n, "W_prep"), K, H, _stream(stream, W_src)))


def proj_add_rmsnorm_fp8(x_q, x_scales, scale_rows: int, W_q, w_scale, residual_inout, norm_w,
                         eps: float, T: int, K: int, H: int, norm_kind: int = PR_NORM_STANDARD,
                         out=None, stream=None) -> None:
    T_, K_, H_ = max(T, 0), max(K, 0), max(H, 0)
    groups = (T_ - 1) // scale_rows + 1 if T_ > 0 and scale_rows > 0 else 0
    _check(_lib().proj_add_rmsnorm_fp8(
        _ptr(x_q, T_ * K_, "x_q"), _ptr(x_scales, 4 * groups, "x_scales"), scale_rows,
        _ptr(W_q, K_ * H_, "W_q"), _ptr(w_scale, 4, "w_scale"),
        _ptr(residual_inout, 4 * T_ * H_, "residual_inout"), _ptr(norm_w, 4 * H_, "norm_w"), eps,
        T, K, H, norm_kind, _ptr(out, 2 * T_ * H_, "out"), _stream(stream, x_q, residual_inout)))


def pr_validate_fp8(x_q, x_scales, scale_rows, W_q, w_scale, residual_inout, norm_w, eps, T, K,
                    H, norm_kind, out) -> int:
    """Returns the code (does not raise)."""
    return _lib().pr_validate_fp8(_ptr(x_q), _ptr(x_scales), scale_rows, _ptr(W_q),
                                  _ptr(w_scale), _ptr(residual_inout), _ptr(norm_w), eps, T, K,
                                  H, norm_kind, _ptr(out))


def pr_device_status(stream=None) -> int:
    """Status bits of single-launch calls since the last read (waits for `stream`)."""
    v = ctypes.c_uint(0)
    _check(_lib().pr_device_status(_stream(stream), ctypes.byref(v)))
    return v.value


def pr_workspace_output() -> Optional[int]:
    return _lib().pr_workspace_output()


def pr_release_workspace() -> None:
    """Frees the library's grown workspaces on the current device (waits for the device)."""
    _check(_lib().pr_release_workspace())


def pr_validate(x, W, residual_inout, norm_w, eps, T, K, H, microchunk, norm_kind, out) -> int:
    """Returns the code (does not raise)."""
    return _lib().pr_validate(_ptr(x), _ptr(W), _ptr(residual_inout), _ptr(norm_w), eps, T, K,
                              H, microchunk, norm_kind, _ptr(out))


def pr_select(T: int, K: int, H: int, microchunk: int) -> dict:
    d = pr_decision()
    _check(_lib().pr_select(T, K, H, microchunk, ctypes.byref(d)))
    return {f: getattr(d, f) for f, _ in pr_decision._fields_}


def _plan(fn, T: int, microchunk: int) -> List[Tuple[str, int, int, int, int]]:
    n = fn(T, microchunk, None, 0)
    if n < 0:
        _check(n)
    ops = (pr_plan_op * max(n, 1))()
    _check(0 if fn(T, microchunk, ops, n) == n else PR_ERR_INVALID_ARG)
    return [(OP_NAMES[o.op], o.stream, o.chunk, o.slot, o.rows) for o in ops[:n]]


def pr_plan(T: int, microchunk: int) -> List[Tuple[str, int, int, int, int]]:
    """The ping-pong pipeline's schedule: (op, stream, chunk, slot, rows) in host order."""
    return _plan(_lib().pr_plan, T, microchunk)


def pr_plan_cu_split(T: int, microchunk: int) -> List[Tuple[str, int, int, int, int]]:
    """The CU-partitioned pipeline's schedule (streams 0 caller, 1 projections, 2 add/norms)."""
    return _plan(_lib().pr_plan_cu_split, T, microchunk)


def pr_set_cu_split(K: int, H: int, microchunk: int, addnorm_cus: int) -> None:
    _check(_lib().pr_set_cu_split(K, H, microchunk, addnorm_cus))


def pr_threshold_from_timings(T_grid: Sequence[int], t_conv, t_fused, spread=None) -> int:
    """t_conv / t_fused / spread: [ngroups][nT] nested sequences (seconds)."""
    ng, nT = len(t_conv), len(T_grid)
    flat = lambda a: (ctypes.c_double * (ng * nT))(*[float(v) for row in a for v in row])
    thr = ctypes.c_int()
    _check(_lib().pr_threshold_from_timings(
        ng, nT, (ctypes.c_int * nT)(*T_grid), flat(t_conv), flat(t_fused),
        flat(spread) if spread is not None else None, ctypes.byref(thr)))
    return thr.value


def pr_set_tuning(K: int, H: int, threshold_tokens: int, max_tokens: int,
                  T_grid: Sequence[int], mc_for_T: Sequence[int]) -> None:
    n = len(T_grid)
    _check(_lib().pr_set_tuning(K, H, threshold_tokens, max_tokens, (ctypes.c_int * n)(*T_grid),
                                (ctypes.c_int * n)(*mc_for_T), n))


def pr_set_chunk_config(K: int, H: int, microchunk: int, tile_m: int, tile_n: int, split_k: int,
                        waves: int) -> None:
    _check(_lib().pr_set_chunk_config(K, H, microchunk, tile_m, tile_n, split_k, waves))


def pr_clear_tuning() -> None:
    _lib().pr_clear_tuning()


def pr_tuning_save(path: str, device_key: Optional[str] = None) -> None:
    _check(_lib().pr_tuning_save(os.fsencode(path),
                                 None if device_key is None else device_key.encode()))


def pr_tuning_load(path: str, device_key: Optional[str] = None) -> None:
    _check(_lib().pr_tuning_load(os.fsencode(path),
                                 None if device_key is None else device_key.encode()))


def pr_tune(Ks: Sequence[int], Hs: Sequence[int], norm_kind: int, T_grid: Sequence[int],
            mc_cand: Sequence[int], reps: int = 10, stream=None) -> dict:
    ng, nT, nmc = len(Ks), len(T_grid), len(mc_cand)
    rep = pr_tune_report()
    nc = 3 + nmc  # conventional, best fused, each chunk size, single launch
    timings = (ctypes.c_double * (ng * nT * nc))()
    _check(_lib().pr_tune((ctypes.c_int * ng)(*Ks), (ctypes.c_int * ng)(*Hs), ng, norm_kind,
                          (ctypes.c_int * nT)(*T_grid), nT, (ctypes.c_int * nmc)(*mc_cand), nmc,
                          reps, ctypes.byref(rep), timings, _stream(stream)))
    t = list(timings)
    table = [[t[(g * nT + i) * nc:(g * nT + i + 1) * nc] for i in range(nT)] for g in range(ng)]
    return {"threshold_tokens": rep.threshold_tokens, "max_tokens": rep.max_tokens,
            "n_checked": rep.n_checked, "n_rejected": rep.n_rejected, "timings": table}


def pr_profile_enable(on: bool = True) -> None:
    _check(_lib().pr_profile_enable(1 if on else 0))


def pr_profile_read() -> dict:
    p = pr_profile()
    _check(_lib().pr_profile_read(ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in pr_profile._fields_}


def pr_strerror(code: int) -> str:
    return _lib().pr_strerror(code).decode()


def pr_last_error() -> str:
    return _lib().pr_last_error().decode()


def pr_version() -> int:
    return _lib().pr_version()
