"""ctypes binding of libdarkprf.so (the C ABI in include/darkprf.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  torch supplies device memory and the current HIP stream.  There
is no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdarkprf.so")

DARK_OK = 0
DARK_ERR_INVALID_ARG = 1
DARK_ERR_UNSUPPORTED = 2
DARK_ERR_WORKSPACE = 3
DARK_ERR_STALE_STATE = 4
DARK_ERR_HIP = 5
DARK_F32 = 0
DARK_BF16 = 1


class DarkPrfDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32),
        ("L", ctypes.c_int32), ("d_h", ctypes.c_int32), ("m", ctypes.c_int32),
        ("r", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("m_per_head", ctypes.c_int32),
        ("q_str", ctypes.c_int64 * 3), ("k_str", ctypes.c_int64 * 3),
        ("v_str", ctypes.c_int64 * 3), ("o_str", ctypes.c_int64 * 3),
        ("proj_tag", ctypes.c_uint64), ("omega_per_head", ctypes.c_int32),
    ]


class DarkPrfProjection(ctypes.Structure):
    _fields_ = [
        ("base_seed", ctypes.c_uint64), ("seed", ctypes.c_uint64), ("tag", ctypes.c_uint64),
        ("draw", ctypes.c_int64), ("forwards", ctypes.c_int64),
        ("m", ctypes.c_int32), ("r", ctypes.c_int32), ("orthogonal", ctypes.c_int32),
        ("interval", ctypes.c_int32), ("fixed", ctypes.c_int32),
    ]


class DarkPrfError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdarkprf.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with random_feature_linear_amd.build.build()")
        # torch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading it
        # first makes this library bind to that same runtime; loading this
        # library first would put a second HIP runtime in the process, and
        # torch's streams and memory would be foreign to it.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.dark_prf_omega.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
        L.dark_prf_omega.restype = ctypes.c_int
        L.dark_prf_omega_device_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.dark_prf_omega_device_workspace_bytes.restype = ctypes.c_size_t
        L.dark_prf_omega_device.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                                            ctypes.c_size_t, P]
        L.dark_prf_omega_device.restype = ctypes.c_int
        L.dark_prf_proj_tag.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.dark_prf_proj_tag.restype = ctypes.c_uint64
        L.dark_prf_head_seed.argtypes = [ctypes.c_uint64, ctypes.c_int32]
        L.dark_prf_head_seed.restype = ctypes.c_uint64
        L.dark_prf_omega_per_head.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, P]
        L.dark_prf_omega_per_head.restype = ctypes.c_int
        L.dark_prf_proj_tag_per_head.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32]
        L.dark_prf_proj_tag_per_head.restype = ctypes.c_uint64
        L.dark_prf_workspace_bytes.argtypes = [ctypes.POINTER(DarkPrfDesc)]
        L.dark_prf_workspace_bytes.restype = ctypes.c_size_t
        L.dark_prf_fwd.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
        L.dark_prf_fwd.restype = ctypes.c_int
        L.dark_prf_fwd_noalloc.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, P, P, P, P, P]
        L.dark_prf_fwd_noalloc.restype = ctypes.c_int
        L.dark_prf_decode_step.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, P, P,
                                           ctypes.c_uint64, P, P]
        L.dark_prf_decode_step.restype = ctypes.c_int
        L.dark_prf_context_state.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, P, P, P,
                                             ctypes.c_size_t, P]
        L.dark_prf_context_state.restype = ctypes.c_int
        L.dark_prf_cross_fwd.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, ctypes.c_uint64,
                                         P, P, P, ctypes.c_size_t, P]
        L.dark_prf_cross_fwd.restype = ctypes.c_int
        L.dark_prf_exact_workspace_bytes.argtypes = [ctypes.POINTER(DarkPrfDesc)]
        L.dark_prf_exact_workspace_bytes.restype = ctypes.c_size_t
        L.dark_prf_exact_fwd.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.dark_prf_exact_fwd.restype = ctypes.c_int
        L.dark_prf_auto_mode.argtypes = [ctypes.POINTER(DarkPrfDesc), ctypes.c_int32]
        L.dark_prf_auto_mode.restype = ctypes.c_int32
        L.dark_prf_auto_workspace_bytes.argtypes = [ctypes.POINTER(DarkPrfDesc), ctypes.c_int32]
        L.dark_prf_auto_workspace_bytes.restype = ctypes.c_size_t
        L.dark_prf_auto_fwd.argtypes = [ctypes.POINTER(DarkPrfDesc), ctypes.c_int32, P, P, P, P, P, P, P, P,
                                        ctypes.c_size_t, P]
        L.dark_prf_auto_fwd.restype = ctypes.c_int
        L.dark_prf_bwd_workspace_bytes.argtypes = [ctypes.POINTER(DarkPrfDesc)]
        L.dark_prf_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.dark_prf_bwd.argtypes = [ctypes.POINTER(DarkPrfDesc), P, P, P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
        L.dark_prf_bwd.restype = ctypes.c_int
        PP = ctypes.POINTER(DarkPrfProjection)
        L.dark_prf_projection_init.argtypes = [PP, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32]
        L.dark_prf_projection_init.restype = ctypes.c_int
        L.dark_prf_projection_forward.argtypes = [PP, ctypes.c_int32]
        L.dark_prf_projection_forward.restype = ctypes.c_int32
        L.dark_prf_projection_redraw.argtypes = [PP, ctypes.c_int32]
        L.dark_prf_projection_redraw.restype = ctypes.c_int32
        L.dark_prf_projection_fix.argtypes = [PP, ctypes.c_int32]
        L.dark_prf_projection_fix.restype = ctypes.c_int
        L.dark_prf_status_str.argtypes = [ctypes.c_int]
        L.dark_prf_status_str.restype = ctypes.c_char_p
        L.dark_prf_timing_begin.argtypes = []
        L.dark_prf_timing_begin.restype = ctypes.c_int
        L.dark_prf_timing_end.argtypes = [P, P]
        L.dark_prf_timing_end.restype = ctypes.c_int
        _lib = L
    return _lib


# ---- the C entry points, same names ------------------------------------------
def dark_prf_status_str(status: int) -> str:
    return lib().dark_prf_status_str(int(status)).decode()


status_str = dark_prf_status_str


def dark_prf_omega(seed: int, m: int, r: int, orthogonal: bool) -> np.ndarray:
    out = np.empty((m, r), dtype=np.float32)
    st = lib().dark_prf_omega(ctypes.c_uint64(seed), m, r, int(bool(orthogonal)),
                              out.ctypes.data_as(ctypes.c_void_p))
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_omega")
    return out


def dark_prf_head_seed(seed: int, h: int) -> int:
    return int(lib().dark_prf_head_seed(ctypes.c_uint64(seed), h))


def dark_prf_omega_per_head(seed: int, H: int, m: int, r: int, orthogonal: bool) -> np.ndarray:
    """Per-head projections [H][m][r]: head h is dark_prf_omega(dark_prf_head_seed(seed, h), ...)."""
    out = np.empty((H, m, r), dtype=np.float32)
    st = lib().dark_prf_omega_per_head(ctypes.c_uint64(seed), H, m, r, int(bool(orthogonal)),
                                       out.ctypes.data_as(ctypes.c_void_p))
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_omega_per_head")
    return out


def dark_prf_proj_tag_per_head(seed: int, H: int, m: int, r: int, orthogonal: bool) -> int:
    return int(lib().dark_prf_proj_tag_per_head(ctypes.c_uint64(seed), H, m, r, int(bool(orthogonal))))


def dark_prf_omega_device_workspace_bytes(m: int, r: int, orthogonal: bool) -> int:
    return int(lib().dark_prf_omega_device_workspace_bytes(m, r, int(bool(orthogonal))))


def dark_prf_omega_device(seed: int, m: int, r: int, orthogonal: bool, omega: int, workspace: int,
                          ws_bytes: int, stream: int) -> int:
    return lib().dark_prf_omega_device(ctypes.c_uint64(seed), m, r, int(bool(orthogonal)), omega or None,
                                       workspace or None, ws_bytes, stream or None)


def omega_on_device(seed: int, m: int, r: int, orthogonal: bool, device="cuda:0"):
    """dark_prf_omega_device into a new fp32 [m][r] device tensor."""
    import torch
    out = torch.empty((m, r), dtype=torch.float32, device=device)
    nb = dark_prf_omega_device_workspace_bytes(m, r, orthogonal)
    ws = torch.empty(max(nb, 8), dtype=torch.uint8, device=device)
    st = dark_prf_omega_device(seed, m, r, orthogonal, out.data_ptr(), ws.data_ptr(), nb,
                               torch.cuda.current_stream(out.device).cuda_stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_omega_device")
    return out


def dark_prf_projection_init(seed: int, m: int, r: int, orthogonal: bool, redraw_interval: int = 0,
                             deterministic: bool = False) -> DarkPrfProjection:
    p = DarkPrfProjection()
    st = lib().dark_prf_projection_init(ctypes.byref(p), ctypes.c_uint64(seed), m, r, int(bool(orthogonal)),
                                        redraw_interval, int(bool(deterministic)))
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_projection_init")
    return p


def dark_prf_projection_forward(p: DarkPrfProjection, training: bool) -> int:
    return int(lib().dark_prf_projection_forward(ctypes.byref(p), int(bool(training))))


def dark_prf_projection_redraw(p: DarkPrfProjection, force: bool = False) -> int:
    return int(lib().dark_prf_projection_redraw(ctypes.byref(p), int(bool(force))))


def dark_prf_projection_fix(p: DarkPrfProjection, fixed: bool) -> int:
    return int(lib().dark_prf_projection_fix(ctypes.byref(p), int(bool(fixed))))


def dark_prf_proj_tag(seed: int, m: int, r: int, orthogonal: bool) -> int:
    return int(lib().dark_prf_proj_tag(ctypes.c_uint64(seed), m, r, int(bool(orthogonal))))


def dark_prf_workspace_bytes(desc: DarkPrfDesc) -> int:
    return int(lib().dark_prf_workspace_bytes(ctypes.byref(desc)))


def dark_prf_fwd(desc: DarkPrfDesc, q: int, k: int, v: int, M: int, omega: int, mask: int,
                 out: int, S_out: int, z_out: int, workspace: int, ws_bytes: int,
                 stream: int) -> int:
    """Raw call with integer device addresses (0 = NULL); returns the status."""
    return lib().dark_prf_fwd(ctypes.byref(desc), q or None, k or None, v or None, M or None,
                              omega or None, mask or None, out or None, S_out or None,
                              z_out or None, workspace or None, ws_bytes, stream or None)


DARK_PRF_SCRATCH_BYTES = 64 << 20   # the static workspace of dark_prf_fwd_noalloc


def dark_prf_fwd_noalloc(desc: DarkPrfDesc, q: int, k: int, v: int, M: int, omega: int, mask: int,
                         out: int, S_out: int, z_out: int, stream: int) -> int:
    """Raw call of the forward that takes its workspace from the library's static
    per-GPU buffer (no workspace argument); returns the status."""
    return lib().dark_prf_fwd_noalloc(ctypes.byref(desc), q or None, k or None, v or None, M or None,
                                      omega or None, mask or None, out or None, S_out or None,
                                      z_out or None, stream or None)


def dark_prf_context_state(desc: DarkPrfDesc, k: int, v: int, M: int, omega: int, context_mask: int,
                           S_out: int, z_out: int, workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().dark_prf_context_state(ctypes.byref(desc), k or None, v or None, M or None,
                                        omega or None, context_mask or None, S_out or None,
                                        z_out or None, workspace or None, ws_bytes, stream or None)


def dark_prf_cross_fwd(desc: DarkPrfDesc, q: int, M: int, omega: int, S: int, z: int, state_tag: int,
                       query_mask: int, out: int, workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().dark_prf_cross_fwd(ctypes.byref(desc), q or None, M or None, omega or None,
                                    S or None, z or None, ctypes.c_uint64(state_tag),
                                    query_mask or None, out or None, workspace or None, ws_bytes,
                                    stream or None)


def dark_prf_exact_workspace_bytes(desc: DarkPrfDesc) -> int:
    return int(lib().dark_prf_exact_workspace_bytes(ctypes.byref(desc)))


def dark_prf_exact_fwd(desc: DarkPrfDesc, q: int, k: int, v: int, M: int, mask: int, out: int,
                       workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().dark_prf_exact_fwd(ctypes.byref(desc), q or None, k or None, v or None, M or None,
                                    mask or None, out or None, workspace or None, ws_bytes, stream or None)


def dark_prf_auto_mode(desc: DarkPrfDesc, exact_threshold: int) -> int:
    return int(lib().dark_prf_auto_mode(ctypes.byref(desc), exact_threshold))


def dark_prf_auto_workspace_bytes(desc: DarkPrfDesc, exact_threshold: int) -> int:
    return int(lib().dark_prf_auto_workspace_bytes(ctypes.byref(desc), exact_threshold))


def dark_prf_auto_fwd(desc: DarkPrfDesc, exact_threshold: int, q: int, k: int, v: int, M: int, omega: int,
                      mask: int, out: int, workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().dark_prf_auto_fwd(ctypes.byref(desc), exact_threshold, q or None, k or None, v or None,
                                   M or None, omega or None, mask or None, out or None, workspace or None,
                                   ws_bytes, stream or None)


def dark_prf_bwd_workspace_bytes(desc: DarkPrfDesc) -> int:
    return int(lib().dark_prf_bwd_workspace_bytes(ctypes.byref(desc)))


def dark_prf_bwd(desc: DarkPrfDesc, q: int, k: int, v: int, M: int, omega: int, mask: int, dout: int,
                 dq: int, dk: int, dv: int, dM: int, workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().dark_prf_bwd(ctypes.byref(desc), q or None, k or None, v or None, M or None, omega or None,
                              mask or None, dout or None, dq or None, dk or None, dv or None, dM or None,
                              workspace or None, ws_bytes, stream or None)


def dark_prf_decode_step(desc: DarkPrfDesc, q: int, k: int, v: int, M: int, omega: int, S: int,
                         z: int, state_tag: int, out: int, stream: int) -> int:
    return lib().dark_prf_decode_step(ctypes.byref(desc), q or None, k or None, v or None,
                                      M or None, omega or None, S or None, z or None,
                                      ctypes.c_uint64(state_tag), out or None, stream or None)


KERNEL_KINDS = ("prep", "kstate", "scan", "qout", "decode", "shift", "bwd_gemm", "bwd_aux")


def dark_prf_timing_begin() -> None:
    st = lib().dark_prf_timing_begin()
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_timing_begin")


def dark_prf_timing_end() -> dict:
    """{kind: (total_ms, launches)} for every kernel kind."""
    ms = (ctypes.c_double * len(KERNEL_KINDS))()
    n = (ctypes.c_int32 * len(KERNEL_KINDS))()
    st = lib().dark_prf_timing_end(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(n, ctypes.c_void_p))
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_timing_end")
    return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(KERNEL_KINDS)}


# ---- torch-tensor conveniences (marshalling only) -----------------------------
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DARK_BF16
    if t.dtype == torch.float32:
        return DARK_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_desc(q, k, v, out, M, omega, causal: bool, proj_tag: int = 0) -> DarkPrfDesc:
    """Descriptor for q [B][H][L][d_h], k/v [B][H_kv][L][d_h] (any strides, d_h contiguous)."""
    B, H, L, d_h = q.shape
    d = DarkPrfDesc()
    d.B, d.H, d.H_kv, d.L, d.d_h = B, H, k.shape[1], L, d_h
    d.m, d.r = omega.shape[-2], omega.shape[-1]
    d.omega_per_head = int(omega.dim() == 3)
    d.dtype = _dtype_code(q)
    d.causal = int(bool(causal))
    d.m_per_head = int(M.dim() == 3)
    for name, t in (("q_str", q), ("k_str", k), ("v_str", v), ("o_str", out)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
        getattr(d, name)[:] = list(t.stride()[:3])
    d.proj_tag = proj_tag
    return d


def prf_attention(q, k, v, M, omega, mask=None, causal: bool = False, return_state: bool = False,
                  proj_tag: int = 0, out=None, workspace=None):
    """dark_prf_fwd on torch device tensors; returns out (and S, z when return_state)."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    desc = make_desc(q, k, v, out, M, omega, causal, proj_tag)
    nbytes = dark_prf_workspace_bytes(desc)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    S = z = None
    if return_state:
        B, H = q.shape[0], q.shape[1]
        S = torch.empty((B, H, desc.m, desc.d_h), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, desc.m), dtype=torch.float32, device=q.device)
    mask_ptr = 0
    if mask is not None:
        if mask.dtype != torch.uint8 or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B][L] tensor")
        mask_ptr = mask.data_ptr()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = dark_prf_fwd(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), M.data_ptr(),
                      omega.data_ptr(), mask_ptr, out.data_ptr(),
                      S.data_ptr() if S is not None else 0, z.data_ptr() if z is not None else 0,
                      workspace.data_ptr(), workspace.numel(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_fwd")
    return (out, S, z) if return_state else out


def decode_step(q, k, v, M, omega, S, z, state_tag: int, proj_tag: int, out=None):
    """dark_prf_decode_step: q [N][H][d_h], k/v [N][H_kv][d_h]; S, z updated in place."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    N, H, d_h = q.shape
    d = DarkPrfDesc()
    d.B, d.H, d.H_kv, d.L, d.d_h = N, H, k.shape[1], 1, d_h
    d.m, d.r = omega.shape[-2], omega.shape[-1]
    d.omega_per_head = int(omega.dim() == 3)
    d.dtype = _dtype_code(q)
    d.causal = 1
    d.m_per_head = int(M.dim() == 3)
    for name, t in (("q_str", q), ("k_str", k), ("v_str", v), ("o_str", out)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
        getattr(d, name)[:] = [t.stride(0), t.stride(1), 0]
    d.proj_tag = proj_tag
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = dark_prf_decode_step(d, q.data_ptr(), k.data_ptr(), v.data_ptr(), M.data_ptr(),
                              omega.data_ptr(), S.data_ptr(), z.data_ptr(), state_tag,
                              out.data_ptr(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_decode_step")
    return out


def _mask_ptr(mask, what: str) -> int:
    import torch
    if mask is None:
        return 0
    if mask.dtype != torch.uint8 or not mask.is_contiguous():
        raise ValueError(f"{what} must be a contiguous uint8 [B][L] tensor")
    return mask.data_ptr()


def context_state(k, v, M, omega, H: int, context_mask=None, proj_tag: int = 0, workspace=None):
    """dark_prf_context_state: k/v [B][H_kv][L_k][d_h] -> S [B][H][m][d_h], z [B][H][m] (fp32)."""
    import torch
    B, H_kv, L_k, d_h = k.shape
    d = DarkPrfDesc()
    d.B, d.H, d.H_kv, d.L, d.d_h = B, H, H_kv, L_k, d_h
    d.m, d.r = omega.shape[-2], omega.shape[-1]
    d.omega_per_head = int(omega.dim() == 3)
    d.dtype = _dtype_code(k)
    d.causal = 0
    d.m_per_head = int(M.dim() == 3)
    for name, t in (("k_str", k), ("v_str", v)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
        getattr(d, name)[:] = list(t.stride()[:3])
    d.q_str[:] = list(k.stride()[:3])   # not used by this call
    d.o_str[:] = list(k.stride()[:3])
    d.proj_tag = proj_tag
    nbytes = dark_prf_workspace_bytes(d)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    S = torch.empty((B, H, d.m, d_h), dtype=torch.float32, device=k.device)
    z = torch.empty((B, H, d.m), dtype=torch.float32, device=k.device)
    stream = torch.cuda.current_stream(k.device).cuda_stream
    st = dark_prf_context_state(d, k.data_ptr(), v.data_ptr(), M.data_ptr(), omega.data_ptr(),
                                _mask_ptr(context_mask, "context_mask"), S.data_ptr(), z.data_ptr(),
                                workspace.data_ptr(), workspace.numel(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_context_state")
    return S, z


def cross_attention(q, M, omega, S, z, state_tag: int, proj_tag: int, query_mask=None, H_kv: int = 1,
                    out=None, workspace=None):
    """dark_prf_cross_fwd: q [B][H][L_q][d_h] against a summary (S, z) -> out [B][H][L_q][d_h]."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    B, H, L_q, d_h = q.shape
    d = DarkPrfDesc()
    d.B, d.H, d.H_kv, d.L, d.d_h = B, H, H_kv, L_q, d_h
    d.m, d.r = omega.shape[-2], omega.shape[-1]
    d.omega_per_head = int(omega.dim() == 3)
    d.dtype = _dtype_code(q)
    d.causal = 0
    d.m_per_head = int(M.dim() == 3)
    for name, t in (("q_str", q), ("o_str", out)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
        getattr(d, name)[:] = list(t.stride()[:3])
    d.k_str[:] = list(q.stride()[:3])   # not used by this call
    d.v_str[:] = list(q.stride()[:3])
    d.proj_tag = proj_tag
    nbytes = dark_prf_workspace_bytes(d)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = dark_prf_cross_fwd(d, q.data_ptr(), M.data_ptr(), omega.data_ptr(), S.data_ptr(), z.data_ptr(),
                            state_tag, _mask_ptr(query_mask, "query_mask"), out.data_ptr(),
                            workspace.data_ptr(), workspace.numel(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_cross_fwd")
    return out


def auto_attention(q, k, v, M, omega, exact_threshold: int, mask=None, causal: bool = False, proj_tag: int = 0,
                   out=None, workspace=None):
    """dark_prf_auto_fwd: exact attention for L <= exact_threshold, linear attention above."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    desc = make_desc(q, k, v, out, M, omega, causal, proj_tag)
    nbytes = dark_prf_auto_workspace_bytes(desc, exact_threshold)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = dark_prf_auto_fwd(desc, exact_threshold, q.data_ptr(), k.data_ptr(), v.data_ptr(), M.data_ptr(),
                           omega.data_ptr(), _mask_ptr(mask, "mask"), out.data_ptr(), workspace.data_ptr(),
                           workspace.numel(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_auto_fwd")
    return out


def prf_attention_backward(q, k, v, M, omega, dout, mask=None, causal: bool = False, workspace=None):
    """dark_prf_bwd on torch device tensors: returns (dq, dk, dv, dM).

    dq, dk and dv take the strides of q, k and v; dout must have the strides of
    q (the forward's output layout); dM is fp32 shaped like M.
    """
    import torch
    if tuple(dout.shape) != tuple(q.shape) or dout.dtype != q.dtype:
        raise ValueError("dout must match q in shape and dtype")
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
    dM = torch.empty(M.shape, dtype=torch.float32, device=M.device)
    desc = make_desc(q, k, v, dout, M, omega, causal)
    nbytes = dark_prf_bwd_workspace_bytes(desc)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = dark_prf_bwd(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), M.data_ptr(), omega.data_ptr(),
                      _mask_ptr(mask, "mask"), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      dM.data_ptr(), workspace.data_ptr(), workspace.numel(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_bwd")
    return dq, dk, dv, dM


def exact_attention(q, k, v, M, mask=None, causal: bool = False, out=None, workspace=None):
    """dark_prf_exact_fwd: softmax attention on u = d_h^(-1/4) M_h x for q and k."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    B, H, L, d_h = q.shape
    d = DarkPrfDesc()
    d.B, d.H, d.H_kv, d.L, d.d_h = B, H, k.shape[1], L, d_h
    d.m, d.r = 16, M.shape[-2]          # m is not used by the exact path
    d.dtype = _dtype_code(q)
    d.causal = int(bool(causal))
    d.m_per_head = int(M.dim() == 3)
    for name, t in (("q_str", q), ("k_str", k), ("v_str", v), ("o_str", out)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous")
        getattr(d, name)[:] = list(t.stride()[:3])
    nbytes = dark_prf_exact_workspace_bytes(d)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = dark_prf_exact_fwd(d, q.data_ptr(), k.data_ptr(), v.data_ptr(), M.data_ptr(),
                            _mask_ptr(mask, "mask"), out.data_ptr(), workspace.data_ptr(),
                            workspace.numel(), stream)
    if st != DARK_OK:
        raise DarkPrfError(st, "dark_prf_exact_fwd")
    return out
