"""Thin ctypes binding over libssd.so (declared in include/ssd.h).

Argument marshalling only: shapes are read off torch tensors, device
pointers and the current HIP stream are passed through, and a non-zero status
raises ``SSDError``.  Every step of the scan runs in the library's HIP
kernels; there is no fallback of any kind.  If libssd.so is missing this
module raises on first use: build it with
``python -m mamba_ssd_scan_chunk_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSD_LIB_PATH names another build of the same library (the tests run the host
# checks once more under a sanitizer build); by default the in-tree build.
LIB_PATH = os.environ.get("SSD_LIB_PATH") or os.path.join(_HERE, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_OK = 0
SSD_ERR_INVALID_ARG = -1
SSD_ERR_UNSUPPORTED = -2
SSD_ERR_ALIGNMENT = -3
SSD_ERR_WORKSPACE = -4
SSD_ERR_HIP = -5
SSD_ERR_TOO_LARGE = -6
NOALLOC_SCRATCH_BYTES = 64 << 20  # SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h

# (name, restype, argtypes) of every entry point in include/ssd.h
_i, _p, _l, _sz, _f = ctypes.c_int, ctypes.c_void_p, ctypes.c_long, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "ssd_prefill": (_i, [_i] * 8 + [_p] * 10 + [_sz, _p]),
    "ssd_prefill_dt_raw": (_i, [_i] * 8 + [_p] * 3 + [_f, _f] + [_p] * 8 + [_sz, _p]),
    "ssd_prefill_workspace_bytes": (_sz, [_i] * 8),
    "ssd_prefill_noalloc": (_i, [_i] * 8 + [_p] * 9 + [_p]),
    "ssd_prefill_varlen": (_i, [_i] * 8 + [_p] * 11 + [_sz, _p]),
    "ssd_prefill_varlen_workspace_bytes": (_sz, [_i] * 8),
    "ssd_prefill_varlen_dt_raw": (_i, [_i] * 8 + [_p] * 4 + [_f, _f] + [_p] * 8 + [_sz, _p]),
    "ssd_decode_step": (_i, [_i] * 6 + [_p] * 8 + [_l] + [_p] * 4 + [_i, _i, _p]),
    "ssd_decode_step_dt_raw": (_i, [_i] * 6 + [_p] * 3 + [_f, _f] + [_p] * 6 + [_l] + [_p] * 4 + [_i, _i, _p]),
    "conv_state_update": (_i, [_i] * 5 + [_p] * 4 + [_i, _p, _p]),
    "conv_state_update_varlen": (_i, [_i] * 5 + [_p] * 5 + [_i, _p, _p, _sz, _p]),
    "conv_state_update_varlen_workspace_bytes": (_sz, [_i, _i]),
    "ssd_gated_rmsnorm": (_i, [_l, _i, _i, _i, _p, _p, _l, _p, _f, _p, _p]),
    "ssd_stage_timing": (_i, [_i]),
    "ssd_stage_times": (_i, [ctypes.POINTER(ctypes.c_float), _i, ctypes.POINTER(_i)]),
    "ssd_stage_name": (ctypes.c_char_p, [_i]),
    "ssd_debug_handoff_ticks": (_i, [ctypes.c_longlong]),
    "ssd_debug_handoff_jitter": (_i, [_i]),
    "ssd_debug_packed_form": (_i, [_i]),
    "ssd_status_string": (ctypes.c_char_p, [_i]),
    "ssd_last_hip_error": (_i, []),
}

_lib = None


class SSDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().ssd_status_string(status).decode()
        if status == SSD_ERR_HIP:
            msg += f" (hipError_t {lib().ssd_last_hip_error()})"
        super().__init__(f"{fn} returned {status}: {msg}")


def lib() -> ctypes.CDLL:
    """The loaded library with typed entry points (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: the HIP library is not built "
                "(python -m mamba_ssd_scan_chunk_amd.build)")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.restype, fn.argtypes = res, args
        _lib = cdll
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(type(t))
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return t.data_ptr()


def _dense(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _want(t, name, shape, dtype, device):
    """Raise unless t is None or a dense tensor of this shape and dtype on
    this device.  The C ABI receives bare pointers and cannot see buffer
    sizes, so a tensor of the wrong size or type would be read or written
    out of bounds by the kernels: every tensor is checked here first."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want_workspace(ws, need, device):
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.dim() != 1 or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.device != device:
        raise ValueError(f"workspace must be on {device}, got {ws.device}")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")


def _want_rows(t, name, rows, cols, dtype, device, stride):
    """x_t / B_t / C_t of a decode step: [rows, cols] with row stride
    ``stride`` elements (0: dense) and contiguous columns."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if stride == 0:
        if not t.is_contiguous() or t.numel() != rows * cols:
            raise ValueError(f"{name} must be dense with {rows}x{cols} elements when in_stride is 0")
        return
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must be a [{rows}, {cols}] view when in_stride is set, got {tuple(t.shape)}")
    if t.stride(1) != 1 or (rows > 1 and t.stride(0) != stride):
        raise ValueError(f"{name} must have row stride {stride} and contiguous columns, got strides {t.stride()}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, rc: int):
    if rc != SSD_OK:
        raise SSDError(fn, rc)


def ssd_prefill_workspace_bytes(B, L, H, P, G, N, Q, dtype) -> int:
    n = lib().ssd_prefill_workspace_bytes(B, L, H, P, G, N, Q, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("ssd_prefill would reject these arguments")
    return n


def ssd_prefill(x, dt, A_log, Bm, Cm, D=None, init_state=None, *, Q, y=None,
                final_state=None, want_final_state=True, workspace=None, stream=None,
                dt_raw=False, dt_bias=None, dt_min=0.0, dt_max=float("inf")):
    """Chunked SSD prefill.  x [B,L,H,P], dt [B,L,H] f32, A_log [H] f32,
    Bm/Cm [B,L,G,N], D [H] f32 or None, init_state [B,H,P,N] f32 or None.
    With ``dt_raw`` the kernels use clamp(softplus(dt + dt_bias), dt_min,
    dt_max) as the step (ssd_prefill_dt_raw).  Returns (y, final_state)."""
    if x.dim() != 4 or Bm.dim() != 4:
        raise ValueError("x must be [B,L,H,P] and Bm [B,L,G,N]")
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    code = _dtype_code(x)
    f32, dv = torch.float32, x.device
    _want(x, "x", (B, L, H, P), x.dtype, dv)
    _want(dt, "dt", (B, L, H), f32, dv)
    _want(A_log, "A_log", (H,), f32, dv)
    _want(Bm, "Bm", (B, L, G, N), x.dtype, dv)
    _want(Cm, "Cm", (B, L, G, N), x.dtype, dv)
    _want(D, "D", (H,), f32, dv)
    _want(init_state, "init_state", (B, H, P, N), f32, dv)
    _want(y, "y", (B, L, H, P), x.dtype, dv)
    _want(final_state, "final_state", (B, H, P, N), f32, dv)
    _want(dt_bias, "dt_bias", (H,), f32, dv)
    need = ssd_prefill_workspace_bytes(B, L, H, P, G, N, Q, code)
    _want_workspace(workspace, need, dv)
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, P, N), dtype=torch.float32, device=x.device)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if dt_raw:
        rc = lib().ssd_prefill_dt_raw(B, L, H, P, G, N, Q, code, _ptr(x), _ptr(dt), _ptr(dt_bias), float(dt_min),
                                      float(dt_max), _ptr(A_log), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state),
                                      _ptr(y), _ptr(final_state), _ptr(workspace), ws_bytes, _stream(stream))
        _check("ssd_prefill_dt_raw", rc)
    else:
        if dt_bias is not None:
            raise ValueError("dt_bias is used only with dt_raw=True")
        rc = lib().ssd_prefill(B, L, H, P, G, N, Q, code, _ptr(x), _ptr(dt), _ptr(A_log), _ptr(Bm),
                               _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state),
                               _ptr(workspace), ws_bytes, _stream(stream))
        _check("ssd_prefill", rc)
    return y, final_state


def ssd_prefill_noalloc(x, dt, A_log, Bm, Cm, D=None, init_state=None, *, Q, y, final_state=None, stream=None):
    """ssd_prefill without a workspace argument: the scratch is the
    library's fixed per-GPU buffer of NOALLOC_SCRATCH_BYTES (for callers that
    cannot allocate device memory).  y, and final_state when wanted, are the
    caller's: this call allocates nothing.  Returns (y, final_state)."""
    if x.dim() != 4 or Bm.dim() != 4:
        raise ValueError("x must be [B,L,H,P] and Bm [B,L,G,N]")
    if y is None:
        raise ValueError("ssd_prefill_noalloc allocates nothing: pass y")
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    code = _dtype_code(x)
    f32, dv = torch.float32, x.device
    _want(x, "x", (B, L, H, P), x.dtype, dv)
    _want(dt, "dt", (B, L, H), f32, dv)
    _want(A_log, "A_log", (H,), f32, dv)
    _want(Bm, "Bm", (B, L, G, N), x.dtype, dv)
    _want(Cm, "Cm", (B, L, G, N), x.dtype, dv)
    _want(D, "D", (H,), f32, dv)
    _want(init_state, "init_state", (B, H, P, N), f32, dv)
    _want(y, "y", (B, L, H, P), x.dtype, dv)
    _want(final_state, "final_state", (B, H, P, N), f32, dv)
    rc = lib().ssd_prefill_noalloc(B, L, H, P, G, N, Q, code, _ptr(x), _ptr(dt), _ptr(A_log), _ptr(Bm), _ptr(Cm),
                                   _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state), _stream(stream))
    _check("ssd_prefill_noalloc", rc)
    return y, final_state


def ssd_prefill_varlen(x, dt, A_log, Bm, Cm, D, cu_seqlens, init_state=None, *, Q, y=None, final_state=None,
                       workspace=None, stream=None, dt_raw=False, dt_bias=None, dt_min=0.0, dt_max=float("inf")):
    """Prefill of B sequences packed without padding: x [T,H,P], dt [T,H],
    Bm/Cm [T,G,N], cu_seqlens [B+1] int32 on the GPU (sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1]).  init_state / final_state [B,H,P,N].
    With ``dt_raw`` the step is clamp(softplus(dt + dt_bias), dt_min, dt_max)
    (ssd_prefill_varlen_dt_raw).  Returns (y [T,H,P], final_state)."""
    if dt_bias is not None and not dt_raw:
        raise ValueError("dt_bias is used only with dt_raw=True")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if x.dim() != 3 or Bm.dim() != 3 or cu_seqlens.dim() != 1:
        raise ValueError("x must be [T,H,P], Bm [T,G,N] and cu_seqlens [B+1]")
    T, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    B = cu_seqlens.numel() - 1
    code = _dtype_code(x)
    f32, dv = torch.float32, x.device
    _want(x, "x", (T, H, P), x.dtype, dv)
    _want(dt, "dt", (T, H), f32, dv)
    _want(A_log, "A_log", (H,), f32, dv)
    _want(Bm, "Bm", (T, G, N), x.dtype, dv)
    _want(Cm, "Cm", (T, G, N), x.dtype, dv)
    _want(D, "D", (H,), f32, dv)
    _want(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32, dv)
    _want(init_state, "init_state", (B, H, P, N), f32, dv)
    _want(y, "y", (T, H, P), x.dtype, dv)
    _want(final_state, "final_state", (B, H, P, N), f32, dv)
    _want(dt_bias, "dt_bias", (H,), f32, dv)
    if y is None:
        y = torch.empty_like(x)
    if final_state is None:
        final_state = torch.empty((B, H, P, N), dtype=torch.float32, device=x.device)
    nws = lib().ssd_prefill_varlen_workspace_bytes(B, T, H, P, G, N, Q, code)
    if nws == ctypes.c_size_t(-1).value:
        raise ValueError("ssd_prefill_varlen would reject these arguments")
    _want_workspace(workspace, nws, dv)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if dt_raw:
        rc = lib().ssd_prefill_varlen_dt_raw(B, T, H, P, G, N, Q, code, _ptr(cu_seqlens), _ptr(x), _ptr(dt),
                                             _ptr(dt_bias), float(dt_min), float(dt_max), _ptr(A_log), _ptr(Bm),
                                             _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state),
                                             _ptr(workspace), ws_bytes, _stream(stream))
        _check("ssd_prefill_varlen_dt_raw", rc)
    else:
        rc = lib().ssd_prefill_varlen(B, T, H, P, G, N, Q, code, _ptr(cu_seqlens), _ptr(x), _ptr(dt), _ptr(A_log),
                                      _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state),
                                      _ptr(workspace), ws_bytes, _stream(stream))
        _check("ssd_prefill_varlen", rc)
    return y, final_state


def ssd_decode_step(x_t, dt_t, A_log, B_t, C_t, D, ssm_state, *, y_t=None, in_stride=0,
                    conv_state_in=None, conv_state_out=None, conv_w=None, conv_b=None,
                    K=4, activation=0, H=None, P=None, G=None, N=None, stream=None,
                    dt_raw=False, dt_bias=None, dt_min=0.0, dt_max=float("inf")):
    """One decode step, in place on ssm_state [B,H,P,N] (and conv_state_out).

    x_t [B,H*P], dt_t [B,H], B_t/C_t [B,G*N] (or views into one [B,C] row with
    ``in_stride`` = C).  With ``dt_raw`` the step is clamp(softplus(dt_t +
    dt_bias), dt_min, dt_max) (ssd_decode_step_dt_raw).  Returns y_t [B,H,P]."""
    if ssm_state.dim() != 4:
        raise ValueError("ssm_state must be [B,H,P,N]")
    Bsz, H_, P_, N_ = ssm_state.shape
    if (H or H_, P or P_, N or N_) != (H_, P_, N_):
        raise ValueError(f"H, P, N given as {(H, P, N)} but ssm_state is {tuple(ssm_state.shape)}")
    H, P, N = H_, P_, N_
    G = G or (B_t.numel() // (Bsz * N) if in_stride == 0 else None)
    if G is None:
        raise ValueError("G must be given when in_stride is set")
    code = _dtype_code(x_t)
    f32, dv, adt = torch.float32, x_t.device, x_t.dtype
    stride = int(in_stride)
    _want_rows(x_t, "x_t", Bsz, H * P, adt, dv, stride)
    _want_rows(B_t, "B_t", Bsz, G * N, adt, dv, stride)
    _want_rows(C_t, "C_t", Bsz, G * N, adt, dv, stride)
    _want(dt_t, "dt_t", (Bsz, H), f32, dv)
    _want(A_log, "A_log", (H,), f32, dv)
    _want(D, "D", (H,), f32, dv)
    _want(ssm_state, "ssm_state", (Bsz, H, P, N), f32, dv)
    _want(y_t, "y_t", (Bsz, H, P), adt, dv)
    _want(dt_bias, "dt_bias", (H,), f32, dv)
    if conv_state_in is not None:
        C = H * P + 2 * G * N
        _want(conv_state_in, "conv_state_in", (Bsz, C, int(K) - 1), adt, dv)
        if conv_state_out is None or conv_w is None:
            raise ValueError("conv_state_out and conv_w are needed with conv_state_in")
        _want(conv_state_out, "conv_state_out", (Bsz, C, int(K) - 1), adt, dv)
        _want(conv_w, "conv_w", (C, int(K)), adt, dv)
        _want(conv_b, "conv_b", (C,), adt, dv)
    if y_t is None:
        y_t = torch.empty((Bsz, H, P), dtype=x_t.dtype, device=x_t.device)
    if dt_raw:
        rc = lib().ssd_decode_step_dt_raw(Bsz, H, P, G, N, code, _ptr(x_t), _ptr(dt_t), _ptr(dt_bias),
                                          float(dt_min), float(dt_max), _ptr(A_log), _ptr(B_t), _ptr(C_t),
                                          _ptr(D), _ptr(ssm_state), _ptr(y_t), int(in_stride),
                                          _ptr(conv_state_in), _ptr(conv_state_out), _ptr(conv_w),
                                          _ptr(conv_b), int(K), int(activation), _stream(stream))
        _check("ssd_decode_step_dt_raw", rc)
    else:
        if dt_bias is not None:
            raise ValueError("dt_bias is used only with dt_raw=True")
        rc = lib().ssd_decode_step(Bsz, H, P, G, N, code, _ptr(x_t), _ptr(dt_t), _ptr(A_log), _ptr(B_t),
                                   _ptr(C_t), _ptr(D), _ptr(ssm_state), _ptr(y_t), int(in_stride),
                                   _ptr(conv_state_in), _ptr(conv_state_out), _ptr(conv_w), _ptr(conv_b),
                                   int(K), int(activation), _stream(stream))
        _check("ssd_decode_step", rc)
    return y_t


def conv_state_update(conv_state, xBC, conv_w, conv_b=None, *, activation=0, out=None,
                      want_out=True, stream=None):
    """Depthwise causal conv over T tokens; conv_state [B,C,K-1] updated in
    place.  xBC [B,T,C], conv_w [C,K].  Returns out [B,T,C] (or None)."""
    if conv_state.dim() != 3 or xBC.dim() != 3:
        raise ValueError("conv_state must be [B,C,K-1] and xBC [B,T,C]")
    B, C, Km1 = conv_state.shape
    T = xBC.shape[1]
    code = _dtype_code(conv_state)
    adt, dv = conv_state.dtype, conv_state.device
    _want(conv_state, "conv_state", (B, C, Km1), adt, dv)
    _want(xBC, "xBC", (B, T, C), adt, dv)
    _want(conv_w, "conv_w", (C, Km1 + 1), adt, dv)
    _want(conv_b, "conv_b", (C,), adt, dv)
    _want(out, "out", (B, T, C), adt, dv)
    if out is None and want_out:
        out = torch.empty_like(xBC)
    rc = lib().conv_state_update(B, T, C, Km1 + 1, code, _ptr(conv_state), _ptr(xBC), _ptr(conv_w),
                                 _ptr(conv_b), int(activation), _ptr(out), _stream(stream))
    _check("conv_state_update", rc)
    return out


def _row_stride(t, D, name):
    """Element stride between consecutive rows of t viewed as [rows, D]
    (channels contiguous, rows evenly spaced)."""
    if t.stride(-1) != 1 or t.shape[-1] != D:
        raise ValueError(f"{name} must have {D} contiguous channels on its last axis")
    if t.dim() == 1:
        return D
    stride = t.stride(-2)
    expect = stride
    for k in range(t.dim() - 2, 0, -1):
        expect *= t.shape[k]
        if t.shape[k - 1] > 1 and t.stride(k - 1) != expect:
            raise ValueError(f"{name}: rows must be evenly spaced")
    return stride


def ssd_gated_rmsnorm(y, z=None, norm_w=None, *, group, eps=1e-5, out=None, stream=None):
    """out = y * silu(z) scaled per group of ``group`` channels to unit RMS
    (plus eps) and by norm_w (fp32 [D]).  y [..., D] contiguous; z of y's
    shape with contiguous channels and evenly spaced rows (a column slice of
    a wider projection is fine) or None; out may be y (in place)."""
    _dense(y, "y")
    _dense(norm_w, "norm_w")
    D = y.shape[-1]
    rows = y.numel() // D if D else 0
    z_stride = 0
    if z is not None:
        if tuple(z.shape) != tuple(y.shape) or z.dtype != y.dtype:
            raise ValueError("z must match y's shape and dtype")
        z_stride = _row_stride(z, D, "z")
    if norm_w is not None and (norm_w.dtype != torch.float32 or tuple(norm_w.shape) != (D,)):
        raise ValueError("norm_w must be fp32 [D]")
    _want(out, "out", tuple(y.shape), y.dtype, y.device)
    if out is None:
        out = torch.empty_like(y)
    rc = lib().ssd_gated_rmsnorm(rows, D, int(group), _dtype_code(y), _ptr(y), _ptr(z), z_stride, _ptr(norm_w),
                                 float(eps), _ptr(out), _stream(stream))
    _check("ssd_gated_rmsnorm", rc)
    return out


def conv_state_update_varlen(conv_state, xBC, cu_seqlens, conv_w, conv_b=None, *, activation=0, out=None,
                             want_out=True, workspace=None, stream=None):
    """conv_state_update over packed sequences: xBC [T,C], cu_seqlens [B+1]
    int32 on the GPU, conv_state [B,C,K-1] updated in place.  Returns out
    [T,C] (or None)."""
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if conv_state.dim() != 3 or xBC.dim() != 2:
        raise ValueError("conv_state must be [B,C,K-1] and xBC [T,C]")
    B, C, Km1 = conv_state.shape
    T = xBC.shape[0]
    code = _dtype_code(conv_state)
    adt, dv = conv_state.dtype, conv_state.device
    _want(conv_state, "conv_state", (B, C, Km1), adt, dv)
    _want(xBC, "xBC", (T, C), adt, dv)
    _want(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32, dv)
    _want(conv_w, "conv_w", (C, Km1 + 1), adt, dv)
    _want(conv_b, "conv_b", (C,), adt, dv)
    _want(out, "out", (T, C), adt, dv)
    if out is None and want_out:
        out = torch.empty_like(xBC)
    nws = lib().conv_state_update_varlen_workspace_bytes(B, T)
    _want_workspace(workspace, nws, dv)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=xBC.device)
    rc = lib().conv_state_update_varlen(B, T, C, Km1 + 1, code, _ptr(cu_seqlens), _ptr(conv_state), _ptr(xBC),
                                        _ptr(conv_w), _ptr(conv_b), int(activation), _ptr(out), _ptr(workspace),
                                        0 if workspace is None else workspace.numel(), _stream(stream))
    _check("conv_state_update_varlen", rc)
    return out


def ssd_status_string(status: int) -> str:
    return lib().ssd_status_string(status).decode()


def ssd_last_hip_error() -> int:
    return lib().ssd_last_hip_error()


def debug_handoff_ticks(ticks: int) -> None:
    """Bound of the chained prefill's hand-off waits for later calls of this
    thread, in 100 MHz device ticks; negative restores the default (0.2 s)."""
    _check("ssd_debug_handoff_ticks", lib().ssd_debug_handoff_ticks(int(ticks)))


def debug_handoff_jitter(max_rounds: int) -> None:
    """Random delays (0 .. max_rounds rounds of s_sleep 8 per point) at the
    chained prefill's hand-off points for later calls of this thread; 0 = off."""
    _check("ssd_debug_handoff_jitter", lib().ssd_debug_handoff_jitter(int(max_rounds)))


def debug_packed_form(form: int) -> None:
    """Form of later packed prefills of this thread that may take the chained
    pass: -1 = chosen on the device from the lengths, 0 = four-kernel, 1 = chained."""
    _check("ssd_debug_packed_form", lib().ssd_debug_packed_form(int(form)))


def stage_timing(enable: bool) -> None:
    """Turn per-kernel event timing of later ssd_prefill calls (this thread) on or off."""
    _check("ssd_stage_timing", lib().ssd_stage_timing(1 if enable else 0))


def stage_times() -> list:
    """[(kernel name, ms)] of the last timed ssd_prefill call, after waiting for it."""
    cap = 16
    ms = (ctypes.c_float * cap)()
    n = _i(0)
    _check("ssd_stage_times", lib().ssd_stage_times(ms, cap, ctypes.byref(n)))
    return [(lib().ssd_stage_name(i).decode(), float(ms[i])) for i in range(min(n.value, cap))]
