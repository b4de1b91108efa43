"""Plain CPU oracle for the Mamba-2 SSD layer scan (fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and it imports nothing from the HIP side.

What it computes (arXiv 2603.09555, "Compiler-First State Space Duality and
Portable O(1) Autoregressive Caching for Inference"; abstract, and the
bqwf.cn article on the compiler-first Mamba-2 implementation §1.1, §2.1,
§2.2): the per-token recurrence, for every batch element b and head h,

    h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t        [P x N]
    y_t = h_t . C_t + D_h * x_t                                      [P]

with A_h = -exp(A_log[h]), plus the depthwise causal convolution over a
(K-1)-token window cache and the step-size chain dt = clip(softplus(dt_raw +
dt_bias), dt_min, dt_max) of §1.2 (``dt_from_raw``), and the layer's closing
gated RMS normalisation of §3.2 and §4.1 (``gated_rmsnorm``).  ``ssd_scan`` is the
prefill (``ssd_scan_varlen`` the same per packed sequence), ``decode_step`` is
one step of the same recurrence after one step of the convolution cache.

All arithmetic is in C (``ssd_oracle.c``), double precision, token by token.
Every function here only marshals arrays.  Pins that tie this oracle to the
pages and to mathematics live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_LIB names a prebuilt copy (the sanitizer build the tests also run
# the pins against); by default the in-tree build, compiled on demand.
_ENV_LIB = os.environ.get("SSD_ORACLE_LIB")
_LIB_PATH = _ENV_LIB or os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build_sanitized(out: str) -> str:
    """Compile ssd_oracle.c with clang's AddressSanitizer and
    UndefinedBehaviorSanitizer (any finding aborts) into `out`; load it by
    setting SSD_ORACLE_LIB, with clang's ASan runtime preloaded."""
    subprocess.check_call(
        ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-Wall", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", out, _SRC, "-lm", "-lpthread"]
    )
    return out


def build(force: bool = False) -> str:
    """Compile ssd_oracle.c with gcc -O2 (no fast-math) into libssd_oracle.so
    (nothing to do when SSD_ORACLE_LIB names a prebuilt copy)."""
    if _ENV_LIB:
        if not os.path.exists(_ENV_LIB):
            raise FileNotFoundError(f"SSD_ORACLE_LIB={_ENV_LIB} does not exist")
        return _ENV_LIB
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm", "-lpthread"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_ssd_scan.restype = ctypes.c_int
        lib.oracle_ssd_scan.argtypes = [ctypes.c_int] * 6 + [_dp] * 9 + [ctypes.c_int]
        lib.oracle_conv_update.restype = ctypes.c_int
        lib.oracle_conv_update.argtypes = [ctypes.c_int] * 4 + [_dp] * 4 + [ctypes.c_int, _dp]
        lib.oracle_dt_from_raw.restype = ctypes.c_int
        lib.oracle_dt_from_raw.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, ctypes.c_double,
                                           ctypes.c_double, _dp]
        lib.oracle_gated_rmsnorm.restype = ctypes.c_int
        lib.oracle_gated_rmsnorm.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _dp, _dp, ctypes.c_long,
                                             _dp, ctypes.c_double, _dp]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    """Exact widening to a C-contiguous float64 array (None passes through)."""
    if a is None:
        return None
    try:
        import torch

        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def ssd_scan(x, dt, A_log, Bm, Cm, D=None, init_state=None, *, want_y=True,
             nthreads=None):
    """Sequential SSD recurrence over a whole sequence (the prefill).

    x [B,L,H,P], dt [B,L,H], A_log [H], Bm/Cm [B,L,G,N], D [H] or None (0),
    init_state [B,H,P,N] or None (0).  Returns (y [B,L,H,P] or None,
    final_state [B,H,P,N]) as float64 arrays.
    """
    x, dt, A_log, Bm, Cm = map(_f64, (x, dt, A_log, Bm, Cm))
    D, init_state = _f64(D), _f64(init_state)
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert dt.shape == (Bsz, L, H) and A_log.shape == (H,)
    assert Bm.shape == (Bsz, L, G, N) and Cm.shape == (Bsz, L, G, N)
    assert D is None or D.shape == (H,)
    assert init_state is None or init_state.shape == (Bsz, H, P, N)
    y = np.empty((Bsz, L, H, P), np.float64) if want_y else None
    fs = np.empty((Bsz, H, P, N), np.float64)
    rc = _load().oracle_ssd_scan(
        Bsz, L, H, P, G, N, _ptr(x), _ptr(dt), _ptr(A_log), _ptr(Bm), _ptr(Cm),
        _ptr(D), _ptr(init_state), _ptr(y), _ptr(fs),
        int(nthreads or default_threads()),
    )
    if rc != 0:
        raise ValueError(f"oracle_ssd_scan failed ({rc})")
    return y, fs


def ssd_scan_varlen(x, dt, A_log, Bm, Cm, cu_seqlens, D=None, init_state=None, *, nthreads=None):
    """The prefill of sequences packed without padding: sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1] of x [T,H,P], dt [T,H], Bm/Cm [T,G,N],
    scanned on its own from init_state[b] (or 0) by ``ssd_scan``.

    Returns (y [T,H,P], final_state [B,H,P,N]) as float64 arrays.
    """
    x, dt, Bm, Cm = map(_f64, (x, dt, Bm, Cm))
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    T, H, P = x.shape
    N = Bm.shape[2]
    nseq = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and all(a <= b for a, b in zip(cu, cu[1:]))
    init = _f64(init_state)
    y = np.empty((T, H, P), np.float64)
    fs = np.empty((nseq, H, P, N), np.float64)
    for b in range(nseq):
        lo, hi = cu[b], cu[b + 1]
        yb, fs[b:b + 1] = ssd_scan(x[None, lo:hi], dt[None, lo:hi], A_log, Bm[None, lo:hi], Cm[None, lo:hi], D,
                                   None if init is None else init[b:b + 1], nthreads=nthreads)
        y[lo:hi] = yb[0]
    return y, fs


def dt_from_raw(dt_raw, dt_bias=None, dt_min=0.0, dt_max=float("inf")):
    """Step size from a raw projection: clip(softplus(dt_raw + dt_bias[h]),
    dt_min, dt_max), the softplus -> clip chain of bqwf.cn §1.2.

    dt_raw [..., H] (any leading shape), dt_bias [H] or None (0).  Returns a
    float64 array of dt_raw's shape.
    """
    raw = _f64(dt_raw)
    H = raw.shape[-1]
    bias = _f64(dt_bias)
    assert bias is None or bias.shape == (H,)
    out = np.empty_like(raw)
    rc = _load().oracle_dt_from_raw(raw.size // H, H, _ptr(raw), _ptr(bias), float(dt_min), float(dt_max),
                                    _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_dt_from_raw failed ({rc})")
    return out


def gated_rmsnorm(y, z=None, w=None, *, group, eps=1e-5):
    """The layer's closing normalisation, gated RMS form (bqwf.cn §3.2,
    §4.1): g = y * silu(z), then each group of ``group`` consecutive channels
    of the last axis is divided by sqrt(mean(g^2) + eps) and multiplied by w.

    y [..., D], z [..., D] or None (no gate), w [D] or None (1).  Returns a
    float64 array of y's shape.
    """
    y = _f64(y)
    D = y.shape[-1]
    z, w = _f64(z), _f64(w)
    assert z is None or z.shape == y.shape
    assert w is None or w.shape == (D,)
    out = np.empty_like(y)
    rc = _load().oracle_gated_rmsnorm(y.size // D, D, int(group), _ptr(y), _ptr(z), D, _ptr(w), float(eps),
                                      _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_gated_rmsnorm failed ({rc})")
    return out


def conv_update(conv_state, xBC, w, bias=None, activation=False):
    """Depthwise causal conv over T new tokens with a (K-1)-token cache.

    conv_state [B,C,K-1] (index K-2 newest), xBC [B,T,C], w [C,K], bias [C].
    Returns (new_state [B,C,K-1], out [B,T,C]) as float64; inputs unchanged.
    """
    st = _f64(conv_state).copy()
    xBC, w, bias = _f64(xBC), _f64(w), _f64(bias)
    Bsz, C, Km1 = st.shape
    T = xBC.shape[1]
    assert xBC.shape == (Bsz, T, C) and w.shape == (C, Km1 + 1)
    out = np.empty((Bsz, T, C), np.float64)
    rc = _load().oracle_conv_update(Bsz, T, C, Km1 + 1, _ptr(st), _ptr(xBC), _ptr(w),
                                    _ptr(bias), int(bool(activation)), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv_update failed ({rc})")
    return st, out


def conv_update_varlen(conv_state, xBC, cu_seqlens, w, bias=None, activation=False):
    """``conv_update`` per packed sequence: sequence b is rows cu_seqlens[b]
    .. cu_seqlens[b+1] of xBC [T,C] and starts from conv_state[b] [C,K-1].
    Returns (new_state [B,C,K-1], out [T,C]) as float64."""
    st = _f64(conv_state)
    xBC = _f64(xBC)
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    assert cu[0] == 0 and cu[-1] == xBC.shape[0] and all(a <= b for a, b in zip(cu, cu[1:]))
    new = np.empty_like(st)
    out = np.empty_like(xBC)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        nb, ob = conv_update(st[b:b + 1], xBC[None, lo:hi], w, bias, activation)
        new[b] = nb[0]
        out[lo:hi] = ob[0]
    return new, out


def decode_step(x_t, dt_t, A_log, B_t, C_t, D, ssm_state, *, conv_state=None,
                conv_w=None, conv_b=None, activation=False, nthreads=None):
    """One cached decode step: conv window step (optional), then one token of
    the recurrence from ``ssm_state``.

    x_t [B,H*P], dt_t [B,H], B_t/C_t [B,G*N], ssm_state [B,H,P,N].  With
    ``conv_state`` [B,C,K-1] (C = H*P + 2*G*N, channels ordered x | B | C),
    x_t/B_t/C_t are the raw pre-convolution inputs.
    Returns (y_t [B,H,P], new_ssm_state, new_conv_state or None).
    """
    ssm_state = _f64(ssm_state)
    Bsz, H, P, N = ssm_state.shape
    x_t, B_t, C_t = _f64(x_t), _f64(B_t), _f64(C_t)
    G = B_t.shape[1] // N
    new_conv = None
    if conv_state is not None:
        xbc = np.concatenate([x_t, B_t, C_t], axis=1)[:, None, :]
        new_conv, out = conv_update(conv_state, xbc, conv_w, conv_b, activation)
        out = out[:, 0, :]
        x_t, B_t, C_t = out[:, :H * P], out[:, H * P:H * P + G * N], out[:, H * P + G * N:]
    y, fs = ssd_scan(
        x_t.reshape(Bsz, 1, H, P), _f64(dt_t).reshape(Bsz, 1, H), A_log,
        B_t.reshape(Bsz, 1, G, N), C_t.reshape(Bsz, 1, G, N), D, ssm_state,
        nthreads=nthreads,
    )
    return y[:, 0], fs, new_conv
