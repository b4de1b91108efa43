"""Seeded synthetic inputs shaped like Mamba-2 SSD layers.

This module draws random numbers and nothing else: it holds none of the scan's
arithmetic, and both the HIP path and the CPU oracle take their inputs from
it.  Values are drawn with numpy's PCG64 (``default_rng(seed)``) in a fixed
order, as float32, and rounded to bfloat16 with round-to-nearest-even (torch
``.to(torch.bfloat16)``) where a workload is bf16.

Distributions (``N(mu, v)`` has variance ``v``):
    x      ~ N(0, 1)
    dt     =  clip(softplus(N(-1, 0.5)), 1e-3, 0.1)   (already discretised)
    A_log  ~ U(0, ln 16), so A = -exp(A_log) lies in [-16, -1]
    Bm, Cm ~ N(0, 1/N)
    D      ~ N(0, 1)
    conv_w ~ N(0, 0.02),  raw conv inputs ~ N(0, 1)
    dt_raw ~ N(0, 1), dt_bias ~ U(ln 1e-3, ln 0.1)   (raw step-size projection)
    z ~ N(0, 1), norm_w ~ U(0.5, 1.5)   (gate branch and normalisation weight)
    packed sequence lengths: log-uniform in [lo, hi]
Variants: "spec" (as above), "d0" (D = 0, so the output is the SSM term
alone), "slow" (A_log ~ U(-7, -4) and dt = 1e-3, so state survives across
thousands of tokens and every chunk hand-off matters), "steep" (A_log ~
U(0, ln 64) and dt = clip(softplus(N(0.5, 0.5)), 0.05, 3), so some heads decay
by up to ~190 per token and others by ~1), "dtzero" (as "spec" but dt = 0 on
every token t with t % 5 == 3).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

VARIANTS = ("spec", "d0", "slow", "steep", "dtzero")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    H: int
    P: int
    N: int
    G: int
    Q: int
    dtype: str  # "f32" or "bf16": storage type of x, Bm, Cm, y (and conv data)
    K: int = 4  # depthwise conv width
    decode_steps: int = 0

    @property
    def conv_channels(self) -> int:
        return self.H * self.P + 2 * self.G * self.N


# Workloads of the pages' problem statement, named by shape.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("ssd-f32-tiny", 1, 256, 2, 16, 16, 1, 64, "f32", decode_steps=16),
        Workload("mamba2-130m-prefill", 1, 4096, 24, 64, 128, 1, 256, "bf16"),
        Workload("mamba2-2.7b-prefill", 1, 4096, 80, 64, 128, 1, 256, "bf16"),
        Workload("mamba2-2.7b-decode-b1", 1, 4096, 80, 64, 128, 1, 256, "bf16", decode_steps=4096),
        Workload("mamba2-2.7b-decode-b16", 16, 4096, 80, 64, 128, 1, 256, "bf16", decode_steps=4096),
        Workload("mamba2-130m-decode-b1", 1, 4096, 24, 64, 128, 1, 256, "bf16", decode_steps=4096),
        Workload("mamba2-130m-decode-b16", 16, 4096, 24, 64, 128, 1, 256, "bf16", decode_steps=4096),
        Workload("mamba2-2.7b-longctx", 8, 16384, 80, 64, 128, 1, 256, "bf16", decode_steps=1024),
        # one long sequence: the four-kernel form (80 chains) at 256 chunks each
        Workload("mamba2-2.7b-prefill-64k", 1, 65536, 80, 64, 128, 1, 256, "bf16"),
    ]
}


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _normal(rng, shape, var=1.0, mean=0.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        a *= np.float32(math.sqrt(var))
    if mean != 0.0:
        a += np.float32(mean)
    return a


def _dt(rng, shape):
    z = rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64)
    z = -1.0 + math.sqrt(0.5) * z
    sp = np.logaddexp(0.0, z)  # softplus, computed stably
    return np.clip(sp, 1e-3, 0.1).astype(np.float32)


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch_dtype(dtype)) if dtype != "f32" else t


def make_prefill(B, L, H, P, G, N, dtype="f32", seed=0, variant="spec"):
    """Inputs of one prefill call as CPU tensors.

    Returns dict(x [B,L,H,P], dt [B,L,H] f32, A_log [H] f32, Bm/Cm [B,L,G,N],
    D [H] f32) with x/Bm/Cm stored in ``dtype``.
    Draw order: x, dt, A_log, Bm, Cm, D.
    """
    if variant not in VARIANTS:
        raise ValueError(variant)
    rng = np.random.default_rng(seed)
    x = _normal(rng, (B, L, H, P))
    dt = _dt(rng, (B, L, H))
    A_log = rng.uniform(0.0, math.log(16.0), size=H).astype(np.float32)
    Bm = _normal(rng, (B, L, G, N), 1.0 / N)
    Cm = _normal(rng, (B, L, G, N), 1.0 / N)
    D = _normal(rng, (H,))
    if variant == "d0":
        D[:] = 0.0
    elif variant == "slow":
        A_log = rng.uniform(-7.0, -4.0, size=H).astype(np.float32)
        dt[:] = np.float32(1e-3)
    elif variant == "steep":
        A_log = rng.uniform(0.0, math.log(64.0), size=H).astype(np.float32)
        z = 0.5 + math.sqrt(0.5) * rng.standard_normal(size=(B, L, H), dtype=np.float32).astype(np.float64)
        dt = np.clip(np.logaddexp(0.0, z), 0.05, 3.0).astype(np.float32)
    elif variant == "dtzero":
        dt[:, 3::5] = np.float32(0.0)
    return dict(
        x=_store(x, dtype), dt=torch.from_numpy(dt), A_log=torch.from_numpy(A_log),
        Bm=_store(Bm, dtype), Cm=_store(Cm, dtype), D=torch.from_numpy(D),
    )


def make_dt_raw(shape, H, seed=0):
    """A raw step-size projection dt_raw [*shape, H] ~ N(0, 1) and a per-head
    bias dt_bias [H] ~ U(ln 1e-3, ln 0.1), both fp32.  With bounds 1e-3 and
    0.1 the preprocessed step lands below, inside and above that range.
    Draw order: dt_raw, dt_bias."""
    rng = np.random.default_rng(seed)
    raw = _normal(rng, tuple(shape) + (H,))
    bias = rng.uniform(math.log(1e-3), math.log(0.1), size=H).astype(np.float32)
    return torch.from_numpy(raw), torch.from_numpy(bias)


def make_gate(shape, D, dtype="f32", seed=0):
    """The gate branch z [*shape, D] ~ N(0, 1) in ``dtype`` and the
    normalisation weight norm_w [D] ~ U(0.5, 1.5) in fp32.
    Draw order: z, norm_w."""
    rng = np.random.default_rng(seed)
    z = _normal(rng, tuple(shape) + (D,))
    w = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    return _store(z, dtype), torch.from_numpy(w)


def make_lengths(nseq, lo, hi, seed=0):
    """Sequence lengths for a packed (varlen) batch: log-uniform in [lo, hi]
    (integers), the mix of prompt lengths a serving batch sees."""
    rng = np.random.default_rng(seed)
    return [int(v) for v in np.exp(rng.uniform(math.log(lo), math.log(hi), size=nseq)).round()]


def make_varlen(lengths, H, P, G, N, dtype="f32", seed=0, variant="spec"):
    """Inputs of a packed prefill: make_prefill of one sequence of sum(lengths)
    tokens, with the batch axis dropped (x [T,H,P], dt [T,H], Bm/Cm [T,G,N]),
    plus cu_seqlens [len(lengths) + 1] int32 (token offsets)."""
    T = int(sum(lengths))
    d = make_prefill(1, T, H, P, G, N, dtype, seed, variant)
    out = {k: (v[0] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in d.items()}
    out["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return out


def make_state(B, H, P, N, seed=0, scale=1.0):
    """A dense fp32 state [B,H,P,N] ~ N(0, scale^2) (for init_state tests)."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(_normal(rng, (B, H, P, N), scale * scale))


def make_conv(C, K, dtype="f32", seed=0, with_bias=False):
    """Depthwise conv weights w [C,K] ~ N(0, 0.02) and optional bias [C]."""
    rng = np.random.default_rng(seed)
    w = _normal(rng, (C, K), 0.02)
    b = _normal(rng, (C,), 0.02) if with_bias else None
    return _store(w, dtype), (None if b is None else _store(b, dtype))


def make_tokens(B, T, C, dtype="f32", seed=0):
    """Raw (pre-convolution) channel inputs xBC [B,T,C] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    return _store(_normal(rng, (B, T, C)), dtype)


def make_decode_stream(steps, B, H, P, G, N, dtype="f32", seed=0, variant="spec"):
    """Per-step decode inputs: raw xBC tokens [steps,B,C] ~ N(0,1) (channels
    x | B | C) and dt [steps,B,H].  With variant "slow", dt = 1e-3."""
    rng = np.random.default_rng(seed)
    C = H * P + 2 * G * N
    xbc = _normal(rng, (steps, B, C))
    dt = _dt(rng, (steps, B, H))
    if variant == "slow":
        dt[:] = np.float32(1e-3)
    return _store(xbc, dtype), torch.from_numpy(dt)
