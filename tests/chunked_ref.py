"""Chunked SSD in numpy fp64, written from the algebra (tests only).

This is NOT the oracle.  It is an independent check of the decomposition the
GPU path uses, so that the oracle's sequential recurrence and the chunked form
can be compared with each other (chunk-size invariance), and so that the GPU's
per-stage outputs have a reference.  Sources: bqwf.cn article on the
compiler-first Mamba-2 implementation, §1.1 (fixed-size chunks, parallel
matrix work inside a chunk, a light sequential scan between chunks; decay
matrix L = tril(exp(segsum(log A)))) and §1.2 (the intra-chunk einsum
Y = einsum('bclhn,bcshn,bhcls,bcshp->bclhp', C, B, L, X), where X is the
discretised input dt * x).

For one chunk with local index l, s in [0, Qc):
    a_l      = dt_l * A_h;        cs_l = sum_{j <= l} a_j           (a1)
    Y_diag   = ((C B^T) o Lmat) (dt o X),  Lmat[l,s] = exp(cs_l - cs_s), l >= s
                                                                   (a2)
    S_c      = sum_s exp(cs_last - cs_s) dt_s x_s (outer) B_s       (a3)
    h_c      = exp(cs_last) h_{c-1} + S_c                           (a4)
    y        = Y_diag + exp(cs_l) C_l . h_{c-1} + D x               (a5)
"""
from __future__ import annotations

import numpy as np


def chunked_ssd(x, dt, A_log, Bm, Cm, D=None, init_state=None, Q=64, want_stages=False):
    x, dt, A_log, Bm, Cm = (np.asarray(a, np.float64) for a in (x, dt, A_log, Bm, Cm))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2:]
    hpg = H // G
    A = -np.exp(A_log)
    Bh = np.repeat(Bm, hpg, axis=2)  # [B,L,H,N], head h uses group h // hpg
    Ch = np.repeat(Cm, hpg, axis=2)
    h = np.zeros((Bsz, H, P, N)) if init_state is None else np.array(init_state, np.float64)
    y = np.zeros_like(x)
    stages = {"cs": [], "S": [], "h_in": []}
    for c0 in range(0, L, Q):
        c1 = min(L, c0 + Q)
        a = dt[:, c0:c1, :] * A                      # [B,Qc,H]
        cs = np.cumsum(a, axis=1)                    # inclusive
        diff = cs[:, :, None, :] - cs[:, None, :, :]  # [B,l,s,H]
        Qc = c1 - c0
        mask = np.tril(np.ones((Qc, Qc), bool))[None, :, :, None]
        Lmat = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
        Xd = dt[:, c0:c1, :, None] * x[:, c0:c1]     # dt o X  [B,Qc,H,P]
        CB = np.einsum("blhn,bshn->blsh", Ch[:, c0:c1], Bh[:, c0:c1])
        y_diag = np.einsum("blsh,bshp->blhp", CB * Lmat, Xd)
        y_off = np.exp(cs)[..., None] * np.einsum("blhn,bhpn->blhp", Ch[:, c0:c1], h)
        w = np.exp(cs[:, -1:, :] - cs)               # [B,Qc,H]
        S = np.einsum("bsh,bshp,bshn->bhpn", w, Xd, Bh[:, c0:c1])
        if want_stages:
            stages["cs"].append(cs)
            stages["S"].append(S)
            stages["h_in"].append(h.copy())
        y[:, c0:c1] = y_diag + y_off
        h = np.exp(cs[:, -1, :])[:, :, None, None] * h + S
    if D is not None:
        y += np.asarray(D, np.float64)[None, None, :, None] * x
    if want_stages:
        return y, h, stages
    return y, h
