"""Float64 emulation of where the bf16 backward rounds (test infrastructure: the tolerance
model of tests/test_parity_bwd_gpu.py; CPU only).

The library's backward (fixed feature map, causal sets) rounds to bf16 at these points,
and computes everything else in fp32. The emulation repeats the chain rule of y = sum_j
w_ij v_j / den_i (the same one the oracle writes out) with the same rounding points, in
float64 otherwise:
  * dy and g = dy / den, as MFMA operands;
  * phi(k) where it enters the forward state S_t = sum phi(k) v^T (and z_t = sum phi(k));
  * the states S_t and the reverse states G when they become MFMA operands;
  * phi(q) where it enters G = sum phi(q) g^T (and h = sum phi(q) c);
  * the softmax weights p (for dv) and their gradients ds (for dq and dk);
  * phi(k) where it enters dv += G^T phi(k);
  * the feature gradients times the map slope, gq and gk, where they enter dq, dk and dW.
Its distance to the exact oracle estimates the rounding error the kernels should show;
den and y are taken exact (the forward's own rounding is not emulated).
"""
from __future__ import annotations

import math

import numpy as np

import oracle as orc


def r16(x):
    """Round to the nearest bf16 (ties to even), returned as float64."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def backward_bf16(q, k, v, Wq, Wk, dy, *, HW, Tc, To, rows=None, keys=None):
    """dq, dk, dv, dWq, dWk with the kernels' bf16 rounding points (causal sets).

    rows / keys: optional subsets; then only dq of those query rows and dk, dv of those keys
    are formed (the rest is NaN) and dW is not returned."""
    q, k, v, dy = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dy))
    Wq, Wk = np.asarray(Wq, dtype=np.float64), np.asarray(Wk, dtype=np.float64)
    N, D = q.shape
    T = N // HW
    s = 1.0 / math.sqrt(D)
    uq, uk = q @ Wq * s, k @ Wk * s
    phq, phk = 1 + uq + 0.5 * uq * uq, 1 + uk + 0.5 * uk * uk
    layout = orc.chunk_layout(T, HW, Tc, To)
    # exact forward quantities
    den = np.zeros(N)
    y = np.zeros_like(q)
    for (r0, r1, lo, hi) in layout:
        ES = np.exp(q[r0:r1] @ k[lo:hi].T * s)
        EL = phq[r0:r1] @ phk[:lo].T
        den[r0:r1] = ES.sum(1) + EL.sum(1)
        y[r0:r1] = (ES @ v[lo:hi] + EL @ v[:lo]) / den[r0:r1, None]
    dyb = r16(dy)
    g = r16(dy / den[:, None])
    dd = (dy * y).sum(1)
    c = dd / den
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    F = Wq.shape[1]
    gq, gk = np.zeros((N, F)), np.zeros((N, F))
    row_on = np.ones(N, dtype=bool) if rows is None else np.isin(np.arange(N), rows)
    key_on = np.ones(N, dtype=bool) if keys is None else np.isin(np.arange(N), keys)
    # window part (rows of P for the dq rows asked for, columns for the keys)
    for (r0, r1, lo, hi) in layout:
        ri = np.nonzero(row_on[r0:r1])[0] + r0
        kj = np.nonzero(key_on[lo:hi])[0] + lo
        if ri.size:
            P = np.exp(q[ri] @ k[lo:hi].T * s) / den[ri, None]
            ds = r16(P * (dyb[ri] @ v[lo:hi].T - dd[ri, None]) * s)
            dq[ri] += ds @ k[lo:hi]
        if kj.size:
            P = np.exp(q[r0:r1] @ k[kj].T * s) / den[r0:r1, None]
            ds = r16(P * (dyb[r0:r1] @ v[kj].T - dd[r0:r1, None]) * s)
            dk[kj] += ds.T @ q[r0:r1]
            dv[kj] += r16(P).T @ dyb[r0:r1]
    # linear part, query side: forward states from bf16 phi(k)
    pk16 = r16(phk)
    for (r0, r1, lo, hi) in layout:
        if lo == 0:
            continue
        S = r16(pk16[:lo].T @ v[:lo])
        z = pk16[:lo].sum(0)
        dphi = g[r0:r1] @ S.T - c[r0:r1, None] * z
        gq[r0:r1] = r16(dphi * (1 + uq[r0:r1]) * s)
    dq += gq @ Wq.T
    # reverse states and the key side
    pq16 = r16(phq)
    for f in range(T):
        f0 = Tc * ((f + 1 + To + Tc - 1) // Tc)
        a, b = f * HW, (f + 1) * HW
        if f0 >= T:
            Gm, h = np.zeros((F, D)), np.zeros(F)
        else:
            Gm = pq16[f0 * HW:].T @ g[f0 * HW:]
            h = pq16[f0 * HW:].T @ c[f0 * HW:]
        G16 = r16(Gm)
        dpsi = v[a:b] @ G16.T - h
        gk[a:b] = r16(dpsi * (1 + uk[a:b]) * s)
        dv[a:b] += r16(phk[a:b]) @ G16
    dk += gk @ Wk.T
    dq[~row_on] = np.nan
    dk[~key_on] = np.nan
    dv[~key_on] = np.nan
    out = {"dq": dq, "dk": dk, "dv": dv}
    if rows is None and keys is None:
        out["dWq"], out["dWk"] = q.T @ gq, k.T @ gk
    return out
