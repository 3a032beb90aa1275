"""Plain float64 oracle of ReHyAt hybrid attention (test infrastructure only).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg; never by the library. Shares no code with the HIP path.

Source: the papernotes.org note "ReHyAt: Recurrent Hybrid Attention for Video Diffusion
Transformers" (CVPR 2026), section "method details", key designs 1, 2 and 4. Notation:

  N  = T*HW tokens, time-major (token f*HW + s is spatial position s of frame f);
  N' = Tc*HW tokens per chunk; the queries of chunk t are rows [t*N', min((t+1)*N', N)).
  Softmax key set of chunk t (key design 2, overlapped set):
        S_t = [lo_t, hi_t),  lo_t = max(t*N' - To*HW, 0),  hi_t = min((t+1)*N', N).
  Linear key set (key design 4, causal):          L_t = [0, lo_t)
               (key design 1, bidirectional):     L_t = [0, lo_t) U [hi_t, N)
                                                  (the complement of the overlapped window).
  Branches (key design 1):  a^S = sum_{j in S_t} exp(q.k_j/sqrt(D)) v_j,  n^S = sum exp(.)
                            a^L = sum_{j in L_t} (phi(q).phi(k_j)) v_j,   n^L = sum phi.phi
  Joint normalisation (key design 1):  y = (a^S + a^L) / (n^S + n^L).
  Feature map used throughout: phi(x)_i = 1 + u_i + u_i^2/2 with u = x W / sqrt(D),
  W a D x F matrix (x a row vector). It is strictly positive: 1+u+u^2/2 = ((1+u)^2+1)/2 >= 1/2.

Readings where the page is silent or inconsistent (each is also listed with its reason in
the design notes of the repository):
  * The softmax stabiliser c_t of key design 1 sits in the softmax branch only, so under the
    joint normalisation it is not result-neutral; the oracle uses the unstabilised form
    (c_t = 0). Any running max used by an implementation must be compensated exactly.
  * n^S and n^L are the sums of the branch weights (the denominators of the recurrence in
    key design 4 are n^S + phi(q) z_t with z_t = sum phi(k_j)).
  * The recurrence of key design 4 as printed adds the whole softmax set S_t to the state;
    with To > 0 that counts the overlap frames in both branches, contradicting the causal
    linear set. The oracle follows the sets: after chunk t the state holds exactly the keys
    j < lo_{t+1}, i.e. s_{t+1} = s_t + sum over [lo_t, lo_{t+1}). For To = 0 this is the
    printed recurrence.
  * No mask inside a chunk: the softmax window is bidirectional, overlap frames included.
  * A last chunk shorter than Tc frames (T not a multiple of Tc) keeps hi = N.

Feature maps. Every function below takes the feature map of the queries and of the keys
as its Wq / Wk arguments: a D x F matrix W selects the fixed map phi(x) = 1 + u + u^2/2,
u = x W / sqrt(D) (per head: an [H, D, F] array); a feature-map object (or one per head)
selects that map. Key design 3 gives two more:
  * EluFeatureMap: 1 + elu(x), elementwise (F = D), the fixed map of earlier linear
    attention that the note compares against.
  * PolyMlpFeatureMap, the learned polynomial map. Reading: the per-head embedding network
    (grouped 1x1 convolution + nonlinearity; "2-layer MLP" in the hyper-parameters) is
    psi(x) = relu(x W1 + b1) W2 + b2 with W1 [D, h], W2 [h, F]; the nonlinearity is not
    named, ReLU is taken. psi is split into P equal parts (degree P = 2 in the note) and
    part i (1-based) is raised elementwise to the power i: phi = [psi_1, psi_2 * psi_2].
    This map can give a negative phi(q).phi(k); the definition is used as it stands.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "chunk_layout", "phi", "hybrid_attention", "hybrid_recurrent",
    "state_direct", "recurrent_init", "recurrent_step", "EluFeatureMap", "PolyMlpFeatureMap",
    "feature", "feature_dim", "hybrid_attention_bwd",
]


def chunk_layout(T: int, HW: int, Tc: int, To: int) -> List[Tuple[int, int, int, int]]:
    """Per chunk t: (row_lo, row_hi, lo_t, hi_t).

    Rows [row_lo, row_hi) are the queries of chunk t (queries are not overlapped, key
    design 2); [lo_t, hi_t) is its overlapped softmax key set (key design 2).
    """
    if min(T, HW, Tc) <= 0 or To < 0:
        raise ValueError("T, HW, Tc must be positive and To non-negative")
    N = T * HW
    Np = Tc * HW
    out = []
    t = 0
    while t * Np < N:
        row_lo = t * Np
        row_hi = min((t + 1) * Np, N)
        lo = max(t * Np - To * HW, 0)
        hi = row_hi
        out.append((row_lo, row_hi, lo, hi))
        t += 1
    return out


def phi(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """phi(x) = 1 + u + u*u/2, u = x W / sqrt(D), rows of x mapped independently."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    D = x.shape[-1]
    u = (x @ W) / math.sqrt(D)
    return 1.0 + u + 0.5 * u * u


class EluFeatureMap:
    """phi(x) = 1 + elu(x) elementwise: x + 1 for x > 0, exp(x) otherwise (F = D)."""

    def __call__(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64)
        return np.where(x > 0, 1.0 + x, np.exp(np.minimum(x, 0.0)))

    def dim(self, D: int) -> int:
        return D


class PolyMlpFeatureMap:
    """Learned polynomial map of key design 3 (reading in the module docstring):
    psi = relu(x W1 + b1) W2 + b2, phi = [psi part i ** i for i = 1 .. P]."""

    def __init__(self, W1, b1, W2, b2, P: int = 2):
        self.W1 = np.asarray(W1, dtype=np.float64)
        self.b1 = np.asarray(b1, dtype=np.float64)
        self.W2 = np.asarray(W2, dtype=np.float64)
        self.b2 = np.asarray(b2, dtype=np.float64)
        self.P = int(P)
        if self.W2.shape[1] % self.P:
            raise ValueError("F must split into P equal parts")

    def __call__(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64)
        hid = np.maximum(x @ self.W1 + self.b1, 0.0)
        psi = hid @ self.W2 + self.b2
        parts = np.split(psi, self.P, axis=-1)
        return np.concatenate([part ** (i + 1) for i, part in enumerate(parts)], axis=-1)

    def dim(self, D: int) -> int:
        return self.W2.shape[1]


def feature(x: np.ndarray, W) -> np.ndarray:
    """Apply the feature map W (a D x F matrix for the fixed map, or a map object)."""
    return W(x) if callable(W) else phi(x, W)


def feature_dim(W, D: int) -> int:
    return W.dim(D) if callable(W) else np.asarray(W).shape[1]


def _linear_ranges(lo: int, hi: int, N: int, causal: bool) -> List[Tuple[int, int]]:
    """Key ranges of the linear set: [0, lo) (causal, key design 4), plus [hi, N) in the
    bidirectional form (complement of the overlapped window, key design 1)."""
    ranges = [(0, lo)] if lo > 0 else []
    if not causal and hi < N:
        ranges.append((hi, N))
    return ranges


def hybrid_attention(q, k, v, Wq, Wk, *, HW: int, Tc: int, To: int, causal: bool = True,
                     rows: Optional[Sequence[int]] = None, block: int = 256,
                     return_stats: bool = False):
    """Hybrid attention of one (batch, head), by the definition, query by query.

    q, k, v: [N, D]; Wq, Wk: [D, F]. For every query the explicit weights over all of its
    keys are formed (exp over the softmax set, phi(q).phi(k) over the linear set) and the
    joint normalisation is applied (key design 1). Queries are processed in blocks of
    `block` rows only to bound memory; nothing else is reordered.

    rows: optional subset of query rows (outputs for other rows are not computed).
    Returns y [len(rows) or N, D] (float64); with return_stats also a dict of the per-row
    numerator/denominator parts nS, nL.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, D = q.shape
    if N % HW:
        raise ValueError("N must be a multiple of HW")
    T = N // HW
    rows_arr = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((rows_arr.size, v.shape[1]), dtype=np.float64)
    nS_out = np.empty(rows_arr.size)
    nL_out = np.empty(rows_arr.size)
    phik = feature(k, Wk)
    inv_sqrt_d = 1.0 / math.sqrt(D)
    for (row_lo, row_hi, lo, hi) in chunk_layout(T, HW, Tc, To):
        sel = np.nonzero((rows_arr >= row_lo) & (rows_arr < row_hi))[0]
        if sel.size == 0:
            continue
        Lr = _linear_ranges(lo, hi, N, causal)
        kS, vS = k[lo:hi], v[lo:hi]
        for b0 in range(0, sel.size, block):
            pos = sel[b0:b0 + block]
            Qb = q[rows_arr[pos]]
            ES = np.exp((Qb @ kS.T) * inv_sqrt_d)          # softmax branch weights, c_t = 0
            num = ES @ vS
            nS = ES.sum(axis=1)
            nL = np.zeros(pos.size)
            if Lr:
                pq = feature(Qb, Wq)
                for (a, b) in Lr:
                    EL = pq @ phik[a:b].T                   # linear branch weights
                    num = num + EL @ v[a:b]
                    nL = nL + EL.sum(axis=1)
            y[pos] = num / (nS + nL)[:, None]
            nS_out[pos] = nS
            nL_out[pos] = nL
    if return_stats:
        return y, {"nS": nS_out, "nL": nL_out}
    return y


def state_direct(k, v, Wk, j_end: int, j_begin: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Recurrent state by its definition (key design 4): the direct sums over keys
    j in [j_begin, j_end) of phi(k_j) v_j^T (an F x D matrix s) and phi(k_j) (z, length F)."""
    k = np.asarray(k, dtype=np.float64)[j_begin:j_end]
    v = np.asarray(v, dtype=np.float64)[j_begin:j_end]
    pk = feature(k, Wk)
    return pk.T @ v, pk.sum(axis=0)


def hybrid_recurrent(q, k, v, Wq, Wk, *, HW: int, Tc: int, To: int,
                     return_states: bool = False):
    """Causal hybrid attention as the chunk-wise RNN of key design 4.

    For chunk t:  y_t = (a^S_t + phi(Q_t) s_t) / (n^S_t + phi(Q_t) z_t), with s_t, z_t the
    state carried from earlier chunks; then the state absorbs the keys that leave reach of
    every later softmax window: s_{t+1} = s_t + sum_{j in [lo_t, lo_{t+1})} phi(k_j) v_j^T
    (and z likewise), so that s_t always equals the sum over the causal linear set
    [0, lo_t). This is an algorithm different from hybrid_attention (state hoisted out of
    the query, sums carried across chunks); the two must agree.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, D = q.shape
    T = N // HW
    layout = chunk_layout(T, HW, Tc, To)
    F = feature_dim(Wq, D)
    s = np.zeros((F, v.shape[1]))
    z = np.zeros(F)
    y = np.empty((N, v.shape[1]))
    states = []
    inv_sqrt_d = 1.0 / math.sqrt(D)
    for t, (row_lo, row_hi, lo, hi) in enumerate(layout):
        states.append((s.copy(), z.copy()))
        Q = q[row_lo:row_hi]
        ES = np.exp((Q @ k[lo:hi].T) * inv_sqrt_d)
        aS = ES @ v[lo:hi]
        nS = ES.sum(axis=1)
        pq = feature(Q, Wq)
        y[row_lo:row_hi] = (aS + pq @ s) / (nS + pq @ z)[:, None]
        lo_next = layout[t + 1][2] if t + 1 < len(layout) else lo
        if lo_next > lo:
            pk = feature(k[lo:lo_next], Wk)
            s = s + pk.T @ v[lo:lo_next]
            z = z + pk.sum(axis=0)
    if return_states:
        return y, states
    return y


# ---------------------------------------------------------------------------------------
# Streaming (one call per chunk), the sampling-time use of the RNN form (key design 4 and
# the framework overview: one chunk of Tc frames generated at a time, state carried).
#
# Carried state after the chunks covering frames [0, f_end):
#   S = sum over keys of frames [0, f_end - To) of phi(k) v^T,  z likewise,
#   tail = the K and V rows of frames [f_end - To, f_end) (the overlap frames the next
#          chunk's softmax window reaches back to; not named on the page, it follows from
#          the overlapped softmax set and the causal linear set).
# ---------------------------------------------------------------------------------------

def recurrent_init(F: int, D: int) -> Dict[str, object]:
    """Empty streaming state (before chunk 0)."""
    return {"S": np.zeros((F, D)), "z": np.zeros(F), "k_tail": np.zeros((0, D)),
            "v_tail": np.zeros((0, D)), "t": 0}


def recurrent_step(state: Dict[str, object], q_c, k_c, v_c, Wq, Wk, *, HW: int, To: int):
    """One chunk of the streaming form.

    q_c, k_c, v_c: the chunk's rows [n_c, D] (n_c a multiple of HW). The softmax window is
    tail + chunk (the overlapped set of key design 2), the linear part is read from the
    state (key design 4). Returns (y_c, new_state); the input state is not modified.
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    k_c = np.asarray(k_c, dtype=np.float64)
    v_c = np.asarray(v_c, dtype=np.float64)
    D = q_c.shape[1]
    S, z = state["S"], state["z"]
    kw = np.concatenate([state["k_tail"], k_c])
    vw = np.concatenate([state["v_tail"], v_c])
    ES = np.exp((q_c @ kw.T) / math.sqrt(D))
    pq = feature(q_c, Wq)
    y = (ES @ vw + pq @ S) / (ES.sum(axis=1) + pq @ z)[:, None]
    # Keys of the window that no later window reaches: all but the last To frames.
    n_keep = min(To * HW, kw.shape[0])
    n_fold = kw.shape[0] - n_keep
    pk = feature(kw[:n_fold], Wk)
    new = {"S": S + pk.T @ vw[:n_fold], "z": z + pk.sum(axis=0),
           "k_tail": kw[n_fold:].copy(), "v_tail": vw[n_fold:].copy(),
           "t": int(state["t"]) + 1}
    return y, new


# ---------------------------------------------------------------------------------------
# Backward of the non-recursive form (the training-time form of key design 4, the form the
# note trains and distils the feature maps with).
#
# For one query i, with w_ij its weight of key j (exp(q_i.k_j/sqrt(D)) on the softmax set,
# phi(q_i).phi(k_j) on the linear set) and den_i = sum_j w_ij:
#     y_i = sum_j w_ij v_j / den_i.
# For a loss with upstream gradient dy_i the chain rule gives
#     dL/dw_ij = dy_i . (v_j - y_i) / den_i,         dL/dv_j += (w_ij / den_i) dy_i,
# and then, through each kind of weight,
#     softmax: dL/ds_ij = w_ij dL/dw_ij  ->  dq_i += dL/ds_ij k_j/sqrt(D),
#                                             dk_j += dL/ds_ij q_i/sqrt(D);
#     linear:  dphi(q_i) += dL/dw_ij phi(k_j),  dphi(k_j) += dL/dw_ij phi(q_i).
# Finally through the fixed map phi = 1 + u + u^2/2, u = x W / sqrt(D) (dphi/du = 1 + u):
#     g = dphi * (1 + u),  dx += g W^T / sqrt(D),  dW += x^T g / sqrt(D).
# ---------------------------------------------------------------------------------------

def hybrid_attention_bwd(q, k, v, Wq, Wk, dy, *, HW: int, Tc: int, To: int,
                         causal: bool = True, block: int = 256,
                         rows: Optional[Sequence[int]] = None,
                         keys: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dy * y) for one (batch, head), y = hybrid_attention(...).

    Returns a dict with dq, dk, dv [N, D]; dphi_q, dphi_k [N, F] (the gradients with
    respect to the feature rows phi(q_i), phi(k_j)); and, for the fixed map (W matrices),
    dWq, dWk [D, F]; with the fixed map dq and dk include the path through phi, with a
    map object they hold the softmax branch only (the map's own backward takes dphi).
    Queries are processed in blocks of `block` rows with the same sets as the forward.

    rows / keys: optional subsets. Only the query rows in `rows` get dq and dphi_q and only
    the keys in `keys` get dk, dv and dphi_k (other entries are NaN; an empty list skips
    that side); dWq needs every row and dWk every key, so each is returned only when its
    side is complete. The sums are the same; only the entries asked for are formed.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    N, D = q.shape
    if N % HW:
        raise ValueError("N must be a multiple of HW")
    T = N // HW
    inv_sqrt_d = 1.0 / math.sqrt(D)
    phik = feature(k, Wk)
    F = phik.shape[1]
    row_on = np.ones(N, dtype=bool) if rows is None else np.isin(np.arange(N), np.asarray(rows, dtype=np.int64))
    key_on = np.ones(N, dtype=bool) if keys is None else np.isin(np.arange(N), np.asarray(keys, dtype=np.int64))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dphi_q = np.zeros((N, F))
    dphi_k = np.zeros((N, F))
    for (row_lo, row_hi, lo, hi) in chunk_layout(T, HW, Tc, To):
        Lr = _linear_ranges(lo, hi, N, causal)
        kS, vS = k[lo:hi], v[lo:hi]
        # keys of each set whose gradients are asked for
        ks_sel = np.nonzero(key_on[lo:hi])[0]
        kl_sel = [np.nonzero(key_on[a:b])[0] for (a, b) in Lr]
        any_keys = ks_sel.size > 0 or any(x.size for x in kl_sel)
        for r0 in range(row_lo, row_hi, block):
            r1 = min(r0 + block, row_hi)
            rsel = np.nonzero(row_on[r0:r1])[0]
            if rsel.size == 0 and not any_keys:
                continue
            Qb, dyb = q[r0:r1], dy[r0:r1]
            # forward weights of the block, as in hybrid_attention
            ES = np.exp((Qb @ kS.T) * inv_sqrt_d)
            num = ES @ vS
            den = ES.sum(axis=1)
            pq = feature(Qb, Wq) if Lr else None
            EL = []
            for (a, b) in Lr:
                E = pq @ phik[a:b].T
                EL.append(E)
                num = num + E @ v[a:b]
                den = den + E.sum(axis=1)
            yb = num / den[:, None]
            # dL/dw_ij = g_i . v_j - c_i with g_i = dy_i / den_i, c_i = dy_i . y_i / den_i
            g = dyb / den[:, None]
            c = (dyb * yb).sum(axis=1) / den
            # softmax set: dL/ds_ij = w_ij dL/dw_ij
            if rsel.size:
                dS_r = (g[rsel] @ vS.T - c[rsel, None]) * ES[rsel]
                dq[r0 + rsel] += (dS_r @ kS) * inv_sqrt_d
            if ks_sel.size:
                dS_k = (g @ vS[ks_sel].T - c[:, None]) * ES[:, ks_sel]
                dk[lo + ks_sel] += (dS_k.T @ Qb) * inv_sqrt_d
                dv[lo + ks_sel] += ES[:, ks_sel].T @ g
            # linear set: dphi(q_i) += dL/dw_ij phi(k_j), dphi(k_j) += dL/dw_ij phi(q_i)
            for (a, b), E, ksel in zip(Lr, EL, kl_sel):
                if rsel.size:
                    dW_r = g[rsel] @ v[a:b].T - c[rsel, None]
                    dphi_q[r0 + rsel] += dW_r @ phik[a:b]
                if ksel.size:
                    dW_k = g @ v[a + ksel].T - c[:, None]
                    dphi_k[a + ksel] += dW_k.T @ pq
                    dv[a + ksel] += E[:, ksel].T @ g
    dq[~row_on] = np.nan
    dphi_q[~row_on] = np.nan
    for arr in (dk, dv, dphi_k):
        arr[~key_on] = np.nan
    out = {"dq": dq, "dk": dk, "dv": dv, "dphi_q": dphi_q, "dphi_k": dphi_k}
    for side, x, W, on in (("q", q, Wq, row_on), ("k", k, Wk, key_on)):
        if callable(W):
            continue
        W = np.asarray(W, dtype=np.float64)
        dphi = out["dphi_" + side]
        sel = np.nonzero(on)[0]
        u = (x[sel] @ W) / math.sqrt(D)
        gx = dphi[sel] * (1.0 + u)
        out["d" + side][sel] += (gx @ W.T) / math.sqrt(D)
        if on.all():
            out["dW" + side] = (x.T @ gx) / math.sqrt(D)
    return out
