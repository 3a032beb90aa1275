"""Pins that tie the float64 oracle to facts fixed by the ReHyAt definition, not by itself.

Each pin takes an attention callable attn(q, k, v, Wq, Wk, HW, Tc, To, causal) -> y [N, Dv]
(float64, one batch-head) and returns the largest deviation it finds. The oracle must give
~1e-12 on every pin; each planted mistake in tests/test_oracle_mutations.py must move at
least one pin far off.

Sources for the definitions: papernotes.org note "ReHyAt: Recurrent Hybrid Attention for
Video Diffusion Transformers", key design 1 (chunked split, joint normalisation), key
design 2 (overlapped softmax set), key design 3 (feature maps), key design 4 (causal linear
set, chunk-wise RNN).

Feature maps are passed as the Wq / Wk arguments: a D x F matrix (the fixed map
1 + u + u^2/2) or a map object; `make_map` builds the map objects of key design 3 from a
plain description, so the pins do not depend on how the oracle implements them.
"""
from __future__ import annotations

import json
import math
import os
from typing import Callable

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked_tiny.json")
GOLDEN_MAPS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "hand_worked_feature_maps.json")

Attn = Callable[..., np.ndarray]


def _eval_formula(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e}))  # noqa: S307 (own fixture)


def pin_golden(attn: Attn) -> float:
    """Hand-derived outputs of tests/golden/hand_worked_tiny.json, both modes."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    worst = 0.0
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        W = np.array(c["W"], dtype=np.float64)
        for mode in ("causal", "bidir"):
            exp_rows = c[mode]
            expected = np.array([[_eval_formula(e) for e in (r if isinstance(r, list) else [r])]
                                 for r in exp_rows])
            y = attn(q, k, v, W, W, c["HW"], c["Tc"], c["To"], mode == "causal")
            worst = max(worst, float(np.abs(y - expected).max()))
    return worst


def _sdpa(q, k, v):
    """Softmax attention by torch's library routine, float64 on the CPU."""
    tq = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    tk = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    tv = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def pin_softmax_special_cases(attn: Attn) -> float:
    """Tc >= T: one chunk, empty linear set in both modes, so y is plain softmax attention.
    Causal form, chunk 0: the linear set is empty (clamp at 0), so chunk 0's rows are
    softmax attention over the chunk's own keys."""
    worst = 0.0
    for (T, HW, D, F, seed) in ((3, 5, 8, 6, 11), (2, 7, 16, 4, 12)):
        N = T * HW
        q, k, v = (_rand((N, D), seed + i, 1.3) for i in range(3))
        W = _rand((D, F), seed + 9, 1 / math.sqrt(D))
        ref = _sdpa(q, k, v)
        for causal in (True, False):
            y = attn(q, k, v, W, W, HW, T, 1, causal)
            worst = max(worst, float(np.abs(y - ref).max()))
    for (T, HW, Tc, To, D, F, seed) in ((5, 4, 2, 1, 8, 8, 21), (7, 3, 3, 2, 16, 5, 22)):
        N = T * HW
        q, k, v = (_rand((N, D), seed + i) for i in range(3))
        W = _rand((D, F), seed + 9, 1 / math.sqrt(D))
        Np = Tc * HW
        y = attn(q, k, v, W, W, HW, Tc, To, True)
        ref = _sdpa(q[:Np], k[:Np], v[:Np])
        worst = max(worst, float(np.abs(y[:Np] - ref).max()))
    return worst


def pin_w_zero_closed_form(attn: Attn) -> float:
    """W = 0 gives phi = 1, so every linear pair weighs F. Then
        y = (Z_S * A_S + F * sum_L v) / (Z_S + F * |L|)
    with A_S the softmax attention over the window (library SDPA) and Z_S = sum_S exp(logit)
    (library logsumexp). Windows taken from the page's set definitions for each chunk."""
    worst = 0.0
    for (T, HW, Tc, To, D, F, seed) in ((6, 3, 2, 1, 8, 5, 31), (7, 2, 3, 2, 4, 7, 32),
                                        (5, 4, 1, 0, 8, 3, 33), (4, 3, 1, 3, 8, 4, 34)):
        N = T * HW
        q, k, v = (_rand((N, D), seed + i) for i in range(3))
        W = np.zeros((D, F))
        Np = Tc * HW
        for causal in (True, False):
            y = attn(q, k, v, W, W, HW, Tc, To, causal)
            ref = np.empty_like(y)
            t = 0
            while t * Np < N:
                r0, r1 = t * Np, min((t + 1) * Np, N)
                lo, hi = max(t * Np - To * HW, 0), r1
                L = list(range(0, lo)) + ([] if causal else list(range(hi, N)))
                A = _sdpa(q[r0:r1], k[lo:hi], v[lo:hi])
                logits = torch.from_numpy(q[r0:r1] @ k[lo:hi].T / math.sqrt(D))
                Z = torch.logsumexp(logits, dim=1).exp().numpy()[:, None]
                sv = v[L].sum(axis=0) if L else np.zeros(v.shape[1])
                ref[r0:r1] = (Z * A + F * sv) / (Z + F * len(L))
                t += 1
            worst = max(worst, float(np.abs(y - ref).max()))
    return worst


def brute_force(q, k, v, Wq, Wk, HW, Tc, To, causal):
    """The definition with pure-Python loops (tiny inputs only): for each query token, walk
    all key tokens, classify each by the set definitions, weigh it by exp(q.k/sqrt(D)) or
    phi(q).phi(k), and normalise jointly."""
    N, D = len(q), len(q[0])
    F = len(Wq[0])
    Np = Tc * HW

    def phi_row(x, W):
        out = []
        for f in range(F):
            u = sum(x[d] * W[d][f] for d in range(D)) / math.sqrt(D)
            out.append(1.0 + u + u * u / 2.0)
        return out

    y = []
    for n in range(N):
        t = n // Np
        lo = max(t * Np - To * HW, 0)
        hi = min((t + 1) * Np, N)
        pq = phi_row(q[n], Wq)
        num = [0.0] * len(v[0])
        den = 0.0
        for j in range(N):
            if lo <= j < hi:
                w = math.exp(sum(q[n][d] * k[j][d] for d in range(D)) / math.sqrt(D))
            elif j < lo or (not causal and j >= hi):
                pk = phi_row(k[j], Wk)
                w = sum(a * b for a, b in zip(pq, pk))
            else:
                continue
            den += w
            for d in range(len(num)):
                num[d] += w * v[j][d]
        y.append([x / den for x in num])
    return np.array(y)


def pin_brute_force(attn: Attn) -> float:
    """Oracle vs pure-Python brute force over every (Tc, To) in {1..4} x {0..3}, both modes,
    ragged lengths included (T not a multiple of Tc)."""
    worst = 0.0
    seed = 100
    for T, HW in ((4, 2), (5, 1)):
        for Tc in range(1, 5):
            for To in range(0, 4):
                seed += 1
                N, D, F = T * HW, 3, 2
                q, k, v = (_rand((N, D), seed + i) for i in range(3))
                Wq = _rand((D, F), seed + 7, 0.8)
                Wk = _rand((D, F), seed + 8, 0.8)
                for causal in (True, False):
                    y = attn(q, k, v, Wq, Wk, HW, Tc, To, causal)
                    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), Wq.tolist(),
                                      Wk.tolist(), HW, Tc, To, causal)
                    worst = max(worst, float(np.abs(y - ref).max()))
    return worst


# ---- feature maps of key design 3 ----------------------------------------------------------

class EluMap:
    """1 + elu(x) elementwise, restated here for the pins."""
    kind = "elu"

    def __call__(self, x):
        x = np.asarray(x, dtype=np.float64)
        return np.where(x > 0, 1.0 + x, np.exp(np.minimum(x, 0.0)))

    def dim(self, D):
        return D


class PolyMlpMap:
    """relu(x W1 + b1) W2 + b2 split into P parts, part i to the power i (restated)."""
    kind = "poly_mlp"

    def __init__(self, W1, b1, W2, b2, P=2):
        self.W1, self.b1 = np.asarray(W1, float), np.asarray(b1, float)
        self.W2, self.b2 = np.asarray(W2, float), np.asarray(b2, float)
        self.P = P

    def __call__(self, x):
        psi = np.maximum(np.asarray(x, float) @ self.W1 + self.b1, 0.0) @ self.W2 + self.b2
        n = psi.shape[-1] // self.P
        return np.concatenate([psi[..., i * n:(i + 1) * n] ** (i + 1) for i in range(self.P)],
                              axis=-1)

    def dim(self, D):
        return self.W2.shape[1]


def make_map(desc):
    if desc["map"] == "elu":
        return EluMap()
    return PolyMlpMap(desc["W1"], desc["b1"], desc["W2"], desc["b2"], desc.get("P", 2))


def pin_golden_feature_maps(attn: Attn) -> float:
    """Hand-derived outputs of tests/golden/hand_worked_feature_maps.json, both modes."""
    with open(GOLDEN_MAPS) as f:
        cases = json.load(f)["cases"]
    worst = 0.0
    for c in cases:
        q, k, v = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v"))
        m = make_map(c)
        for mode in ("causal", "bidir"):
            expected = np.array([[_eval_formula(e)] for e in c[mode]])
            y = attn(q, k, v, m, m, c["HW"], c["Tc"], c["To"], mode == "causal")
            worst = max(worst, float(np.abs(y - expected).max()))
    return worst


def pin_constant_map_closed_form(attn: Attn) -> float:
    """W2 = 0 makes the learned map constant, phi = [b2 part 1, (b2 part 2)^2]: every linear
    pair weighs c = |phi|^2, so y = (Z_S * A_S + c * sum_L v) / (Z_S + c * |L|) with A_S
    and Z_S from the library (SDPA, logsumexp) over each chunk's window."""
    worst = 0.0
    for (T, HW, Tc, To, D, h, F, seed) in ((6, 3, 2, 1, 8, 5, 4, 41), (5, 2, 1, 2, 4, 3, 6, 42)):
        N = T * HW
        q, k, v = (_rand((N, D), seed + i) for i in range(3))
        b2 = _rand((F,), seed + 5)
        m = PolyMlpMap(_rand((D, h), seed + 6), _rand((h,), seed + 7), np.zeros((h, F)), b2)
        c = float((b2[:F // 2] ** 2).sum() + (b2[F // 2:] ** 4).sum())
        Np = Tc * HW
        for causal in (True, False):
            y = attn(q, k, v, m, m, HW, Tc, To, causal)
            ref = np.empty_like(y)
            t = 0
            while t * Np < N:
                r0, r1 = t * Np, min((t + 1) * Np, N)
                lo, hi = max(t * Np - To * HW, 0), r1
                L = list(range(0, lo)) + ([] if causal else list(range(hi, N)))
                A = _sdpa(q[r0:r1], k[lo:hi], v[lo:hi])
                logits = torch.from_numpy(q[r0:r1] @ k[lo:hi].T / math.sqrt(D))
                Z = torch.logsumexp(logits, dim=1).exp().numpy()[:, None]
                sv = v[L].sum(axis=0) if L else np.zeros(v.shape[1])
                ref[r0:r1] = (Z * A + c * sv) / (Z + c * len(L))
                t += 1
            worst = max(worst, float(np.abs(y - ref).max()))
    return worst


def _phi_row_loops(x, m):
    """A map of key design 3 applied to one row with pure-Python loops."""
    if m.kind == "elu":
        return [1.0 + a if a > 0 else math.exp(a) for a in x]
    W1, b1, W2, b2 = m.W1.tolist(), m.b1.tolist(), m.W2.tolist(), m.b2.tolist()
    hid = [max(sum(x[d] * W1[d][j] for d in range(len(x))) + b1[j], 0.0) for j in range(len(b1))]
    psi = [sum(hid[j] * W2[j][f] for j in range(len(hid))) + b2[f] for f in range(len(b2))]
    n = len(psi) // m.P
    return [psi[f] ** (f // n + 1) for f in range(len(psi))]


def brute_force_maps(q, k, v, mq, mk, HW, Tc, To, causal):
    """Like brute_force, with feature maps of key design 3 computed by loops."""
    N, D = len(q), len(q[0])
    Np = Tc * HW
    y = []
    for n in range(N):
        t = n // Np
        lo = max(t * Np - To * HW, 0)
        hi = min((t + 1) * Np, N)
        pq = _phi_row_loops(q[n], mq)
        num = [0.0] * len(v[0])
        den = 0.0
        for j in range(N):
            if lo <= j < hi:
                w = math.exp(sum(q[n][d] * k[j][d] for d in range(D)) / math.sqrt(D))
            elif j < lo or (not causal and j >= hi):
                w = sum(a * b for a, b in zip(pq, _phi_row_loops(k[j], mk)))
            else:
                continue
            den += w
            for d in range(len(num)):
                num[d] += w * v[j][d]
        y.append([x / den for x in num])
    return np.array(y)


def pin_brute_force_feature_maps(attn: Attn) -> float:
    """Oracle vs pure-Python brute force with the elu map and with learned maps (separate
    maps for queries and keys), several (Tc, To), both modes, a ragged last chunk."""
    worst = 0.0
    seed = 300
    for (T, HW, Tc, To) in ((4, 2, 1, 0), (5, 1, 2, 1), (4, 2, 3, 2), (5, 2, 2, 3)):
        seed += 1
        N, D, h, F = T * HW, 3, 4, 4
        q, k, v = (_rand((N, D), seed + i) for i in range(3))
        maps = [(EluMap(), EluMap())]
        mq = PolyMlpMap(_rand((D, h), seed + 5, 0.7), _rand((h,), seed + 6, 0.3),
                        _rand((h, F), seed + 7, 0.6), _rand((F,), seed + 8, 0.5) + 1.0)
        mk = PolyMlpMap(_rand((D, h), seed + 9, 0.7), _rand((h,), seed + 10, 0.3),
                        _rand((h, F), seed + 11, 0.6), _rand((F,), seed + 12, 0.5) + 1.0)
        maps.append((mq, mk))
        for (a, b) in maps:
            for causal in (True, False):
                y = attn(q, k, v, a, b, HW, Tc, To, causal)
                ref = brute_force_maps(q.tolist(), k.tolist(), v.tolist(), a, b, HW, Tc, To,
                                       causal)
                worst = max(worst, float(np.abs(y - ref).max()))
    return worst


ALL_PINS = {
    "golden": pin_golden,
    "softmax_special_cases": pin_softmax_special_cases,
    "w_zero_closed_form": pin_w_zero_closed_form,
    "brute_force": pin_brute_force,
    "golden_feature_maps": pin_golden_feature_maps,
    "constant_map_closed_form": pin_constant_map_closed_form,
    "brute_force_feature_maps": pin_brute_force_feature_maps,
}
