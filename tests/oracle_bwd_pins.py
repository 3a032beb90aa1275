"""Pins of the oracle's backward (hybrid_attention_bwd) to facts outside it (CPU only).

Each pin takes a backward callable

    bwd(q, k, v, Wq, Wk, dy, HW, Tc, To, causal) -> dict of dq, dk, dv, dphi_q, dphi_k,
                                                   dWq, dWk (the last two for W matrices)

and returns the largest error it finds (0 for an exact match). A pin never re-derives the
chain rule the oracle writes out:
  * golden: gradients worked by hand as formulas (tests/golden/hand_worked_backward.json);
  * finite differences of the forward oracle (itself pinned by tests/oracle_pins.py), for
    the inputs, both maps' matrices, both modes and several (Tc, To);
  * feature-row gradients: with an affine map phi(x) = 1 + x A (a map object, so dq and dk
    hold the softmax branch only) the total input gradient is dq + dphi_q A^T; finite
    differences of the forward check that sum;
  * softmax special case: with Tc >= T every key is in the window and the method is
    softmax attention, whose gradients torch's autograd gives (float64, CPU); there is no
    linear set, so dphi and dW vanish.
"""
from __future__ import annotations

import json
import math
import os
from typing import Callable, Dict

import numpy as np

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_backward.json")

Bwd = Callable[..., Dict[str, np.ndarray]]


def _eval_formula(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e}))  # noqa: S307 (own fixture)


def pin_golden_backward(bwd: Bwd) -> float:
    err = 0.0
    for c in json.load(open(GOLDEN))["cases"]:
        arr = {n: np.array(c[n], dtype=np.float64) for n in ("q", "k", "v", "dy", "Wq", "Wk")}
        out = bwd(arr["q"], arr["k"], arr["v"], arr["Wq"], arr["Wk"], arr["dy"], c["HW"], c["Tc"],
                  c["To"], c["causal"])
        for name, rows in c["expected"].items():
            expected = np.array([_eval_formula(r) for r in rows]).reshape(np.shape(out[name]))
            err = max(err, float(np.abs(out[name] - expected).max()))
    return err


def _forward_loss(dy, HW, Tc, To, causal):
    def loss(q, k, v, Wq, Wk):
        y = orc.hybrid_attention(q, k, v, Wq, Wk, HW=HW, Tc=Tc, To=To, causal=causal)
        return float((dy * y).sum())
    return loss


def _fd(loss, args, which, h=1e-6):
    A = args[which]
    out = np.zeros_like(A)
    for idx in np.ndindex(A.shape):
        ap, am = list(args), list(args)
        ap[which] = A.copy()
        am[which] = A.copy()
        ap[which][idx] += h
        am[which][idx] -= h
        out[idx] = (loss(*ap) - loss(*am)) / (2 * h)
    return out


FD_CASES = [
    # (T, HW, Tc, To, causal)
    (4, 2, 2, 1, True), (4, 2, 2, 1, False), (3, 2, 1, 0, True), (3, 1, 1, 2, False),
    (5, 1, 2, 3, True), (4, 2, 3, 1, True),
]


def pin_finite_differences(bwd: Bwd) -> float:
    """Relative error of every gradient against central differences of the forward."""
    rng = np.random.default_rng(11)
    worst = 0.0
    for (T, HW, Tc, To, causal) in FD_CASES:
        N, D, F = T * HW, 3, 2
        q, k, v, dy = (rng.normal(size=(N, D)) for _ in range(4))
        Wq, Wk = rng.normal(size=(D, F)), rng.normal(size=(D, F))
        out = bwd(q, k, v, Wq, Wk, dy, HW, Tc, To, causal)
        loss = _forward_loss(dy, HW, Tc, To, causal)
        args = [q, k, v, Wq, Wk]
        for i, name in enumerate(("dq", "dk", "dv", "dWq", "dWk")):
            fd = _fd(loss, args, i)
            worst = max(worst, float(np.abs(out[name] - fd).max() / max(np.abs(fd).max(), 1e-3)))
    return worst


class AffineMap:
    """phi(x) = 1 + x A: a feature-map object with a known Jacobian (A)."""

    def __init__(self, A):
        self.A = np.asarray(A, dtype=np.float64)

    def __call__(self, x):
        return 1.0 + np.asarray(x, dtype=np.float64) @ self.A

    def dim(self, D):
        return self.A.shape[1]


def pin_feature_row_gradients(bwd: Bwd) -> float:
    """With map objects, dq + dphi_q A^T and dk + dphi_k A^T are the total input gradients."""
    rng = np.random.default_rng(12)
    worst = 0.0
    for (T, HW, Tc, To, causal) in FD_CASES[:4]:
        N, D, F = T * HW, 3, 2
        q, k, v, dy = (rng.normal(size=(N, D)) for _ in range(4))
        mq, mk = AffineMap(0.2 * rng.normal(size=(D, F))), AffineMap(0.2 * rng.normal(size=(D, F)))
        out = bwd(q, k, v, mq, mk, dy, HW, Tc, To, causal)
        if "dWq" in out or "dWk" in out:
            return math.inf   # a map object has no W gradient here
        loss = _forward_loss(dy, HW, Tc, To, causal)
        args = [q, k, v, mq, mk]
        total_q = out["dq"] + out["dphi_q"] @ mq.A.T
        total_k = out["dk"] + out["dphi_k"] @ mk.A.T
        for which, got in ((0, total_q), (1, total_k), (2, out["dv"])):
            fd = _fd(loss, args, which)
            worst = max(worst, float(np.abs(got - fd).max() / max(np.abs(fd).max(), 1e-3)))
    return worst


def pin_softmax_autograd(bwd: Bwd) -> float:
    """Tc >= T: the gradients of softmax attention (torch autograd, float64)."""
    import torch
    rng = np.random.default_rng(13)
    worst = 0.0
    for (T, HW, D, F, Tc) in ((3, 4, 5, 3, 3), (2, 5, 4, 6, 7)):
        N = T * HW
        q, k, v, dy = (rng.normal(size=(N, D)) for _ in range(4))
        Wq, Wk = rng.normal(size=(D, F)), rng.normal(size=(D, F))
        out = bwd(q, k, v, Wq, Wk, dy, HW, Tc, 1, True)
        qt, kt, vt = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        y = torch.softmax(qt @ kt.T / math.sqrt(D), dim=-1) @ vt
        (y * torch.tensor(dy)).sum().backward()
        for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
            worst = max(worst, float(np.abs(out[name] - t.grad.numpy()).max()))
        for name in ("dphi_q", "dphi_k", "dWq", "dWk"):
            worst = max(worst, float(np.abs(out[name]).max()))
    return worst


ALL_BWD_PINS = {
    "golden_backward": pin_golden_backward,
    "finite_differences": pin_finite_differences,
    "feature_row_gradients": pin_feature_row_gradients,
    "softmax_autograd": pin_softmax_autograd,
}


def oracle_bwd(q, k, v, Wq, Wk, dy, HW, Tc, To, causal):
    return orc.hybrid_attention_bwd(q, k, v, Wq, Wk, dy, HW=HW, Tc=Tc, To=To, causal=causal)
