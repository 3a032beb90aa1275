"""Planted mistakes in a copy of the oracle must each fail at least one pin (CPU only).

The copy below restates the oracle's definition with switches that plant one plausible
mistake at a time (a dropped term, a wrong sign, scale or index, a swapped operand). The
pins of tests/oracle_pins.py are then run against every variant: a pin set that lets a
variant through would not protect the oracle from that mistake.
"""
import math

import numpy as np
import pytest

from tests import oracle_pins as pins


def _map(x, m, bug):
    """The feature maps of key design 3 (objects from tests/oracle_pins.py), restated."""
    x = np.asarray(x, dtype=np.float64)
    if isinstance(m, pins.EluMap):
        if bug == "elu_minus_one":
            return np.where(x > 0, x, np.exp(np.minimum(x, 0.0)) - 1.0)
        if bug == "elu_no_exp_branch":
            return 1.0 + x
        return np.where(x > 0, 1.0 + x, np.exp(np.minimum(x, 0.0)))
    pre = x @ m.W1 + (0.0 if bug == "mlp_no_bias1" else m.b1)
    hid = pre if bug == "mlp_no_relu" else np.maximum(pre, 0.0)
    psi = hid @ m.W2 + (0.0 if bug == "mlp_no_bias2" else m.b2)
    if bug == "mlp_no_power":
        return psi
    n = psi.shape[-1] // m.P
    parts = [psi[..., i * n:(i + 1) * n] for i in range(m.P)]
    if bug == "mlp_power_on_first_part":
        parts = parts[::-1]
        return np.concatenate([p ** (i + 1) for i, p in enumerate(parts)][::-1], axis=-1)
    return np.concatenate([p ** (i + 1) for i, p in enumerate(parts)], axis=-1)


def _phi(x, W, bug):
    if isinstance(W, (pins.EluMap, pins.PolyMlpMap)):
        return _map(x, W, bug)
    D = x.shape[-1]
    if bug == "phi_transposed_w":
        u = x @ W.T / math.sqrt(D)
    elif bug == "phi_scale_d":
        u = x @ W / D
    else:
        u = x @ W / math.sqrt(D)
    if bug == "phi_no_half":
        return 1.0 + u + u * u
    if bug == "phi_sign":
        return 1.0 - u + 0.5 * u * u
    if bug == "phi_no_const":
        return u + 0.5 * u * u + 0.5
    return 1.0 + u + 0.5 * u * u


def mutant_attention(bug):
    def attn(q, k, v, Wq, Wk, HW, Tc, To, causal):
        N, D = q.shape
        Np = Tc * HW
        if bug == "swap_wq_wk":
            Wq, Wk = Wk, Wq
        y = np.empty((N, v.shape[1]))
        t = 0
        while t * Np < N:
            r0, r1 = t * Np, min((t + 1) * Np, N)
            lo = max(t * Np - To * HW, 0)
            hi = r1
            if bug == "no_overlap":
                lo = t * Np
            if bug == "overlap_forward":
                hi = min(r1 + To * HW, N)
            if bug == "overlap_off_by_one_frame":
                lo = max(t * Np - (To + 1) * HW, 0)
            scale = 1.0 / (D if bug == "logit_scale_d" else math.sqrt(D))
            Lidx = list(range(0, lo))
            if bug == "linear_set_off_by_one_frame":
                Lidx = list(range(0, max(lo - HW, 0)))
            if not causal and bug != "bidir_drops_future":
                Lidx += list(range(hi, N))
            if bug == "linear_includes_window":
                Lidx += list(range(lo, hi))
            Q = q[r0:r1]
            s = Q @ k[lo:hi].T * scale
            if bug == "causal_mask_in_chunk":
                qi = np.arange(r0, r1)[:, None]
                kj = np.arange(lo, hi)[None, :]
                s = np.where(kj <= qi, s, -np.inf)
            if bug == "uncompensated_max":
                s = s - s.max(axis=1, keepdims=True)
            ES = np.exp(s)
            if bug == "drop_softmax_after_chunk0" and t > 0:
                ES = ES * 0.0
            num = ES @ v[lo:hi]
            den = ES.sum(axis=1)
            if Lidx and bug != "drop_linear":
                EL = _phi(Q, Wq, bug) @ _phi(k[Lidx], Wk, bug).T
                if bug == "linear_values_from_keys":
                    num = num + EL @ k[Lidx]
                else:
                    num = num + EL @ v[Lidx]
                if bug != "linear_missing_from_denominator":
                    den = den + EL.sum(axis=1)
            y[r0:r1] = num / den[:, None]
            t += 1
        return y
    return attn


BUGS = [
    "phi_transposed_w", "phi_scale_d", "phi_no_half", "phi_sign", "phi_no_const",
    "swap_wq_wk", "no_overlap", "overlap_forward", "overlap_off_by_one_frame",
    "logit_scale_d", "linear_set_off_by_one_frame", "bidir_drops_future",
    "linear_includes_window", "causal_mask_in_chunk", "uncompensated_max",
    "drop_softmax_after_chunk0", "drop_linear", "linear_values_from_keys",
    "linear_missing_from_denominator",
    "elu_minus_one", "elu_no_exp_branch", "mlp_no_relu", "mlp_no_bias1", "mlp_no_bias2",
    "mlp_no_power", "mlp_power_on_first_part",
]


def test_unmutated_copy_passes_every_pin():
    attn = mutant_attention(None)
    for name, pin in pins.ALL_PINS.items():
        assert pin(attn) < 1e-12, name


@pytest.mark.parametrize("bug", BUGS)
def test_each_planted_mistake_fails_a_pin(bug):
    attn = mutant_attention(bug)
    caught = []
    for name, pin in pins.ALL_PINS.items():
        try:
            err = pin(attn)
        except Exception:  # a shape error is a caught mistake too
            err = math.inf
        if not err < 1e-6:
            caught.append(name)
    assert caught, f"no pin catches {bug}"
