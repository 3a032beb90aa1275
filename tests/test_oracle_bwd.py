"""The oracle's backward against its pins, and planted mistakes in a restated copy of it
(CPU only). See tests/oracle_bwd_pins.py for what each pin fixes."""
import math

import numpy as np
import pytest

from tests import oracle_bwd_pins as pins
import oracle as orc


@pytest.mark.parametrize("name", sorted(pins.ALL_BWD_PINS))
def test_oracle_backward_pin(name):
    err = pins.ALL_BWD_PINS[name](pins.oracle_bwd)
    assert err < 1e-6, f"{name}: {err:.3e}"


def mutant_bwd(bug):
    """The chain rule of y = sum_j w_ij v_j / sum_j w_ij, restated with one switchable
    mistake (sets and weights as in the forward oracle)."""
    def bwd(q, k, v, Wq, Wk, dy, HW, Tc, To, causal):
        q, k, v, dy = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dy))
        N, D = q.shape
        T = N // HW
        s = 1.0 / math.sqrt(D)
        phik = orc.feature(k, Wk)
        phiq = orc.feature(q, Wq)
        F = phik.shape[1]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        dpq, dpk = np.zeros((N, F)), np.zeros((N, F))
        for (r0, r1, lo, hi) in orc.chunk_layout(T, HW, Tc, To):
            L = list(range(0, lo)) + ([] if causal else list(range(hi, N)))
            if bug == "linear_set_includes_window":
                L = list(range(0, hi))
            Sset = list(range(lo, hi))
            for i in range(r0, r1):
                ws = np.exp(q[i] @ k[Sset].T * s)
                wl = phiq[i] @ phik[L].T if L else np.zeros(0)
                den = ws.sum() + (0.0 if bug == "den_without_linear" else wl.sum())
                y = (ws @ v[Sset] + (wl @ v[L] if L else 0.0)) / den
                g = dy[i] / den
                c = 0.0 if bug == "no_mean_term" else float(dy[i] @ y) / den
                if bug == "mean_term_sign":
                    c = -c
                dws = v[Sset] @ g - c
                ds = dws * ws
                dq[i] += (ds @ k[Sset]) * (1.0 if bug == "dq_no_scale" else s)
                dk[Sset] += np.outer(ds, q[i]) * s
                dv[Sset] += np.outer(ws, dy[i] if bug == "dv_no_den" else g)
                if L:
                    dwl = v[L] @ g - c
                    dpq[i] += dwl @ phik[L]
                    dpk[L] += np.outer(dwl, phik[L][0] if bug == "dphik_uses_phik" else phiq[i])
                    if bug != "dv_drops_linear":
                        dv[L] += np.outer(wl, g)
        out = {"dq": dq, "dk": dk, "dv": dv, "dphi_q": dpq, "dphi_k": dpk}
        for x, W, dp, dn, wn in ((q, Wq, dpq, "dq", "dWq"), (k, Wk, dpk, "dk", "dWk")):
            if callable(W):
                continue
            W = np.asarray(W, dtype=np.float64)
            u = x @ W * s
            gg = dp if bug == "map_no_slope" else dp * (1.0 + u)
            if bug == "map_slope_sign":
                gg = dp * (1.0 - u)
            out[dn] = out[dn] + gg @ W.T * s
            out[wn] = x.T @ gg * (1.0 if bug == "dW_no_scale" else s)
        if bug == "swap_dWq_dWk" and "dWq" in out:
            out["dWq"], out["dWk"] = out["dWk"], out["dWq"]
        return out
    return bwd


BUGS = ["linear_set_includes_window", "den_without_linear", "no_mean_term", "mean_term_sign",
        "dq_no_scale", "dv_no_den", "dphik_uses_phik", "dv_drops_linear", "map_no_slope",
        "map_slope_sign", "dW_no_scale", "swap_dWq_dWk"]


def test_unmutated_backward_copy_passes_every_pin():
    for name, pin in pins.ALL_BWD_PINS.items():
        assert pin(mutant_bwd(None)) < 1e-6, name


@pytest.mark.parametrize("bug", BUGS)
def test_each_planted_backward_mistake_fails_a_pin(bug):
    caught = []
    for name, pin in pins.ALL_BWD_PINS.items():
        try:
            err = pin(mutant_bwd(bug))
        except Exception:  # a shape error is a caught mistake too
            err = math.inf
        if not err < 1e-6:
            caught.append(name)
    assert caught, f"no pin catches {bug}"


def test_backward_subsets_match_full():
    """rows / keys restrict which entries are formed, not the sums."""
    rng = np.random.default_rng(5)
    T, HW, D, F, Tc, To = 7, 5, 6, 4, 2, 1
    N = T * HW
    q, k, v, dy = (rng.normal(size=(N, D)) for _ in range(4))
    Wq, Wk = 0.3 * rng.normal(size=(D, F)), 0.3 * rng.normal(size=(D, F))
    for causal in (True, False):
        full = orc.hybrid_attention_bwd(q, k, v, Wq, Wk, dy, HW=HW, Tc=Tc, To=To, causal=causal)
        rows, keys = [0, 3, 11, 20, 34], [1, 9, 10, 22, 33]
        sub = orc.hybrid_attention_bwd(q, k, v, Wq, Wk, dy, HW=HW, Tc=Tc, To=To, causal=causal,
                                       rows=rows, keys=keys, block=4)
        for name, sel in (("dq", rows), ("dphi_q", rows), ("dk", keys), ("dv", keys),
                          ("dphi_k", keys)):
            assert np.allclose(sub[name][sel], full[name][sel], rtol=1e-12, atol=1e-12), name
        assert "dWq" not in sub and "dWk" not in sub
        assert np.isnan(sub["dq"][1]).all() and np.isnan(sub["dk"][0]).all()
