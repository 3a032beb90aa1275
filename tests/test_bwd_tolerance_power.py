"""The sharp bar of the backward's GPU parity test can see the plausible mistakes (CPU).

For the strong-map shapes of tests/test_parity_bwd_gpu.py, every planted mistake of the
restated backward (tests/test_oracle_bwd.py) plus dropping the path through phi on either
side moves some output by more than the bar, 4 x the emulated bf16 rounding error
(tests/bwd_emulation.py); and the emulated error itself stays inside the worst-case bound
2^-6 M of the same test.
"""
import math

import numpy as np
import pytest

import oracle as orc
import synthetic as syn
from synthetic import to_f64
from tests import bwd_emulation as em
from tests.test_oracle_bwd import BUGS, mutant_bwd

NAMES = ("dq", "dk", "dv", "dWq", "dWk")
SHAPES = [(12, 16, 64, 2, 1, 12.0), (9, 40, 64, 2, 1, 12.0)]


def _case(T, HW, F, Tc, To, gain):
    inp = syn.make_custom(1, 1, T * HW, 128, F, seed=3, dtype="bf16", HW=HW,
                          w_std=gain / math.sqrt(128))
    q, k, v = (to_f64(inp[n][0, 0]) for n in ("q", "k", "v"))
    W = to_f64(inp["W"])
    dy = to_f64(syn.make_upstream((1, 1, T * HW, 128), seed=5, dtype="f32"))[0, 0]
    return q, k, v, W, dy


def _drop_map_path(ref, side, x, W):
    u = x @ W / math.sqrt(x.shape[1])
    out = dict(ref)
    out["d" + side] = ref["d" + side] - (ref["dphi_" + side] * (1 + u)) @ W.T / math.sqrt(x.shape[1])
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=["T12HW16", "T9HW40"])
def test_planted_backward_mistakes_exceed_the_bar(shape):
    from tests.test_parity_bwd_gpu import BAR_REL, EMUL_FACTOR, _magnitudes
    T, HW, F, Tc, To, gain = shape
    q, k, v, W, dy = _case(*shape)
    ref = orc.hybrid_attention_bwd(q, k, v, W, W, dy, HW=HW, Tc=Tc, To=To)
    emu = em.backward_bf16(q, k, v, W, W, dy, HW=HW, Tc=Tc, To=To)
    mag = _magnitudes(q, k, v, W, W, dy, HW, Tc, To)
    bar = {n: EMUL_FACTOR * float(np.abs(emu[n] - ref[n]).max()) + 1e-6 for n in NAMES}
    for n in NAMES:   # the emulated rounding error is inside the worst-case bound
        assert (np.abs(emu[n] - ref[n]) <= BAR_REL * mag[n] + 1e-6).all(), n
    variants = {b: mutant_bwd(b)(q, k, v, W, W, dy, HW, Tc, To, True) for b in BUGS}
    variants["drop_dq_map_path"] = _drop_map_path(ref, "q", q, W)
    variants["drop_dk_map_path"] = _drop_map_path(ref, "k", k, W)
    for bug, out in variants.items():
        worst = max(float(np.abs(out[n] - ref[n]).max()) / bar[n] for n in NAMES)
        assert worst > 1.0, f"{bug} stays inside the bar ({worst:.2f})"
