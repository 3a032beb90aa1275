"""The float64 oracle against facts the ReHyAt definition fixes (CPU only).

Definitions: papernotes.org note "ReHyAt: Recurrent Hybrid Attention for Video Diffusion
Transformers", key designs 1, 2 and 4.
"""
import math

import numpy as np
import pytest

import oracle as orc
from tests import oracle_pins as pins

TOL = 1e-12


def oracle_map(m):
    """The oracle's own map object for a pin's map description (matrices pass through)."""
    if isinstance(m, pins.EluMap):
        return orc.EluFeatureMap()
    if isinstance(m, pins.PolyMlpMap):
        return orc.PolyMlpFeatureMap(m.W1, m.b1, m.W2, m.b2, m.P)
    return m


def attn_oracle(q, k, v, Wq, Wk, HW, Tc, To, causal):
    return orc.hybrid_attention(q, k, v, oracle_map(Wq), oracle_map(Wk), HW=HW, Tc=Tc, To=To,
                                causal=causal)


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_oracle_pin(name):
    assert pins.ALL_PINS[name](attn_oracle) < TOL


def test_chunk_layout_hand_enumerated():
    # Tc=2, To=1, HW=2: chunk 1 queries tokens 4..7 and its softmax keys are 2..7.
    assert orc.chunk_layout(4, 2, 2, 1) == [(0, 4, 0, 4), (4, 8, 2, 8)]
    # ragged: 5 frames, last chunk has one frame; its window still reaches one frame back.
    assert orc.chunk_layout(5, 2, 2, 1) == [(0, 4, 0, 4), (4, 8, 2, 8), (8, 10, 6, 10)]
    # no overlap: the window is the chunk itself.
    assert orc.chunk_layout(4, 3, 2, 0) == [(0, 6, 0, 6), (6, 12, 6, 12)]
    # overlap longer than a chunk is clamped at token 0.
    assert orc.chunk_layout(3, 2, 1, 3) == [(0, 2, 0, 2), (2, 4, 0, 4), (4, 6, 0, 6)]
    # the 21x30x52 workload: 7 chunks of 4680 tokens, windows of 6240 after chunk 0.
    lay = orc.chunk_layout(21, 1560, 3, 1)
    assert len(lay) == 7
    assert lay[1] == (4680, 9360, 3120, 9360)
    assert all(hi - lo == 6240 for (_, _, lo, hi) in lay[1:])


def test_phi_hand_values_and_positivity():
    # W = sqrt(D) * I makes u = x: phi(2) = 1+2+2 = 5, phi(-1) = 1-1+1/2 = 1/2.
    D = 2
    W = np.eye(D) * math.sqrt(D)
    assert np.array_equal(orc.phi(np.array([[2.0, -1.0]]), W), np.array([[5.0, 0.5]]))
    # 1+u+u^2/2 = ((1+u)^2+1)/2 >= 1/2 with equality at u = -1.
    x = np.random.default_rng(0).standard_normal((500, 8)) * 10
    Wr = np.random.default_rng(1).standard_normal((8, 16))
    assert orc.phi(x, Wr).min() >= 0.5


def test_recurrence_equals_pairwise():
    rng = np.random.default_rng(5)
    for (T, HW, Tc, To, D, F) in ((6, 5, 2, 1, 8, 6), (7, 4, 3, 1, 16, 8), (9, 3, 3, 2, 8, 4),
                                  (10, 2, 2, 0, 4, 4), (5, 3, 1, 1, 8, 8)):
        N = T * HW
        q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
        Wq = rng.standard_normal((D, F)) / math.sqrt(D)
        Wk = rng.standard_normal((D, F)) / math.sqrt(D)
        y1 = orc.hybrid_attention(q, k, v, Wq, Wk, HW=HW, Tc=Tc, To=To, causal=True)
        y2 = orc.hybrid_recurrent(q, k, v, Wq, Wk, HW=HW, Tc=Tc, To=To)
        assert np.abs(y1 - y2).max() < 1e-12


def test_state_is_direct_sum_brute_force():
    rng = np.random.default_rng(6)
    T, HW, Tc, To, D, F = 7, 3, 3, 1, 4, 3
    N = T * HW
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    W = rng.standard_normal((D, F))
    _, states = orc.hybrid_recurrent(q, k, v, W, W, HW=HW, Tc=Tc, To=To, return_states=True)
    for t, (row_lo, _, lo, _) in enumerate(orc.chunk_layout(T, HW, Tc, To)):
        S, z = states[t]
        # brute force: loop over keys j < lo_t, accumulate phi(k_j) v_j^T entry by entry
        Sb = [[0.0] * D for _ in range(F)]
        zb = [0.0] * F
        for j in range(lo):
            u = [sum(k[j][d] * W[d][f] for d in range(D)) / math.sqrt(D) for f in range(F)]
            p = [1 + x + x * x / 2 for x in u]
            for f in range(F):
                zb[f] += p[f]
                for d in range(D):
                    Sb[f][d] += p[f] * v[j][d]
        assert np.abs(S - np.array(Sb)).max() < 1e-12
        assert np.abs(z - np.array(zb)).max() < 1e-12
        S2, z2 = orc.state_direct(k, v, W, lo)
        assert np.abs(S - S2).max() < 1e-12 and np.abs(z - z2).max() < 1e-12


def _page_recurrence_verbatim(q, k, v, W, HW, Tc, To):
    """The chunk-wise RNN exactly as printed in key design 4: after chunk t the state adds
    phi(k_j) v_j^T over the chunk's whole softmax set."""
    N, D = q.shape
    Np = Tc * HW
    F = W.shape[1]
    s, z = np.zeros((F, v.shape[1])), np.zeros(F)
    y = np.empty_like(v)
    t = 0
    while t * Np < N:
        r0, r1 = t * Np, min((t + 1) * Np, N)
        lo = max(t * Np - To * HW, 0)
        E = np.exp(q[r0:r1] @ k[lo:r1].T / math.sqrt(D))
        pq = orc.phi(q[r0:r1], W)
        y[r0:r1] = (E @ v[lo:r1] + pq @ s) / (E.sum(1) + pq @ z)[:, None]
        pk = orc.phi(k[lo:r1], W)
        s = s + pk.T @ v[lo:r1]
        z = z + pk.sum(0)
        t += 1
    return y


def test_page_recurrence_verbatim_when_no_overlap():
    rng = np.random.default_rng(7)
    T, HW, Tc, D, F = 8, 4, 2, 8, 8
    N = T * HW
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    W = rng.standard_normal((D, F)) / math.sqrt(D)
    y0 = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=0)
    assert np.abs(y0 - _page_recurrence_verbatim(q, k, v, W, HW, Tc, 0)).max() < 1e-12
    # With overlap the printed update double-counts the overlap frames; the oracle follows
    # the sets instead, so the two must differ.
    y1 = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=1)
    assert np.abs(y1 - _page_recurrence_verbatim(q, k, v, W, HW, Tc, 1)).max() > 1e-4


def test_streaming_equals_whole_sequence_and_resume():
    rng = np.random.default_rng(8)
    for (T, HW, Tc, To) in ((9, 4, 3, 1), (8, 3, 3, 2), (7, 2, 2, 0), (10, 3, 3, 1)):
        D, F = 8, 6
        N = T * HW
        q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
        W = rng.standard_normal((D, F)) / math.sqrt(D)
        whole = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, causal=True)
        st = orc.recurrent_init(F, D)
        outs, snaps = [], []
        for (r0, r1, _, _) in orc.chunk_layout(T, HW, Tc, To):
            snaps.append(st)
            y, st = orc.recurrent_step(st, q[r0:r1], k[r0:r1], v[r0:r1], W, W, HW=HW, To=To)
            outs.append(y)
        assert np.abs(np.concatenate(outs) - whole).max() < 1e-12
        # resume from a snapshot taken before chunk 1: identical results
        lay = orc.chunk_layout(T, HW, Tc, To)
        r0, r1 = lay[1][0], lay[1][1]
        y_again, _ = orc.recurrent_step(snaps[1], q[r0:r1], k[r0:r1], v[r0:r1], W, W, HW=HW, To=To)
        assert np.array_equal(y_again, outs[1])
        # the carried state is the direct sum over the causal linear set of the next chunk
        S, z = snaps[2]["S"], snaps[2]["z"]
        S2, z2 = orc.state_direct(k, v, W, lay[2][2])
        assert np.abs(S - S2).max() < 1e-12 and np.abs(z - z2).max() < 1e-12


def test_causality_and_last_chunk_modes():
    rng = np.random.default_rng(9)
    T, HW, Tc, To, D, F = 9, 3, 3, 1, 8, 8
    N, Np = T * HW, Tc * HW
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    W = rng.standard_normal((D, F)) / math.sqrt(D)
    y = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, causal=True)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[Np:] += rng.standard_normal(a[Np:].shape)
    y2 = orc.hybrid_attention(q2, k2, v2, W, W, HW=HW, Tc=Tc, To=To, causal=True)
    assert np.array_equal(y[:Np], y2[:Np])
    yb = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, causal=False)
    assert np.abs(yb[-Np:] - y[-Np:]).max() < 1e-12
    assert np.abs(yb[:Np] - y[:Np]).max() > 1e-3


def test_in_frame_permutation_equivariance():
    rng = np.random.default_rng(10)
    T, HW, Tc, To, D, F = 6, 5, 2, 1, 8, 4
    N = T * HW
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    W = rng.standard_normal((D, F)) / math.sqrt(D)
    perm_s = rng.permutation(HW)
    perm = (np.arange(T)[:, None] * HW + perm_s[None, :]).reshape(-1)
    for causal in (True, False):
        y = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, causal=causal)
        yp = orc.hybrid_attention(q[perm], k[perm], v[perm], W, W, HW=HW, Tc=Tc, To=To,
                                  causal=causal)
        assert np.abs(yp - y[perm]).max() < 1e-12


def test_constant_values_and_convex_hull():
    rng = np.random.default_rng(11)
    T, HW, Tc, To, D, F = 7, 4, 3, 2, 8, 8
    N = T * HW
    q, k = (rng.standard_normal((N, D)) * 2 for _ in range(2))
    W = rng.standard_normal((D, F))
    c = rng.standard_normal(D)
    for causal in (True, False):
        y = orc.hybrid_attention(q, k, np.tile(c, (N, 1)), W, W, HW=HW, Tc=Tc, To=To,
                                 causal=causal)
        assert np.abs(y - c).max() < 1e-12
        v = rng.standard_normal((N, D))
        y = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, causal=causal)
        # all weights are positive (exp > 0, phi >= 1/2), so y is a convex combination
        assert (y <= v.max(0) + 1e-12).all() and (y >= v.min(0) - 1e-12).all()


def test_rows_subset_matches_full():
    rng = np.random.default_rng(12)
    T, HW, Tc, To, D, F = 7, 4, 3, 1, 8, 8
    N = T * HW
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    W = rng.standard_normal((D, F)) / math.sqrt(D)
    rows = [0, 5, 12, 13, 27]
    y = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To)
    ys = orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, rows=rows)
    assert np.abs(ys - y[rows]).max() < 1e-13


def test_feature_maps_hand_values():
    # 1 + elu(x): x + 1 above zero, exp(x) at or below it.
    e = orc.EluFeatureMap()(np.array([[0.0, 1.0, -1.0, 2.5]]))
    assert np.allclose(e, [[1.0, 2.0, math.exp(-1.0), 3.5]], rtol=0, atol=1e-15)
    # learned map, D = h = 2, F = 2, P = 2: pre-activation x W1 + b1 with W1 = I, b1 = (0, -1);
    # x = (1, 2): relu(1, 1) = (1, 1); psi = (1, 1) W2 + b2 = (1 + 0.5, 2 + 1 + 0) = (1.5, 3);
    # phi = (1.5, 3^2) = (1.5, 9). x = (-1, 0.5): relu(-1, -0.5) = 0, psi = b2 = (0.5, 0).
    m = orc.PolyMlpFeatureMap(np.eye(2), [0.0, -1.0], [[1.0, 2.0], [0.0, 1.0]], [0.5, 0.0], P=2)
    assert np.array_equal(m(np.array([[1.0, 2.0], [-1.0, 0.5]])), np.array([[1.5, 9.0], [0.5, 0.0]]))
    # P = 1 is the plain 2-layer network; P = 2 with F = 4 squares the last two outputs.
    m1 = orc.PolyMlpFeatureMap(np.eye(2), [0.0, -1.0], [[1.0, 2.0], [0.0, 1.0]], [0.5, 0.0], P=1)
    assert np.array_equal(m1(np.array([[1.0, 2.0]])), np.array([[1.5, 3.0]]))
    m4 = orc.PolyMlpFeatureMap([[1.0]], [0.0], [[1.0, -1.0, 2.0, -3.0]], [0.0, 0.0, 0.0, 0.0], P=2)
    assert np.array_equal(m4(np.array([[2.0]])), np.array([[2.0, -2.0, 16.0, 36.0]]))
    assert orc.feature_dim(m4, 1) == 4 and orc.feature_dim(orc.EluFeatureMap(), 7) == 7


def test_feature_map_recurrence_and_state():
    """The chunk-wise RNN and the direct state sums agree with the pairwise definition for
    the maps of key design 3 (separate query and key maps)."""
    rng = np.random.default_rng(9)
    T, HW, Tc, To, D, h, F = 7, 3, 2, 1, 8, 6, 4
    N = T * HW
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    mq = orc.PolyMlpFeatureMap(rng.standard_normal((D, h)) / 3, rng.standard_normal(h) * 0.2,
                               rng.standard_normal((h, F)) / 2, rng.standard_normal(F) * 0.3 + 1)
    mk = orc.PolyMlpFeatureMap(rng.standard_normal((D, h)) / 3, rng.standard_normal(h) * 0.2,
                               rng.standard_normal((h, F)) / 2, rng.standard_normal(F) * 0.3 + 1)
    for (a, b) in ((orc.EluFeatureMap(), orc.EluFeatureMap()), (mq, mk)):
        y = orc.hybrid_attention(q, k, v, a, b, HW=HW, Tc=Tc, To=To, causal=True)
        yr, states = orc.hybrid_recurrent(q, k, v, a, b, HW=HW, Tc=Tc, To=To, return_states=True)
        assert np.abs(y - yr).max() < 1e-12
        for t, (lo_t) in enumerate(l[2] for l in orc.chunk_layout(T, HW, Tc, To)):
            S, z = orc.state_direct(k, v, b, lo_t)
            assert np.abs(states[t][0] - S).max() < 1e-12 and np.abs(states[t][1] - z).max() < 1e-12
