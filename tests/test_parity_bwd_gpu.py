"""GPU parity of the backward of the causal non-recursive form (rehyat_hybrid_fwd_stats +
rehyat_hybrid_bwd through the C ABI) against the float64 oracle's hybrid_attention_bwd on
the same seeded bf16 inputs and upstream gradient.

Tolerances (per output tensor; the derivation is in tests/bwd_emulation.py):
  * sharp bar: max-abs error <= 4 x the max-abs error of a float64 emulation of the
    kernels' bf16 rounding points (tests/bwd_emulation.py) against the exact oracle, on
    the same inputs. tests/test_bwd_tolerance_power.py shows on the CPU that every planted
    mistake of the backward moves some output by more than this bar on the strong-map
    cases below;
  * worst-case bar: |err| <= 2^-6 M elementwise, M the sum of the absolute values of the
    terms of each entry (each term passes through at most four bf16 roundings of <= 2^-9,
    so 2^-7 M bounds the rounding error; 2x margin for fp32 accumulation and the forward's
    rounding of y inside dy . y);
  * the bf16 bar 3e-2 on every entry.
"""
import math

import numpy as np
import pytest
import torch

from hybrid_softmax_linear_amd import torch_api as ta
import oracle as orc
import synthetic as syn
from synthetic import to_f64
from tests import bwd_emulation as em
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128
BAR_REL = 2.0 ** -6


def _inputs(B, H, T, HW, F, seed, *, w_per_head=False, separate_wk=False, w_gain=1.0):
    # w_gain scales W ~ N(0, w_gain^2 / D): gain 12 gives u ~ N(0, ~1), a strongly varying
    # map, so that the gradient through phi stands out of the rounding noise
    inp = syn.make_custom(B, H, T * HW, D, F, seed=seed, dtype="bf16", HW=HW,
                          w_std=w_gain / math.sqrt(D))
    g = torch.Generator().manual_seed(seed + 1000)
    if w_per_head:
        inp["W"] = (torch.randn((H, D, F), generator=g) * (w_gain / math.sqrt(D))).to(torch.bfloat16)
    if separate_wk:
        shape = (H, D, F) if w_per_head else (D, F)
        inp["Wk"] = (torch.randn(shape, generator=g) * (w_gain / math.sqrt(D))).to(torch.bfloat16)
    return inp


def _w(W, h):
    W = to_f64(W)
    return W if W.ndim == 2 else W[h]


def _magnitudes(q, k, v, Wq, Wk, dy, HW, Tc, To):
    """Sums of the absolute values of the terms of each gradient entry (causal sets)."""
    N = q.shape[0]
    T = N // HW
    s = 1.0 / math.sqrt(D)
    pq, pk = orc.phi(q, Wq), orc.phi(k, Wk)
    M = {n: np.zeros_like(q) for n in ("dq", "dk", "dv")}
    mq, mk = np.zeros_like(pq), np.zeros_like(pk)
    ady, av = np.abs(dy), np.abs(v)
    for (r0, r1, lo, hi) in orc.chunk_layout(T, HW, Tc, To):
        Q = q[r0:r1]
        ES = np.exp(Q @ k[lo:hi].T * s)
        EL = pq[r0:r1] @ pk[:lo].T
        den = ES.sum(1) + EL.sum(1)
        y = (ES @ v[lo:hi] + EL @ v[:lo]) / den[:, None]
        dd = np.abs((dy[r0:r1] * y).sum(1))
        aS = ady[r0:r1] @ av[lo:hi].T + dd[:, None]        # bound of |dP - dy.y|
        PS = ES / den[:, None]
        M["dq"][r0:r1] += (PS * aS) @ np.abs(k[lo:hi]) * s
        M["dk"][lo:hi] += (PS * aS).T @ np.abs(Q) * s
        M["dv"][lo:hi] += PS.T @ ady[r0:r1]
        if lo:
            aL = (ady[r0:r1] @ av[:lo].T + dd[:, None]) / den[:, None]
            mq[r0:r1] += aL @ pk[:lo]
            mk[:lo] += aL.T @ pq[r0:r1]
            M["dv"][:lo] += (EL / den[:, None]).T @ ady[r0:r1]
    uq, uk = q @ Wq * s, k @ Wk * s
    gq, gk = mq * np.abs(1 + uq) * s, mk * np.abs(1 + uk) * s
    M["dq"] += gq @ np.abs(Wq).T
    M["dk"] += gk @ np.abs(Wk).T
    M["dWq"] = np.abs(q).T @ gq
    M["dWk"] = np.abs(k).T @ gk
    return M


def _run(inp, *, HW, Tc, To, y_dtype=torch.float32):
    B, H, N, _ = inp["q"].shape
    dy = syn.make_upstream((B, H, N, D), seed=N + H, dtype="f32" if y_dtype == torch.float32 else "bf16")
    d = {n: t.to(DEV) for n, t in inp.items() if isinstance(t, torch.Tensor)}
    Wq, Wk = d["W"], d.get("Wk", d["W"])
    y, lse = ta.hybrid_fwd_stats(d["q"], d["k"], d["v"], Wq, Wk, HW=HW, Tc=Tc, To=To, y_dtype=y_dtype)
    out = ta.hybrid_bwd(d["q"], d["k"], d["v"], Wq, Wk, y, lse, dy.to(DEV), HW=HW, Tc=Tc, To=To)
    torch.cuda.synchronize()
    return dy, {n: t.double().cpu().numpy() for n, t in out.items()}


EMUL_FACTOR = 4.0


def _compare(name, got, ref, mag, emul, label):
    err = np.abs(got - ref)
    ratio = float((err / (BAR_REL * mag + 1e-6)).max())
    ebar = EMUL_FACTOR * float(np.abs(emul - ref).max()) + 1e-6
    print(f"[{label}] {name}: max-abs {err.max():.3e} (sharp bar {ebar:.3e}), max|ref| "
          f"{np.abs(ref).max():.3e}, worst err / worst-case bound {ratio:.3f}", flush=True)
    assert np.isfinite(got).all(), name
    assert err.max() <= pu.BF16_BAR, name
    assert ratio <= 1.0, name
    assert err.max() <= ebar, name


CASES = [
    # (B, H, T, HW, F, Tc, To, extra)
    (1, 2, 7, 100, 128, 3, 1, {}),            # 3 chunks, ragged tiles
    (1, 2, 8, 100, 128, 3, 2, {}),            # short last chunk, To = 2
    (2, 3, 9, 40, 64, 2, 1, {}),              # F = 64, many chunks
    (1, 2, 10, 60, 256, 7, 3, {}),            # F = 256, wide chunk
    (1, 2, 6, 50, 128, 1, 0, {}),             # Tc = 1, no overlap
    (1, 2, 6, 50, 128, 1, 2, {}),             # overlap longer than a chunk
    (1, 2, 5, 64, 128, 5, 1, {}),             # one chunk: softmax only
    (1, 1, 12, 1, 128, 3, 1, {}),             # HW = 1
    (1, 2, 7, 100, 128, 3, 1, {"w_per_head": True, "separate_wk": True}),
    # strong maps: the gradient through phi well above the rounding noise
    (1, 1, 12, 16, 64, 2, 1, {"w_gain": 12.0}),
    (1, 2, 9, 40, 64, 2, 1, {"w_gain": 12.0, "separate_wk": True}),
    (1, 2, 7, 100, 128, 3, 1, {"w_gain": 16.0, "w_per_head": True}),
]


def _check_all(inp, *, HW, Tc, To, y_dtype, label):
    """Every entry of dq, dk, dv, dWq and dWk against the oracle (all heads)."""
    B, H = inp["q"].shape[:2]
    dy, got = _run(inp, HW=HW, Tc=Tc, To=To, y_dtype=y_dtype)
    q, k, v = (to_f64(inp[n]) for n in ("q", "k", "v"))
    dyf = to_f64(dy)
    Wq_t, Wk_t = inp["W"], inp.get("Wk", inp["W"])
    names = ("dq", "dk", "dv", "dWq", "dWk")
    ref, mag, emu = ({n: np.zeros_like(got[n]) for n in names} for _ in range(3))
    per_head = Wq_t.dim() == 3
    for b in range(B):
        for h in range(H):
            Wq, Wk = _w(Wq_t, h), _w(Wk_t, h)
            args = (q[b, h], k[b, h], v[b, h], Wq, Wk, dyf[b, h])
            o = orc.hybrid_attention_bwd(*args, HW=HW, Tc=Tc, To=To)
            m = _magnitudes(*args, HW, Tc, To)
            e = em.backward_bf16(*args, HW=HW, Tc=Tc, To=To)
            for n in names:
                for dst, src in ((ref, o), (mag, m), (emu, e)):
                    if n in ("dq", "dk", "dv"):
                        dst[n][b, h] = src[n]
                    elif per_head:
                        dst[n][h] += src[n]
                    else:
                        dst[n] += src[n]
    for n in names:
        _compare(n, got[n], ref[n], mag[n], emu[n], label)


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16], ids=["y32", "y16"])
def test_hybrid_bwd_small(case, y_dtype):
    B, H, T, HW, F, Tc, To, extra = case
    inp = _inputs(B, H, T, HW, F, seed=hash(case[:7]) % 10000, **extra)
    _check_all(inp, HW=HW, Tc=Tc, To=To, y_dtype=y_dtype,
               label=f"bwd {case[:7]} {extra} {'y16' if y_dtype == torch.bfloat16 else 'y32'}")


@pytest.mark.parametrize("extra", [{}, {"w_gain": 12.0, "w_per_head": True, "separate_wk": True}],
                         ids=["workload_map", "strong_per_head_maps"])
def test_hybrid_bwd_mid_size_every_entry(extra):
    """A mid-size shape (B1 H3, 9 frames of 520 tokens: 3 chunks of 1560 queries, Tc3 To1,
    F128) with every entry of dq, dk, dv and of the feature-map gradients dWq, dWk checked:
    the full-size test samples rows of one head and cannot check dW, which sums over all
    rows and heads."""
    inp = _inputs(1, 3, 9, 520, 128, seed=77, **extra)
    _check_all(inp, HW=520, Tc=3, To=1, y_dtype=torch.float32, label=f"bwd mid-size {extra}")



def test_hybrid_bwd_full_size_sampled():
    """The 21x30x52 workload (B2 H12 N32760 F128, Tc3 To1), as bench.py times the backward:
    dq on sampled query rows and dk, dv on sampled keys of two heads, against the oracle's
    row / key subsets, with the sharp bar formed from the emulation of the same head. The
    heads are the ones with the smallest (batch item 1, head 11) and the largest (batch item
    0, head 2) per-head scale of the seeded draw."""
    cfg = syn.config(3)
    inp = syn.make_inputs(cfg)
    dy, got = _run(inp, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To)
    rows = pu.sample_rows(cfg.T, cfg.HW, cfg.Tc, per_edge=8, n_random=32, seed=4)
    keys = pu.sample_rows(cfg.T, cfg.HW, 1, per_edge=4, n_random=32, seed=5)   # frame edges
    W = to_f64(inp["W"])
    for b, h in ((1, cfg.H - 1), (0, 2)):
        q, k, v = (to_f64(inp[n][b, h]) for n in ("q", "k", "v"))
        dyf = to_f64(dy[b, h])
        o = orc.hybrid_attention_bwd(q, k, v, W, W, dyf, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To,
                                     rows=rows, keys=keys)
        e = em.backward_bf16(q, k, v, W, W, dyf, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To, rows=rows,
                             keys=keys)
        for n, sel in (("dq", rows), ("dk", keys), ("dv", keys)):
            g_, r_, e_ = got[n][b, h][sel], o[n][sel], e[n][sel]
            err = float(np.abs(g_ - r_).max())
            ebar = EMUL_FACTOR * float(np.abs(e_ - r_).max()) + 1e-6
            print(f"[full c3 batch {b} head {h}] {n}: max-abs {err:.3e} (sharp bar "
                  f"{ebar:.3e}), max|ref| {np.abs(r_).max():.3e}", flush=True)
            assert np.isfinite(got[n]).all(), n
            assert err <= pu.BF16_BAR, n
            assert err <= ebar, n
