"""GPU parity of the other feature maps of key design 3 (papernotes.org ReHyAt note): the
1 + elu map and the learned polynomial map (psi = relu(x W1 + b1) W2 + b2 split into parts
raised to the powers 1..P), evaluated ahead into bf16 rows by the library, against the
float64 oracle's EluFeatureMap / PolyMlpFeatureMap on the same bf16 inputs and parameters.

Tolerances
  * phi rows: the hidden activations enter the second product as bf16 (<= 2^-9 relative
    each) and the first product accumulates in fp32, so |d psi| <= 2^-8 (|h| @ |W2|) plus
    2^-16 of the magnitude sums; the part power i scales that by i |psi|^(i-1); the stored
    phi is rounded once more (2^-9, taken as 2^-8).
  * state sums: those phi errors times |v|, plus fp32 accumulation (1e-4).
  * attention: the bars of the fixed map (tests/parity_util.py), multiplied by the
    conditioning cond = max over rows of (n^S + sum_f |phi_f(q)| sum_L |phi_f(k)|) /
    |n^S + n^L|. With features of one sign cond = 1 and the derivation for positive weights
    holds as it stands; a signed map perturbs numerator and denominator by amounts that
    scale with the absolute mass, relative to the (smaller) signed denominator.
"""
import zlib

import numpy as np
import pytest
import torch

from hybrid_softmax_linear_amd import torch_api as ta
import oracle as orc
import synthetic as syn
from synthetic import to_f64
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _params(F, hid, P, seed, heads=None, psi_mean=None):
    return syn.make_mlp_map_params(D, hid, F, seed=seed, P=P, heads=heads, psi_mean=psi_mean)


def _oracle_map(p, P, h=None):
    sel = (lambda t: to_f64(t)) if h is None else (lambda t: to_f64(t[h]))
    return orc.PolyMlpFeatureMap(sel(p["W1"]), sel(p["b1"]), sel(p["W2"]), sel(p["b2"]), P=P)


def _map_tol(x, p, P, h=None):
    """Elementwise bound on |phi_kernel - phi_oracle| for the learned map (module doc)."""
    sel = (lambda t: to_f64(t)) if h is None else (lambda t: to_f64(t[h]))
    W1, b1, W2, b2 = sel(p["W1"]), sel(p["b1"]), sel(p["W2"]), sel(p["b2"])
    pre = x @ W1 + b1
    hid = np.maximum(pre, 0.0)
    mag1 = np.abs(x) @ np.abs(W1) + np.abs(b1)
    psi = hid @ W2 + b2
    tol_psi = 2.0 ** -8 * (hid @ np.abs(W2)) + 2.0 ** -16 * (mag1 @ np.abs(W2) + np.abs(b2))
    F = W2.shape[1]
    power = np.repeat(np.arange(1, P + 1), F // P)
    phi = psi ** power
    tol = power * (np.abs(psi) + tol_psi) ** (power - 1) * tol_psi + 2.0 ** -8 * np.abs(phi)
    return tol + 1e-7


# ---- phi rows -----------------------------------------------------------------------------

def test_phi_elu():
    inp = syn.make_custom(2, 3, 333, D, D, seed=21, dtype="bf16")
    x = inp["q"]
    x[0, 0, 0, :8] = torch.tensor([0.0, -0.0, 1e-3, -1e-3, 20.0, -20.0, -90.0, 3.0])
    out = ta.phi(x.to(DEV), None, fmap=ta.elu_map(D)).float().cpu().numpy().astype(np.float64)
    ref = orc.EluFeatureMap()(to_f64(x))
    assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-38)


@pytest.mark.parametrize("F,hid,P,per_head", [(64, 64, 2, False), (128, 128, 2, False),
                                              (256, 256, 2, False), (128, 64, 4, True),
                                              (64, 256, 1, False), (256, 128, 2, True)])
def test_phi_learned_map(F, hid, P, per_head):
    B, H, n = 2, 3, 600
    inp = syn.make_custom(B, H, n, D, F, seed=22, dtype="bf16")
    psi_mean = [0.1] + [0.3] * (P - 1)
    p = _params(F, hid, P, seed=23, heads=H if per_head else None, psi_mean=psi_mean)
    block = ta.mlp_param_block(p["W1"], p["b1"], p["W2"], p["b2"]).to(DEV)
    out = ta.phi(inp["q"].to(DEV), block, fmap=ta.mlp_map(F, hid, P))
    out = out.float().cpu().numpy().astype(np.float64)
    x = to_f64(inp["q"])
    worst = 0.0
    for b in range(B):
        for h in range(H):
            hh = h if per_head else None
            ref = _oracle_map(p, P, hh)(x[b, h])
            tol = _map_tol(x[b, h], p, P, hh)
            err = np.abs(out[b, h] - ref)
            worst = max(worst, float((err / tol).max()))
            assert np.all(err <= tol), (b, h, float(err.max()))
    print(f"[phi F{F} h{hid} P{P}] worst error / bound {worst:.3f}", flush=True)


# ---- state sums ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,F,hid,P,n", [("elu", 128, 0, 0, 1000), ("mlp", 64, 64, 2, 513),
                                           ("mlp", 256, 128, 2, 77), ("mlp", 128, 256, 4, 700)])
def test_state_update_maps(kind, F, hid, P, n):
    B, H = 2, 2
    inp = syn.make_custom(B, H, n, D, F, seed=24, dtype="bf16")
    S0 = torch.randn((B, H, F, D), generator=torch.Generator().manual_seed(3))
    z0 = torch.rand((B, H, F), generator=torch.Generator().manual_seed(4))
    S, z = S0.to(DEV), z0.to(DEV)
    k, v = to_f64(inp["k"]), to_f64(inp["v"])
    if kind == "elu":
        ta.state_update(inp["k"].to(DEV), inp["v"].to(DEV), None, S, z, fmap=ta.elu_map(D))
        fmap = orc.EluFeatureMap()
        tolf = lambda x: 2.0 ** -8 * np.abs(fmap(x)) + 1e-38
    else:
        p = _params(F, hid, P, seed=25, psi_mean=[0.1] + [0.3] * (P - 1))
        block = ta.mlp_param_block(p["W1"], p["b1"], p["W2"], p["b2"]).to(DEV)
        ta.state_update(inp["k"].to(DEV), inp["v"].to(DEV), block, S, z,
                        fmap=ta.mlp_map(F, hid, P))
        fmap = _oracle_map(p, P)
        tolf = lambda x: _map_tol(x, p, P)
    S, z = S.cpu().numpy().astype(np.float64), z.cpu().numpy().astype(np.float64)
    for b in range(B):
        for h in range(H):
            Sr, zr = orc.state_direct(k[b, h], v[b, h], fmap, n)
            Sr = Sr + S0[b, h].double().numpy()
            zr = zr + z0[b, h].double().numpy()
            tphi = tolf(k[b, h])
            assert (np.abs(S[b, h] - Sr) <= tphi.T @ np.abs(v[b, h]) + 1e-4).all()
            assert (np.abs(z[b, h] - zr) <= tphi.sum(0) + 1e-4).all()


# ---- whole-sequence attention -------------------------------------------------------------

def _maps_for_case(kind, F, hid, P, H, *, per_head=False, separate_wk=False, psi_k=None, seed=0):
    """(device W for q, device W for k, fmap, oracle map of q for head h, same for k)."""
    if kind == "elu":
        m = orc.EluFeatureMap()
        return None, None, ta.elu_map(D), (lambda h: m), (lambda h: m)
    heads = H if per_head else None
    pq = _params(F, hid, P, seed=seed + 1, heads=heads)
    pk = _params(F, hid, P, seed=seed + 2, heads=heads, psi_mean=psi_k) \
        if (separate_wk or psi_k is not None) else pq
    bq = ta.mlp_param_block(pq["W1"], pq["b1"], pq["W2"], pq["b2"]).to(DEV)
    bk = ta.mlp_param_block(pk["W1"], pk["b1"], pk["W2"], pk["b2"]).to(DEV) if pk is not pq else bq
    fq = lambda h: _oracle_map(pq, P, h if per_head else None)
    fk = lambda h: _oracle_map(pk, P, h if per_head else None)
    return bq, bk, ta.mlp_map(F, hid, P), fq, fk


def _cond(q, k, mq, mk, HW, Tc, To, causal, nS, nL, rows=None):
    """max over rows of (n^S + sum_f |phi_f(q)| sum_L |phi_f(k)|) / |n^S + n^L| (nS, nL of
    the given rows, default all)."""
    N = q.shape[0]
    T = N // HW
    rows = np.arange(N) if rows is None else np.asarray(rows)
    pq, pk = np.abs(mq(q[rows])), np.abs(mk(k))
    mass = np.zeros(rows.size)
    for (r0, r1, lo, hi) in orc.chunk_layout(T, HW, Tc, To):
        sel = (rows >= r0) & (rows < r1)
        zabs = pk[:lo].sum(0)
        if not causal:
            zabs = zabs + pk[hi:].sum(0)
        mass[sel] = pq[sel] @ zabs
    return float(np.max((nS + mass) / np.abs(nS + nL)))


def _run_case(B, H, T, HW, F, Tc, To, causal, kind, hid=0, P=0, y_dtype=torch.float32, **mk):
    seed = zlib.crc32(repr((B, H, T, HW, F, Tc, To, causal, kind, hid, P, mk)).encode()) % 10000
    inp = syn.make_custom(B, H, T * HW, D, F, seed=seed, dtype="bf16", HW=HW)
    bq, bk, fmap, fq, fk = _maps_for_case(kind, F, hid, P, H, seed=seed, **mk)
    d = {n: inp[n].to(DEV) for n in ("q", "k", "v")}
    y = ta.hybrid_fwd(d["q"], d["k"], d["v"], bq, bk, HW=HW, Tc=Tc, To=To, causal=causal,
                      y_dtype=y_dtype, fmap=fmap)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    ref = np.empty_like(y)
    cond = 1.0
    for b in range(B):
        for h in range(H):
            q, k, v = (to_f64(inp[n][b, h]) for n in ("q", "k", "v"))
            ref[b, h], st = orc.hybrid_attention(q, k, v, fq(h), fk(h), HW=HW, Tc=Tc, To=To,
                                                 causal=causal, return_stats=True)
            cond = max(cond, _cond(q, k, fq(h), fk(h), HW, Tc, To, causal, st["nS"], st["nL"]))
    return inp, y, ref, cond


def _check(inp, y, ref, cond, *, T, HW, Tc, y_bf16, label):
    rows = list(range(T * HW))
    errs = pu.chunk_errors(y, ref, rows, T, HW, Tc)
    err = max(e["max_abs"] for e in errs)
    rel = max(pu.chunk_rel_errors(errs))
    print(f"[{label}] cond {cond:.3f}; max-abs {err:.3e}, per-chunk relative {rel:.2e}; "
          f"{pu.describe(errs)}", flush=True)
    assert np.isfinite(y).all()
    pu.assert_bf16(errs, y_bf16, cond)


MAP_CASES = [
    # (B, H, T, HW, F, Tc, To, causal, kind, hid, P, extra)
    (1, 2, 7, 100, 128, 3, 1, True, "elu", 0, 0, {}),
    (1, 2, 7, 100, 128, 3, 1, False, "elu", 0, 0, {}),
    (1, 2, 8, 100, 128, 3, 2, True, "elu", 0, 0, {}),            # short last chunk
    (2, 3, 9, 40, 64, 2, 1, True, "mlp", 64, 2, {}),
    (1, 2, 7, 100, 128, 3, 1, False, "mlp", 128, 2, {}),
    (1, 2, 10, 60, 256, 7, 3, True, "mlp", 256, 2, {}),
    (1, 2, 10, 60, 256, 7, 3, False, "mlp", 128, 2, {}),
    (1, 2, 7, 100, 128, 3, 1, True, "mlp", 64, 4, {}),           # powers 1..4
    (1, 2, 7, 100, 128, 3, 1, True, "mlp", 256, 1, {}),          # P = 1: psi itself
    (1, 2, 7, 100, 128, 3, 1, True, "mlp", 128, 2, {"per_head": True, "separate_wk": True}),
    (1, 2, 6, 50, 128, 1, 0, False, "mlp", 128, 2, {}),          # Tc = 1, no overlap
    (1, 2, 7, 100, 64, 3, 1, True, "mlp", 64, 2, {"psi_k": [-0.02, 0.0]}),   # n^L < 0
    (1, 2, 7, 100, 64, 3, 1, False, "mlp", 64, 2, {"psi_k": [-0.02, 0.0]}),
]


@pytest.mark.parametrize("case", MAP_CASES, ids=[str(i) for i in range(len(MAP_CASES))])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16], ids=["y32", "y16"])
def test_hybrid_fwd_maps(case, y_dtype):
    B, H, T, HW, F, Tc, To, causal, kind, hid, P, extra = case
    inp, y, ref, cond = _run_case(B, H, T, HW, F, Tc, To, causal, kind, hid, P,
                                  y_dtype=y_dtype, **extra)
    _check(inp, y, ref, cond, T=T, HW=HW, Tc=Tc, y_bf16=y_dtype == torch.bfloat16,
           label=f"map {case[:11]} {extra}")


def test_signed_case_has_negative_linear_mass():
    """The signed cases above do exercise n^L < 0 (checked on the oracle)."""
    B, H, T, HW, F, Tc, To = 1, 1, 7, 100, 64, 3, 1
    inp = syn.make_custom(B, H, T * HW, D, F, seed=5, dtype="bf16", HW=HW)
    _, _, _, fq, fk = _maps_for_case("mlp", F, 64, 2, H, psi_k=[-0.02, 0.0], seed=5)
    q, k, v = (to_f64(inp[n][0, 0]) for n in ("q", "k", "v"))
    _, st = orc.hybrid_attention(q, k, v, fq(0), fk(0), HW=HW, Tc=Tc, To=To, causal=True,
                                 return_stats=True)
    assert (st["nL"] < 0).sum() > HW


# ---- the chunk-wise RNN form --------------------------------------------------------------

@pytest.mark.parametrize("kind,T,HW,F,Tc,To,hid,P", [("elu", 9, 80, 128, 3, 1, 0, 0),
                                                    ("mlp", 8, 80, 128, 3, 2, 128, 2),
                                                    ("mlp", 10, 60, 256, 7, 3, 256, 2),
                                                    ("mlp", 6, 50, 64, 2, 0, 64, 2)])
def test_recurrent_maps_equal_whole_sequence(kind, T, HW, F, Tc, To, hid, P):
    B, H = 1, 2
    inp = syn.make_custom(B, H, T * HW, D, F, seed=26, dtype="bf16", HW=HW)
    bq, bk, fmap, fq, fk = _maps_for_case(kind, F, hid, P, H, separate_wk=True, seed=27)
    d = {n: inp[n].to(DEV) for n in ("q", "k", "v")}
    whole = ta.hybrid_fwd(d["q"], d["k"], d["v"], bq, bk, HW=HW, Tc=Tc, To=To, causal=True,
                          fmap=fmap)
    rec = ta.Recurrent(B, H, D, F, T=T, HW=HW, Tc=Tc, To=To, fmap=fmap)
    outs = []
    Np = Tc * HW
    for t in range(-(-T // Tc)):
        r0, r1 = t * Np, min((t + 1) * Np, T * HW)
        outs.append(rec.step(d["q"][:, :, r0:r1].contiguous(), d["k"][:, :, r0:r1].contiguous(),
                             d["v"][:, :, r0:r1].contiguous(), bq, bk))
    torch.cuda.synchronize()
    streamed = torch.cat(outs, dim=2)
    # phi rows are computed row by row with the same instructions in both forms, and the
    # state is summed frame by frame in the same order: bitwise equal
    assert torch.equal(streamed, whole)
    y = streamed.double().cpu().numpy()
    ref = np.empty_like(y)
    cond = 1.0
    for h in range(H):
        q, k, v = (to_f64(inp[n][0, h]) for n in ("q", "k", "v"))
        ref[0, h], st = orc.hybrid_attention(q, k, v, fq(h), fk(h), HW=HW, Tc=Tc, To=To,
                                             causal=True, return_stats=True)
        cond = max(cond, _cond(q, k, fq(h), fk(h), HW, Tc, To, True, st["nS"], st["nL"]))
    _check(inp, y, ref, cond, T=T, HW=HW, Tc=Tc, y_bf16=False, label=f"stream {kind} T{T}")


# ---- full size: the 21x30x52 latent, 12 heads ------------------------------------------------

@pytest.mark.parametrize("kind", ["elu", "mlp"])
def test_full_size_maps_sampled_rows(kind):
    cfg = syn.config(3)
    inp = syn.make_inputs(cfg)
    F = cfg.D if kind == "elu" else cfg.F
    bq, bk, fmap, fq, fk = _maps_for_case(kind, F, 128, 2, cfg.H, separate_wk=True, seed=28)
    d = {n: inp[n].to(DEV) for n in ("q", "k", "v")}
    y = ta.hybrid_fwd(d["q"], d["k"], d["v"], bq, bk, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To,
                      causal=cfg.mode == "causal", fmap=fmap)
    torch.cuda.synchronize()
    rows = pu.sample_rows(cfg.T, cfg.HW, cfg.Tc, per_edge=8, n_random=24, seed=3)
    heads = [(0, 0), (0, cfg.H - 1)]
    y_rows = y[:, :, rows].double().cpu().numpy()
    errs_all = []
    cond = 1.0
    causal = cfg.mode == "causal"
    for (b, h) in heads:
        q, k, v = (to_f64(inp[n][b, h]) for n in ("q", "k", "v"))
        ref, st = orc.hybrid_attention(q, k, v, fq(h), fk(h), HW=cfg.HW, Tc=cfg.Tc, To=cfg.To,
                                       causal=causal, rows=rows, return_stats=True)
        cond = max(cond, _cond(q, k, fq(h), fk(h), cfg.HW, cfg.Tc, cfg.To, causal, st["nS"],
                               st["nL"], rows=rows))
        errs = pu.chunk_errors(y_rows[b:b + 1, h:h + 1], ref[None, None], rows, cfg.T, cfg.HW,
                               cfg.Tc)
        errs_all += errs
        print(f"[full {kind} head {h}] {pu.describe(errs)}", flush=True)
        assert np.isfinite(y_rows[b, h]).all()
    err = max(e["max_abs"] for e in errs_all)
    print(f"[full {kind}] cond {cond:.3f}, max-abs {err:.3e}", flush=True)
    assert err <= pu.BF16_BAR
    assert max(pu.chunk_rel_errors(errs_all)) <= cond * pu.chunk_rel_bar(False)
