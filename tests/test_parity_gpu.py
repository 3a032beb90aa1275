"""GPU parity: the librehyat HIP kernels (through the C ABI) against the float64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds, spanning several tiles
with ragged tails, plus edge cases and GPU-side invariants.

Tolerances and their derivation: tests/parity_util.py.
"""
import math

import numpy as np
import pytest
import torch

import hybrid_softmax_linear_amd as hs
from hybrid_softmax_linear_amd import torch_api as ta
import oracle as orc
import synthetic as syn
from synthetic import to_f64
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(B, H, T, HW, D, F, *, seed, dtype, w_per_head=False, separate_wk=False, q_scale=1.0,
            k_scale=1.0, w_zero=False):
    inp = syn.make_custom(B, H, T * HW, D, F, seed=seed, dtype=dtype, HW=HW)
    if q_scale != 1.0:
        inp["q"] = (inp["q"].float() * q_scale).to(inp["q"].dtype)
    if k_scale != 1.0:
        inp["k"] = (inp["k"].float() * k_scale).to(inp["k"].dtype)
    g = torch.Generator().manual_seed(seed + 1000)
    if w_per_head:
        inp["W"] = (torch.randn((H, D, F), generator=g) / math.sqrt(D)).to(inp["q"].dtype)
    if separate_wk:
        shape = (H, D, F) if w_per_head else (D, F)
        inp["Wk"] = (torch.randn(shape, generator=g) / math.sqrt(D)).to(inp["q"].dtype)
    if w_zero:
        inp["W"] = torch.zeros_like(inp["W"])
    return inp


def _oracle_w(inp, h=None):
    return inp["W"], inp.get("Wk", inp["W"])


def _run_fwd(inp, *, HW, Tc, To, causal, y_dtype=torch.float32):
    d = {k: v.to(DEV) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    y = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], d.get("Wk", d["W"]), HW=HW, Tc=Tc, To=To,
                      causal=causal, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(y, ref, inp, *, bf16, y_bf16, T, HW, Tc, rows=None, label=""):
    rows = list(range(T * HW)) if rows is None else rows
    errs = pu.chunk_errors(y, ref, rows, T, HW, Tc)
    err = max(e["max_abs"] for e in errs)
    rel = max(pu.chunk_rel_errors(errs))
    print(f"[{label}] max-abs {err:.3e}, max per-chunk relative {rel:.2e}; {pu.describe(errs)}",
          flush=True)
    assert np.isfinite(y).all()
    if bf16:
        pu.assert_bf16(errs, y_bf16)
    else:
        assert err <= pu.F32_BAR, f"max-abs {err:.3e} > {pu.F32_BAR}"
    return err


# ---- small shapes: every row against the oracle --------------------------------------------

BF16_CASES = [
    # (B, H, T, HW, F, Tc, To, causal, extra)
    (1, 2, 7, 100, 128, 3, 1, True, {}),          # 3 chunks, ragged q and k tiles
    (1, 2, 8, 100, 128, 3, 1, True, {}),          # short last chunk (8 = 3+3+2)
    (1, 2, 7, 100, 128, 3, 1, False, {}),         # bidirectional
    (2, 3, 9, 40, 64, 2, 1, True, {}),            # F = 64, many small chunks
    (1, 2, 10, 60, 256, 7, 3, True, {}),          # F = 256, wide chunk, To = 3
    (1, 2, 10, 60, 256, 7, 3, False, {}),
    (1, 2, 6, 50, 128, 2, 0, True, {}),           # no overlap
    (1, 2, 6, 50, 128, 1, 0, True, {}),           # Tc = 1: window = own frame
    (1, 2, 6, 50, 128, 1, 2, False, {}),          # overlap longer than a chunk
    (1, 2, 5, 64, 128, 5, 1, True, {}),           # Tc = T: plain softmax
    (1, 2, 5, 64, 128, 9, 1, False, {}),          # Tc > T
    (1, 1, 12, 1, 128, 3, 1, True, {}),           # HW = 1
    (1, 2, 7, 100, 128, 3, 1, True, {"w_per_head": True, "separate_wk": True}),
    (1, 2, 7, 100, 128, 3, 1, False, {"separate_wk": True}),
    (1, 2, 7, 100, 128, 3, 1, True, {"q_scale": 3.0, "k_scale": 3.0}),   # large logits
    (1, 2, 7, 100, 128, 3, 1, True, {"q_scale": 0.0}),                   # uniform softmax
    (1, 2, 7, 100, 128, 3, 1, False, {"w_zero": True}),                  # phi = 1
]


@pytest.mark.parametrize("case", BF16_CASES, ids=[str(i) for i in range(len(BF16_CASES))])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16], ids=["y32", "y16"])
def test_hybrid_fwd_bf16_small(case, y_dtype):
    B, H, T, HW, F, Tc, To, causal, extra = case
    inp = _inputs(B, H, T, HW, 128, F, seed=hash(case[:8]) % 10000, dtype="bf16", **extra)
    y = _run_fwd(inp, HW=HW, Tc=Tc, To=To, causal=causal, y_dtype=y_dtype)
    ref = pu.oracle_rows(inp, HW=HW, Tc=Tc, To=To, causal=causal)
    _check(y, ref, inp, bf16=True, y_bf16=y_dtype == torch.bfloat16, T=T, HW=HW, Tc=Tc,
           label=f"bf16 {case}")


F32_CASES = [
    (1, 2, 6, 64, 64, 64, 2, 1, True, {}),        # the tiny fp32 workload's shape
    (1, 2, 7, 50, 128, 128, 3, 1, True, {}),
    (1, 2, 7, 50, 128, 128, 3, 1, False, {}),
    (2, 2, 9, 30, 64, 32, 2, 2, True, {"w_per_head": True, "separate_wk": True}),
    (1, 2, 10, 40, 128, 256, 7, 3, True, {}),
    (1, 2, 5, 33, 64, 48, 1, 0, False, {}),
    (1, 2, 4, 40, 128, 128, 4, 1, True, {"q_scale": 3.0, "k_scale": 3.0}),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[str(i) for i in range(len(F32_CASES))])
def test_hybrid_fwd_f32_small(case):
    B, H, T, HW, D, F, Tc, To, causal, extra = case
    inp = _inputs(B, H, T, HW, D, F, seed=hash(case[:9]) % 10000, dtype="f32", **extra)
    y = _run_fwd(inp, HW=HW, Tc=Tc, To=To, causal=causal)
    ref = pu.oracle_rows(inp, HW=HW, Tc=Tc, To=To, causal=causal)
    _check(y, ref, inp, bf16=False, y_bf16=False, T=T, HW=HW, Tc=Tc, label=f"f32 {case}")


def test_tiny_fp32_workload_all_rows():
    cfg = syn.config(1)
    inp = syn.make_inputs(cfg)
    y = _run_fwd(inp, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To, causal=True)
    ref = pu.oracle_rows(inp, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To, causal=True)
    _check(y, ref, inp, bf16=False, y_bf16=False, T=cfg.T, HW=cfg.HW, Tc=cfg.Tc, label=cfg.name)


# ---- feature map and state update ------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,F", [("bf16", 128, 64), ("bf16", 128, 128), ("bf16", 128, 256),
                                       ("f32", 64, 64), ("f32", 128, 96)])
def test_phi(dtype, D, F):
    n = 333
    inp = syn.make_custom(2, 3, n, D, F, seed=7, dtype=dtype)
    x = inp["q"].to(DEV)
    out = ta.phi(x, inp["W"].to(DEV)).float().cpu().numpy().astype(np.float64)
    ref = orc.phi(to_f64(inp["q"]), to_f64(inp["W"]))
    rel = np.abs(out - ref) / np.abs(ref)
    # bf16 output: one rounding (<= 2^-9 relative) on an fp32-accumulated value
    assert rel.max() <= (2.0 ** -8 if dtype == "bf16" else 1e-5), rel.max()


@pytest.mark.parametrize("dtype,D,F,n", [("bf16", 128, 128, 1000), ("bf16", 128, 256, 77),
                                         ("bf16", 128, 64, 513), ("f32", 64, 64, 300),
                                         ("f32", 128, 128, 700)])
def test_state_update(dtype, D, F, n):
    B, H = 2, 2
    inp = syn.make_custom(B, H, n, D, F, seed=8, dtype=dtype)
    S0 = torch.randn((B, H, F, D), generator=torch.Generator().manual_seed(3))
    z0 = torch.rand((B, H, F), generator=torch.Generator().manual_seed(4))
    S, z = S0.to(DEV), z0.to(DEV)
    ta.state_update(inp["k"].to(DEV), inp["v"].to(DEV), inp["W"].to(DEV), S, z)
    S, z = S.cpu().numpy().astype(np.float64), z.cpu().numpy().astype(np.float64)
    k, v, W = to_f64(inp["k"]), to_f64(inp["v"]), to_f64(inp["W"])
    for b in range(B):
        for h in range(H):
            Sr, zr = orc.state_direct(k[b, h], v[b, h], W, n)
            Sr = Sr + S0[b, h].double().numpy()
            zr = zr + z0[b, h].double().numpy()
            pk = orc.phi(k[b, h], W)
            # bf16: phi(k) rounded once (<= 2^-9 relative) before the fp32 sums
            tol_S = (2.0 ** -8 if dtype == "bf16" else 1e-5) * (pk.T @ np.abs(v[b, h])) + 1e-4
            tol_z = (2.0 ** -8 if dtype == "bf16" else 1e-5) * pk.sum(0) + 1e-4
            assert (np.abs(S[b, h] - Sr) <= tol_S).all()
            assert (np.abs(z[b, h] - zr) <= tol_z).all()


# ---- the chunk-wise RNN form --------------------------------------------------------------

@pytest.mark.parametrize("dtype,T,HW,F,Tc,To,fused", [
    ("bf16", 9, 80, 128, 3, 1, False), ("bf16", 9, 80, 128, 3, 1, True),
    ("bf16", 8, 80, 128, 3, 2, False), ("bf16", 8, 80, 128, 3, 2, True),
    ("bf16", 10, 60, 256, 7, 3, False), ("bf16", 10, 60, 256, 7, 3, True),
    ("bf16", 6, 50, 64, 2, 0, False), ("bf16", 6, 50, 64, 2, 0, True),
    ("f32", 8, 40, 64, 2, 1, False)])
def test_recurrent_steps_equal_whole_sequence(dtype, T, HW, F, Tc, To, fused):
    """rehyat_recurrent_step (fused=False) and rehyat_recurrent_step_fused, chunk by chunk."""
    B, H = 1, 2
    D = 128 if dtype == "bf16" else 64
    inp = syn.make_custom(B, H, T * HW, D, F, seed=9, dtype=dtype, HW=HW)
    d = {k: v.to(DEV) for k, v in inp.items()}
    whole = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], HW=HW, Tc=Tc, To=To, causal=True)
    rec = ta.Recurrent(B, H, D, F, T=T, HW=HW, Tc=Tc, To=To, dtype=syn.TORCH_DTYPE[dtype],
                       fused=fused)
    outs = []
    Np = Tc * HW
    for t in range(-(-T // Tc)):
        r0, r1 = t * Np, min((t + 1) * Np, T * HW)
        outs.append(rec.step(d["q"][:, :, r0:r1].contiguous(), d["k"][:, :, r0:r1].contiguous(),
                             d["v"][:, :, r0:r1].contiguous(), d["W"]))
    torch.cuda.synchronize()
    streamed = torch.cat(outs, dim=2)
    # same kernels, same key order and same per-frame state sums: bitwise equal
    assert torch.equal(streamed, whole)
    # and the carried state equals the direct sum over keys before lo of the next chunk
    lo_next = max(T * HW - To * HW, 0)
    k, v, W = to_f64(inp["k"]), to_f64(inp["v"]), to_f64(inp["W"])
    S = rec.S.double().cpu().numpy()
    for h in range(H):
        Sr, zr = orc.state_direct(k[0, h], v[0, h], W, lo_next)
        pk = orc.phi(k[0, h, :lo_next], W)
        tol = (2.0 ** -8 if dtype == "bf16" else 1e-5) * (pk.T @ np.abs(v[0, h, :lo_next])) + 1e-4
        assert (np.abs(S[0, h] - Sr) <= tol).all()
    ref = pu.oracle_rows(inp, HW=HW, Tc=Tc, To=To, causal=True)
    _check(streamed.double().cpu().numpy(), ref, inp, bf16=dtype == "bf16", y_bf16=False, T=T,
           HW=HW, Tc=Tc, label=f"stream {dtype} T{T} Tc{Tc} To{To} fused={fused}")


def test_recurrent_snapshot_resume():
    B, H, T, HW, F, Tc, To = 1, 2, 9, 64, 128, 3, 1
    inp = syn.make_custom(B, H, T * HW, 128, F, seed=10, dtype="bf16", HW=HW)
    d = {k: v.to(DEV) for k, v in inp.items()}
    rec = ta.Recurrent(B, H, 128, F, T=T, HW=HW, Tc=Tc, To=To)
    Np = Tc * HW
    sl = lambda x, t: x[:, :, t * Np:(t + 1) * Np].contiguous()
    rec.step(sl(d["q"], 0), sl(d["k"], 0), sl(d["v"], 0), d["W"])
    snap = rec.snapshot()
    y1 = rec.step(sl(d["q"], 1), sl(d["k"], 1), sl(d["v"], 1), d["W"])
    y2 = rec.step(sl(d["q"], 2), sl(d["k"], 2), sl(d["v"], 2), d["W"])
    rec.restore(snap)
    y1b = rec.step(sl(d["q"], 1), sl(d["k"], 1), sl(d["v"], 1), d["W"])
    y2b = rec.step(sl(d["q"], 2), sl(d["k"], 2), sl(d["v"], 2), d["W"])
    assert torch.equal(y1, y1b) and torch.equal(y2, y2b)


# ---- invariants on the GPU ----------------------------------------------------------------

def test_causality_and_determinism():
    B, H, T, HW, F, Tc, To = 1, 2, 9, 70, 128, 3, 1
    inp = syn.make_custom(B, H, T * HW, 128, F, seed=11, dtype="bf16", HW=HW)
    d = {k: v.to(DEV) for k, v in inp.items()}
    y = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], HW=HW, Tc=Tc, To=To)
    y_again = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], HW=HW, Tc=Tc, To=To)
    assert torch.equal(y, y_again)
    Np = Tc * HW
    q2, k2, v2 = d["q"].clone(), d["k"].clone(), d["v"].clone()
    for x in (q2, k2, v2):
        x[:, :, Np:] = torch.randn_like(x[:, :, Np:].float()).to(x.dtype)
    y2 = ta.hybrid_fwd(q2, k2, v2, d["W"], HW=HW, Tc=Tc, To=To)
    assert torch.equal(y[:, :, :Np], y2[:, :, :Np])
    yb = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], HW=HW, Tc=Tc, To=To, causal=False)
    assert torch.equal(yb[:, :, -Np:], y[:, :, -Np:])


def test_overflow_fallback_outlier_key():
    """A key whose logit for one query exceeds the first window block's maximum by far more
    than 127 (log2 units) overflows the fixed-reference accumulation; the workgroup must
    recompute with the exact row maximum. Whole-sequence form against the oracle, and the
    multi-launch and single-launch recurrent forms bit for bit against it (the outlier sits
    in chunk 1, whose window spans the carried tail and the chunk)."""
    B, H, T, HW, F, Tc, To = 1, 2, 6, 64, 128, 2, 1
    inp = syn.make_custom(B, H, T * HW, 128, F, seed=21, dtype="bf16", HW=HW)
    Np = Tc * HW
    qi = Np + 5                       # a query of chunk 1
    kj = 2 * Np - 3                   # a late key of chunk 1's window (not in its first block)
    for h in range(H):
        inp["k"][0, h, kj] = (inp["q"][0, h, qi].float() * 13.0).to(torch.bfloat16)
    q, k = to_f64(inp["q"][0, 0]), to_f64(inp["k"][0, 0])
    logit = q[qi] @ k[kj] / math.sqrt(128)
    lo = Np - To * HW
    block0 = (q[qi] @ k[lo:lo + 32].T / math.sqrt(128)).max()
    assert (logit - block0) * math.log2(math.e) > 160     # far past the fp32 range of 2^x
    d = {n: t.to(DEV) for n, t in inp.items()}
    whole = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], HW=HW, Tc=Tc, To=To, causal=True)
    torch.cuda.synchronize()
    y = whole.double().cpu().numpy()
    assert np.isfinite(y).all()
    ref = pu.oracle_rows(inp, HW=HW, Tc=Tc, To=To, causal=True)
    err = float(np.abs(y - ref).max())
    print(f"[outlier key] max-abs vs oracle {err:.3e}; y[qi] vs v[kj] "
          f"{float(np.abs(y[0, 0, qi] - to_f64(inp['v'][0, 0, kj])).max()):.3e}", flush=True)
    pu.assert_bf16(pu.chunk_errors(y, ref, list(range(T * HW)), T, HW, Tc), False)
    for fused in (False, True):
        rec = ta.Recurrent(B, H, 128, F, T=T, HW=HW, Tc=Tc, To=To, fused=fused)
        outs = [rec.step(*(d[n][:, :, t * Np:(t + 1) * Np].contiguous() for n in ("q", "k", "v")),
                         d["W"]) for t in range(T // Tc)]
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(outs, dim=2), whole), f"fused={fused}"
