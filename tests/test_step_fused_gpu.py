"""GPU parity of the single-launch recurrent step (rehyat_recurrent_step_fused through the
C ABI): the same per-chunk outputs, carried state S, z and tail (the single-launch form writes
it to a second buffer) as the multi-launch step (rehyat_recurrent_step), bit for bit, on
every chunk; the streamed outputs equal the
whole-sequence form bit for bit and match the float64 oracle within the bf16 bars of
tests/parity_util.py; the completion counters at the start of the workspace are zero
after every call.

The bitwise equality is by construction: the fused kernel runs the attention workgroup
code of the step with the same operand values (the linear-branch slabs are staged from W
and the fp32 state in the image layout) and the state kernel's per-frame partials and
fold order.
"""
import math

import numpy as np
import pytest
import torch

import hybrid_softmax_linear_amd as hs
from hybrid_softmax_linear_amd import torch_api as ta
import synthetic as syn
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _inputs(B, H, T, HW, F, seed, *, w_per_head=False, separate_wk=False):
    inp = syn.make_custom(B, H, T * HW, D, F, seed=seed, dtype="bf16", HW=HW)
    g = torch.Generator().manual_seed(seed + 1000)
    if w_per_head:
        inp["W"] = (torch.randn((H, D, F), generator=g) / math.sqrt(D)).to(torch.bfloat16)
    if separate_wk:
        shape = (H, D, F) if w_per_head else (D, F)
        inp["Wk"] = (torch.randn(shape, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    return inp


CASES = [
    # (B, H, T, HW, F, Tc, To, extra)
    (1, 2, 9, 80, 128, 3, 1, {}),              # 3 chunks, frames of 80 rows (ragged tiles)
    (1, 2, 8, 80, 128, 3, 2, {}),              # short last chunk (2 frames), To = 2
    (2, 3, 10, 60, 256, 7, 3, {}),             # F = 256, wide chunk, B = 2
    (1, 2, 6, 50, 64, 2, 0, {}),               # F = 64, no overlap (no tail)
    (1, 2, 7, 64, 128, 1, 1, {}),              # Tc = 1: one frame per chunk
    (1, 1, 12, 1, 128, 3, 1, {}),              # HW = 1
    (1, 2, 9, 100, 128, 3, 1, {"w_per_head": True, "separate_wk": True}),
    (2, 12, 6, 130, 128, 3, 1, {}),            # many heads: fold and attention blocks interleave
]


def _stream(rec, d, T, HW, Tc):
    Np = Tc * HW
    outs, states = [], []
    for t in range(-(-T // Tc)):
        r0, r1 = t * Np, min((t + 1) * Np, T * HW)
        y = rec.step(d["q"][:, :, r0:r1].contiguous(), d["k"][:, :, r0:r1].contiguous(),
                     d["v"][:, :, r0:r1].contiguous(), d["W"], d.get("Wk", d["W"]))
        outs.append(y.clone())
        states.append((rec.S.clone(), rec.z.clone(), rec.k_tail.clone(), rec.v_tail.clone()))
        if rec.fused:
            BH = rec.S.shape[0] * rec.S.shape[1]
            assert int(rec.ws[:4 * BH].view(torch.int32).abs().sum()) == 0, f"counters after chunk {t}"
    torch.cuda.synchronize()
    return outs, states


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_fused_step_equals_multi_launch(case):
    B, H, T, HW, F, Tc, To, extra = case
    inp = _inputs(B, H, T, HW, F, seed=hash(case[:7]) % 10000, **extra)
    d = {n: t.to(DEV) for n, t in inp.items() if isinstance(t, torch.Tensor)}
    per_head = inp["W"].dim() == 3
    kw = dict(T=T, HW=HW, Tc=Tc, To=To, w_per_head=per_head, device=DEV)
    fused = ta.Recurrent(B, H, D, F, fused=True, **kw)
    multi = ta.Recurrent(B, H, D, F, fused=False, **kw)
    yf, sf = _stream(fused, d, T, HW, Tc)
    ym, sm = _stream(multi, d, T, HW, Tc)
    for t, (a, b) in enumerate(zip(yf, ym)):
        assert torch.equal(a, b), f"y of chunk {t} differs"
    for t, (a, b) in enumerate(zip(sf, sm)):
        for name, x, y in zip(("S", "z", "k_tail", "v_tail"), a, b):
            assert torch.equal(x, y), f"{name} after chunk {t} differs"
    # the streamed outputs are the whole-sequence form's, and match the oracle
    whole = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], d.get("Wk", d["W"]), HW=HW, Tc=Tc,
                          To=To, causal=True)
    streamed = torch.cat(yf, dim=2)
    assert torch.equal(streamed, whole)
    rows = pu.sample_rows(T, HW, Tc, per_edge=4, n_random=24, seed=7)
    ref = pu.oracle_rows(inp, HW=HW, Tc=Tc, To=To, causal=True, rows=rows)
    y = streamed[:, :, rows].double().cpu().numpy()
    errs = pu.chunk_errors(y, ref, rows, T, HW, Tc)
    err = max(e["max_abs"] for e in errs)
    rel = max(pu.chunk_rel_errors(errs))
    print(f"[fused step {case[:7]} {extra}] max-abs vs oracle {err:.3e}, per-chunk relative "
          f"{rel:.2e}; {pu.describe(errs)}", flush=True)
    assert np.isfinite(y).all()
    pu.assert_bf16(errs, False)


def test_fused_step_reuses_workspace_across_videos():
    """One workspace for two videos of different lengths in turn: the counters the first
    leaves behind are zero, so the second reproduces a fresh run."""
    B, H, HW, F, Tc, To = 1, 2, 70, 128, 3, 1
    kw = dict(HW=HW, Tc=Tc, To=To, device=DEV)
    rec = ta.Recurrent(B, H, D, F, T=9, fused=True, **kw)
    a = _inputs(B, H, 9, HW, F, seed=31)
    da = {n: t.to(DEV) for n, t in a.items() if isinstance(t, torch.Tensor)}
    _stream(rec, da, 9, HW, Tc)
    b = _inputs(B, H, 7, HW, F, seed=32)
    db = {n: t.to(DEV) for n, t in b.items() if isinstance(t, torch.Tensor)}
    again = ta.Recurrent(B, H, D, F, T=7, fused=True, **kw)
    again.ws = rec.ws        # the used workspace (large enough: same B, H, F, Tc)
    fresh = ta.Recurrent(B, H, D, F, T=7, fused=True, **kw)
    y1, _ = _stream(again, db, 7, HW, Tc)
    y2, _ = _stream(fresh, db, 7, HW, Tc)
    for t, (x, y) in enumerate(zip(y1, y2)):
        assert torch.equal(x, y), f"chunk {t}"


def test_fused_step_rejects_unsupported():
    B, H, T, HW, F, Tc, To = 1, 1, 6, 16, 128, 3, 1
    desc = hs.Desc(B=B, H=H, T=T, HW=HW, D=D, F=F, Tc=Tc, To=To, dtype=hs.BF16, y_dtype=hs.F32,
                   mode=hs.CAUSAL, phi_kind=hs.PHI_ELU)
    x = torch.zeros((B, H, Tc * HW, D), dtype=torch.bfloat16, device=DEV)
    S = torch.zeros((B, H, F, D), dtype=torch.float32, device=DEV)
    z = torch.zeros((B, H, F), dtype=torch.float32, device=DEV)
    tail = torch.zeros((B, H, To * HW, D), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((B, H, Tc * HW, D), dtype=torch.float32, device=DEV)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError, match="UNSUPPORTED|unsupported|supports"):
        hs.rehyat_recurrent_step_fused(desc, 0, x, x, x, None, None, S, z, tail, tail.clone(),
                                       tail.clone(), tail.clone(), y, ws)
