"""GPU parity over the chunk-size / overlap grid of the pages' ablation (Tc in {1, 2, 3, 5,
7}, To in {0, 1, 2, 3}; papernotes.org ReHyAt note, key hyper-parameters and ablation
sections) at the 21x20x30 latent (320x480), causal form, bf16 inputs, fp32 output, in the
launch configuration bench.py --sweep times. To > Tc (a window reaching further back
than one chunk) is part of the grid.

Sampled query rows (first and last rows of every chunk plus random rows) of three heads
are checked against the float64 oracle with the same bars as the other bf16 tests.
"""
import pytest
import torch

import synthetic as syn
from hybrid_softmax_linear_amd import torch_api as ta
from tests import parity_util as pu

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRID = [(tc, to) for tc in (1, 2, 3, 5, 7) for to in (0, 1, 2, 3)]


@pytest.fixture(scope="module")
def inputs():
    cfg = syn.config(2)   # 21x20x30, B1 H12 D128 F128
    inp = syn.make_inputs(cfg)
    dev = {k: v.to(DEV) for k, v in inp.items() if k in ("q", "k", "v", "W")}
    return cfg, inp, dev


@pytest.mark.parametrize("Tc,To", GRID, ids=[f"Tc{a}_To{b}" for a, b in GRID])
def test_sweep_grid_sampled_rows(inputs, Tc, To):
    cfg, inp, d = inputs
    y = ta.hybrid_fwd(d["q"], d["k"], d["v"], d["W"], HW=cfg.HW, Tc=Tc, To=To, causal=True,
                      y_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = pu.sample_rows(cfg.T, cfg.HW, Tc, per_edge=4, n_random=16, seed=Tc * 10 + To)
    heads = [(0, 0), (0, 5), (0, 11)]
    y_rows = y[:, :, rows].double().cpu().numpy()
    ref = pu.oracle_rows(inp, HW=cfg.HW, Tc=Tc, To=To, causal=True, rows=rows, heads=heads)
    sel = [h for (_, h) in heads]
    errs = pu.chunk_errors(y_rows[:, sel], ref[:, sel], rows, cfg.T, cfg.HW, Tc)
    err = max(e["max_abs"] for e in errs)
    rel = max(pu.chunk_rel_errors(errs))
    print(f"[Tc={Tc} To={To}] max-abs {err:.3e}, max per-chunk relative {rel:.2e}", flush=True)
    pu.assert_bf16(errs, False)
