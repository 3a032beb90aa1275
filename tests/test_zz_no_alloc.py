"""GPU check of rehyat_recurrent_step_fused_noalloc (the single-launch recurrent step with its
scratch in the library's static device array) through the C ABI: on consecutive calls, the
second one smaller than the first, its output y, the updated S and z and the new tail are
bit for bit those of rehyat_recurrent_step_fused on the same inputs with a workspace.

The first call leaves the static array holding a larger problem's state and partials; the
smaller call that follows must not read any of it (its counters start at zero because every
call leaves them zero).
"""
import pytest
import torch

import hybrid_softmax_linear_amd as hs
import synthetic as syn

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _case(B, H, T, HW, F, Tc, To, seed):
    """Inputs of chunk t = 1 of a (B, H, T*HW) sequence, with the state S, z and tail that
    chunk 0 leaves (computed by the workspace form)."""
    inp = syn.make_custom(B, H, T * HW, D, F, seed=seed, dtype="bf16", HW=HW)
    d = {n: x.to(DEV) for n, x in inp.items()}
    desc = hs.Desc(B=B, H=H, T=T, HW=HW, D=D, F=F, Tc=Tc, To=To, dtype=hs.BF16, y_dtype=hs.F32,
                   mode=hs.CAUSAL)
    Np = Tc * HW
    chunk = {n: [d[n][:, :, t * Np:(t + 1) * Np].contiguous() for t in range(2)]
             for n in ("q", "k", "v")}
    S = torch.zeros((B, H, F, D), dtype=torch.float32, device=DEV)
    z = torch.zeros((B, H, F), dtype=torch.float32, device=DEV)
    tail = [torch.zeros((B, H, max(To * HW, 1), D), dtype=torch.bfloat16, device=DEV)
            for _ in range(4)]
    y0 = torch.empty((B, H, Np, D), dtype=torch.float32, device=DEV)
    ws = torch.zeros(hs.rehyat_recurrent_step_fused_workspace(desc), dtype=torch.uint8,
                     device=DEV)
    hs.rehyat_recurrent_step_fused(desc, 0, chunk["q"][0], chunk["k"][0], chunk["v"][0], d["W"],
                                   d["W"], S, z, tail[0], tail[1], tail[2], tail[3], y0, ws)
    torch.cuda.synchronize()
    return desc, d["W"], {n: chunk[n][1] for n in chunk}, S, z, (tail[2], tail[3]), ws


def _run(desc, W, c, S0, z0, tails, ws):
    """One call of chunk 1, with a workspace (ws) or on the static array (ws None)."""
    S, z = S0.clone(), z0.clone()
    kt, vt = tails
    ko, vo = torch.full_like(kt, 7.0), torch.full_like(vt, 7.0)
    y = torch.full(c["q"].shape, float("nan"), dtype=torch.float32, device=DEV)
    args = (desc, 1, c["q"], c["k"], c["v"], W, W, S, z, kt, vt, ko, vo, y)
    if ws is None:
        hs.rehyat_recurrent_step_fused_noalloc(*args)
    else:
        hs.rehyat_recurrent_step_fused(*args, ws)
    torch.cuda.synchronize()
    return {"y": y, "S": S, "z": z, "k_tail": ko, "v_tail": vo}


def test_noalloc_step_matches_workspace_step_on_two_calls():
    cases = [
        (2, 12, 9, 130, 256, 3, 1, 501),   # larger first: B2 H12, F = 256, ragged tiles
        (1, 3, 6, 64, 128, 2, 1, 502),     # then smaller: fewer heads, F = 128, shorter chunk
    ]
    for (B, H, T, HW, F, Tc, To, seed) in cases:
        desc, W, c, S0, z0, tails, ws = _case(B, H, T, HW, F, Tc, To, seed)
        assert hs.rehyat_recurrent_step_fused_workspace(desc) <= hs.STATIC_SCRATCH_BYTES
        print(f"[noalloc] B{B} H{H} T{T} HW{HW} F{F} Tc{Tc} To{To} chunk 1", flush=True)
        ref = _run(desc, W, c, S0, z0, tails, ws)
        got = _run(desc, W, c, S0, z0, tails, None)
        assert torch.isfinite(got["y"]).all()
        for name in ("y", "S", "z", "k_tail", "v_tail"):
            assert torch.equal(got[name], ref[name]), f"{name} differs (B{B} H{H} F{F})"
    # the same small call again: the static array's counters were left zero
    got2 = _run(desc, W, c, S0, z0, tails, None)
    for name in ("y", "S", "z", "k_tail", "v_tail"):
        assert torch.equal(got2[name], ref[name]), f"{name} differs on a repeated call"


def test_noalloc_step_rejects_oversized_scratch():
    """A descriptor whose scratch exceeds the static array is refused before any launch."""
    desc = hs.Desc(B=8, H=32, T=6, HW=16, D=D, F=256, Tc=3, To=1, dtype=hs.BF16,
                   y_dtype=hs.F32, mode=hs.CAUSAL)
    assert hs.rehyat_recurrent_step_fused_workspace(desc) > hs.STATIC_SCRATCH_BYTES
    x = torch.zeros((8, 32, 48, D), dtype=torch.bfloat16, device=DEV)
    S = torch.zeros((8, 32, 256, D), dtype=torch.float32, device=DEV)
    z = torch.zeros((8, 32, 256), dtype=torch.float32, device=DEV)
    W = torch.zeros((D, 256), dtype=torch.bfloat16, device=DEV)
    tails = [torch.zeros((8, 32, 16, D), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    y = torch.empty((8, 32, 48, D), dtype=torch.float32, device=DEV)
    with pytest.raises(hs.RehyatError, match="WORKSPACE"):
        hs.rehyat_recurrent_step_fused_noalloc(desc, 0, x, x.clone(), x.clone(), W, W, S, z,
                                               *tails, y)
