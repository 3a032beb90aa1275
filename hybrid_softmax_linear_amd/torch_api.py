"""Convenience wrappers over the librehyat binding for torch device tensors.

They allocate outputs and workspaces with torch (device memory only) and call the C entry
points; no arithmetic happens here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import (BF16, BIDIR, CAUSAL, F32, PHI_ELU, PHI_MLP, PHI_POLY2, Desc, rehyat_hybrid_bwd,
               rehyat_hybrid_bwd_workspace, rehyat_hybrid_fwd, rehyat_hybrid_fwd_stats,
               rehyat_hybrid_fwd_workspace, rehyat_phi, rehyat_recurrent_step,
               rehyat_recurrent_step_workspace, rehyat_recurrent_step_fused,
               rehyat_recurrent_step_fused_workspace, rehyat_state_update,
               rehyat_state_update_workspace)

_DT = {torch.float32: F32, torch.bfloat16: BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DT[t.dtype]


@dataclasses.dataclass(frozen=True)
class FeatureMap:
    """Which feature map phi the library evaluates (rehyat_desc.phi_kind and its sizes).
    The fixed map (the default) takes F from its W [D, F] / [H, D, F]."""
    kind: int = PHI_POLY2
    F: int = 0
    hidden: int = 0
    parts: int = 0


def elu_map(D: int = 128) -> FeatureMap:
    """phi = 1 + elu(x), F = D; it takes no parameters (pass W = None)."""
    return FeatureMap(PHI_ELU, F=D)


def mlp_map(F: int, hidden: int, parts: int = 2) -> FeatureMap:
    """The learned polynomial map; its W is a parameter block from mlp_param_block."""
    return FeatureMap(PHI_MLP, F=F, hidden=hidden, parts=parts)


def mlp_param_block(W1, b1, W2, b2) -> torch.Tensor:
    """Concatenate W1 [D, h], b1 [h], W2 [h, F], b2 [F] (or the same with a leading head
    dimension) into the bf16 parameter block the library reads ([n] or [H, n])."""
    per_head = W1.dim() == 3
    lead = (W1.shape[0],) if per_head else ()
    parts = [t.reshape(lead + (-1,)) for t in (W1, b1, W2, b2)]
    return torch.cat(parts, dim=-1).to(torch.bfloat16).contiguous()


def _map_fields(W: Optional[torch.Tensor], fmap: Optional[FeatureMap]):
    """(F, w_per_head, phi_kind, phi_hidden, phi_parts) of a W argument."""
    if fmap is None or fmap.kind == PHI_POLY2:
        return W.shape[-1], 1 if W.dim() == 3 else 0, PHI_POLY2, 0, 0
    per_head = 1 if (fmap.kind == PHI_MLP and W is not None and W.dim() == 2) else 0
    return fmap.F, per_head, fmap.kind, fmap.hidden, fmap.parts


def make_desc(q: torch.Tensor, W: Optional[torch.Tensor], *, T: int, HW: int, Tc: int, To: int,
              causal: bool = True, y_dtype: torch.dtype = torch.float32,
              fmap: Optional[FeatureMap] = None) -> Desc:
    B, H, _, D = q.shape
    F, wph, kind, hid, parts = _map_fields(W, fmap)
    return Desc(B=B, H=H, T=T, HW=HW, D=D, F=F, Tc=Tc, To=To, dtype=_dtype_code(q),
                y_dtype=_DT[y_dtype], mode=CAUSAL if causal else BIDIR, w_per_head=wph,
                phi_kind=kind, phi_hidden=hid, phi_parts=parts)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def hybrid_fwd(q, k, v, Wq, Wk=None, *, HW: int, Tc: int, To: int, causal: bool = True,
               y_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None,
               fmap: Optional[FeatureMap] = None) -> torch.Tensor:
    """Whole-sequence hybrid attention of q, k, v [B, H, N, D] (N a multiple of HW)."""
    Wk = Wq if Wk is None else Wk
    N = q.shape[2]
    if N % HW:
        raise ValueError("N must be a multiple of HW")
    d = make_desc(q, Wq, T=N // HW, HW=HW, Tc=Tc, To=To, causal=causal, y_dtype=y_dtype,
                  fmap=fmap)
    y = torch.empty(q.shape, dtype=y_dtype, device=q.device) if out is None else out
    if ws is None:
        ws = workspace(rehyat_hybrid_fwd_workspace(d), q.device)
    rehyat_hybrid_fwd(d, q, k, v, Wq, Wk, y, ws)
    return y


def hybrid_fwd_stats(q, k, v, Wq, Wk=None, *, HW: int, Tc: int, To: int, causal: bool = True,
                     y_dtype: torch.dtype = torch.float32):
    """(y, lse): the whole-sequence forward and log2 of each row's joint normaliser."""
    Wk = Wq if Wk is None else Wk
    N = q.shape[2]
    d = make_desc(q, Wq, T=N // HW, HW=HW, Tc=Tc, To=To, causal=causal, y_dtype=y_dtype)
    y = torch.empty(q.shape, dtype=y_dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws = workspace(rehyat_hybrid_fwd_workspace(d), q.device)
    rehyat_hybrid_fwd_stats(d, q, k, v, Wq, Wk, y, lse, ws)
    return y, lse


def hybrid_bwd(q, k, v, Wq, Wk, y, lse, dy, *, HW: int, Tc: int, To: int):
    """Gradients of sum(dy * y) of the causal form: dict of dq, dk, dv (fp32 [B,H,N,D]) and
    dWq, dWk (fp32, shaped like W)."""
    Wk = Wq if Wk is None else Wk
    N = q.shape[2]
    d = make_desc(q, Wq, T=N // HW, HW=HW, Tc=Tc, To=To, causal=True, y_dtype=y.dtype)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(q.shape, **f32),
           "dv": torch.empty(q.shape, **f32), "dWq": torch.empty(Wq.shape, **f32),
           "dWk": torch.empty(Wk.shape, **f32)}
    ws = workspace(rehyat_hybrid_bwd_workspace(d), q.device)
    rehyat_hybrid_bwd(d, q, k, v, Wq, Wk, y, lse, dy, out["dq"], out["dk"], out["dv"], out["dWq"],
                      out["dWk"], ws)
    return out


def phi(x, W, fmap: Optional[FeatureMap] = None) -> torch.Tensor:
    B, H, n, D = x.shape
    d = make_desc(x, W, T=1, HW=1, Tc=1, To=0, fmap=fmap)
    out = torch.empty((B, H, n, d.F), dtype=x.dtype, device=x.device)
    rehyat_phi(d, x, n, W, out)
    return out


def state_update(k, v, Wk, S, z, fmap: Optional[FeatureMap] = None) -> None:
    """S += sum phi(k) v^T, z += sum phi(k) (in place)."""
    n = k.shape[2]
    d = make_desc(k, Wk, T=1, HW=1, Tc=1, To=0, fmap=fmap)
    ws = workspace(rehyat_state_update_workspace(d, n), k.device)
    rehyat_state_update(d, k, v, n, Wk, S, z, ws)


class Recurrent:
    """Chunk-wise RNN form: carries S [B,H,F,D], z [B,H,F] (fp32) and the K/V tail of the
    last To frames; memory is allocated once, at construction.

    fused: run each step as one launch (rehyat_recurrent_step_fused, which writes the new
    tail to a second buffer: the two alternate); None picks it where it is supported (bf16
    inputs, the fixed feature map)."""

    def __init__(self, B: int, H: int, D: int, F: int, *, T: int, HW: int, Tc: int, To: int,
                 dtype: torch.dtype = torch.bfloat16, y_dtype: torch.dtype = torch.float32,
                 w_per_head: bool = False, device="cuda", fmap: Optional[FeatureMap] = None,
                 fused: Optional[bool] = None):
        fm = fmap or FeatureMap()
        self.desc = Desc(B=B, H=H, T=T, HW=HW, D=D, F=F, Tc=Tc, To=To, dtype=_DT[dtype],
                         y_dtype=_DT[y_dtype], mode=CAUSAL, w_per_head=int(w_per_head),
                         phi_kind=fm.kind, phi_hidden=fm.hidden, phi_parts=fm.parts)
        self.S = torch.zeros((B, H, F, D), dtype=torch.float32, device=device)
        self.z = torch.zeros((B, H, F), dtype=torch.float32, device=device)
        if fused is None:
            fused = dtype == torch.bfloat16 and fm.kind == PHI_POLY2
        self.fused = bool(fused)
        rows = max(To * HW, 1)
        self._tails = [(torch.zeros((B, H, rows, D), dtype=dtype, device=device),
                        torch.zeros((B, H, rows, D), dtype=dtype, device=device))
                       for _ in range(2 if self.fused else 1)]
        self._cur = 0
        if self.fused:
            # completion counters at its start: zero before the first call, left zero
            self.ws = torch.zeros(max(rehyat_recurrent_step_fused_workspace(self.desc), 16),
                                  dtype=torch.uint8, device=device)
        else:
            self.ws = workspace(rehyat_recurrent_step_workspace(self.desc), device)
        self.y_dtype = y_dtype
        self.t = 0

    @property
    def k_tail(self) -> torch.Tensor:
        return self._tails[self._cur][0]

    @property
    def v_tail(self) -> torch.Tensor:
        return self._tails[self._cur][1]

    def step(self, q_c, k_c, v_c, Wq, Wk=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        Wk = Wq if Wk is None else Wk
        y = torch.empty(q_c.shape, dtype=self.y_dtype, device=q_c.device) if out is None else out
        has_tail = self.desc.To > 0
        kt, vt = (self.k_tail, self.v_tail) if has_tail else (None, None)
        if self.fused:
            nxt = 1 - self._cur
            ko, vo = self._tails[nxt] if has_tail else (None, None)
            rehyat_recurrent_step_fused(self.desc, self.t, q_c, k_c, v_c, Wq, Wk, self.S, self.z,
                                        kt, vt, ko, vo, y, self.ws)
            self._cur = nxt
        else:
            rehyat_recurrent_step(self.desc, self.t, q_c, k_c, v_c, Wq, Wk, self.S, self.z, kt,
                                  vt, y, self.ws)
        self.t += 1
        return y

    def snapshot(self):
        return (self.t, self.S.clone(), self.z.clone(), self.k_tail.clone(), self.v_tail.clone())

    def restore(self, snap) -> None:
        t, S, z, kt, vt = snap
        self.t = t
        self.S.copy_(S)
        self.z.copy_(z)
        self.k_tail.copy_(kt)
        self.v_tail.copy_(vt)
