"""Convenience wrappers over the librehyat binding for torch device tensors.

They allocate outputs and workspaces with torch (device memory only) and call the C entry
points; no arithmetic happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (BF16, BIDIR, CAUSAL, F32, Desc, rehyat_hybrid_fwd, rehyat_hybrid_fwd_workspace,
               rehyat_phi, rehyat_recurrent_step, rehyat_recurrent_step_workspace,
               rehyat_state_update, rehyat_state_update_workspace)

_DT = {torch.float32: F32, torch.bfloat16: BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DT[t.dtype]


def make_desc(q: torch.Tensor, W: torch.Tensor, *, T: int, HW: int, Tc: int, To: int,
              causal: bool = True, y_dtype: torch.dtype = torch.float32) -> Desc:
    B, H, _, D = q.shape
    return Desc(B=B, H=H, T=T, HW=HW, D=D, F=W.shape[-1], Tc=Tc, To=To, dtype=_dtype_code(q),
                y_dtype=_DT[y_dtype], mode=CAUSAL if causal else BIDIR,
                w_per_head=1 if W.dim() == 3 else 0)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def hybrid_fwd(q, k, v, Wq, Wk=None, *, HW: int, Tc: int, To: int, causal: bool = True,
               y_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Whole-sequence hybrid attention of q, k, v [B, H, N, D] (N a multiple of HW)."""
    Wk = Wq if Wk is None else Wk
    N = q.shape[2]
    if N % HW:
        raise ValueError("N must be a multiple of HW")
    d = make_desc(q, Wq, T=N // HW, HW=HW, Tc=Tc, To=To, causal=causal, y_dtype=y_dtype)
    y = torch.empty(q.shape, dtype=y_dtype, device=q.device) if out is None else out
    if ws is None:
        ws = workspace(rehyat_hybrid_fwd_workspace(d), q.device)
    rehyat_hybrid_fwd(d, q, k, v, Wq, Wk, y, ws)
    return y


def phi(x, W) -> torch.Tensor:
    B, H, n, D = x.shape
    d = Desc(B=B, H=H, T=1, HW=1, D=D, F=W.shape[-1], Tc=1, To=0, dtype=_dtype_code(x),
             w_per_head=1 if W.dim() == 3 else 0)
    out = torch.empty((B, H, n, W.shape[-1]), dtype=x.dtype, device=x.device)
    rehyat_phi(d, x, n, W, out)
    return out


def state_update(k, v, Wk, S, z) -> None:
    """S += sum phi(k) v^T, z += sum phi(k) (in place)."""
    B, H, n, D = k.shape
    d = Desc(B=B, H=H, T=1, HW=1, D=D, F=Wk.shape[-1], Tc=1, To=0, dtype=_dtype_code(k),
             w_per_head=1 if Wk.dim() == 3 else 0)
    ws = workspace(rehyat_state_update_workspace(d, n), k.device)
    rehyat_state_update(d, k, v, n, Wk, S, z, ws)


class Recurrent:
    """Chunk-wise RNN form: carries S [B,H,F,D], z [B,H,F] (fp32) and the K/V tail of the
    last To frames; memory is allocated once, at construction."""

    def __init__(self, B: int, H: int, D: int, F: int, *, T: int, HW: int, Tc: int, To: int,
                 dtype: torch.dtype = torch.bfloat16, y_dtype: torch.dtype = torch.float32,
                 w_per_head: bool = False, device="cuda"):
        self.desc = Desc(B=B, H=H, T=T, HW=HW, D=D, F=F, Tc=Tc, To=To, dtype=_DT[dtype],
                         y_dtype=_DT[y_dtype], mode=CAUSAL, w_per_head=int(w_per_head))
        self.S = torch.zeros((B, H, F, D), dtype=torch.float32, device=device)
        self.z = torch.zeros((B, H, F), dtype=torch.float32, device=device)
        rows = max(To * HW, 1)
        self.k_tail = torch.zeros((B, H, rows, D), dtype=dtype, device=device)
        self.v_tail = torch.zeros((B, H, rows, D), dtype=dtype, device=device)
        self.ws = workspace(rehyat_recurrent_step_workspace(self.desc), device)
        self.y_dtype = y_dtype
        self.t = 0

    def step(self, q_c, k_c, v_c, Wq, Wk=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        Wk = Wq if Wk is None else Wk
        y = torch.empty(q_c.shape, dtype=self.y_dtype, device=q_c.device) if out is None else out
        tail_k = self.k_tail if self.desc.To > 0 else None
        tail_v = self.v_tail if self.desc.To > 0 else None
        rehyat_recurrent_step(self.desc, self.t, q_c, k_c, v_c, Wq, Wk, self.S, self.z, tail_k,
                              tail_v, y, self.ws)
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
