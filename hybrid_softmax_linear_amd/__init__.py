"""ReHyAt temporally chunked hybrid attention on MI355X: Python binding of librehyat.

Argument marshalling only: every step of the computation runs in the HIP kernels of
librehyat.so (built in-tree by hybrid_softmax_linear_amd.build). PyTorch supplies device
memory and the current HIP stream. There is no CPU fallback: if the library is missing or
a call fails, an exception is raised.

The functions carry the names of the C entry points (include/rehyat.h):
    rehyat_phi, rehyat_state_update, rehyat_hybrid_fwd, rehyat_hybrid_fwd_stats,
    rehyat_hybrid_bwd, rehyat_recurrent_step, rehyat_recurrent_step_fused
plus *_workspace helpers, rehyat_timing_enable / rehyat_timing_read.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

__all__ = [
    "RehyatError", "Desc", "lib", "library_path", "exported_symbols",
    "rehyat_phi", "rehyat_state_update", "rehyat_state_update_workspace",
    "rehyat_hybrid_fwd", "rehyat_hybrid_fwd_workspace",
    "rehyat_recurrent_step", "rehyat_recurrent_step_workspace",
    "rehyat_recurrent_step_fused", "rehyat_recurrent_step_fused_workspace",
    "rehyat_recurrent_step_fused_noalloc", "STATIC_SCRATCH_BYTES",
    "rehyat_hybrid_fwd_stats", "rehyat_hybrid_bwd", "rehyat_hybrid_bwd_workspace",
    "rehyat_timing_enable", "rehyat_timing_read", "F32", "BF16", "CAUSAL", "BIDIR",
    "PHI_POLY2", "PHI_ELU", "PHI_MLP",
]

F32, BF16 = 0, 1
STATIC_SCRATCH_BYTES = 16 * 1024 * 1024   # REHYAT_STATIC_SCRATCH_BYTES of include/rehyat.h
CAUSAL, BIDIR = 0, 1
PHI_POLY2, PHI_ELU, PHI_MLP = 0, 1, 2

_PKG = os.path.dirname(os.path.abspath(__file__))
# REHYAT_LIBRARY names another build of the same library (e.g. the host-sanitized copy that
# hybrid_softmax_linear_amd.build.build_host_sanitized makes for the host tests)
library_path = os.environ.get("REHYAT_LIBRARY") or os.path.join(_PKG, "librehyat.so")


class RehyatError(RuntimeError):
    """A librehyat call returned a status other than REHYAT_OK."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}" if detail else name)
        self.status = status
        self.name = name


class _CDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "T", "HW", "D", "F", "Tc", "To", "dtype", "y_dtype", "mode",
                 "w_per_head", "phi_kind", "phi_hidden", "phi_parts")]


@dataclasses.dataclass(frozen=True)
class Desc:
    """Problem description (mirror of rehyat_desc)."""
    B: int
    H: int
    T: int
    HW: int
    D: int
    F: int
    Tc: int
    To: int
    dtype: int = BF16
    y_dtype: int = F32
    mode: int = CAUSAL
    w_per_head: int = 0
    phi_kind: int = PHI_POLY2
    phi_hidden: int = 0
    phi_parts: int = 0

    @property
    def N(self) -> int:
        return self.T * self.HW

    @property
    def n_chunks(self) -> int:
        return -(-self.T // self.Tc)

    def c(self) -> _CDesc:
        return _CDesc(*(int(getattr(self, f[0])) for f in _CDesc._fields_))


_lib: Optional[ctypes.CDLL] = None

_SIGS = {
    "rehyat_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "rehyat_last_error": (ctypes.c_char_p, []),
    "rehyat_phi": (ctypes.c_int, [ctypes.POINTER(_CDesc), ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "rehyat_state_update_workspace": (ctypes.c_size_t, [ctypes.POINTER(_CDesc), ctypes.c_int64]),
    "rehyat_state_update": (ctypes.c_int, [ctypes.POINTER(_CDesc), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]),
    "rehyat_hybrid_fwd_workspace": (ctypes.c_size_t, [ctypes.POINTER(_CDesc)]),
    "rehyat_hybrid_fwd": (ctypes.c_int, [ctypes.POINTER(_CDesc)] + [ctypes.c_void_p] * 7 +
                          [ctypes.c_size_t, ctypes.c_void_p]),
    "rehyat_recurrent_step_workspace": (ctypes.c_size_t, [ctypes.POINTER(_CDesc)]),
    "rehyat_recurrent_step_fused_workspace": (ctypes.c_size_t, [ctypes.POINTER(_CDesc)]),
    "rehyat_recurrent_step": (ctypes.c_int, [ctypes.POINTER(_CDesc), ctypes.c_int32] +
                              [ctypes.c_void_p] * 11 + [ctypes.c_size_t, ctypes.c_void_p]),
    "rehyat_recurrent_step_fused": (ctypes.c_int, [ctypes.POINTER(_CDesc), ctypes.c_int32] +
                                    [ctypes.c_void_p] * 13 + [ctypes.c_size_t, ctypes.c_void_p]),
    "rehyat_recurrent_step_fused_noalloc": (ctypes.c_int, [ctypes.POINTER(_CDesc), ctypes.c_int32] +
                                            [ctypes.c_void_p] * 13),
    "rehyat_hybrid_fwd_stats": (ctypes.c_int, [ctypes.POINTER(_CDesc)] + [ctypes.c_void_p] * 8 +
                                [ctypes.c_size_t, ctypes.c_void_p]),
    "rehyat_hybrid_bwd_workspace": (ctypes.c_size_t, [ctypes.POINTER(_CDesc)]),
    "rehyat_hybrid_bwd": (ctypes.c_int, [ctypes.POINTER(_CDesc)] + [ctypes.c_void_p] * 14 +
                          [ctypes.c_size_t, ctypes.c_void_p]),
    "rehyat_timing_enable": (ctypes.c_int, [ctypes.c_int32]),
    "rehyat_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64)]),
}


def lib() -> ctypes.CDLL:
    """The loaded librehyat.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m hybrid_softmax_linear_amd.build`")
        # torch first: librehyat.so then binds to the HIP runtime torch has loaded, the one
        # that owns the streams and device memory handed to it (loaded the other way round,
        # the process would hold two runtimes)
        import torch  # noqa: F401
        L = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    """Names of the C entry points bound here."""
    return sorted(_SIGS)


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise RehyatError(status, L.rehyat_status_str(status).decode(),
                          f"{what}: {L.rehyat_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None for None); raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to librehyat must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def rehyat_phi(desc: Desc, x, n: int, W, phi, stream=None) -> None:
    """phi [B,H,n,F] of the feature map desc.phi_kind names (see include/rehyat.h)."""
    _check(lib().rehyat_phi(ctypes.byref(desc.c()), _ptr(x), int(n), _ptr(W), _ptr(phi),
                            _stream(stream)), "rehyat_phi")


def rehyat_state_update_workspace(desc: Desc, n: int) -> int:
    return int(lib().rehyat_state_update_workspace(ctypes.byref(desc.c()), int(n)))


def rehyat_state_update(desc: Desc, k, v, n: int, Wk, S, z, ws, ws_bytes: Optional[int] = None,
                        stream=None) -> None:
    """S += sum phi(k) v^T, z += sum phi(k) over n rows per head (see include/rehyat.h)."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib().rehyat_state_update(ctypes.byref(desc.c()), _ptr(k), _ptr(v), int(n), _ptr(Wk),
                                     _ptr(S), _ptr(z), _ptr(ws), nb, _stream(stream)),
           "rehyat_state_update")


def rehyat_hybrid_fwd_workspace(desc: Desc) -> int:
    return int(lib().rehyat_hybrid_fwd_workspace(ctypes.byref(desc.c())))


def rehyat_hybrid_fwd(desc: Desc, q, k, v, Wq, Wk, y, ws, ws_bytes: Optional[int] = None,
                      stream=None) -> None:
    """Whole-sequence hybrid attention into y (see include/rehyat.h)."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib().rehyat_hybrid_fwd(ctypes.byref(desc.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(Wq),
                                   _ptr(Wk), _ptr(y), _ptr(ws), nb, _stream(stream)),
           "rehyat_hybrid_fwd")


def rehyat_hybrid_fwd_stats(desc: Desc, q, k, v, Wq, Wk, y, lse, ws,
                            ws_bytes: Optional[int] = None, stream=None) -> None:
    """rehyat_hybrid_fwd that also writes lse = log2 of each row's normaliser."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib().rehyat_hybrid_fwd_stats(ctypes.byref(desc.c()), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(Wq), _ptr(Wk), _ptr(y), _ptr(lse), _ptr(ws), nb,
                                         _stream(stream)),
           "rehyat_hybrid_fwd_stats")


def rehyat_hybrid_bwd_workspace(desc: Desc) -> int:
    return int(lib().rehyat_hybrid_bwd_workspace(ctypes.byref(desc.c())))


def rehyat_hybrid_bwd(desc: Desc, q, k, v, Wq, Wk, y, lse, dy, dq, dk, dv, dWq, dWk, ws,
                      ws_bytes: Optional[int] = None, stream=None) -> None:
    """Gradients of sum(dy * y) of the causal form (see include/rehyat.h)."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib().rehyat_hybrid_bwd(ctypes.byref(desc.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(Wq),
                                   _ptr(Wk), _ptr(y), _ptr(lse), _ptr(dy), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(dWq), _ptr(dWk), _ptr(ws), nb,
                                   _stream(stream)),
           "rehyat_hybrid_bwd")


def rehyat_recurrent_step_workspace(desc: Desc) -> int:
    return int(lib().rehyat_recurrent_step_workspace(ctypes.byref(desc.c())))


def rehyat_recurrent_step(desc: Desc, chunk_index: int, q_c, k_c, v_c, Wq, Wk, S, z, k_tail,
                          v_tail, y_c, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    """One chunk of the chunk-wise RNN form (see include/rehyat.h)."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib().rehyat_recurrent_step(ctypes.byref(desc.c()), int(chunk_index), _ptr(q_c),
                                       _ptr(k_c), _ptr(v_c), _ptr(Wq), _ptr(Wk), _ptr(S), _ptr(z),
                                       _ptr(k_tail), _ptr(v_tail), _ptr(y_c), _ptr(ws), nb,
                                       _stream(stream)),
           "rehyat_recurrent_step")


def rehyat_recurrent_step_fused_workspace(desc: Desc) -> int:
    return int(lib().rehyat_recurrent_step_fused_workspace(ctypes.byref(desc.c())))


def rehyat_recurrent_step_fused(desc: Desc, chunk_index: int, q_c, k_c, v_c, Wq, Wk, S, z,
                                k_tail, v_tail, k_tail_out, v_tail_out, y_c, ws,
                                ws_bytes: Optional[int] = None, stream=None) -> None:
    """One chunk of the chunk-wise RNN form in a single launch (see include/rehyat.h): the
    tail is read from k_tail, v_tail and the new one written to k_tail_out, v_tail_out; ws
    must be zeroed once before its first use."""
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib().rehyat_recurrent_step_fused(ctypes.byref(desc.c()), int(chunk_index), _ptr(q_c),
                                             _ptr(k_c), _ptr(v_c), _ptr(Wq), _ptr(Wk), _ptr(S),
                                             _ptr(z), _ptr(k_tail), _ptr(v_tail),
                                             _ptr(k_tail_out), _ptr(v_tail_out), _ptr(y_c),
                                             _ptr(ws), nb, _stream(stream)),
           "rehyat_recurrent_step_fused")


def rehyat_recurrent_step_fused_noalloc(desc: Desc, chunk_index: int, q_c, k_c, v_c, Wq, Wk,
                                        S, z, k_tail, v_tail, k_tail_out, v_tail_out, y_c,
                                        stream=None) -> None:
    """rehyat_recurrent_step_fused with its scratch in the library's static device array
    (no workspace, nothing allocated; see include/rehyat.h for the size limit and the
    sharing rules)."""
    _check(lib().rehyat_recurrent_step_fused_noalloc(ctypes.byref(desc.c()), int(chunk_index),
                                                     _ptr(q_c), _ptr(k_c), _ptr(v_c), _ptr(Wq),
                                                     _ptr(Wk), _ptr(S), _ptr(z), _ptr(k_tail),
                                                     _ptr(v_tail), _ptr(k_tail_out),
                                                     _ptr(v_tail_out), _ptr(y_c),
                                                     _stream(stream)),
           "rehyat_recurrent_step_fused_noalloc")


def rehyat_timing_enable(enable, kernel: int = 1) -> None:
    """Time the launches of one kernel: 1 attention (forward and step), 2 backward dk/dv,
    3 backward dq, 4 the single-launch step (enable=False disables)."""
    _check(lib().rehyat_timing_enable(int(kernel) if enable else 0), "rehyat_timing_enable")


def rehyat_timing_read() -> Tuple[float, int]:
    """(summed attention-kernel milliseconds, launches) since the last enable/read."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().rehyat_timing_read(ctypes.byref(ms), ctypes.byref(n)), "rehyat_timing_read")
    return ms.value, n.value
