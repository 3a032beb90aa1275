"""librehyat C ABI on the host: the library loads, exports every declared entry point, and
rejects bad arguments with the documented status before anything is launched.

No call here reaches a kernel launch (each one fails validation first), so these run
without a GPU.
"""
import ctypes
import os
import re

import pytest

import hybrid_softmax_linear_amd as hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rehyat.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_ALIAS = range(9)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rehyat_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = hs.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    # the binding wraps every declared entry point and nothing else
    assert set(hs.exported_symbols()) == set(names)


def test_status_strings():
    L = hs.lib()
    names = [L.rehyat_status_str(i).decode() for i in range(9)]
    assert names == ["REHYAT_OK", "REHYAT_ERR_NULL", "REHYAT_ERR_SHAPE", "REHYAT_ERR_DTYPE",
                     "REHYAT_ERR_ALIGN", "REHYAT_ERR_UNSUPPORTED", "REHYAT_ERR_WORKSPACE",
                     "REHYAT_ERR_HIP", "REHYAT_ERR_ALIAS"]


def _desc(**kw):
    base = dict(B=2, H=3, T=7, HW=10, D=128, F=128, Tc=3, To=1, dtype=hs.BF16, y_dtype=hs.F32,
                mode=hs.CAUSAL, w_per_head=0)
    base.update(kw)
    return hs.Desc(**base)


# Fake, well-separated, 16-byte aligned "device addresses": validation never dereferences them.
P = [0x10000000 * (i + 1) for i in range(16)]


def fwd(desc, q=P[0], k=P[1], v=P[2], Wq=P[3], Wk=P[4], y=P[5], ws=P[6], ws_bytes=None):
    L = hs.lib()
    if ws_bytes is None:
        ws_bytes = L.rehyat_hybrid_fwd_workspace(ctypes.byref(desc.c())) if desc else 0
    d = ctypes.byref(desc.c()) if desc is not None else None
    return L.rehyat_hybrid_fwd(d, q, k, v, Wq, Wk, y, ws, ws_bytes, None)


def step(desc, t=1, q=P[0], k=P[1], v=P[2], Wq=P[3], Wk=P[4], S=P[5], z=P[6], kt=P[7], vt=P[8],
         y=P[9], ws=P[10], ws_bytes=None):
    L = hs.lib()
    if ws_bytes is None:
        ws_bytes = L.rehyat_recurrent_step_workspace(ctypes.byref(desc.c()))
    return L.rehyat_recurrent_step(ctypes.byref(desc.c()), t, q, k, v, Wq, Wk, S, z, kt, vt, y,
                                   ws, ws_bytes, None)


def test_hybrid_fwd_validation():
    d = _desc()
    assert fwd(None) == ERR_NULL
    assert "desc" in hs.lib().rehyat_last_error().decode()
    assert fwd(d, q=None) == ERR_NULL
    assert fwd(d, y=None) == ERR_NULL
    assert fwd(_desc(dtype=7)) == ERR_DTYPE
    assert fwd(_desc(y_dtype=2)) == ERR_DTYPE
    assert fwd(_desc(mode=3)) == ERR_DTYPE
    assert fwd(_desc(B=0)) == ERR_SHAPE
    assert fwd(_desc(To=-1)) == ERR_SHAPE
    assert fwd(_desc(Tc=0)) == ERR_SHAPE
    assert fwd(_desc(w_per_head=2)) == ERR_SHAPE
    assert fwd(_desc(D=64)) == ERR_UNSUP            # bf16 path: D = 128 only
    assert fwd(_desc(F=96)) == ERR_UNSUP
    assert fwd(_desc(dtype=hs.F32, D=96)) == ERR_UNSUP
    assert fwd(_desc(dtype=hs.F32, F=40)) == ERR_UNSUP
    assert fwd(_desc(B=1 << 12, H=1 << 10)) == ERR_SHAPE   # > 2^31 elements
    assert fwd(d, q=P[0] + 8) == ERR_ALIGN
    assert fwd(d, ws=None) == ERR_WS
    need = hs.lib().rehyat_hybrid_fwd_workspace(ctypes.byref(d.c()))
    assert fwd(d, ws_bytes=need - 1) == ERR_WS
    assert fwd(d, y=P[0]) == ERR_ALIAS              # y aliases q
    assert fwd(d, ws=P[1] + 64) == ERR_ALIAS        # workspace inside k


def test_workspace_sizes():
    L = hs.lib()
    d = _desc()
    E = d.F * d.D + d.F
    BH = d.B * d.H
    img = d.F * 256                       # one bf16 S^T or W^T image (F rows of 128 d)
    queue = 256                           # work counters of the persistent attention launch
    assert L.rehyat_hybrid_fwd_workspace(ctypes.byref(d.c())) == (
        BH * (d.T + d.n_chunks) * E * 4 + BH * d.n_chunks * img + img + queue)
    gather = 2 * BH * 40 * d.D * 2        # gathered K and V windows of (Tc + To) HW = 40 rows
    assert L.rehyat_recurrent_step_workspace(ctypes.byref(d.c())) == (
        BH * d.Tc * E * 4 + gather + BH * img + img)
    dh = _desc(w_per_head=1)              # one W^T image per head
    assert L.rehyat_recurrent_step_workspace(ctypes.byref(dh.c())) == (
        BH * d.Tc * E * 4 + gather + BH * img + d.H * img)
    assert L.rehyat_state_update_workspace(ctypes.byref(d.c()), 1000) == BH * 2 * E * 4
    assert L.rehyat_state_update_workspace(ctypes.byref(d.c()), 0) == 0
    assert L.rehyat_hybrid_fwd_workspace(ctypes.byref(_desc(D=64).c())) == 0   # invalid desc


def test_recurrent_step_validation():
    d = _desc()
    assert step(_desc(To=4)) == ERR_UNSUP                  # To > Tc
    assert step(d, t=-1) == ERR_SHAPE
    assert step(d, t=d.n_chunks) == ERR_SHAPE
    assert step(_desc(T=7, Tc=3, To=2), t=2) == ERR_UNSUP  # last chunk has 1 frame < To
    assert step(d, kt=None) == ERR_NULL
    assert step(d, S=None) == ERR_NULL
    assert step(d, z=P[5] + 4) == ERR_ALIGN
    assert step(d, ws_bytes=0) == ERR_WS
    assert step(d, y=P[2]) == ERR_ALIAS                    # y_c aliases v_c
    assert step(d, S=P[5], z=P[5] + 16) == ERR_ALIAS       # z inside S


def step_fused(desc, t=1, q=P[0], k=P[1], v=P[2], Wq=P[3], Wk=P[4], S=P[5], z=P[6], kt=P[7],
               vt=P[8], y=P[9], ws=P[10], ko=P[11], vo=P[12], ws_bytes=None):
    L = hs.lib()
    if ws_bytes is None:
        ws_bytes = L.rehyat_recurrent_step_fused_workspace(ctypes.byref(desc.c()))
    return L.rehyat_recurrent_step_fused(ctypes.byref(desc.c()), t, q, k, v, Wq, Wk, S, z, kt, vt,
                                         ko, vo, y, ws, ws_bytes, None)


def test_recurrent_step_fused_validation():
    """The single-launch step takes the step's checks, and supports bf16 with the fixed map
    only; every case below returns before any launch."""
    d = _desc()
    assert step_fused(_desc(To=4)) == ERR_UNSUP
    assert step_fused(d, t=-1) == ERR_SHAPE
    assert step_fused(d, t=d.n_chunks) == ERR_SHAPE
    assert step_fused(_desc(T=7, Tc=3, To=2), t=2) == ERR_UNSUP
    assert step_fused(d, kt=None) == ERR_NULL
    assert step_fused(d, z=P[5] + 4) == ERR_ALIGN
    assert step_fused(d, ws=P[10] + 8) == ERR_ALIGN
    assert step_fused(d, ws_bytes=0) == ERR_WS
    assert step_fused(d, y=P[2]) == ERR_ALIAS
    assert step_fused(_desc(dtype=hs.F32, D=64)) == ERR_UNSUP
    assert step_fused(_desc(phi_kind=hs.PHI_ELU)) == ERR_UNSUP
    assert step_fused(_desc(phi_kind=hs.PHI_MLP, phi_hidden=128, phi_parts=2)) == ERR_UNSUP
    assert step_fused(d, ko=None) == ERR_NULL                  # new tail needed when To > 0
    assert step_fused(d, vo=P[12] + 8) == ERR_ALIGN
    assert step_fused(d, ko=P[7]) == ERR_ALIAS                 # new tail over the carried one
    assert step_fused(d, vo=P[1]) == ERR_ALIAS                 # new tail over k_c
    assert step_fused(d, ko=P[11], vo=P[11] + 16) == ERR_ALIAS
    L = hs.lib()
    BH, E = d.B * d.H, d.F * d.D + d.F
    # per-head counters (rounded up to 256 bytes), then the new state and two frames' partials
    assert L.rehyat_recurrent_step_fused_workspace(ctypes.byref(d.c())) == (
        max(256, -(-BH * 4 // 256) * 256) + 3 * BH * E * 4)
    assert L.rehyat_recurrent_step_fused_workspace(ctypes.byref(_desc(D=64).c())) == 0


def step_noalloc(desc, t=1, q=P[0], k=P[1], v=P[2], Wq=P[3], Wk=P[4], S=P[5], z=P[6], kt=P[7],
                 vt=P[8], y=P[9], ko=P[11], vo=P[12]):
    L = hs.lib()
    return L.rehyat_recurrent_step_fused_noalloc(ctypes.byref(desc.c()), t, q, k, v, Wq, Wk, S, z,
                                                 kt, vt, ko, vo, y, None)


def test_recurrent_step_fused_noalloc_validation():
    """The no-allocation step checks every argument (and its scratch size against the static
    array) before it looks the array up on a device: every case below returns first."""
    src = open(HEADER).read()
    m = re.search(r"#define REHYAT_STATIC_SCRATCH_BYTES \((\d+) \* (\d+) \* (\d+)\)", src)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == hs.STATIC_SCRATCH_BYTES
    L = hs.lib()
    d = _desc()
    assert step_noalloc(_desc(To=4)) == ERR_UNSUP
    assert step_noalloc(d, t=d.n_chunks) == ERR_SHAPE
    assert step_noalloc(d, kt=None) == ERR_NULL
    assert step_noalloc(d, z=P[5] + 4) == ERR_ALIGN
    assert step_noalloc(d, y=P[2]) == ERR_ALIAS
    assert step_noalloc(d, ko=P[7]) == ERR_ALIAS
    assert step_noalloc(_desc(phi_kind=hs.PHI_ELU)) == ERR_UNSUP
    # the largest B*H whose scratch fits at F = 256 is accepted by the size check, one more
    # head is refused with REHYAT_ERR_WORKSPACE
    def need(B, H, F):
        return L.rehyat_recurrent_step_fused_workspace(ctypes.byref(_desc(B=B, H=H, F=F).c()))
    H = 1
    while need(1, H + 1, 256) <= hs.STATIC_SCRATCH_BYTES:
        H += 1
    assert need(1, H, 256) <= hs.STATIC_SCRATCH_BYTES < need(1, H + 1, 256)
    assert step_noalloc(_desc(B=1, H=H + 1, F=256)) == ERR_WS
    assert "static" in L.rehyat_last_error().decode()
    assert step_noalloc(_desc(B=1, H=H + 1, F=256), kt=None) == ERR_WS   # size checked first
    # the 81-frame streaming workload (B1 H12 F128) and B2 H12 at F = 256 fit
    assert need(1, 12, 128) <= hs.STATIC_SCRATCH_BYTES
    assert need(2, 12, 256) <= hs.STATIC_SCRATCH_BYTES


def test_phi_and_state_update_validation():
    L = hs.lib()
    d = _desc()
    # n = 0 is a no-op that succeeds without touching the device
    assert L.rehyat_phi(ctypes.byref(d.c()), P[0], 0, P[1], P[2], None) == OK
    assert L.rehyat_phi(ctypes.byref(d.c()), None, 10, P[1], P[2], None) == ERR_NULL
    assert L.rehyat_phi(ctypes.byref(d.c()), P[0], -1, P[1], P[2], None) == ERR_SHAPE
    assert L.rehyat_phi(ctypes.byref(d.c()), P[0], 10, P[1], P[0], None) == ERR_ALIAS
    assert L.rehyat_phi(ctypes.byref(d.c()), P[0] + 2, 10, P[1], P[2], None) == ERR_ALIGN
    ws = L.rehyat_state_update_workspace(ctypes.byref(d.c()), 100)
    assert L.rehyat_state_update(ctypes.byref(d.c()), P[0], P[1], 0, P[2], P[3], P[4], None, 0,
                                 None) == OK
    assert L.rehyat_state_update(ctypes.byref(d.c()), P[0], P[1], 100, P[2], P[3], P[4], P[5],
                                 ws - 4, None) == ERR_WS
    assert L.rehyat_state_update(ctypes.byref(d.c()), P[0], P[1], 100, P[2], None, P[4], P[5], ws,
                                 None) == ERR_NULL
    assert L.rehyat_state_update(ctypes.byref(d.c()), P[0], P[1], 100, P[2], P[0], P[4], P[5], ws,
                                 None) == ERR_ALIAS


def test_python_binding_raises():
    d = _desc()
    with pytest.raises(hs.RehyatError) as e:
        hs.rehyat_hybrid_fwd(d, P[0], P[1], P[2], P[3], P[4], P[5], None, 0, stream=0)
    assert e.value.name == "REHYAT_ERR_WORKSPACE"


def test_feature_map_kind_validation():
    assert fwd(_desc(phi_kind=3)) == ERR_DTYPE
    assert fwd(_desc(phi_kind=hs.PHI_ELU, dtype=hs.F32)) == ERR_UNSUP    # bf16 only
    assert fwd(_desc(phi_kind=hs.PHI_ELU, F=64)) == ERR_SHAPE            # 1 + elu: F = D
    assert fwd(_desc(phi_kind=hs.PHI_MLP, phi_hidden=96, phi_parts=2)) == ERR_UNSUP
    assert fwd(_desc(phi_kind=hs.PHI_MLP, phi_hidden=128, phi_parts=0)) == ERR_SHAPE
    assert fwd(_desc(phi_kind=hs.PHI_MLP, phi_hidden=128, phi_parts=3)) == ERR_SHAPE  # 128 % 3
    assert fwd(_desc(phi_kind=hs.PHI_MLP, phi_hidden=128, phi_parts=32)) == ERR_UNSUP  # 4 per part
    # the fixed map and the learned map need W; 1 + elu has no parameters
    assert fwd(_desc(), Wq=None) == ERR_NULL
    assert fwd(_desc(phi_kind=hs.PHI_MLP, phi_hidden=64, phi_parts=2), Wk=None) == ERR_NULL
    # W = NULL passes the pointer checks for 1 + elu (each call then fails a later check)
    L = hs.lib()
    de = _desc(phi_kind=hs.PHI_ELU)
    assert L.rehyat_phi(ctypes.byref(de.c()), P[0] + 2, 10, None, P[2], None) == ERR_ALIGN
    assert fwd(de, Wq=None, Wk=None, ws=None) == ERR_WS
    assert step(de, Wq=None, Wk=None, ws_bytes=0) == ERR_WS
    # the learned map's parameter block [W1 D*h][b1 h][W2 h*F][b2 F] (bf16) is alias-checked
    dm = _desc(phi_kind=hs.PHI_MLP, phi_hidden=64, phi_parts=2)
    block = (128 * 64 + 64 + 64 * 128 + 128) * 2
    assert L.rehyat_phi(ctypes.byref(dm.c()), P[0], 10, P[3], P[3] + block - 16, None) == ERR_ALIAS
    assert fwd(dm, y=P[3] + block - 16) == ERR_ALIAS


def test_feature_map_workspace_sizes():
    L = hs.lib()
    base = _desc()
    BH = base.B * base.H
    E = base.F * base.D + base.F
    N = base.T * base.HW
    img = base.F * 256
    gather = 2 * BH * 40 * base.D * 2
    for kw in (dict(phi_kind=hs.PHI_ELU), dict(phi_kind=hs.PHI_MLP, phi_hidden=128, phi_parts=2)):
        d = _desc(**kw)
        rows = BH * d.F * 2                      # bytes of one bf16 phi row for every head
        # whole sequence: S^T images but no W^T image, phi(k) and phi(q) of all N rows
        assert L.rehyat_hybrid_fwd_workspace(ctypes.byref(d.c())) == (
            BH * (d.T + d.n_chunks) * E * 4 + BH * d.n_chunks * img + 2 * N * rows + 256)
        # one chunk: phi(q_c) of Tc*HW rows and phi of the (Tc + To)*HW window keys
        assert L.rehyat_recurrent_step_workspace(ctypes.byref(d.c())) == (
            BH * d.Tc * E * 4 + gather + BH * img + (30 + 40) * rows)
        assert L.rehyat_state_update_workspace(ctypes.byref(d.c()), 1000) == (
            BH * 2 * E * 4 + 1000 * rows)


def bwd(desc, **kw):
    L = hs.lib()
    names = ("q", "k", "v", "Wq", "Wk", "y", "lse", "dy", "dq", "dk", "dv", "dWq", "dWk", "ws")
    ptrs = {n: P[i] for i, n in enumerate(names)}
    ptrs.update(kw)
    need = L.rehyat_hybrid_bwd_workspace(ctypes.byref(desc.c()))
    ws_bytes = kw.pop("ws_bytes", need) if "ws_bytes" in kw else need
    return L.rehyat_hybrid_bwd(ctypes.byref(desc.c()), *[ptrs[n] for n in names], ws_bytes, None)


def test_backward_validation():
    d = _desc()
    assert bwd(_desc(mode=hs.BIDIR)) == ERR_UNSUP
    assert bwd(_desc(dtype=hs.F32, D=64)) == ERR_UNSUP
    assert bwd(_desc(phi_kind=hs.PHI_ELU)) == ERR_UNSUP
    assert bwd(d, lse=None) == ERR_NULL
    assert bwd(d, dWk=None) == ERR_NULL
    assert bwd(d, dq=P[0] + 8) == ERR_ALIGN
    assert bwd(d, ws_bytes=16) == ERR_WS
    assert bwd(d, dq=P[0]) == ERR_ALIAS              # dq over q
    assert bwd(d, dv=P[8] + 64) == ERR_ALIAS         # dv inside dq
    L = hs.lib()
    # stats forward: lse required, not overlapping y
    need = L.rehyat_hybrid_fwd_workspace(ctypes.byref(d.c()))
    assert L.rehyat_hybrid_fwd_stats(ctypes.byref(d.c()), P[0], P[1], P[2], P[3], P[4], P[5], None,
                                     P[6], need, None) == ERR_NULL
    assert L.rehyat_hybrid_fwd_stats(ctypes.byref(d.c()), P[0], P[1], P[2], P[3], P[4], P[5],
                                     P[5] + 16, P[6], need, None) == ERR_ALIAS


def test_backward_workspace_size():
    L = hs.lib()
    d = _desc()
    BH, N, T, E, F = d.B * d.H, d.T * d.HW, d.T, d.F * d.D + d.F, d.F
    r = lambda n: (n + 255) // 256 * 256
    expect = sum(r(x) for x in (BH * T * E * 4, BH * d.n_chunks * E * 4, BH * T * E * 4,
                                BH * d.n_chunks * F * d.D * 2, BH * T * F * d.D * 2, F * d.D * 2,
                                F * d.D * 2, BH * N * d.D * 2, BH * N * d.D * 2, BH * N * 4,
                                BH * N * 4, BH * N * F * 2, BH * N * F * 2, BH * N * F * 2,
                                BH * F * d.D * 4, BH * F * 4))
    assert L.rehyat_hybrid_bwd_workspace(ctypes.byref(d.c())) == expect
