"""The C ABI on the host: the library loads, exports every symbol include/moe.h
declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import oracle
from top_routing_expert_router_amd import binding as B
from top_routing_expert_router_amd.synth import recipes

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_validate",
              "moe_capacity", "moe_max_rows", "moe_workspace_bytes"):
        assert n in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(B._build.LIB)
    for n in _declared():
        assert hasattr(L, n), n


def _cfg(**kw):
    base = dict(T=1024, H=256, E=8, k=2, F=512, dtype=B.BF16, gate_mode=B.SOFTMAX_TOPK, act=B.GELU, dropless=0,
                capacity_factor=1.25, min_capacity=0)
    base.update(kw)
    return B.MoEConfig(**base)


@pytest.mark.parametrize("kw", [
    dict(k=0), dict(k=17, E=32), dict(k=5, E=4), dict(E=0), dict(E=1025), dict(T=-1), dict(H=0), dict(F=0),
    dict(T=2**30, k=2), dict(dtype=2), dict(gate_mode=3), dict(act=3), dict(dropless=2), dict(min_capacity=-1),
    dict(capacity_factor=0.0), dict(capacity_factor=-1.0), dict(capacity_factor=float("nan")),
    dict(capacity_factor=float("inf")), dict(aux_mode=2), dict(aux_mode=-1), dict(aux_coeff=float("nan")),
    dict(z_coeff=float("inf")), dict(score_fn=2), dict(drop_policy=2), dict(drop_policy=-1),
    dict(second_policy=2), dict(second_policy=1, k=1), dict(second_policy=1, k=3), dict(shared_F=-1),
])
def test_validate_rejects(kw):
    c = _cfg(**kw)
    assert B.validate(c) == B.MOE_ERR_INVALID_ARG
    assert B.capacity(c) == -2
    assert B.max_rows(c) == -1
    assert B.workspace_bytes(c) == 0


def test_validate_accepts_edge_configs():
    for kw in (dict(T=0), dict(E=1, k=1), dict(E=1024, k=16), dict(dropless=1, capacity_factor=0.0),
               dict(H=1, F=1), dict(H=7, F=9), dict(T=2**30 - 1, k=2)):
        assert B.validate(_cfg(**kw)) == B.MOE_OK, kw


@pytest.mark.parametrize("name", list(recipes.RUNS))
def test_capacity_and_rows_match_oracle(name):
    r = recipes.RUNS[name]
    c = B.MoEConfig.from_run(r)
    C = oracle.capacity(r.T, r.k, r.E, r.cf, r.min_capacity, r.dropless)
    assert B.capacity(c) == C
    rmax = r.T * r.k if C < 0 else min(r.T * r.k, r.E * C)
    assert B.max_rows(c) == rmax
    assert B.workspace_bytes(c) >= rmax * r.F * r.elem_bytes


@pytest.mark.parametrize("name", list(recipes.RUNS))
def test_saved_act_bytes(name):
    """moe_saved_act_bytes: u (and v for SwiGLU) of every packed row, bf16."""
    r = recipes.RUNS[name]
    c = B.MoEConfig.from_run(r)
    m1 = 2 if r.act == recipes.SWIGLU else 1
    assert B.saved_act_bytes(c) == m1 * B.max_rows(c) * r.F * 2
    assert B.saved_act_bytes(_cfg(k=0)) == 0


def test_min_capacity_floor():
    c = _cfg(T=10, E=8, k=1, capacity_factor=1.0, min_capacity=4)
    assert B.capacity(c) == 4


class _Null:
    def data_ptr(self):
        return 0


def test_entry_points_reject_before_launch():
    """Argument errors come back as status codes with nothing enqueued (no GPU needed)."""
    L = B.lib()
    c = _cfg()
    cc = c.c()
    plan = B._Plan()  # all NULL
    st = L.moe_route(ctypes.byref(cc), 16, 16, None, ctypes.byref(plan), 16, 1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG
    good = B._Plan(*([256] * 8 + [None]))
    assert L.moe_route(ctypes.byref(cc), 256, 256, None, ctypes.byref(good), 256, 16, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_route(ctypes.byref(cc), 256, 256, None, ctypes.byref(good), None, 1 << 40, None) == \
        B.MOE_ERR_WORKSPACE
    bad = _cfg(k=0).c()
    assert L.moe_route(ctypes.byref(bad), 256, 256, None, ctypes.byref(good), 256, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARG
    # SwiGLU needs W3; non-SwiGLU must not get one
    sw = _cfg(act=B.SWIGLU).c()
    assert L.moe_expert_ffn(ctypes.byref(sw), 256, ctypes.byref(good), 256, None, 256, 256, 256, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(ctypes.byref(cc), 256, ctypes.byref(good), 256, 256, 256, 256, 256, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(ctypes.byref(cc), 256, ctypes.byref(good), 256, None, 256, 256, 256, 8, None) == \
        B.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(ctypes.byref(cc), None, ctypes.byref(good), 256, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(cc), 256, ctypes.byref(good), None, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward(ctypes.byref(cc), 256, None, None, 256, None, 256, None, 256, ctypes.byref(good), 256, 256,
                         256, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_validate(None) == B.MOE_ERR_INVALID_ARG
    # moe_forward_save: act required; only the tiled bf16 path keeps pre-activations
    assert L.moe_forward_save(ctypes.byref(cc), 256, 256, None, 256, None, 256, None, 256, ctypes.byref(good), 256,
                              256, None, 256, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    f32 = _cfg(dtype=B.F32).c()
    assert L.moe_forward_save(ctypes.byref(f32), 256, 256, None, 256, None, 256, None, 256, ctypes.byref(good), 256,
                              256, 256, 256, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    odd = _cfg(H=96).c()  # H % 64 != 0: not the tiled path
    assert L.moe_forward_save(ctypes.byref(odd), 256, 256, None, 256, None, 256, None, 256, ctypes.byref(good), 256,
                              256, 256, 256, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    # shared expert: needs shared_F > 0, its weights (Ws3 iff SwiGLU) and the workspace
    sh = _cfg(shared_F=384)
    shc = sh.c()
    ws_need = B.workspace_bytes(sh)
    assert ws_need >= sh.T * sh.shared_F * 2 + sh.T * sh.H * 2
    assert L.moe_shared_expert(ctypes.byref(cc), 256, 256, None, 256, 256, 256, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_shared_expert(ctypes.byref(shc), 256, None, None, 256, 256, 256, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_shared_expert(ctypes.byref(shc), 256, 256, 256, 256, 256, 256, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_shared_expert(ctypes.byref(shc), 256, 256, None, 256, 256, 256, ws_need - 1, None) == \
        B.MOE_ERR_WORKSPACE
    assert L.moe_combine_shared(ctypes.byref(shc), 256, ctypes.byref(good), None, None, 256, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_shared(ctypes.byref(cc), 256, 256, None, 256, None, 256, 256, None, 256, None, 256,
                                ctypes.byref(good), 256, 256, 256, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_shared(ctypes.byref(shc), 256, 256, None, 256, None, 256, 256, None, 256, None, 256,
                                ctypes.byref(good), 256, 256, 256, ws_need - 1, None) == B.MOE_ERR_WORKSPACE


def test_status_strings():
    for s in range(5):
        assert B.status_str(s)
    with pytest.raises(B.MoEError):
        B._check(B.MOE_ERR_INVALID_ARG, "x")
