"""moe_route_noalloc (route on the library's static device scratch, nothing allocated)
against moe_route (caller's workspace): identical plans, logits and gates, bit for bit,
on two calls in a row (the second with fewer tokens, over the scratch the first left)."""
import numpy as np
import pytest

from tests import gpu_util as U
from top_routing_expert_router_amd import binding as B
from top_routing_expert_router_amd.synth import recipes

pytestmark = pytest.mark.gpu

PLAN_OUT = U.PLAN_INT + ("row_token", "topk_gate", "logits")


def _route_both(r, gpu, cfg_kw=None):
    import torch

    cfg = B.MoEConfig.from_run(r)
    for key, val in (cfg_kw or {}).items():
        setattr(cfg, key, val)
    x = U.dev(recipes.gen_x(r), gpu)
    wg, bias = recipes.gen_router(r)
    wg, bias = U.dev(wg, gpu), U.dev(bias, gpu)
    ref = B.alloc_plan(cfg, gpu, logits=True)
    got = B.alloc_plan(cfg, gpu, logits=True)
    for n in got:  # stale contents must not leak into the result
        got[n].fill_(-7)
    B.route(cfg, x, wg, bias, ref, B.alloc_workspace(cfg, gpu))
    B.route_noalloc(cfg, x, wg, bias, got)
    torch.cuda.synchronize()
    for n in PLAN_OUT:
        a, b = U.host(ref[n]), U.host(got[n])
        if n == "row_token":
            R = int(U.host(ref["offsets"])[-1])
            a, b = a[:R], b[:R]
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), (r.name, n)
    return int(U.host(ref["n_dropped"])[0])


@pytest.mark.parametrize("name,small", [("2", "2"), ("5", "5"), ("3a", "3a"), ("1", "1")])
def test_route_noalloc_equals_route_twice(gpu, name, small):
    """Full-size run then a smaller one on the same device (the second call reuses the
    scratch the first one filled)."""
    big = recipes.RUNS[name]
    dropped = _route_both(big, gpu)
    little = recipes.SMALL[small].scaled(name=f"{small}-second", T=max(1, recipes.SMALL[small].T // 3))
    _route_both(little, gpu)
    print(f"[noalloc] run {name}: full size ({dropped} dropped) then T={little.T}: identical", flush=True)


def test_route_noalloc_variants(gpu):
    """The exact path ("probs" policy under a capacity), then the split router with the
    training terms' buffers unused, in a row."""
    r = recipes.SMALL["3a"]
    _route_both(r, gpu, {"drop_policy": 1})
    _route_both(recipes.SMALL["5"].scaled(name="5-second", T=100), gpu)


def test_route_noalloc_rejects_oversized(gpu):
    """A configuration whose route scratch exceeds the static array is refused before
    anything is enqueued, with the sizes in the message."""
    import torch

    r = recipes.SMALL["5"].scaled(name="huge", T=65536, E=128, H=256)
    cfg = B.MoEConfig.from_run(r)
    plan = B.alloc_plan(cfg, gpu)
    x = torch.zeros((r.T, r.H), dtype=torch.bfloat16, device=gpu)
    wg = torch.zeros((r.H, r.E), dtype=torch.float32, device=gpu)
    with pytest.raises(B.MoEError) as ei:
        B.route_noalloc(cfg, x, wg, None, plan)
    assert ei.value.status == B.MOE_ERR_WORKSPACE and "static scratch" in str(ei.value)
