"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing plans (expert ids, slot positions, drop sets, counts, offsets,
row_token) must match bit-exactly; gates within 1e-5 relative; logits within
1e-5 relative L2 (bit-identical in practice); layer outputs within the bf16 /
fp32 tolerances of tests/gpu_util.py, measured on the residual-free output.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as U
from top_routing_expert_router_amd import binding as B
from top_routing_expert_router_amd import synth
from top_routing_expert_router_amd.synth import recipes

pytestmark = pytest.mark.gpu

SMALL = list(recipes.SMALL)


def _cap(r):
    return None if r.dropless else oracle.capacity(r.T, r.k, r.E, r.cf, r.min_capacity)


def _oracle_route(r, x, wg, bias):
    return oracle.route(x, r.dtype, wg, bias, r.k, r.gate_mode, _cap(r))


def _gpu_route(r, gpu, x, wg, bias):
    import torch

    cfg = B.MoEConfig.from_run(r)
    plan = B.alloc_plan(cfg, gpu, logits=True)
    ws = B.alloc_workspace(cfg, gpu)
    B.route(cfg, U.dev(x, gpu), U.dev(wg, gpu), U.dev(bias, gpu), plan, ws)
    torch.cuda.synchronize()
    return cfg, plan


def _exact_path(r):
    """The runs whose router computes every logit and gate as defined (fp32 activations, or H
    not a multiple of 64): logits and gates are then bit-identical to the oracle's."""
    return r.dtype == recipes.F32 or r.H % 64 != 0


def _check_route(r, gplan, oplan):
    if _exact_path(r):
        _check_exact_route(r, gplan, oplan, f"run {r.name}")
        return
    gl = U.host(gplan["logits"])
    nd = int((gl != oplan["logits"]).sum())
    _, rel = U.err_stats(gl.astype(np.float64), oplan["logits"].astype(np.float64))
    print(f"[parity] run {r.name}: logits rel-L2 {rel:.2e}, {nd} of {gl.size} not bit-identical; "
          f"R={oplan['R']} dropped={int(oplan['n_dropped'][0])}", flush=True)
    assert rel <= U.LOGIT_RELL2
    U.assert_plan_equal(gplan, oplan, f"run {r.name}")


@pytest.mark.parametrize("name", SMALL)
def test_route_small(gpu, name):
    r = recipes.SMALL[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    _, gplan = _gpu_route(r, gpu, x, wg, bias)
    _check_route(r, gplan, _oracle_route(r, x, wg, bias))


@pytest.mark.parametrize("name", list(recipes.RUNS))
def test_route_full_size(gpu, name):
    """Routing of the full workloads, every token compared."""
    r = recipes.RUNS[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    _, gplan = _gpu_route(r, gpu, x, wg, bias)
    _check_route(r, gplan, _oracle_route(r, x, wg, bias))


# Split router with more than 64 experts: the h chunks are split over 1, 2, 4 or 8
# workgroups per 256-token x 64-expert tile (as many as keep the grid within 256
# workgroups and divide the chunk count), their binary64 parts added at
# certification.  One shape per split count, and one with an odd chunk count.
_HSPLIT_SHAPES = {
    "hs8": dict(T=700, E=256, H=512),     # 12 tiles, 8 chunks
    "hs4": dict(T=333, E=256, H=256),     # 8 tiles, 4 chunks
    "hs2": dict(T=8192, E=256, H=256),    # 128 tiles
    "hs1": dict(T=16384, E=256, H=128),   # 256 tiles
    "odd": dict(T=700, E=96, H=192),      # 3 chunks
}


@pytest.mark.parametrize("name", list(_HSPLIT_SHAPES))
def test_split_router_h_split(gpu, name):
    """Routing through the split-h logits kernel, every token compared with the oracle (plan
    bit-exact, logits and gates within tolerance)."""
    r = recipes.SMALL["5"].scaled(name=f"5-{name}", **_HSPLIT_SHAPES[name])
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    _, gplan = _gpu_route(r, gpu, x, wg, bias)
    _check_route(r, gplan, _oracle_route(r, x, wg, bias))


@pytest.mark.parametrize("name", ["2", "3b", "5"])
def test_dispatch_bit_exact(gpu, name):
    import torch

    r = recipes.SMALL[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    oplan = _oracle_route(r, x, wg, bias)
    cfg = B.MoEConfig.from_run(r)
    gp = U.plan_to_device(oplan, cfg, gpu)
    Xd = torch.zeros((B.max_rows(cfg), r.H), dtype=torch.bfloat16, device=gpu)
    B.dispatch(cfg, U.dev(x, gpu), gp, Xd)
    torch.cuda.synchronize()
    assert np.array_equal(U.host(Xd)[:oplan["R"]], oracle.dispatch(x, r.dtype, oplan))


@pytest.mark.parametrize("name", SMALL)
def test_expert_ffn(gpu, name):
    import torch

    r = recipes.SMALL[name]
    d = recipes.gen_all(r)
    oplan = _oracle_route(r, d["x"], d["wg"], d["bias"])
    X = oracle.dispatch(d["x"], r.dtype, oplan)
    Yref = oracle.expert_ffn(X, oplan["offsets"], r.dtype, r.act, d["w1"], d["w3"], d["w2"])
    cfg = B.MoEConfig.from_run(r)
    gp = U.plan_to_device(oplan, cfg, gpu)
    rmax = B.max_rows(cfg)
    Xd = torch.zeros((rmax, r.H), dtype=torch.bfloat16 if r.dtype == recipes.BF16 else torch.float32, device=gpu)
    Xd[:oplan["R"]].copy_(U.dev(X, "cpu"))
    Yd = torch.zeros_like(Xd)
    ws = B.alloc_workspace(cfg, gpu)
    B.expert_ffn(cfg, Xd, gp, U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu), Yd, ws)
    torch.cuda.synchronize()
    U.assert_close(U.host(Yd)[:oplan["R"]], Yref, r.dtype == recipes.BF16, f"expert FFN run {r.name}")


@pytest.mark.parametrize("name", ["1", "3a", "5"])
@pytest.mark.parametrize("with_residual", [False, True])
def test_combine(gpu, name, with_residual):
    import torch

    r = recipes.SMALL[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    oplan = _oracle_route(r, x, wg, bias)
    dt = recipes.act_dtype(r)
    Yh = synth.normal(4242, oplan["R"] * r.H, 0.7, dt).reshape(oplan["R"], r.H)
    res = x if with_residual else None
    yref = oracle.combine(U.as_f64(Yh), oplan, r.dtype, residual=res)
    cfg = B.MoEConfig.from_run(r)
    gp = U.plan_to_device(oplan, cfg, gpu)
    tdt = torch.bfloat16 if r.dtype == recipes.BF16 else torch.float32
    Yd = torch.zeros((B.max_rows(cfg), r.H), dtype=tdt, device=gpu)
    Yd[:oplan["R"]].copy_(U.dev(Yh, "cpu"))
    yd = torch.empty((r.T, r.H), dtype=tdt, device=gpu)
    B.combine(cfg, Yd, gp, U.dev(res, gpu), yd)
    torch.cuda.synchronize()
    U.assert_close(U.host(yd), yref, r.dtype == recipes.BF16, f"combine run {r.name} residual={with_residual}")


def _gpu_forward(r, gpu, d, residual=False, weights=None):
    import torch

    cfg = B.MoEConfig.from_run(r)
    tdt = torch.bfloat16 if r.dtype == recipes.BF16 else torch.float32
    rmax = B.max_rows(cfg)
    xd = U.dev(d["x"], gpu)
    if weights is None:
        weights = (U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu))
    plan = B.alloc_plan(cfg, gpu, logits=True)
    X = torch.empty((max(rmax, 1), r.H), dtype=tdt, device=gpu)
    Y = torch.empty_like(X)
    y = torch.empty((r.T, r.H), dtype=tdt, device=gpu)
    ws = B.alloc_workspace(cfg, gpu)
    B.forward(cfg, xd, U.dev(d["wg"], gpu), U.dev(d["bias"], gpu), *weights, xd if residual else None, y, plan, X, Y,
              ws)
    torch.cuda.synchronize()
    return plan, y


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(gpu, name):
    r = recipes.SMALL[name]
    d = recipes.gen_all(r)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, _cap(r))
    gplan, y = _gpu_forward(r, gpu, d)
    _check_route(r, gplan, oplan)
    U.assert_close(U.host(y), yref, r.dtype == recipes.BF16, f"forward run {r.name}")
    # with the residual: a token all of whose assignments were dropped passes x through bit-exactly
    gplan2, y2 = _gpu_forward(r, gpu, d, residual=True)
    dropped = (oplan["dst_row"] < 0).all(1)
    if dropped.any():
        assert np.array_equal(U.host(y2)[dropped], d["x"][dropped])


@pytest.mark.parametrize("name", ["1", "2", "3a", "3b", "3c"])
def test_forward_full_size_all_tokens(gpu, name):
    """Full workload on the GPU in the benchmark's launch configuration; routing and the
    output of every token compared with the oracle's whole-layer forward."""
    r = recipes.RUNS[name]
    d = recipes.gen_all(r)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, _cap(r))
    gplan, y = _gpu_forward(r, gpu, d)
    _check_route(r, gplan, oplan)
    U.assert_close(U.host(y), yref, r.dtype == recipes.BF16, f"forward full-size run {r.name}, all {r.T} tokens")
    dropped = (oplan["dst_row"] < 0).all(1)
    if dropped.any():  # a fully dropped token's residual-free output is zero
        assert not U.as_f64(U.host(y)[dropped]).any()


@pytest.mark.parametrize("name", ["4", "5"])
def test_forward_full_size_sampled(gpu, name):
    """Full workload on the GPU in the benchmark's launch configuration; routing compared
    on every token, outputs on the tokens of the first and last row of every 128-row
    m-tile of every non-empty expert (also the edges of 256-row tiles) plus random ones."""
    r = recipes.RUNS[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    oplan = _oracle_route(r, x, wg, bias)
    toks = U.tile_boundary_tokens(oplan, r.T, int(r.run_id))
    weights, yref = U.upload_weights_with_reference(r, gpu, x, oplan, toks)
    gplan, y = _gpu_forward(r, gpu, dict(x=x, wg=wg, bias=bias), weights=weights)
    _check_route(r, gplan, oplan)
    nonempty = int((oplan["kept"] > 0).sum())
    U.assert_close(U.host(y)[toks], yref, r.dtype == recipes.BF16,
                   f"forward full-size run {r.name}: {len(toks)} tokens covering {nonempty} non-empty experts")


@pytest.mark.parametrize("name", ["2", "3a", "5"])
def test_route_full_size_deterministic(gpu, name):
    """Two routings of the same full-size batch give the same bits (logits, choices, gates,
    plan), also where undecided tokens go through the global refinement queue (256 experts, top-8)."""
    r = recipes.RUNS[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    _, p1 = _gpu_route(r, gpu, x, wg, bias)
    _, p2 = _gpu_route(r, gpu, x, wg, bias)
    for n in ("logits", "topk_gate"):
        assert np.array_equal(U.host(p1[n]).view(np.uint32), U.host(p2[n]).view(np.uint32)), n
    for n in U.PLAN_INT:
        assert np.array_equal(U.host(p1[n]), U.host(p2[n])), n
    R = int(U.host(p1["offsets"])[-1])  # rows past R are not written
    assert np.array_equal(U.host(p1["row_token"])[:R], U.host(p2["row_token"])[:R])


@pytest.mark.parametrize("shape", [
    # top-1, bf16, H % 64 == 0, F % 64 == 0: the second GEMM writes y itself;
    # one shape per tiled kernel it can run in (128-row pipe, 256-row pipe,
    # split-ring), with drops (cf < 1) so that the dropped-token pass matters
    dict(name="pipe128", T=2048, H=256, E=16, F=512, cf=1.0),
    dict(name="pipe256", T=4096, H=256, E=8, F=256, cf=0.5),
    dict(name="ring", T=16384, H=768, E=8, F=256, cf=0.5),
    # the Switch workload itself (the benchmark's configuration)
    dict(name="switch", T=16384, H=768, E=64, F=3072, cf=1.0),
])
@pytest.mark.parametrize("residual", [False, True])
def test_forward_top1_fused_equals_stages(gpu, shape, residual):
    """moe_forward (combine folded into the second GEMM) against the stage entry
    points route -> dispatch -> expert_ffn -> combine: bit-identical y."""
    import torch

    kw = dict(shape)
    r = recipes.RUNS["2"].scaled(name="top1-" + kw.pop("name"), **kw)
    d = recipes.gen_all(r)
    gplan, y = _gpu_forward(r, gpu, d, residual=residual)
    cfg = B.MoEConfig.from_run(r)
    xd = U.dev(d["x"], gpu)
    w = (U.dev(d["w1"], gpu), None, U.dev(d["w2"], gpu))
    plan = B.alloc_plan(cfg, gpu)
    ws = B.alloc_workspace(cfg, gpu)
    rmax = B.max_rows(cfg)
    X = torch.zeros((rmax, r.H), dtype=torch.bfloat16, device=gpu)
    Y = torch.zeros_like(X)
    ys = torch.empty((r.T, r.H), dtype=torch.bfloat16, device=gpu)
    B.route(cfg, xd, U.dev(d["wg"], gpu), U.dev(d["bias"], gpu), plan, ws)
    B.dispatch(cfg, xd, plan, X)
    B.expert_ffn(cfg, X, plan, *w, Y, ws)
    B.combine(cfg, Y, plan, xd if residual else None, ys)
    torch.cuda.synchronize()
    nd = int(U.host(plan["n_dropped"])[0])
    print(f"[parity] top-1 fused {r.name} residual={residual}: dropped {nd} of {r.T}", flush=True)
    assert nd > 0 or r.cf >= 1.0
    assert np.array_equal(U.host(plan["dst_row"]), U.host(gplan["dst_row"]))
    assert np.array_equal(U.host(y).view(np.uint16), U.host(ys).view(np.uint16))


@pytest.mark.parametrize("name", ["2", "3a"])
def test_forward_in_place(gpu, name):
    """y, the residual and x as one buffer (top-1 with the combine in the second
    GEMM, and top-4 with the separate combine): the same y as with three buffers."""
    import torch

    r = recipes.SMALL[name]
    d = recipes.gen_all(r)
    _, y = _gpu_forward(r, gpu, d, residual=True)
    cfg = B.MoEConfig.from_run(r)
    rmax = B.max_rows(cfg)
    xd = U.dev(d["x"], gpu)
    plan = B.alloc_plan(cfg, gpu)
    X = torch.empty((max(rmax, 1), r.H), dtype=xd.dtype, device=gpu)
    Y = torch.empty_like(X)
    ws = B.alloc_workspace(cfg, gpu)
    B.forward(cfg, xd, U.dev(d["wg"], gpu), U.dev(d["bias"], gpu), U.dev(d["w1"], gpu), U.dev(d["w3"], gpu),
              U.dev(d["w2"], gpu), xd, xd, plan, X, Y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(U.host(xd), U.host(y))


def test_determinism(gpu):
    r = recipes.SMALL["3a"]
    d = recipes.gen_all(r)
    p1, y1 = _gpu_forward(r, gpu, d)
    p2, y2 = _gpu_forward(r, gpu, d)
    assert np.array_equal(U.host(y1), U.host(y2))
    for n in U.PLAN_INT + ("topk_gate", "logits"):
        assert np.array_equal(U.host(p1[n]), U.host(p2[n])), n
    R = int(U.host(p1["offsets"])[-1])
    assert np.array_equal(U.host(p1["row_token"])[:R], U.host(p2["row_token"])[:R])


# --------------------------------------------------------------------------- edge cases


def _run_edge(gpu, r):
    d = recipes.gen_all(r)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, _cap(r))
    gplan, y = _gpu_forward(r, gpu, d)
    _check_route(r, gplan, oplan)
    if r.T:
        U.assert_close(U.host(y), yref, r.dtype == recipes.BF16, f"edge {r.name}")
    return gplan, oplan


@pytest.mark.parametrize("kw", [
    dict(name="T1", T=1), dict(name="T63", T=63), dict(name="T65", T=65),
    dict(name="E1", E=1, k=1), dict(name="kE", E=6, k=6), dict(name="k16", E=20, k=16, T=90),
    dict(name="ragged", H=37, F=45), dict(name="H1", H=1, F=3, T=70), dict(name="bigE", E=1024, k=3, T=130, H=64),
    dict(name="tinycf", cf=0.05), dict(name="mincap", cf=0.05, min_capacity=7),
    # 33..64 experts, a multiple of 4: the router loads the fp32 weights itself
    # (48: padded expert columns; 36 and T=1: a single, mostly empty token tile)
    dict(name="E48", E=48, k=2, T=333), dict(name="E36", E=36, k=3, T=1), dict(name="E64H128", E=64, k=1, H=128),
    dict(name="E44", E=44, k=4, T=257, H=192),
    # tiled GEMMs whose output width is 8 mod 16: the last 8-column group of a
    # row is stored by the lower half-wave only (F=72 for the first GEMM, H=72
    # for the second)
    dict(name="F72", H=128, F=72, T=300), dict(name="H72", H=72, F=128, T=300),
])
def test_edge_shapes(gpu, kw):
    base = recipes.SMALL["5"].scaled(T=200, H=64, F=96, E=16, k=4)
    name = kw.pop("name")
    dl = 0 if ("cf" in kw or "min_capacity" in kw) else base.dropless
    r = base.scaled(name=f"edge-{name}", dropless=dl, **kw)
    _run_edge(gpu, r)


def test_fp32_ragged_and_gelu(gpu):
    r = recipes.RUNS["1"].scaled(name="edge-f32", T=300, H=20, F=28, E=5, k=2, act=recipes.GELU)
    _run_edge(gpu, r)


def test_empty_batch(gpu):
    r = recipes.SMALL["3a"].scaled(name="edge-T0", T=0)
    gplan, _ = _gpu_forward(r, gpu, recipes.gen_all(r))
    assert (U.host(gplan["demand"]) == 0).all() and (U.host(gplan["offsets"]) == 0).all()
    assert U.host(gplan["n_dropped"])[0] == 0


def test_designed_ties_break_to_lower_index(gpu):
    """x = 0 makes every logit equal to the bias exactly, on both sides."""
    r = recipes.SMALL["5"].scaled(name="ties", T=130, H=32, F=16, E=12, k=4, bias="none")
    d = recipes.gen_all(r)
    d["x"] = np.zeros_like(d["x"])
    d["bias"] = np.array([0, 1, 1, 0.5, 1, 0, 0.5, 1, 0, 0, 1, 0.5], np.float32)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, None)
    assert (oplan["topk_idx"] == np.array([1, 2, 4, 7])).all()
    gplan, y = _gpu_forward(r, gpu, d)
    _check_route(r, gplan, oplan)


def test_capacity_calculator_scenario_on_gpu(gpu):
    """The capacity calculator's worked example (T=1024, E=64, k=2, cf=1.25: 472 of 2048
    assignments dropped) built through x and Wg so that logits are exact."""
    import torch

    T, E, k, H = 1024, 64, 2, 64
    x = np.zeros((T, H), np.float32)
    for t in range(T):
        a, b = (0, 1 + t % 63) if t < 512 else (1 + t % 63, 1 + (t + 1) % 63)
        x[t, a], x[t, b] = 1.0, 0.5
    wg = np.eye(H, E, dtype=np.float32) * 10.0
    r = recipes.SMALL["2"].scaled(name="calc", T=T, H=H, E=E, k=k, F=32, cf=1.25, gate_mode=recipes.TOPK_SOFTMAX)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact in bf16
    oplan = oracle.route(xb, r.dtype, wg, None, k, r.gate_mode, oracle.capacity(T, k, E, 1.25))
    assert int(oplan["n_dropped"][0]) == 472
    _, gplan = _gpu_route(r, gpu, xb, wg, None)
    _check_route(r, gplan, oplan)
    assert U.host(gplan["n_dropped"])[0] == 472
    assert U.host(gplan["offsets"])[-1] == 2048 - 472


@pytest.mark.parametrize("act,F,H", [(recipes.GELU, 3328, 128), (recipes.SWIGLU, 1664, 128), (recipes.RELU, 1280, 256)])
def test_expert_ffn_large_tiles(gpu, act, F, H):
    """Expert FFN on shapes that take the 256-row pipelined tiles (many rows per expert),
    every output element compared."""
    import torch

    r = recipes.SMALL["4"].scaled(name=f"tiles-{act}", T=4096, H=H, F=F, E=4, k=1, act=act, dropless=1,
                                  gate_mode=recipes.SOFTMAX_TOPK, bias="n1")
    d = recipes.gen_all(r)
    oplan = _oracle_route(r, d["x"], d["wg"], d["bias"])
    X = oracle.dispatch(d["x"], r.dtype, oplan)
    Yref = oracle.expert_ffn(X, oplan["offsets"], r.dtype, r.act, d["w1"], d["w3"], d["w2"])
    cfg = B.MoEConfig.from_run(r)
    gp = U.plan_to_device(oplan, cfg, gpu)
    Xd = torch.zeros((B.max_rows(cfg), r.H), dtype=torch.bfloat16, device=gpu)
    Xd[:oplan["R"]].copy_(U.dev(X, "cpu"))
    Yd = torch.zeros_like(Xd)
    ws = B.alloc_workspace(cfg, gpu)
    B.expert_ffn(cfg, Xd, gp, U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu), Yd, ws)
    torch.cuda.synchronize()
    U.assert_close(U.host(Yd)[:oplan["R"]], Yref, True, f"expert FFN large tiles act={act}")


# Row counts on both sides of every 32-row token-fragment boundary of the
# 128- and 256-row tiles (a wave multiplies only its fragments that hold rows
# of the tile), with empty experts between them.
_FRAG_ROWS = [1, 31, 32, 33, 0, 63, 64, 65, 95, 96, 97, 127, 128, 0, 129, 159, 160, 161, 191, 192, 193, 223, 224,
              225, 255, 256, 257, 300, 5, 0, 40, 90]


@pytest.mark.parametrize("act,E", [(recipes.SWIGLU, 32), (recipes.GELU, 32), (recipes.SWIGLU, 16),
                                   (recipes.RELU, 16)])
def test_expert_ffn_fragment_boundaries(gpu, act, E):
    """Expert FFN on experts of 0..300 rows placed around every 32-row fragment edge; E = 32 puts the
    experts of at most 128 rows in 128-row tiles and the others in 256-row ones, E = 16 (the last 16
    counts, more than 128 rows per expert on average) every expert in 256-row tiles.  Every output
    element compared with the oracle."""
    import torch

    counts = np.array(_FRAG_ROWS[-E:], np.int32)
    R = int(counts.sum())
    r = recipes.SMALL["4"].scaled(name=f"frag-{act}-{E}", T=R, H=256, F=320, E=E, k=1, act=act, dropless=1,
                                  gate_mode=recipes.SOFTMAX_TOPK, bias="n1")
    d = recipes.gen_all(r)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    X = d["x"]  # R token rows, read as the expert-contiguous rows
    Yref = oracle.expert_ffn(X, offsets, r.dtype, r.act, d["w1"], d["w3"], d["w2"])
    cfg = B.MoEConfig.from_run(r)
    gp = B.alloc_plan(cfg, gpu)
    gp["offsets"].copy_(torch.from_numpy(offsets))
    Xd = torch.zeros((B.max_rows(cfg), r.H), dtype=torch.bfloat16, device=gpu)
    Xd[:R].copy_(U.dev(X, "cpu"))
    Yd = torch.full_like(Xd, float("nan"))
    ws = B.alloc_workspace(cfg, gpu)
    B.expert_ffn(cfg, Xd, gp, U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu), Yd, ws)
    torch.cuda.synchronize()
    U.assert_close(U.host(Yd)[:R], Yref, True, f"expert FFN fragment edges act={act} E={E}")



@pytest.mark.parametrize("act,H,F,counts", [
    (recipes.SWIGLU, 250, 500, [1, 63, 64, 65, 0, 700, 7, 1300]),
    (recipes.RELU, 128, 200, [64, 0, 1290, 31, 1292, 5]),
    (recipes.GELU, 100, 140, [3, 2500, 0, 2400]),
    (recipes.SWIGLU, 37, 45, [1, 63, 64, 65, 0, 130, 7]),  # below the tiles' size threshold
])
def test_expert_ffn_f32_tiles(gpu, act, H, F, counts):
    """fp32 expert FFN with row counts around the 64-row tile edge and k and output widths that
    are not multiples of the tile: the LDS-tiled kernel (at least 2^26 multiply-adds per GEMM) and
    the one-thread-per-output kernel below that, every output element against the oracle."""
    import torch

    counts = np.array(counts, np.int32)
    R = int(counts.sum())
    r = recipes.RUNS["1"].scaled(name=f"f32tiles-{act}-{H}", T=R, H=H, F=F, E=len(counts), k=1, act=act,
                                 dropless=1)
    d = recipes.gen_all(r)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Yref = oracle.expert_ffn(d["x"], offsets, r.dtype, r.act, d["w1"], d["w3"], d["w2"])
    cfg = B.MoEConfig.from_run(r)
    gp = B.alloc_plan(cfg, gpu)
    gp["offsets"].copy_(torch.from_numpy(offsets))
    Xd = torch.zeros((B.max_rows(cfg), r.H), dtype=torch.float32, device=gpu)
    Xd[:R].copy_(torch.from_numpy(d["x"]))
    Yd = torch.full_like(Xd, float("nan"))
    ws = B.alloc_workspace(cfg, gpu)
    B.expert_ffn(cfg, Xd, gp, U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu), Yd, ws)
    torch.cuda.synchronize()
    U.assert_close(U.host(Yd)[:R], Yref, False, f"fp32 expert FFN act={act} H={H} F={F}")

# --------------------------------------------------------------------------- split-bf16 router


def _radius(x, wg, bias, v):
    """Certified radius of an approximate logit (bf16 x, H % 64 == 0): c1 ||x|| ||w_e|| + c2 |v| + c3 |b_e|,
    with c1 = 1.01 ((65 (1 + 2^-7) + 129 2^-7) 2^-23 + (1 + 2^-6) 2^-24) + 4 H 2^-53 (per 64-wide h chunk,
    an fp32 chain of the 64 exact products with the leading bf16 piece and one of the 128 with the two
    trailing pieces, the two chain sums added in fp32), c2 = 2^-24 + 2^-44 and c3 = H 2^-52."""
    H = x.shape[1]
    xf = U.as_f64(x)
    xn = np.sqrt((xf * xf).sum(1))
    wn = np.sqrt((wg.astype(np.float64) ** 2).sum(0))
    c1 = 1.01 * ((65 * (1 + 2.0 ** -7) + 129 * 2.0 ** -7) * 2.0 ** -23 + (1 + 2.0 ** -6) * 2.0 ** -24) + 4 * H * 2.0 ** -53
    b = np.zeros(wg.shape[1]) if bias is None else np.abs(bias.astype(np.float64))
    return c1 * xn[:, None] * wn[None, :] + (2.0 ** -24 + 2.0 ** -44) * np.abs(v) + H * 2.0 ** -52 * b[None, :]


@pytest.mark.parametrize("name", ["2", "3a", "4", "5"])
def test_split_router_error_within_radius(gpu, name):
    """Every logit the split router leaves approximate lies inside its certified radius of the
    binary64-defined logit, by a wide margin; routing stays bit-exact."""
    r = recipes.SMALL[name] if name in recipes.SMALL else recipes.SMALL["3a"]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    _, gplan = _gpu_route(r, gpu, x, wg, bias)
    oplan = _oracle_route(r, x, wg, bias)
    gl = U.host(gplan["logits"]).astype(np.float64)
    ol = oplan["logits"].astype(np.float64)
    rho = _radius(x, wg, bias, ol)
    ratio = float((np.abs(gl - ol) / rho).max())
    print(f"[split] run {r.name}: max |approx - exact| / radius = {ratio:.3e}", flush=True)
    assert ratio < 0.25
    U.assert_plan_equal(gplan, oplan, f"split router {r.name}")


def test_split_router_pieces_exact(gpu):
    """One-hot rows of x make logit (t, e) equal to Wg[t][e]: the three bf16 pieces of every fp32
    weight, with exponents spread over 2^-60 .. 2^20, must add back to it exactly."""
    H, E = 256, 64
    rng = np.random.default_rng(7)
    mant = rng.integers(1 << 23, 1 << 24, size=(H, E)).astype(np.float64)
    ex = rng.integers(-60, 20, size=(H, E))
    sign = np.where(rng.random((H, E)) < 0.5, -1.0, 1.0)
    wg = (sign * mant * np.exp2(ex - 23)).astype(np.float32)
    x = np.zeros((H, H), np.uint16)
    x[np.arange(H), np.arange(H)] = 0x3F80  # bf16 1.0
    r = recipes.SMALL["2"].scaled(name="pieces", T=H, H=H, E=E, k=2, gate_mode=recipes.TOPK_SOFTMAX, bias="none")
    _, gplan = _gpu_route(r, gpu, x, wg, None)
    assert np.array_equal(U.host(gplan["logits"]), wg)
    U.assert_plan_equal(gplan, _oracle_route(r, x, wg, None), "pieces")


def test_split_router_exact_and_near_ties(gpu):
    """Duplicated router columns tie exactly for every token; a copy perturbed in one weight by one
    ulp ties within rounding.  The recomputed logits decide both, lower index first on exact ties."""
    r = recipes.SMALL["5"].scaled(name="coltie", T=777, H=256, E=16, k=4, bias="none")
    x = recipes.gen_x(r)
    wg, _ = recipes.gen_router(r)
    wg[:, 2] *= 3.0
    wg[:, 5] = wg[:, 2]
    wg[:, 9] = wg[:, 2]
    wg[17, 9] = np.nextafter(wg[17, 9], np.float32(np.inf))
    wg[:, 12] = wg[:, 2]
    wg[200, 12] = np.nextafter(wg[200, 12], np.float32(-np.inf))
    oplan = _oracle_route(r, x, wg, None)
    sel = oplan["topk_idx"].reshape(r.T, r.k)
    assert (sel == 2).any() and ((sel == 5).any(1) & (sel == 2).any(1)).any()
    _, gplan = _gpu_route(r, gpu, x, wg, None)
    _check_route(r, gplan, oplan)


# --------------------------------------------------------------------------- router training terms


def _gpu_route_losses(r, gpu, x, wg, bias, aux_mode, aux_coeff, z_coeff):
    import torch

    cfg = B.MoEConfig.from_run(r)
    cfg.aux_mode, cfg.aux_coeff, cfg.z_coeff = aux_mode, aux_coeff, z_coeff
    plan = B.alloc_plan(cfg, gpu, logits=True, losses=True)
    ws = B.alloc_workspace(cfg, gpu)
    B.route(cfg, U.dev(x, gpu), U.dev(wg, gpu), U.dev(bias, gpu), plan, ws)
    torch.cuda.synchronize()
    return plan


@pytest.mark.parametrize("name", SMALL + ["full-2", "full-5"])
@pytest.mark.parametrize("aux_mode", [0, 1])
def test_router_losses(gpu, name, aux_mode):
    """Load-balancing loss and z-loss against the oracle: on the oracle's own routing (1e-5
    relative), and on the GPU's logits and choices (1e-6 relative: only the fp32 exp/log differ)."""
    r = recipes.RUNS[name[5:]] if name.startswith("full-") else recipes.SMALL[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    gplan = _gpu_route_losses(r, gpu, x, wg, bias, aux_mode, 0.01, 0.001)
    got = U.host(gplan["losses"])
    oplan = _oracle_route(r, x, wg, bias)
    U.assert_plan_equal(gplan, oplan, f"losses routing {r.name}")
    ref = oracle.router_losses(oplan["logits"], oplan["topk_idx"], oplan["demand"], r.k, aux_mode, 0.01, 0.001)
    own = oracle.router_losses(U.host(gplan["logits"]), U.host(gplan["topk_idx"]), U.host(gplan["demand"]), r.k,
                               aux_mode, 0.01, 0.001)
    print(f"[losses] run {r.name} mode {aux_mode}: gpu {got[0]:.9g} {got[1]:.9g}  oracle {ref[0]:.9g} {ref[1]:.9g}",
          flush=True)
    for i in range(2):
        assert abs(got[i] - ref[i]) <= 1e-5 * abs(ref[i]), (i, got[i], ref[i])
        assert abs(got[i] - own[i]) <= 1e-6 * abs(own[i]), (i, got[i], own[i])


def test_router_losses_uniform_and_empty(gpu):
    """x = 0 and no bias: every probability is 1/E, so the load-balancing loss is the
    coefficient itself, and the z-loss is coeff * (ln E)^2; T = 0 gives zeros."""
    import math

    r = recipes.SMALL["3a"].scaled(name="lossuni", T=300, bias="none")
    x = np.zeros_like(recipes.gen_x(r))
    wg, _ = recipes.gen_router(r)
    for mode in (0, 1):
        got = U.host(_gpu_route_losses(r, gpu, x, wg, None, mode, 0.01, 0.001)["losses"])
        zref = 0.001 * math.log(r.E) ** 2
        assert abs(got[0] - 0.01) <= 1e-8 and abs(got[1] - zref) <= 1e-6 * zref, (got, zref)
    r0 = r.scaled(name="loss-T0", T=0)
    got = U.host(_gpu_route_losses(r0, gpu, x[:0], wg, None, 0, 0.01, 0.001)["losses"])
    assert (got == 0).all()


# --------------------------------------------------------------------------- routing variants


def _gpu_route_cfg(cfg, gpu, x, wg, bias):
    import torch

    plan = B.alloc_plan(cfg, gpu, logits=True)
    ws = B.alloc_workspace(cfg, gpu)
    B.route(cfg, U.dev(x, gpu), U.dev(wg, gpu), U.dev(bias, gpu), plan, ws)
    torch.cuda.synchronize()
    return plan


@pytest.mark.parametrize("name", ["1", "2", "3a", "4", "5"])
@pytest.mark.parametrize("gate_mode", [0, 1, 2])
def test_sigmoid_scoring_route(gpu, name, gate_mode):
    """Sigmoid scores: same choices as softmax, gates are the scores (or renormalised)."""
    r = recipes.SMALL[name].scaled(name=f"sig-{name}-{gate_mode}", gate_mode=gate_mode)
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    cfg = B.MoEConfig.from_run(r)
    cfg.score_fn = 1
    gplan = _gpu_route_cfg(cfg, gpu, x, wg, bias)
    oplan = oracle.route(x, r.dtype, wg, bias, r.k, gate_mode, _cap(r), oracle.SIGMOID)
    _check_route(r, gplan, oplan)


def test_sigmoid_scoring_forward(gpu):
    import torch

    r = recipes.SMALL["5"].scaled(name="sig-fwd")
    d = recipes.gen_all(r)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, _cap(r), score_fn=oracle.SIGMOID)
    cfg = B.MoEConfig.from_run(r)
    cfg.score_fn = 1
    gp = {"x": U.dev(d["x"], gpu), "wg": U.dev(d["wg"], gpu), "bias": U.dev(d["bias"], gpu),
          "w1": U.dev(d["w1"], gpu), "w3": U.dev(d["w3"], gpu), "w2": U.dev(d["w2"], gpu)}
    plan = B.alloc_plan(cfg, gpu, logits=True)
    rmax = max(B.max_rows(cfg), 1)
    X = torch.empty((rmax, r.H), dtype=torch.bfloat16, device=gpu)
    Y = torch.empty_like(X)
    y = torch.empty((r.T, r.H), dtype=torch.bfloat16, device=gpu)
    ws = B.alloc_workspace(cfg, gpu)
    B.forward(cfg, gp["x"], gp["wg"], gp["bias"], gp["w1"], gp["w3"], gp["w2"], None, y, plan, X, Y, ws)
    torch.cuda.synchronize()
    _check_route(r, plan, oplan)
    U.assert_close(U.host(y), yref, True, "sigmoid forward")


def _check_exact_route(r, gplan, oplan, what):
    """Exact path (every logit and gate computed as defined): logits and gates bit-identical
    to the oracle's, the plan bit-exact."""
    gl = U.host(gplan["logits"])
    assert np.array_equal(gl.view(np.uint32), oplan["logits"].view(np.uint32)), \
        f"{what}: {int((gl != oplan['logits']).sum())} logits not bit-identical"
    gg = U.host(gplan["topk_gate"]).reshape(oplan["topk_gate"].shape)
    assert np.array_equal(gg.view(np.uint32), oplan["topk_gate"].view(np.uint32)), \
        f"{what}: {int((gg != oplan['topk_gate']).sum())} gates not bit-identical"
    U.assert_plan_equal(gplan, oplan, what)
    print(f"[exact] {what}: logits, gates and plan bit-identical; R={oplan['R']} "
          f"dropped={int(oplan['n_dropped'][0])}", flush=True)


@pytest.mark.parametrize("name", ["1", "2", "3a", "3b", "3c", "full-3a", "full-3c", "full-2"])
def test_probs_drop_policy(gpu, name):
    """"probs" policy: the gate values decide which assignments are kept, so the plan must
    equal the oracle's bit for bit, with gates bit-identical."""
    r = recipes.RUNS[name[5:]] if name.startswith("full-") else recipes.SMALL[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    cfg = B.MoEConfig.from_run(r)
    cfg.drop_policy = 1
    gplan = _gpu_route_cfg(cfg, gpu, x, wg, bias)
    oplan = oracle.route(x, r.dtype, wg, bias, r.k, r.gate_mode, _cap(r), drop_policy=oracle.DROP_PROBS)
    assert oplan["n_dropped"][0] > 0
    _check_exact_route(r, gplan, oplan, f"probs run {r.name}")


def test_probs_drop_policy_ties_and_dropless(gpu):
    """Repeated token rows give equal gates across tokens, so the position tie-break decides;
    dropless, probs equals position."""
    r = recipes.SMALL["3a"].scaled(name="probs-ties", cf=0.5)
    x = recipes.gen_x(r)
    x[:] = x[np.arange(r.T) % 37]
    wg, bias = recipes.gen_router(r)
    cfg = B.MoEConfig.from_run(r)
    cfg.drop_policy = 1
    gplan = _gpu_route_cfg(cfg, gpu, x, wg, bias)
    oplan = oracle.route(x, r.dtype, wg, bias, r.k, r.gate_mode, _cap(r), drop_policy=oracle.DROP_PROBS)
    _check_exact_route(r, gplan, oplan, "probs ties")
    rd = r.scaled(name="probs-dropless", dropless=1)
    cfg = B.MoEConfig.from_run(rd)
    cfg.drop_policy = 1
    gplan = _gpu_route_cfg(cfg, gpu, x, wg, bias)
    U.assert_plan_equal(gplan, _oracle_route(rd, x, wg, bias), "probs dropless")


def _second_u(r, seed):
    """Seeded uniforms in [0, 1) for GShard's second choice, as drawn (no adjustment)."""
    return np.random.default_rng(seed).random(r.T).astype(np.float32)


def _gpu_route_gshard(r, gpu, x, wg, bias, u):
    import torch

    cfg = B.MoEConfig.from_run(r)
    cfg.second_policy = 1
    plan = B.alloc_plan(cfg, gpu, logits=True)
    plan["second_u"] = U.dev(u, gpu)
    ws = B.alloc_workspace(cfg, gpu)
    B.route(cfg, U.dev(x, gpu), U.dev(wg, gpu), U.dev(bias, gpu), plan, ws)
    torch.cuda.synchronize()
    return plan


_GSHARD = {
    "4": lambda: recipes.SMALL["4"],
    "3a-k2": lambda: recipes.SMALL["3a"].scaled(name="3a-k2", k=2),
    "2-k2": lambda: recipes.SMALL["2"].scaled(name="2-k2", k=2, gate_mode=recipes.SOFTMAX_TOPK_RENORM),
    "1-k2": lambda: recipes.RUNS["1"].scaled(name="1-k2", k=2, T=500),
    # more than 64 experts (one token's experts span several lanes' registers)
    "E96-k2": lambda: recipes.SMALL["5"].scaled(name="E96-k2", E=96, k=2, T=1000),
    # few experts, H a multiple of 256 and fewer than 16384 tokens (32-token tiles of the split router)
    "E12-k2-T4000": lambda: recipes.SMALL["3a"].scaled(name="E12-k2-T4000", k=2, T=4000, H=512),
    # full-size Mixtral-like routing with capacity
    "full-4-cap": lambda: recipes.RUNS["4"].scaled(name="full-4-cap", dropless=0, cf=1.0),
}


@pytest.mark.parametrize("name", list(_GSHARD))
def test_gshard_random_second_choice(gpu, name):
    r = _GSHARD[name]()
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    u = _second_u(r, 21)
    plan = _gpu_route_gshard(r, gpu, x, wg, bias, u)
    oplan = oracle.route(x, r.dtype, wg, bias, r.k, r.gate_mode, _cap(r), second_u=u)
    absent = int((oplan["dst_row"][:, 1] < 0).sum())
    print(f"[gshard] run {r.name}: {absent} of {r.T} second choices not taken", flush=True)
    assert 0 < absent < r.T
    _check_exact_route(r, plan, oplan, f"gshard run {r.name}")


@pytest.mark.parametrize("name", ["3a-k2", "2-k2", "E96-k2"])
def test_gshard_uniforms_on_the_threshold(gpu, name):
    """Uniforms placed on GShard's threshold 2 g2 / (g1 + g2) computed from the oracle's gates
    (the fp32 value nearest to it, and its two neighbours): the decision then rests on the
    last bits of the gates, and the GPU must take the oracle's on every token."""
    r = _GSHARD[name]()
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    og = oracle.route(x, r.dtype, wg, bias, r.k, r.gate_mode, _cap(r))["topk_gate"].astype(np.float64)
    thr = 2.0 * og[:, 1] / (og[:, 0] + og[:, 1])
    u0 = thr.astype(np.float32)
    shift = np.arange(r.T) % 3  # 0: nearest, 1: one ulp below, 2: one ulp above
    u = np.where(shift == 1, np.nextafter(u0, np.float32(0)), np.where(shift == 2, np.nextafter(u0, np.float32(1)), u0))
    u = np.minimum(u, np.float32(np.nextafter(np.float32(1), np.float32(0)))).astype(np.float32)
    plan = _gpu_route_gshard(r, gpu, x, wg, bias, u)
    oplan = oracle.route(x, r.dtype, wg, bias, r.k, r.gate_mode, _cap(r), second_u=u)
    absent = (oplan["dst_row"][:, 1] < 0)
    print(f"[gshard-threshold] run {r.name}: {int(absent.sum())} of {r.T} second choices not taken", flush=True)
    assert 0 < absent.sum() < r.T
    _check_exact_route(r, plan, oplan, f"gshard threshold run {r.name}")


def test_gshard_random_second_choice_forward(gpu):
    import torch

    r = recipes.SMALL["4"].scaled(name="gshard-fwd", dropless=0, cf=1.0)
    d = recipes.gen_all(r)
    u = _second_u(r, 5)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, _cap(r), second_u=u)
    cfg = B.MoEConfig.from_run(r)
    cfg.second_policy = 1
    plan = B.alloc_plan(cfg, gpu, logits=True)
    plan["second_u"] = U.dev(u, gpu)
    rmax = max(B.max_rows(cfg), 1)
    X = torch.empty((rmax, r.H), dtype=torch.bfloat16, device=gpu)
    Y = torch.empty_like(X)
    y = torch.empty((r.T, r.H), dtype=torch.bfloat16, device=gpu)
    ws = B.alloc_workspace(cfg, gpu)
    B.forward(cfg, U.dev(d["x"], gpu), U.dev(d["wg"], gpu), U.dev(d["bias"], gpu), U.dev(d["w1"], gpu),
              U.dev(d["w3"], gpu), U.dev(d["w2"], gpu), None, y, plan, X, Y, ws)
    torch.cuda.synchronize()
    _check_exact_route(r, plan, oplan, "gshard forward")
    U.assert_close(U.host(y), yref, True, "gshard forward")


# ---- shared expert: a dense FFN on every token, added to the routed output
def _shared_weights(r, Fs):
    s1 = recipes.gen_shared_weight(r, "s1", Fs)
    s3 = recipes.gen_shared_weight(r, "s3", Fs) if r.act == recipes.SWIGLU else None
    s2 = recipes.gen_shared_weight(r, "s2", Fs)
    return s1, s3, s2


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("width", ["F", "ragged"])
def test_shared_expert(gpu, name, width):
    import torch

    r = recipes.SMALL[name]
    Fs = r.F if width == "F" else r.F + 40  # ragged: not a whole number of 64-wide k steps
    x = recipes.gen_x(r)
    sw = _shared_weights(r, Fs)
    cfg = B.MoEConfig.from_run(r)
    cfg.shared_F = Fs
    tdt = torch.bfloat16 if r.dtype == recipes.BF16 else torch.float32
    Ys = torch.empty((r.T, r.H), dtype=tdt, device=gpu)
    B.shared_expert(cfg, U.dev(x, gpu), *(U.dev(a, gpu) for a in sw), Ys, B.alloc_workspace(cfg, gpu))
    torch.cuda.synchronize()
    ref = oracle.shared_expert(x, r.dtype, r.act, *sw)
    U.assert_close(U.host(Ys), ref, r.dtype == recipes.BF16, f"shared expert run {r.name} Fs={Fs}")


def _gpu_forward_shared(r, gpu, d, sw, Fs, weights=None, residual=False):
    import torch

    cfg = B.MoEConfig.from_run(r)
    cfg.shared_F = Fs
    tdt = torch.bfloat16 if r.dtype == recipes.BF16 else torch.float32
    rmax = B.max_rows(cfg)
    xd = U.dev(d["x"], gpu)
    if weights is None:
        weights = (U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu))
    plan = B.alloc_plan(cfg, gpu, logits=True)
    X = torch.empty((max(rmax, 1), r.H), dtype=tdt, device=gpu)
    Y = torch.empty_like(X)
    y = torch.empty((r.T, r.H), dtype=tdt, device=gpu)
    B.forward_shared(cfg, xd, U.dev(d["wg"], gpu), U.dev(d["bias"], gpu), *weights, *(U.dev(a, gpu) for a in sw),
                     xd if residual else None, y, plan, X, Y, B.alloc_workspace(cfg, gpu))
    torch.cuda.synchronize()
    return plan, y


@pytest.mark.parametrize("name", SMALL)
def test_forward_shared_small(gpu, name):
    r = recipes.SMALL[name]
    d = recipes.gen_all(r)
    Fs = r.F
    sw = _shared_weights(r, Fs)
    yref, oplan, _, _ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k,
                                       r.gate_mode, r.act, _cap(r), shared=sw)
    gplan, y = _gpu_forward_shared(r, gpu, d, sw, Fs)
    _check_route(r, gplan, oplan)
    U.assert_close(U.host(y), yref, r.dtype == recipes.BF16, f"forward+shared run {r.name}")


@pytest.mark.parametrize("name", ["2", "5"])
def test_forward_shared_full_size_sampled(gpu, name):
    """Full workload with a shared expert of the routed experts' width (one shared expert
    next to the routed ones, as in the DeepSeek-R1 shape); routing on every token,
    outputs on a sample of tokens."""
    r = recipes.RUNS[name]
    x = recipes.gen_x(r)
    wg, bias = recipes.gen_router(r)
    oplan = _oracle_route(r, x, wg, bias)
    rng = np.random.default_rng(int(r.run_id) + 7)
    toks = set(rng.choice(r.T, size=96, replace=False).tolist()) | {0, r.T - 1}
    dropped = np.nonzero((oplan["dst_row"] < 0).all(1))[0]
    toks |= set(dropped[:4].tolist())
    toks = np.array(sorted(toks), np.int64)
    need = sorted(set(oplan["topk_idx"][toks].ravel().tolist()))
    w1, k1 = U.upload_expert_weight(r, "w1", gpu, keep=need)
    w3, k3 = U.upload_expert_weight(r, "w3", gpu, keep=need) if r.act == recipes.SWIGLU else (None, {})
    w2, k2 = U.upload_expert_weight(r, "w2", gpu, keep=need)
    sw = _shared_weights(r, r.F)
    gplan, y = _gpu_forward_shared(r, gpu, dict(x=x, wg=wg, bias=bias), sw, r.F, weights=(w1, w3, w2))
    _check_route(r, gplan, oplan)
    remap = {e: i for i, e in enumerate(need)}
    sub = {n: oplan[n][toks] for n in ("topk_gate", "dst_row")}
    sub["topk_idx"] = np.vectorize(remap.get)(oplan["topk_idx"][toks]).astype(np.int32)
    cw1 = np.stack([k1[e] for e in need])
    cw3 = np.stack([k3[e] for e in need]) if w3 is not None else None
    cw2 = np.stack([k2[e] for e in need])
    yref = oracle.token_outputs(np.arange(len(toks)), x[toks], r.dtype, r.act, sub, cw1, cw3, cw2)
    yref = yref + oracle.shared_expert(x, r.dtype, r.act, *sw, tokens=toks)
    U.assert_close(U.host(y)[toks], yref, r.dtype == recipes.BF16, f"forward+shared full-size run {r.name} sample")


def test_forward_graph_replay(gpu):
    """The whole layer captured in a HIP graph: every replay (with eager work and
    synchronisations in between) gives the eager result bit for bit."""
    import torch

    r = recipes.SMALL["2"]
    d = recipes.gen_all(r)
    cfg = B.MoEConfig.from_run(r)
    tdt = torch.bfloat16
    xd = U.dev(d["x"], gpu)
    wgt = (U.dev(d["wg"], gpu), U.dev(d["bias"], gpu), U.dev(d["w1"], gpu), None, U.dev(d["w2"], gpu))
    plan = B.alloc_plan(cfg, gpu)
    rmax = B.max_rows(cfg)
    X = torch.empty((rmax, r.H), dtype=tdt, device=gpu)
    Y = torch.empty_like(X)
    y = torch.empty((r.T, r.H), dtype=tdt, device=gpu)
    ws = B.alloc_workspace(cfg, gpu)
    s = torch.cuda.Stream()

    def step():
        B.forward(cfg, xd, *wgt, xd, y, plan, X, Y, ws, stream=s)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    dst_eager = plan["dst_row"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        plan["dst_row"].fill_(-7)
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
        assert torch.equal(plan["dst_row"], dst_eager), f"replay {i} plan"
        with torch.cuda.stream(s):  # eager work between replays
            step()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
    yref, *_ = oracle.forward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.k, r.gate_mode,
                              r.act, _cap(r), residual=d["x"])
    U.assert_close(U.host(y_eager), yref, True, "graph replay forward")
