"""GPU parity of moe_backward with the backward oracle (oracle/backward.py).

For each workload's reduced shape (the routing structure of every workload: dtype,
activation, gate mode, capacity and drops) the GPU routes (bit-exact with the
oracle, asserted here again), then moe_backward takes dy and the plan; the oracle
takes the same inputs and its own plan.  Every gradient is compared element by
element in relative L2 and max-abs over the tensor's norm.

Tolerances.  Generic path (fp32 runs, shapes off the 64-grid, unaligned x):
every intermediate is fp32 (inputs are the exact bf16 / fp32 values), each
product an fp32 sum of at most a few thousand terms in a fixed order (error
~ sqrt(K) 2^-24 relative for random signs), the transcendental functions within
a few ulp: near 1e-6 along the chain; bound 1e-4.  Matrix-core path (bf16, H
and F multiples of 64): the intermediates u, v, g z, dzr, du, dv and dX are
stored in bf16, each rounding an rms 2^-9 / sqrt(3) ~ 1.1e-3 relative; a
gradient's chain crosses at most four of them (dx: u, dzr, du, dX), about 2.3e-3
in quadrature; bound 1e-2.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as OB
from tests import gpu_util as U
from top_routing_expert_router_amd import binding as B
from top_routing_expert_router_amd.synth import recipes

pytestmark = pytest.mark.gpu

GRAD_RELL2 = 1e-4  # generic path
GRAD_RELL2_MC = 1e-2  # matrix-core path (bf16 intermediates)


def _cap(r):
    return None if r.dropless else oracle.capacity(r.T, r.k, r.E, r.cf, r.min_capacity)


def _inputs(r):
    d = recipes.gen_all(r)
    d["dy"] = recipes.gen_dy(r)
    return d


def _fast(r):
    return r.dtype == recipes.BF16 and r.H % 64 == 0 and r.F % 64 == 0


def _unaligned(a, gpu):
    """A device copy of `a` that starts 2 bytes past a 16-byte boundary (the backward
    then takes its generic path)."""
    import torch

    t = U.dev(a, gpu)
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=gpu)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def _gpu_backward(r, gpu, d, losses=None, score_fn=0, dg=True, generic=False):
    import torch

    cfg = B.MoEConfig.from_run(r)
    cfg.score_fn = score_fn
    if losses is not None:
        cfg.aux_mode, cfg.aux_coeff, cfg.z_coeff = losses
    plan = B.alloc_plan(cfg, gpu, logits=True, losses=losses is not None)
    ws = B.alloc_workspace(cfg, gpu)
    x = _unaligned(d["x"], gpu) if generic else U.dev(d["x"], gpu)
    wg = U.dev(d["wg"], gpu)
    B.route(cfg, x, wg, U.dev(d["bias"], gpu), plan, ws)
    grads = B.alloc_grads(cfg, gpu, bias=True, dg=dg)
    bws = torch.empty(max(B.backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=gpu)
    B.backward(cfg, x, wg, U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu), plan,
               U.dev(d["dy"], gpu), grads, bws)
    torch.cuda.synchronize()
    return plan, {n: t.cpu().numpy().astype(np.float64) for n, t in grads.items()}


def _oracle_backward(r, d, losses=None, score_fn=0):
    plan = oracle.route(d["x"], r.dtype, d["wg"], d["bias"], r.k, r.gate_mode, _cap(r), score_fn=score_fn)
    X = oracle.dispatch(d["x"], r.dtype, plan)
    Y = oracle.expert_ffn(X, plan["offsets"], r.dtype, r.act, d["w1"], d["w3"], d["w2"])
    am, ac, zc = losses if losses is not None else (0, 0.0, 0.0)
    g = OB.layer_backward(d["x"], r.dtype, d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], r.act, r.gate_mode, plan,
                          X, Y, d["dy"], score_fn, am, ac, zc)
    return plan, g


NAMES = dict(dx="dx", dWg="dWg", dbias="dbias", dW1="dW1", dW3="dW3", dW2="dW2", dg="dg")


def _compare(what, got, ref, tol=GRAD_RELL2):
    for n, on in NAMES.items():
        if n not in got or ref.get(on) is None:
            continue
        g, o = got[n].reshape(ref[on].shape), ref[on]
        d = g - o
        nref = float(np.linalg.norm(o))
        rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
        mx = float(np.abs(d).max()) / (float(np.abs(o).max()) + 1e-30) if d.size else 0.0
        print(f"[backward] {what} {n}: rel-L2 {rel:.2e}, max-abs/max {mx:.2e}", flush=True)
        assert rel <= tol, (what, n, rel)
        assert mx <= 10 * tol, (what, n, mx)


@pytest.mark.parametrize("name", ["2", "3a", "4", "5"])
def test_backward_with_kept_preactivations(gpu, name):
    """moe_forward_save keeps the first expert GEMM's pre-activations (u, and v for
    SwiGLU) of every kept row.  Its layer output equals moe_forward's bit for bit; the
    kept values are the oracle's X W1_e^T (X W3_e^T) within their bf16 rounding; and
    moe_backward given them returns, bit for bit, the gradients it computes when it
    recomputes them (both come from the same k-ordered products)."""
    import torch

    r = recipes.SMALL[name]
    d = _inputs(r)
    cfg = B.MoEConfig.from_run(r)
    R_max = B.max_rows(cfg)
    x, wg, bias = U.dev(d["x"], gpu), U.dev(d["wg"], gpu), U.dev(d["bias"], gpu)
    w1, w3, w2 = U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu)
    plan = B.alloc_plan(cfg, gpu, logits=True)
    X = torch.empty((max(R_max, 1), r.H), dtype=torch.bfloat16, device=gpu)
    Y = torch.empty_like(X)
    y0 = torch.empty((r.T, r.H), dtype=torch.bfloat16, device=gpu)
    y1 = torch.empty_like(y0)
    ws = B.alloc_workspace(cfg, gpu)
    B.forward(cfg, x, wg, bias, w1, w3, w2, x, y0, plan, X, Y, ws)
    m1 = 2 if r.act == recipes.SWIGLU else 1
    assert B.saved_act_bytes(cfg) == m1 * R_max * r.F * 2
    act = torch.full((m1, R_max, r.F), float("nan"), dtype=torch.bfloat16, device=gpu)
    B.forward_save(cfg, x, wg, bias, w1, w3, w2, x, y1, plan, X, Y, act, ws)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), "forward_save changed y"

    oplan = oracle.route(d["x"], r.dtype, d["wg"], d["bias"], r.k, r.gate_mode, _cap(r))
    U.assert_plan_equal(plan, oplan, f"kept {name}")
    R, off = oplan["R"], oplan["offsets"]
    Xo = U.as_f64(oracle.dispatch(d["x"], r.dtype, oplan))
    kept = U.as_f64(U.host(act))
    for j, wn in enumerate(["w1", "w3"][:m1]):
        W = U.as_f64(d[wn])
        ref = np.zeros((R, r.F))
        for e in range(r.E):
            ref[off[e]:off[e + 1]] = Xo[off[e]:off[e + 1]] @ W[e].T
        U.assert_close(kept[j, :R], ref, True, f"kept {name} {'uv'[j]}")

    dy = U.dev(d["dy"], gpu)
    bws = torch.empty(max(B.backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=gpu)
    outs = []
    for a in (None, act):
        grads = B.alloc_grads(cfg, gpu, bias=True, dg=True)
        B.backward(cfg, x, wg, w1, w3, w2, plan, dy, grads, bws, act=a)
        torch.cuda.synchronize()
        outs.append({n: t.cpu() for n, t in grads.items()})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), (name, n)
    print(f"[backward] kept pre-activations {name}: gradients equal to the recomputed path", flush=True)


@pytest.mark.parametrize("name", ["1", "2", "3a", "3b", "3c", "4", "5"])
def test_backward_matches_oracle(gpu, name):
    r = recipes.SMALL[name]
    d = _inputs(r)
    gplan, got = _gpu_backward(r, gpu, d)
    oplan, ref = _oracle_backward(r, d)
    U.assert_plan_equal(gplan, oplan, f"backward run {name}")
    if not r.dropless and name != "1":
        assert int(oplan["n_dropped"][0]) > 0
    _compare(f"run {name}", got, ref, GRAD_RELL2_MC if _fast(r) else GRAD_RELL2)


@pytest.mark.parametrize("name", ["2", "4", "5"])
def test_backward_generic_path_bf16(gpu, name):
    """The same bf16 workloads through the generic path (x not 16-byte aligned): fp32
    intermediates, the tight bound."""
    r = recipes.SMALL[name]
    d = _inputs(r)
    _, got = _gpu_backward(r, gpu, d, generic=True)
    _, ref = _oracle_backward(r, d)
    _compare(f"run {name} generic", got, ref, GRAD_RELL2)


@pytest.mark.parametrize("name", ["2", "5"])
def test_training_step_graph_replay(gpu, name):
    """A training step of the layer (moe_forward_save, then moe_backward given the kept
    pre-activations) captured in a HIP graph: every replay, with eager steps and
    synchronisations in between, gives the eager y and gradients bit for bit."""
    import torch

    r = recipes.SMALL[name]
    d = _inputs(r)
    cfg = B.MoEConfig.from_run(r)
    R_max = max(B.max_rows(cfg), 1)
    x, wg, bias, dy = (U.dev(d[n], gpu) for n in ("x", "wg", "bias", "dy"))
    w1, w3, w2 = U.dev(d["w1"], gpu), U.dev(d["w3"], gpu), U.dev(d["w2"], gpu)
    plan = B.alloc_plan(cfg, gpu, logits=True)
    X = torch.empty((R_max, r.H), dtype=torch.bfloat16, device=gpu)
    Y = torch.empty_like(X)
    y = torch.empty((r.T, r.H), dtype=torch.bfloat16, device=gpu)
    ws = B.alloc_workspace(cfg, gpu)
    act = torch.empty(B.saved_act_bytes(cfg), dtype=torch.uint8, device=gpu)
    grads = B.alloc_grads(cfg, gpu, bias=True, dg=True)
    bws = torch.empty(max(B.backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=gpu)
    s = torch.cuda.Stream()

    def step():
        B.forward_save(cfg, x, wg, bias, w1, w3, w2, x, y, plan, X, Y, act, ws, stream=s)
        B.backward(cfg, x, wg, w1, w3, w2, plan, dy, grads, bws, stream=s, act=act)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    g_eager = {n: t.clone() for n, t in grads.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        y.zero_()
        for t in grads.values():
            t.fill_(float("nan"))
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} y"
        for n, t in grads.items():
            assert torch.equal(t, g_eager[n]), f"replay {i} {n}"
        with torch.cuda.stream(s):  # eager work between replays
            step()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
    # and the eager step is the oracle's gradient within the matrix-core bound
    _, ref = _oracle_backward(r, d)
    _compare(f"graph run {name}", {n: t.cpu().numpy().astype(np.float64) for n, t in g_eager.items()}, ref,
             GRAD_RELL2_MC)


def test_generic_path_ignores_kept_preactivations(gpu):
    """Off the matrix-core path (here: x not 16-byte aligned) moe_backward recomputes its
    fp32 intermediates whether or not kept bf16 pre-activations are passed: the same
    gradients bit for bit."""
    import torch

    r = recipes.SMALL["5"]
    d = _inputs(r)
    cfg = B.MoEConfig.from_run(r)
    plan = B.alloc_plan(cfg, gpu, logits=True)
    ws = B.alloc_workspace(cfg, gpu)
    x = _unaligned(d["x"], gpu)
    wg, w1, w3, w2 = (U.dev(d[n], gpu) for n in ("wg", "w1", "w3", "w2"))
    B.route(cfg, x, wg, U.dev(d["bias"], gpu), plan, ws)
    act = torch.zeros(B.saved_act_bytes(cfg), dtype=torch.uint8, device=gpu)  # deliberately not the forward's
    bws = torch.empty(max(B.backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=gpu)
    outs = []
    for a in (None, act):
        grads = B.alloc_grads(cfg, gpu, bias=True, dg=True)
        B.backward(cfg, x, wg, w1, w3, w2, plan, U.dev(d["dy"], gpu), grads, bws, act=a)
        torch.cuda.synchronize()
        outs.append({n: t.cpu() for n, t in grads.items()})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


@pytest.mark.parametrize("name", ["3a", "5"])
def test_backward_off_grid_shapes(gpu, name):
    """H or F off the 64-grid (generic path) with the routing structure of the run."""
    r = recipes.SMALL[name].scaled(name=f"{name}-offgrid", H=200, F=136)
    d = _inputs(r)
    _, got = _gpu_backward(r, gpu, d)
    _, ref = _oracle_backward(r, d)
    _compare(f"run {r.name}", got, ref, GRAD_RELL2)


@pytest.mark.parametrize("name,losses", [("2", (0, 0.01, 0.001)), ("5", (0, 0.02, 0.001)), ("3a", (1, 0.05, 0.0))])
def test_backward_with_training_terms(gpu, name, losses):
    r = recipes.SMALL[name]
    d = _inputs(r)
    _, got = _gpu_backward(r, gpu, d, losses=losses)
    _, ref = _oracle_backward(r, d, losses=losses)
    _compare(f"run {name} losses {losses}", got, ref, GRAD_RELL2_MC if _fast(r) else GRAD_RELL2)


@pytest.mark.parametrize("name", ["3a", "5"])
def test_backward_sigmoid_scores(gpu, name):
    r = recipes.SMALL[name]
    d = _inputs(r)
    _, got = _gpu_backward(r, gpu, d, losses=(0, 0.05, 0.0), score_fn=1)
    _, ref = _oracle_backward(r, d, losses=(0, 0.05, 0.0), score_fn=1)
    _compare(f"run {name} sigmoid", got, ref, GRAD_RELL2_MC if _fast(r) else GRAD_RELL2)


def test_backward_is_deterministic(gpu):
    r = recipes.SMALL["5"]
    d = _inputs(r)
    _, a = _gpu_backward(r, gpu, d)
    _, b = _gpu_backward(r, gpu, d)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_backward_empty_batch_and_refusals(gpu):
    import torch

    r = recipes.SMALL["2"].scaled(name="empty", T=0)
    cfg = B.MoEConfig.from_run(r)
    plan = B.alloc_plan(cfg, gpu, logits=True)
    grads = B.alloc_grads(cfg, gpu)
    bws = torch.empty(max(B.backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=gpu)
    d = recipes.gen_all(recipes.SMALL["2"])
    for t in grads.values():
        t.fill_(7.0)
    B.backward(cfg, None, U.dev(d["wg"], gpu), U.dev(d["w1"], gpu), None, U.dev(d["w2"], gpu), plan, None, grads, bws)
    torch.cuda.synchronize()
    for n, t in grads.items():  # no tokens: every weight gradient is zero
        assert t.numel() == 0 or bool((t == 0).all()), n
    # a too-small workspace is refused
    r2 = recipes.SMALL["2"]
    cfg2 = B.MoEConfig.from_run(r2)
    with pytest.raises(B.MoEError):
        B.backward(cfg2, U.dev(d["x"], gpu), U.dev(d["wg"], gpu), U.dev(d["w1"], gpu), None, U.dev(d["w2"], gpu),
                   B.alloc_plan(cfg2, gpu, logits=True), U.dev(recipes.gen_dy(r2), gpu), B.alloc_grads(cfg2, gpu),
                   torch.empty(16, dtype=torch.uint8, device=gpu))


@pytest.mark.parametrize("name", ["2", "4", "5"])
def test_backward_full_size_sampled(gpu, name):
    """Full-size runs: the weight gradients of the largest, a median and the smallest
    non-empty expert (the oracle on exactly those experts' rows) and of an empty expert
    (exactly zero), and dx, dg of 64 sampled tokens (expert and router paths: the oracle
    takes each token's choices one by one).  The router weight and bias gradients need
    every token's expert outputs and are compared at the reduced sizes above."""
    import torch

    r = recipes.RUNS[name]
    cfg = B.MoEConfig.from_run(r)
    x_h = recipes.gen_x(r)
    wg_h, bias_h = recipes.gen_router(r)
    dy_h = recipes.gen_dy(r)
    x, wg, dy = U.dev(x_h, gpu), U.dev(wg_h, gpu), U.dev(dy_h, gpu)
    names = ("w1", "w3", "w2") if r.act == recipes.SWIGLU else ("w1", "w2")
    w = {n: U.upload_expert_weight(r, n, gpu)[0] for n in names}
    plan = B.alloc_plan(cfg, gpu, logits=True)
    B.route(cfg, x, wg, U.dev(bias_h, gpu), plan, B.alloc_workspace(cfg, gpu))
    grads = B.alloc_grads(cfg, gpu, dg=True)
    bws = torch.empty(B.backward_workspace_bytes(cfg), dtype=torch.uint8, device=gpu)
    B.backward(cfg, x, wg, w["w1"], w.get("w3"), w["w2"], plan, dy, grads, bws)
    torch.cuda.synchronize()
    oplan = oracle.route(x_h, r.dtype, wg_h, bias_h, r.k, r.gate_mode, _cap(r))
    U.assert_plan_equal(plan, oplan, f"full run {name}")
    kept, off, rt = oplan["kept"], oplan["offsets"], oplan["row_token"]
    dst, idx, gate = oplan["dst_row"], oplan["topk_idx"], oplan["topk_gate"]
    order = np.argsort(kept, kind="stable")
    nonempty = order[kept[order] > 0]
    experts = sorted({int(nonempty[-1]), int(nonempty[len(nonempty) // 2]), int(nonempty[0])})
    empty = [int(e) for e in order[kept[order] == 0][:1]]
    # row -> (token, choice)
    choice_of_row = np.full(oplan["R"], -1, np.int64)
    kt, kr = np.nonzero(dst >= 0)
    choice_of_row[dst[kt, kr]] = kr
    dyf = U.as_f64(dy_h)
    for e in experts:
        rows = np.arange(off[e], off[e + 1])
        toks = rt[rows]
        wts = {n: recipes.gen_expert_weight(r, n, experts=[e])[e][None] for n in names}
        Xe = x_h[toks]
        dYe = gate[toks, choice_of_row[rows]][:, None].astype(np.float64) * dyf[toks]
        _, dW1, dW3, dW2 = OB.expert_backward(Xe, np.array([0, rows.size]), r.act, wts["w1"], wts.get("w3"), wts["w2"],
                                              dYe)
        got = {"dW1": grads["dW1"][e].cpu().numpy().astype(np.float64)[None],
               "dW2": grads["dW2"][e].cpu().numpy().astype(np.float64)[None]}
        ref = {"dW1": dW1, "dW2": dW2}
        if r.act == recipes.SWIGLU:
            got["dW3"] = grads["dW3"][e].cpu().numpy().astype(np.float64)[None]
            ref["dW3"] = dW3
        _compare(f"full run {name} expert {e} ({rows.size} rows)", got, ref, GRAD_RELL2_MC)
    for e in empty:
        for n in ("dW1", "dW3", "dW2"):
            if n in grads:
                assert bool((grads[n][e] == 0).all()), (n, e)
    # sampled tokens: dg from the token's own expert outputs, dx from its kept rows
    # (expert path) plus dl Wg^T (router path, dl from the gate Jacobian of its dg)
    rng = np.random.default_rng(int(name.encode()[0]))
    toks = np.sort(rng.choice(r.T, size=64, replace=False))
    cache = {}

    def wt(e):  # the expert's weights, as generated and in binary64 (converted once)
        if e not in cache:
            raw = {n: recipes.gen_expert_weight(r, n, experts=[e])[e][None] for n in names}
            cache[e] = (raw, {n: OB._f64(v) for n, v in raw.items()})
        return cache[e]

    dg_ref = np.zeros((r.T, r.k))
    dx_ref = np.zeros((toks.size, r.H))
    for i, t in enumerate(toks):
        for c in range(r.k):
            if dst[t, c] < 0:
                continue
            e = int(idx[t, c])
            raw, w64 = wt(e)
            Yrow = oracle.expert_rows(x_h[t:t + 1], [0], r.dtype, r.act, raw["w1"], raw.get("w3"), raw["w2"])[0]
            dg_ref[t, c] = float(Yrow @ dyf[t])
            dX, _, _, _ = OB.expert_backward(x_h[t:t + 1], np.array([0, 1]), r.act, w64["w1"], w64.get("w3"),
                                             w64["w2"], float(gate[t, c]) * dyf[t:t + 1])
            dx_ref[i] += dX[0]
    dl = OB.gate_backward(oplan["logits"], oplan, dg_ref, r.gate_mode)
    dx_ref += dl[toks] @ wg_h.astype(np.float64).T
    got = {"dx": grads["dx"].cpu().numpy().astype(np.float64)[toks],
           "dg": grads["dg"].cpu().numpy().astype(np.float64)[toks]}
    _compare(f"full run {name} tokens", got, {"dx": dx_ref, "dg": dg_ref[toks]}, GRAD_RELL2_MC)
