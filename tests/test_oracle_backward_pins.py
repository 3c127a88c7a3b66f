"""Pins of the backward oracle (oracle/backward.py) to things other than itself.

- Central finite differences of the forward oracle (moe_oracle.c, a separately
  pinned function) on tiny fp32 layers: the loss sum(dy * y) + the training terms,
  differentiated in every input tensor at sampled entries, with the routing held
  fixed (an entry whose perturbation changes the plan is skipped).  This catches a
  dropped term, a sign, a transposed operand or a wrong activation derivative.
- Invariants of the gate Jacobians: softmax-based gates give logit gradients that
  sum to zero per token; one expert with k = 1 has a constant gate (no router
  gradient); the bias gradient is the column sum of the logit gradient.
- The two transposes of the all-to-all paragraph ("Expert-parallel MoE training"
  explainer): the combine's backward scatters g * dy to the kept rows and the
  dispatch's backward sums each token's rows, checked against brute force.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as OB

F32 = oracle.F32


def _layer(seed, T=12, H=16, E=4, k=2, F=12, act=oracle.SWIGLU, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (rng.standard_normal((H, E)) * 0.5).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None
    w1 = (rng.standard_normal((E, F, H)) / np.sqrt(H)).astype(np.float32)
    w3 = (rng.standard_normal((E, F, H)) / np.sqrt(H)).astype(np.float32) if act == oracle.SWIGLU else None
    w2 = (rng.standard_normal((E, H, F)) / np.sqrt(F)).astype(np.float32)
    dy = rng.standard_normal((T, H))
    return dict(x=x, wg=wg, bias=b, w1=w1, w3=w3, w2=w2, dy=dy)


def _loss(p, k, gate_mode, act, C, score_fn, aux_mode, aux_coeff, z_coeff):
    y, plan, X, Y = oracle.forward(p["x"], F32, p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], k, gate_mode, act, C,
                                   score_fn=score_fn)
    aux, z = oracle.router_losses(plan["logits"], plan["topk_idx"], plan["demand"], k, aux_mode, aux_coeff, z_coeff,
                                  score_fn)
    return float((p["dy"] * y).sum()) + aux + z, plan, X, Y


def _step(scale):
    """A perturbation of 2^-9 of the tensor's typical magnitude (large against the fp32
    rounding of the logits and gates it moves, small against the curvature)."""
    return float(2.0 ** (np.floor(np.log2(scale)) - 9))


CASES = [
    # (act, gate_mode, score_fn, capacity, aux_mode, aux_coeff, z_coeff)
    (oracle.SWIGLU, oracle.SOFTMAX_TOPK_RENORM, oracle.SOFTMAX, None, 0, 0.1, 0.01),
    (oracle.SWIGLU, oracle.TOPK_SOFTMAX, oracle.SOFTMAX, None, 0, 0.0, 0.0),
    (oracle.GELU, oracle.SOFTMAX_TOPK, oracle.SOFTMAX, 5, 1, 0.2, 0.05),
    (oracle.RELU, oracle.SOFTMAX_TOPK, oracle.SOFTMAX, 6, 0, 0.0, 0.0),
    (oracle.GELU, oracle.SOFTMAX_TOPK, oracle.SIGMOID, None, 0, 0.3, 0.0),
    (oracle.SWIGLU, oracle.SOFTMAX_TOPK_RENORM, oracle.SIGMOID, 5, 0, 0.3, 0.02),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_layer_gradient_matches_finite_differences(case):
    act, gm, sf, C, aux_mode, aux_c, z_c = CASES[case]
    p = _layer(100 + case, act=act)
    k = 2
    L0, plan, X, Y = _loss(p, k, gm, act, C, sf, aux_mode, aux_c, z_c)
    if C is not None:
        assert int(plan["n_dropped"][0]) > 0, "the capped cases must drop choices"
    g = OB.layer_backward(p["x"], F32, p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], act, gm, plan, X, Y, p["dy"],
                          sf, aux_mode, aux_c, z_c)
    grads = dict(x=g["dx"], wg=g["dWg"], bias=g["dbias"], w1=g["dW1"], w3=g["dW3"], w2=g["dW2"])
    rng = np.random.default_rng(7 + case)
    checked = 0
    for name in ("x", "wg", "bias", "w1", "w3", "w2"):
        if p[name] is None:
            continue
        flat = p[name].reshape(-1)
        scale = float(np.abs(grads[name]).max()) + 1e-30
        h = _step(float(np.sqrt(np.mean(flat.astype(np.float64) ** 2))))
        for i in rng.choice(flat.size, size=min(8, flat.size), replace=False):
            v = float(flat[i])
            vals = []
            for s in (+1, -1):
                q = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in p.items()}
                qf = q[name].reshape(-1)
                qf[i] = np.float32(v + s * h)
                Ls, pl, _, _ = _loss(q, k, gm, act, C, sf, aux_mode, aux_c, z_c)
                same = (np.array_equal(pl["topk_idx"], plan["topk_idx"]) and
                        np.array_equal(pl["dst_row"], plan["dst_row"]))
                vals.append((Ls, same, float(qf[i])))
            if not (vals[0][1] and vals[1][1]):
                continue  # the routing moved: not differentiable there
            # divided by the perturbation the fp32 entry actually took
            fd = (vals[0][0] - vals[1][0]) / (vals[0][2] - vals[1][2])
            an = float(grads[name].reshape(-1)[i])
            assert abs(fd - an) <= 2e-3 * scale + 2e-3 * abs(an), (name, i, fd, an, scale)
            checked += 1
    assert checked >= 30


def test_softmax_gate_gradients_sum_to_zero_per_token():
    p = _layer(5, T=20, E=6, k=3)
    for gm in (oracle.SOFTMAX_TOPK, oracle.SOFTMAX_TOPK_RENORM, oracle.TOPK_SOFTMAX):
        plan = oracle.route(p["x"], F32, p["wg"], p["bias"], 3, gm, None)
        dg = np.random.default_rng(1).standard_normal((20, 3))
        dl = OB.gate_backward(plan["logits"], plan, dg, gm)
        assert np.abs(dl.sum(1)).max() < 1e-12
        la = OB.losses_backward(plan["logits"], plan, 3, 0, 0.5, 0.0)
        assert np.abs(la.sum(1)).max() < 1e-12  # the load-balancing term too (z-loss does not)


def test_single_expert_has_no_router_gradient():
    p = _layer(9, E=1, k=1)
    plan = oracle.route(p["x"], F32, p["wg"], p["bias"], 1, oracle.SOFTMAX_TOPK, None)
    assert np.all(plan["topk_gate"] == 1.0)
    dl = OB.gate_backward(plan["logits"], plan, np.ones((12, 1)), oracle.SOFTMAX_TOPK)
    assert np.abs(dl).max() < 1e-15


def test_bias_gradient_is_column_sum_and_router_transpose():
    p = _layer(11)
    dl = np.random.default_rng(2).standard_normal((12, 4))
    dx, dWg, db = OB.router_backward(p["x"], p["wg"], dl)
    assert np.allclose(db, dl.sum(0), rtol=0, atol=1e-12)
    # brute force of d/dx and d/dWg of sum(dl * (x Wg))
    x, W = p["x"].astype(np.float64), p["wg"].astype(np.float64)
    for t, h in ((0, 0), (5, 7), (11, 15)):
        assert abs(dx[t, h] - sum(dl[t, e] * W[h, e] for e in range(4))) < 1e-12
    for h, e in ((0, 0), (9, 3)):
        assert abs(dWg[h, e] - sum(x[t, h] * dl[t, e] for t in range(12))) < 1e-12


def test_combine_and_dispatch_backward_are_the_all_to_all_transposes():
    """The combine's backward has the dispatch's shape and vice versa: checked as the
    adjoints of the forward combine and dispatch (<dy, combine(Y)> = <combine^T dy, Y>)."""
    p = _layer(13, T=16, E=4, k=2)
    plan = oracle.route(p["x"], F32, p["wg"], p["bias"], 2, oracle.SOFTMAX_TOPK, 5)
    assert int(plan["n_dropped"][0]) > 0
    R = plan["R"]
    rng = np.random.default_rng(3)
    Y = rng.standard_normal((R, 16))
    dy = rng.standard_normal((16, 16))
    y = oracle.combine(Y, plan, F32)
    dY, dg = OB.combine_backward(dy, Y, plan)
    assert abs((dy * y).sum() - (dY * Y).sum()) < 1e-10
    # dg is the derivative of <dy, y> in each kept gate, zero for dropped choices
    for t in range(16):
        for r in range(2):
            d = plan["dst_row"][t, r]
            want = float(Y[d] @ dy[t]) if d >= 0 else 0.0
            assert abs(dg[t, r] - want) < 1e-12
    x = rng.standard_normal((16, 16)).astype(np.float32)
    X = oracle.dispatch(x, F32, plan).astype(np.float64)
    dX = rng.standard_normal((R, 16))
    dx = OB.dispatch_backward(dX, plan, 16)
    assert abs((dX * X).sum() - (dx * x.astype(np.float64)).sum()) < 1e-10
