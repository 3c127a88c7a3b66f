"""CPU oracle of the MoE layer's backward pass.  TEST INFRASTRUCTURE ONLY (like the
rest of this package: only tests/, __graft_entry__.smoke() and the cpu_baseline leg
of bench.py may use it; the GPU library never does).

It is the gradient of the forward this package defines (moe_oracle.c: binary64 on
the given input values, gates from the fp32 logits), taken the way the training
frameworks the pages describe take it:

  - The walk through one MoE layer in the "Expert-parallel MoE training" explainer
    (router -> dispatch -> experts -> unpermute, gate-weighted sum, residual) fixes
    the chain; its all-to-all paragraph gives the two transposes: the backward of
    the combine has the dispatch's shape (each kept choice's row receives its gate
    times the token's output gradient) and the backward of the dispatch has the
    combine's shape (each token sums the input gradients of its kept rows).
  - The same explainer's router section: the load-balancing loss reaches the
    router only through P_e (f_e comes from the top-k selection and has no
    gradient), and the z-loss acts on the logits directly.
  - The routing decision (top-k selection, capacity drops, GShard's second-choice
    draw) is piecewise constant in the inputs and is held fixed; roundings (the
    fp32 logits and gates) are taken as the identity.  A dropped or absent choice
    contributes nothing to the output, so its gate gets no gradient from the
    output, but it still enters the Jacobian of the other gates.
  - The residual enters the output with coefficient one, so its gradient is dy
    itself (returned by nobody: the caller owns it).

Everything is binary64 with numpy matrix products as the only library primitive.
Weight layouts are the forward's: W1, W3 [E][F][H], W2 [E][H][F], Wg [H][E].
"""
import numpy as np

from . import SOFTMAX_TOPK, SOFTMAX_TOPK_RENORM, TOPK_SOFTMAX, RELU, GELU, SWIGLU, SOFTMAX, SIGMOID, BF16

SQRT2 = np.sqrt(2.0)


def _f64(a, dtype=None):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64, copy=False)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _act(u, act):
    if act == RELU:
        return np.maximum(u, 0.0)
    from scipy.special import erf

    return 0.5 * u * (1.0 + erf(u / SQRT2))


def _act_grad(u, act):
    """d act / du: ReLU's is 0 at u = 0 (the forward's u > 0 test); exact-erf GELU's is
    Phi(u) + u phi(u)."""
    if act == RELU:
        return (u > 0.0).astype(np.float64)
    from scipy.special import erf

    return 0.5 * (1.0 + erf(u / SQRT2)) + u * np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)


def _silu_grad(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def combine_backward(dy, Y, plan):
    """Backward of y[t] = res[t] + sum_{kept r} g[t,r] Y[dst_row[t,r]].
    dy [T][H], Y [R][H] (the expert outputs, any float).  Returns (dY [R][H], dg [T][k]):
    dY[dst_row[t,r]] = g[t,r] dy[t]; dg[t,r] = <Y[dst_row[t,r]], dy[t]> (0 if not kept)."""
    dy = _f64(dy)
    Y = _f64(Y)
    g = np.asarray(plan["topk_gate"], np.float64)
    dst = np.asarray(plan["dst_row"])
    T, k = dst.shape
    R = Y.shape[0]
    dY = np.zeros((R, dy.shape[1]))
    dg = np.zeros((T, k))
    for r in range(k):
        kept = np.nonzero(dst[:, r] >= 0)[0]
        rows = dst[kept, r]
        dY[rows] = g[kept, r][:, None] * dy[kept]
        dg[kept, r] = np.einsum("ij,ij->i", Y[rows], dy[kept])
    return dY, dg


def expert_backward(X, offsets, act, w1, w3, w2, dY):
    """Backward of the expert FFN on the packed rows (expert e owns rows offsets[e] ..
    offsets[e+1]-1): 2-matrix Y = act(X W1_e^T) W2_e^T, SwiGLU Y = (silu(X W1_e^T) *
    (X W3_e^T)) W2_e^T.  Returns (dX [R][H], dW1, dW3 or None, dW2), binary64."""
    X = _f64(X)
    dY = _f64(dY)
    W1, W2 = _f64(w1), _f64(w2)
    W3 = _f64(w3) if w3 is not None else None
    dX = np.zeros_like(X)
    dW1, dW2 = np.zeros_like(W1), np.zeros_like(W2)
    dW3 = np.zeros_like(W3) if W3 is not None else None
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        Xe, dYe = X[lo:hi], dY[lo:hi]
        u = Xe @ W1[e].T  # [n][F]
        dz = dYe @ W2[e]  # [n][F]
        if act == SWIGLU:
            v = Xe @ W3[e].T
            z = _silu(u) * v
            du = dz * v * _silu_grad(u)
            dv = dz * _silu(u)
            dW3[e] = dv.T @ Xe
            dX[lo:hi] = du @ W1[e] + dv @ W3[e]
        else:
            z = _act(u, act)
            du = dz * _act_grad(u, act)
            dX[lo:hi] = du @ W1[e]
        dW2[e] = dYe.T @ z
        dW1[e] = du.T @ Xe
    return dX, dW1, dW3, dW2


def dispatch_backward(dX, plan, T):
    """Backward of X[row] = x[row_token[row]]: dx[t] = sum over the token's kept rows of dX."""
    dX = _f64(dX)
    dst = np.asarray(plan["dst_row"])
    dx = np.zeros((T, dX.shape[1]))
    for r in range(dst.shape[1]):
        kept = np.nonzero(dst[:, r] >= 0)[0]
        dx[kept] += dX[dst[kept, r]]
    return dx


def _softmax(l):
    m = l.max(1, keepdims=True)
    p = np.exp(l - m)
    return p / p.sum(1, keepdims=True)


def gate_backward(logits, plan, dg, gate_mode, score_fn=SOFTMAX):
    """dL/dlogits from dL/dg through the gate definitions of the forward (moe_oracle.c
    gates()): softmax over all E then the chosen p (SOFTMAX_TOPK); the chosen p over
    their sum (SOFTMAX_TOPK_RENORM), which equals the softmax over the chosen logits
    (TOPK_SOFTMAX); with sigmoid scores the chosen sigma, or sigma over their sum."""
    l = _f64(logits)
    idx = np.asarray(plan["topk_idx"])
    T, E = l.shape
    k = idx.shape[1]
    dg = np.asarray(dg, np.float64)
    dl = np.zeros((T, E))
    tt = np.arange(T)[:, None]
    if score_fn == SIGMOID and gate_mode != TOPK_SOFTMAX:
        s = 1.0 / (1.0 + np.exp(-l[tt, idx]))  # [T][k] chosen scores
        ds_dl = s * (1.0 - s)
        if gate_mode == SOFTMAX_TOPK:
            dsc = dg
        else:
            S = s.sum(1, keepdims=True)
            g = s / S
            dsc = (dg - (g * dg).sum(1, keepdims=True)) / S
        np.add.at(dl, (np.broadcast_to(tt, idx.shape), idx), dsc * ds_dl)
        return dl
    if gate_mode == SOFTMAX_TOPK:
        p = _softmax(l)
        g = p[tt, idx]
        np.add.at(dl, (np.broadcast_to(tt, idx.shape), idx), g * dg)
        dl -= p * (g * dg).sum(1, keepdims=True)
        return dl
    # RENORM and TOPK_SOFTMAX: g = softmax over the chosen logits
    lc = l[tt, idx]
    g = _softmax(lc)
    dlc = g * (dg - (g * dg).sum(1, keepdims=True))
    np.add.at(dl, (np.broadcast_to(tt, idx.shape), idx), dlc)
    return dl


def losses_backward(logits, plan, k, aux_mode=0, aux_coeff=0.0, z_coeff=0.0, score_fn=SOFTMAX):
    """dL/dlogits of aux_coeff * E * sum_e f_e P_e + z_coeff * mean_t logsumexp(l_t)^2
    (oracle_router_losses): f_e is constant; P_e = mean_t q_e(t) with q the softmax, or
    the sigmoid scores over their sum."""
    l = _f64(logits)
    T, E = l.shape
    dl = np.zeros((T, E))
    if T == 0:
        return dl
    idx = np.asarray(plan["topk_idx"])
    if aux_coeff != 0.0:
        if aux_mode == 0:
            f = np.asarray(plan["demand"], np.float64) / (T * k)
        else:
            f = np.bincount(idx[:, 0], minlength=E).astype(np.float64) / T
        c = aux_coeff * E * f / T  # dL/dq_e(t)
        if score_fn == SIGMOID:
            s = 1.0 / (1.0 + np.exp(-l))
            S = s.sum(1, keepdims=True)
            dl += s * (1.0 - s) / S * (c[None, :] - (c[None, :] * s).sum(1, keepdims=True) / S)
        else:
            p = _softmax(l)
            dl += p * (c[None, :] - (p * c[None, :]).sum(1, keepdims=True))
    if z_coeff != 0.0:
        m = l.max(1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(l - m).sum(1))
        dl += z_coeff * 2.0 / T * lse[:, None] * _softmax(l)
    return dl


def router_backward(x, wg, dl):
    """Backward of l = bias + x Wg: (dx [T][H], dWg [H][E], dbias [E])."""
    xf = _f64(x)
    W = _f64(wg)
    return dl @ W.T, xf.T @ dl, dl.sum(0)


def layer_backward(x, dtype, wg, bias, w1, w3, w2, act, gate_mode, plan, X, Y, dy, score_fn=SOFTMAX,
                   aux_mode=0, aux_coeff=0.0, z_coeff=0.0):
    """Whole-layer backward for the upstream gradient dy [T][H] (plus the training terms
    with their coefficients): returns dict(dx, dWg, dbias, dW1, dW3, dW2, dlogits, dg)."""
    T, k = np.asarray(plan["dst_row"]).shape
    dY, dg = combine_backward(dy, Y, plan)
    dX, dW1, dW3, dW2 = expert_backward(X, plan["offsets"], act, w1, w3, w2, dY)
    dx = dispatch_backward(dX, plan, T)
    dl = gate_backward(plan["logits"], plan, dg, gate_mode, score_fn)
    dl += losses_backward(plan["logits"], plan, k, aux_mode, aux_coeff, z_coeff, score_fn)
    dxr, dWg, dbias = router_backward(x, wg, dl)
    return dict(dx=dx + dxr, dWg=dWg, dbias=dbias, dW1=dW1, dW3=dW3, dW2=dW2, dlogits=dl, dg=dg)
