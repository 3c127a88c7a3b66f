"""CPU oracle of the MoE FFN layer forward (ctypes over liboracle.so, built from moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  It shares no code with the
GPU library; the only thing both sides share is the seeded input generator.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
SOFTMAX_TOPK, SOFTMAX_TOPK_RENORM, TOPK_SOFTMAX = 0, 1, 2
RELU, GELU, SWIGLU = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1
DROP_POSITION, DROP_PROBS = 0, 1
SECOND_ALWAYS, SECOND_RANDOM = 0, 1

_lib = None


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-o", LIB_PATH + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.oracle_capacity.restype = i64
        L.oracle_capacity.argtypes = [i64, i64, i64, dbl, i64, i32]
        L.oracle_logits.restype = None
        L.oracle_logits.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp]
        L.oracle_route_from_logits.restype = i64
        L.oracle_route_from_logits.argtypes = [i64, i64, i32, i32, i32, i32, i32, vp, i64, vp] + [vp] * 8
        L.oracle_dispatch.restype = None
        L.oracle_router_losses.restype = None
        L.oracle_router_losses.argtypes = [i64, i64, i32, i32, vp, vp, vp, i32, dbl, dbl, vp]
        L.oracle_dispatch.argtypes = [i64, i64, i32, vp, vp, vp]
        L.oracle_expert_rows.restype = None
        L.oracle_expert_rows.argtypes = [i64, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [i64, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, i64, vp, vp]
        L.oracle_token_outputs.restype = None
        L.oracle_token_outputs.argtypes = [i64, vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dt is not None:
        assert a.dtype == dt, (a.dtype, dt)
    return a


def _act_np(dtype):
    return np.uint16 if dtype == BF16 else np.float32


def capacity(T, k, E, cf, min_capacity=0, dropless=0):
    return int(lib().oracle_capacity(T, k, E, float(cf), min_capacity, int(dropless)))


def logits(x, dtype, wg, bias=None):
    x = _c(x, _act_np(dtype))
    wg = _c(wg, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = wg.shape[1]
    out = np.empty((T, E), np.float32)
    lib().oracle_logits(T, H, E, dtype, _p(x), _p(wg), _p(bias), _p(out))
    return out


def route_from_logits(lg, k, gate_mode, C, score_fn=SOFTMAX, drop_policy=DROP_POSITION, second_u=None):
    """C: capacity, or None for dropless; second_u: uniforms [T] for GShard's random second
    choice (k = 2), or None.  Returns the routing plan as numpy arrays."""
    lg = _c(lg, np.float32)
    T, E = lg.shape
    Cc = -1 if C is None else int(C)
    tk = T * k
    plan = dict(
        topk_idx=np.empty((T, k), np.int32),
        topk_gate=np.empty((T, k), np.float32),
        dst_row=np.empty((T, k), np.int32),
        demand=np.empty(E, np.int32),
        kept=np.empty(E, np.int32),
        offsets=np.empty(E + 1, np.int32),
        row_token=np.full(max(tk, 1), -1, np.int32),
        n_dropped=np.zeros(1, np.int32),
    )
    su = None if second_u is None else _c(second_u, np.float32)
    R = lib().oracle_route_from_logits(T, E, k, gate_mode, score_fn, drop_policy, 0 if su is None else 1,
                                       None if su is None else _p(su), Cc, _p(lg), *[_p(plan[n]) for n in (
        "topk_idx", "topk_gate", "dst_row", "demand", "kept", "offsets", "row_token", "n_dropped")])
    if R < 0:
        raise ValueError("bad routing arguments")
    plan["R"] = int(R)
    plan["row_token"] = plan["row_token"][:R].copy()
    return plan


def router_losses(logits, topk_idx, demand, k, aux_mode=0, aux_coeff=1.0, z_coeff=1.0, score_fn=SOFTMAX):
    """(load-balancing loss, z-loss) of a routing: see oracle_router_losses."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = _c(np.asarray(topk_idx).reshape(T, k), np.int32)
    dem = _c(demand, np.int32)
    out = np.zeros(2, np.float64)
    lib().oracle_router_losses(T, E, k, int(score_fn), _p(lg), _p(idx), _p(dem), int(aux_mode), float(aux_coeff),
                               float(z_coeff), _p(out))
    return float(out[0]), float(out[1])


def route(x, dtype, wg, bias, k, gate_mode, C, score_fn=SOFTMAX, drop_policy=DROP_POSITION, second_u=None):
    lg = logits(x, dtype, wg, bias)
    plan = route_from_logits(lg, k, gate_mode, C, score_fn, drop_policy, second_u)
    plan["logits"] = lg
    return plan


def dispatch(x, dtype, plan):
    x = _c(x, _act_np(dtype))
    T, H = x.shape
    R = plan["R"]
    X = np.empty((R, H), x.dtype)
    rt = _c(plan["row_token"], np.int32)
    lib().oracle_dispatch(R, H, dtype, _p(x), _p(rt), _p(X))
    return X


def expert_ffn(X, offsets, dtype, act, w1, w3, w2):
    X = _c(X, _act_np(dtype))
    offsets = _c(offsets, np.int32)
    E = offsets.size - 1
    R = int(offsets[-1])
    H = w1.shape[2]
    F = w1.shape[1]
    Y = np.empty((R, H), np.float64)
    w1, w2 = _c(w1, _act_np(dtype)), _c(w2, _act_np(dtype))
    w3 = _c(w3, _act_np(dtype)) if w3 is not None else None
    lib().oracle_expert_ffn(E, _p(offsets), H, F, dtype, act, _p(X), _p(w1), _p(w3), _p(w2), _p(Y))
    return Y


def expert_rows(xrows, experts, dtype, act, w1, w3, w2):
    xrows = _c(xrows, _act_np(dtype))
    ex = _c(np.asarray(experts, np.int32), np.int32)
    n, H = xrows.shape
    F = w1.shape[1]
    Y = np.empty((n, H), np.float64)
    w1, w2 = _c(w1, _act_np(dtype)), _c(w2, _act_np(dtype))
    w3 = _c(w3, _act_np(dtype)) if w3 is not None else None
    lib().oracle_expert_rows(n, _p(ex), H, F, dtype, act, _p(xrows), _p(w1), _p(w3), _p(w2), _p(Y))
    return Y


def combine(Y, plan, dtype, residual=None, tokens=None):
    Y = _c(Y, np.float64)
    T, k = plan["topk_idx"].shape
    H = Y.shape[1] if Y.ndim == 2 and Y.shape[0] else (residual.shape[1] if residual is not None else 0)
    if Y.size == 0:
        Y = np.zeros((1, max(H, 1)), np.float64)
    res = _c(residual, _act_np(dtype)) if residual is not None else None
    tok = None if tokens is None else _c(np.asarray(tokens, np.int64), np.int64)
    n = T if tok is None else tok.size
    y = np.empty((n, H), np.float64)
    lib().oracle_combine(T, H, k, dtype, _p(Y), _p(_c(plan["topk_gate"], np.float32)),
                         _p(_c(plan["dst_row"], np.int32)), _p(res), n, _p(tok), _p(y))
    return y


def token_outputs(tokens, x, dtype, act, plan, w1, w3, w2, residual=None):
    x = _c(x, _act_np(dtype))
    tok = _c(np.asarray(tokens, np.int64), np.int64)
    T, H = x.shape
    F = w1.shape[1]
    k = plan["topk_idx"].shape[1]
    y = np.empty((tok.size, H), np.float64)
    w1, w2 = _c(w1, _act_np(dtype)), _c(w2, _act_np(dtype))
    w3 = _c(w3, _act_np(dtype)) if w3 is not None else None
    res = _c(residual, _act_np(dtype)) if residual is not None else None
    lib().oracle_token_outputs(tok.size, _p(tok), H, F, k, dtype, act, _p(x),
                               _p(_c(plan["topk_idx"], np.int32)), _p(_c(plan["topk_gate"], np.float32)),
                               _p(_c(plan["dst_row"], np.int32)), _p(w1), _p(w3), _p(w2), _p(res), _p(y))
    return y


def shared_expert(x, dtype, act, ws1, ws3, ws2, tokens=None):
    """The shared expert ("Expert-parallel MoE training" explainer, layer walk-through:
    a dense MLP outside the router and the all-to-all, computed on every token and
    added to the routed experts' output; Megatron-Core SharedExpertMLP, DeepSpeed's
    Residual-MoE dense branch).  Read here as one more FFN of the routed experts' form
    (same activation; ws1/ws3 [1, Fs, H], ws2 [1, H, Fs]) applied to every token (or
    to the listed tokens), in binary64 like expert_rows.  Returns [n, H] float64."""
    x = _c(x, _act_np(dtype))
    rows = x if tokens is None else x[np.asarray(tokens, np.int64)]
    return expert_rows(rows, np.zeros(rows.shape[0], np.int32), dtype, act, ws1, ws3, ws2)


def forward(x, dtype, wg, bias, w1, w3, w2, k, gate_mode, act, C, residual=None, score_fn=SOFTMAX,
            drop_policy=DROP_POSITION, second_u=None, shared=None):
    """Whole layer: route -> dispatch -> expert FFN -> combine (+ the shared expert's
    output when shared = (ws1, ws3, ws2)).  Returns (y float64, plan, X, Y)."""
    plan = route(x, dtype, wg, bias, k, gate_mode, C, score_fn, drop_policy, second_u)
    X = dispatch(x, dtype, plan)
    Y = expert_ffn(X, plan["offsets"], dtype, act, w1, w3, w2)
    y = combine(Y, plan, dtype, residual)
    if shared is not None:
        y = y + shared_expert(x, dtype, act, *shared)
    return y, plan, X, Y
