"""ctypes binding of libmoe_hip.so (include/moe.h): argument marshalling only.

Every step of the layer runs in the library's HIP kernels; PyTorch supplies
device memory (tensor.data_ptr()) and the current HIP stream.  There is no CPU
fallback: without the built library every call raises.
"""
import ctypes
import os
from dataclasses import dataclass

from . import _build

F32, BF16 = 0, 1
SOFTMAX_TOPK, SOFTMAX_TOPK_RENORM, TOPK_SOFTMAX = 0, 1, 2
RELU, GELU, SWIGLU = 0, 1, 2

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)

EXPORTS = ("moe_validate", "moe_capacity", "moe_max_rows", "moe_workspace_bytes", "moe_status_str",
           "moe_last_error", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
           "moe_shared_expert", "moe_combine_shared", "moe_forward_shared", "moe_route_noalloc",
           "moe_backward_workspace_bytes", "moe_backward", "moe_saved_act_bytes", "moe_forward_save")


class MoEError(RuntimeError):
    def __init__(self, status, where, detail=""):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)}){' ' + detail if detail else ''}")


class _Config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("F", ctypes.c_int32), ("dtype", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dropless", ctypes.c_int32), ("min_capacity", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double), ("aux_mode", ctypes.c_int32), ("aux_coeff", ctypes.c_double),
                ("z_coeff", ctypes.c_double), ("score_fn", ctypes.c_int32), ("drop_policy", ctypes.c_int32),
                ("second_policy", ctypes.c_int32), ("shared_F", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_gate", "dst_row", "demand", "kept", "offsets",
                                               "row_token", "n_dropped", "logits", "losses", "second_u")]


class _Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dWg", "dbias", "dW1", "dW3", "dW2", "dg")]


@dataclass
class MoEConfig:
    T: int
    H: int
    E: int
    k: int
    F: int
    dtype: int = BF16
    gate_mode: int = SOFTMAX_TOPK
    act: int = GELU
    dropless: int = 0
    capacity_factor: float = 1.0
    min_capacity: int = 0
    aux_mode: int = 0  # 0: every choice / (T*k); 1: first choice / T
    aux_coeff: float = 1e-2
    z_coeff: float = 1e-3
    score_fn: int = 0  # 0: softmax, 1: sigmoid
    drop_policy: int = 0  # 0: position, 1: probs
    second_policy: int = 0  # 0: plain top-k, 1: GShard's random second choice (k = 2, plan["second_u"])
    shared_F: int = 0  # width of the shared expert, 0 = none

    def c(self):
        return _Config(self.T, self.H, self.E, self.k, self.F, self.dtype, self.gate_mode, self.act, self.dropless,
                       self.min_capacity, float(self.capacity_factor), self.aux_mode, float(self.aux_coeff),
                       float(self.z_coeff), self.score_fn, self.drop_policy, self.second_policy, self.shared_F)

    @classmethod
    def from_run(cls, run):
        return cls(run.T, run.H, run.E, run.k, run.F, run.dtype, run.gate_mode, run.act, run.dropless,
                   run.cf if not run.dropless else 1.0, run.min_capacity)


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(_build.LIB)
        vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
        cfgp = ctypes.POINTER(_Config)
        planp = ctypes.POINTER(_Plan)
        L.moe_validate.restype = ctypes.c_int
        L.moe_validate.argtypes = [cfgp]
        L.moe_capacity.restype = i64
        L.moe_capacity.argtypes = [cfgp]
        L.moe_max_rows.restype = i64
        L.moe_max_rows.argtypes = [cfgp]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [cfgp]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [cfgp, vp, vp, vp, planp, vp, sz, vp]
        L.moe_route_noalloc.restype = ctypes.c_int
        L.moe_route_noalloc.argtypes = [cfgp, vp, vp, vp, planp, vp]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [cfgp, vp, planp, vp, vp]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [cfgp, vp, planp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [cfgp, vp, planp, vp, vp, vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, planp, vp, vp, vp, sz, vp]
        L.moe_shared_expert.restype = ctypes.c_int
        L.moe_shared_expert.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine_shared.restype = ctypes.c_int
        L.moe_combine_shared.argtypes = [cfgp, vp, planp, vp, vp, vp, vp]
        L.moe_forward_shared.restype = ctypes.c_int
        L.moe_forward_shared.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, planp, vp, vp, vp, sz, vp]
        L.moe_backward_workspace_bytes.restype = sz
        L.moe_backward_workspace_bytes.argtypes = [cfgp]
        L.moe_backward.restype = ctypes.c_int
        L.moe_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, planp, vp, vp, ctypes.POINTER(_Grads), vp, sz, vp]
        L.moe_saved_act_bytes.restype = sz
        L.moe_saved_act_bytes.argtypes = [cfgp]
        L.moe_forward_save.restype = ctypes.c_int
        L.moe_forward_save.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, planp, vp, vp, vp, vp, sz, vp]
        _lib = L
    return _lib


def status_str(s):
    return lib().moe_status_str(int(s)).decode()


def _ptr(t):
    return None if t is None else (t if isinstance(t, int) else t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(st, where):
    if st != MOE_OK:
        detail = lib().moe_last_error().decode() if st == MOE_ERR_HIP else ""
        raise MoEError(st, where, detail)


def validate(cfg: MoEConfig):
    return lib().moe_validate(ctypes.byref(cfg.c()))


def capacity(cfg: MoEConfig):
    return int(lib().moe_capacity(ctypes.byref(cfg.c())))


def max_rows(cfg: MoEConfig):
    return int(lib().moe_max_rows(ctypes.byref(cfg.c())))


def workspace_bytes(cfg: MoEConfig):
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg.c())))


def _plan_struct(plan):
    return _Plan(*[_ptr(plan.get(n)) for n in ("topk_idx", "topk_gate", "dst_row", "demand", "kept", "offsets",
                                               "row_token", "n_dropped", "logits", "losses", "second_u")])


def alloc_plan(cfg: MoEConfig, device, logits=False, losses=False):
    """Device tensors of a routing plan for cfg (caller-owned memory); `losses` adds the
    two router training terms (load-balancing loss, z-loss) as a float64 tensor of 2."""
    import torch

    T, E, k = cfg.T, cfg.E, cfg.k
    i32 = torch.int32
    plan = dict(
        topk_idx=torch.empty((T, k), dtype=i32, device=device),
        topk_gate=torch.empty((T, k), dtype=torch.float32, device=device),
        dst_row=torch.empty((T, k), dtype=i32, device=device),
        demand=torch.empty(E, dtype=i32, device=device),
        kept=torch.empty(E, dtype=i32, device=device),
        offsets=torch.empty(E + 1, dtype=i32, device=device),
        row_token=torch.empty(max(max_rows(cfg), 1), dtype=i32, device=device),
        n_dropped=torch.empty(1, dtype=i32, device=device),
    )
    if logits:
        plan["logits"] = torch.empty((T, E), dtype=torch.float32, device=device)
    if losses:
        plan["losses"] = torch.empty(2, dtype=torch.float64, device=device)
    return plan


def alloc_workspace(cfg: MoEConfig, device):
    import torch

    return torch.empty(max(workspace_bytes(cfg), 1), dtype=torch.uint8, device=device)


def route(cfg, x, wg, bias, plan, ws, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    st = lib().moe_route(ctypes.byref(c), _ptr(x), _ptr(wg), _ptr(bias), ctypes.byref(p), _ptr(ws),
                         ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "moe_route")


def route_noalloc(cfg, x, wg, bias, plan, stream=None):
    """moe_route on the library's static scratch (no workspace argument, nothing allocated)."""
    c, p = cfg.c(), _plan_struct(plan)
    st = lib().moe_route_noalloc(ctypes.byref(c), _ptr(x), _ptr(wg), _ptr(bias), ctypes.byref(p), _stream(stream))
    if st != MOE_OK:
        raise MoEError(st, "moe_route_noalloc", lib().moe_last_error().decode())


def dispatch(cfg, x, plan, X, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    _check(lib().moe_dispatch(ctypes.byref(c), _ptr(x), ctypes.byref(p), _ptr(X), _stream(stream)), "moe_dispatch")


def expert_ffn(cfg, X, plan, w1, w3, w2, Y, ws, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    st = lib().moe_expert_ffn(ctypes.byref(c), _ptr(X), ctypes.byref(p), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(Y),
                              _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "moe_expert_ffn")


def combine(cfg, Y, plan, residual, y, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    _check(lib().moe_combine(ctypes.byref(c), _ptr(Y), ctypes.byref(p), _ptr(residual), _ptr(y), _stream(stream)),
           "moe_combine")


def forward(cfg, x, wg, bias, w1, w3, w2, residual, y, plan, X, Y, ws, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    st = lib().moe_forward(ctypes.byref(c), _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2),
                           _ptr(residual), _ptr(y), ctypes.byref(p), _ptr(X), _ptr(Y), _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "moe_forward")


def saved_act_bytes(cfg: MoEConfig):
    return int(lib().moe_saved_act_bytes(ctypes.byref(cfg.c())))


def forward_save(cfg, x, wg, bias, w1, w3, w2, residual, y, plan, X, Y, act, ws, stream=None):
    """moe_forward_save: moe_forward that also keeps the first GEMM's pre-activations in act
    (a uint8 or bf16 device tensor of saved_act_bytes bytes)."""
    c, p = cfg.c(), _plan_struct(plan)
    st = lib().moe_forward_save(ctypes.byref(c), _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2),
                                _ptr(residual), _ptr(y), ctypes.byref(p), _ptr(X), _ptr(Y), _ptr(act), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "moe_forward_save")


def shared_expert(cfg, x, ws1, ws3, ws2, Ys, ws, stream=None):
    c = cfg.c()
    st = lib().moe_shared_expert(ctypes.byref(c), _ptr(x), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(Ys), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "moe_shared_expert")


def combine_shared(cfg, Y, plan, residual, Ys, y, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    _check(lib().moe_combine_shared(ctypes.byref(c), _ptr(Y), ctypes.byref(p), _ptr(residual), _ptr(Ys), _ptr(y),
                                    _stream(stream)), "moe_combine_shared")


def forward_shared(cfg, x, wg, bias, w1, w3, w2, ws1, ws3, ws2, residual, y, plan, X, Y, ws, stream=None):
    c, p = cfg.c(), _plan_struct(plan)
    st = lib().moe_forward_shared(ctypes.byref(c), _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2),
                                  _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(residual), _ptr(y), ctypes.byref(p), _ptr(X),
                                  _ptr(Y), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "moe_forward_shared")


def backward_workspace_bytes(cfg: MoEConfig):
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(cfg.c())))


def alloc_grads(cfg: MoEConfig, device, bias=True, dg=False):
    """fp32 device tensors for the gradients moe_backward writes."""
    import torch

    f32 = torch.float32
    g = dict(dx=torch.empty((cfg.T, cfg.H), dtype=f32, device=device),
             dWg=torch.empty((cfg.H, cfg.E), dtype=f32, device=device),
             dW1=torch.empty((cfg.E, cfg.F, cfg.H), dtype=f32, device=device),
             dW2=torch.empty((cfg.E, cfg.H, cfg.F), dtype=f32, device=device))
    if cfg.act == SWIGLU:
        g["dW3"] = torch.empty((cfg.E, cfg.F, cfg.H), dtype=f32, device=device)
    if bias:
        g["dbias"] = torch.empty(cfg.E, dtype=f32, device=device)
    if dg:
        g["dg"] = torch.empty((cfg.T, cfg.k), dtype=f32, device=device)
    return g


def backward(cfg, x, wg, w1, w3, w2, plan, dy, grads, ws, stream=None, act=None):
    """moe_backward: grads is a dict of device tensors (see alloc_grads); act: the
    pre-activations forward_save kept, or None to recompute them."""
    c, p = cfg.c(), _plan_struct(plan)
    gs = _Grads(*[_ptr(grads.get(n)) for n in ("dx", "dWg", "dbias", "dW1", "dW3", "dW2", "dg")])
    st = lib().moe_backward(ctypes.byref(c), _ptr(x), _ptr(wg), _ptr(w1), _ptr(w3), _ptr(w2), ctypes.byref(p),
                            _ptr(dy), _ptr(act), ctypes.byref(gs), _ptr(ws), ws.numel() if ws is not None else 0,
                            _stream(stream))
    _check(st, "moe_backward")
