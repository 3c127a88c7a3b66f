"""The seeded synthetic workloads: shapes, value distributions and seeds.

Workload shapes follow the pages' examples:
  1   tiny top-1 Switch layer in fp32, router skewed by a +2 logit bias on
      expert 0 so that capacity drops occur;
  2   Switch-style top-1, bf16 activations/weights, fp32 router, GELU experts;
  3x  the shape of the DeepSpeed discussion "The MoE spends too much time on the
      gate network" (32768 tokens, 12 experts, top-4) at capacity factors
      1.0 / 0.5 / 0.25;
  4   Mixtral-like dropless top-2 with SwiGLU experts;
  5   DeepSeek-R1-shaped routed experts (256 experts, top-8, SwiGLU 7168->2048).

Weights follow the Switch initialisation rule (Switch Transformers explainer,
section 2.2: sigma = sqrt(s / fan_in)); s = 0.1 where the workload names the
Switch scale, else s = 1.  x ~ N(0, 1).  Routers and their biases are fp32.
"""
from dataclasses import dataclass, replace
import math

import numpy as np

from . import normal, tensor_seed

# Enum values of the C ABI (include/moe.h).
F32, BF16 = 0, 1
SOFTMAX_TOPK, SOFTMAX_TOPK_RENORM, TOPK_SOFTMAX = 0, 1, 2
RELU, GELU, SWIGLU = 0, 1, 2

J_X, J_WG, J_BIAS, J_W1, J_W3, J_W2 = 0, 1, 2, 3, 4, 5
J_S1, J_S3, J_S2 = 6, 7, 8  # shared expert
J_DY = 9  # upstream gradient of the layer output (backward)


@dataclass(frozen=True)
class Run:
    name: str
    run_id: int          # seeds are 1000*run_id + tensor index
    T: int
    H: int
    E: int
    k: int
    F: int
    act: int
    dtype: int
    gate_mode: int
    dropless: int
    cf: float
    min_capacity: int
    bias: str            # "none", "skew2" (+2 on expert 0), "n0.5", "n1" (normal, given variance)
    s: float             # init scale

    @property
    def m(self):
        return 3 if self.act == SWIGLU else 2

    @property
    def elem_bytes(self):
        return 4 if self.dtype == F32 else 2

    def scaled(self, name=None, **kw):
        return replace(self, name=name or (self.name + "-small"), **kw)


RUNS = {
    "1": Run("1", 1, 256, 64, 4, 1, 128, RELU, F32, SOFTMAX_TOPK, 0, 1.25, 0, "skew2", 0.1),
    "2": Run("2", 2, 16384, 768, 64, 1, 3072, GELU, BF16, SOFTMAX_TOPK, 0, 1.0, 0, "none", 0.1),
    "3a": Run("3a", 3, 32768, 512, 12, 4, 2048, GELU, BF16, SOFTMAX_TOPK, 0, 1.0, 0, "n0.5", 1.0),
    "3b": Run("3b", 3, 32768, 512, 12, 4, 2048, GELU, BF16, SOFTMAX_TOPK, 0, 0.5, 0, "n0.5", 1.0),
    "3c": Run("3c", 3, 32768, 512, 12, 4, 2048, GELU, BF16, SOFTMAX_TOPK, 0, 0.25, 0, "n0.5", 1.0),
    "4": Run("4", 4, 8192, 4096, 8, 2, 14336, SWIGLU, BF16, TOPK_SOFTMAX, 1, 0.0, 0, "none", 1.0),
    "5": Run("5", 5, 4096, 7168, 256, 8, 2048, SWIGLU, BF16, SOFTMAX_TOPK_RENORM, 1, 0.0, 0, "n1", 1.0),
}

# Reduced shapes the oracle finishes in seconds; they keep each run's routing
# structure (E, k, gate mode, capacity rule, activation, dtype) and span several
# GPU tiles plus a ragged tail in T, rows per expert, H and F.
SMALL = {
    "1": RUNS["1"],
    "2": RUNS["2"].scaled(T=1000, H=256, F=384),
    "3a": RUNS["3a"].scaled(T=1500, H=192, F=320),
    "3b": RUNS["3b"].scaled(T=1500, H=192, F=320),
    "3c": RUNS["3c"].scaled(T=1500, H=192, F=320),
    "4": RUNS["4"].scaled(T=700, H=384, F=448),
    "5": RUNS["5"].scaled(T=333, H=256, F=192),
}


def act_dtype(run: Run) -> str:
    return "f32" if run.dtype == F32 else "bf16"


def gen_x(run: Run):
    return normal(tensor_seed(run.run_id, J_X), run.T * run.H, 1.0, act_dtype(run)).reshape(run.T, run.H)


def gen_router(run: Run):
    wg = normal(tensor_seed(run.run_id, J_WG), run.H * run.E, math.sqrt(run.s / run.H), "f32").reshape(run.H, run.E)
    if run.bias == "none":
        bias = None
    elif run.bias == "skew2":
        bias = np.zeros(run.E, np.float32)
        bias[0] = 2.0
    elif run.bias.startswith("n"):
        var = float(run.bias[1:])
        bias = normal(tensor_seed(run.run_id, J_BIAS), run.E, math.sqrt(var), "f32")
    else:
        raise ValueError(run.bias)
    return wg, bias


def gen_expert_weight(run: Run, which: str, experts=None):
    """Expert weights, every matrix stored [out_features, in_features] row-major.

    which: "w1" (gate / W_in, [E,F,H]), "w3" (SwiGLU up, [E,F,H]), "w2" (down / W_out, [E,H,F]).
    experts: optional iterable of expert ids; returns {e: [out,in]} with just those
    experts (the generator is counter-based, so any expert's slice stands alone).
    """
    j = {"w1": J_W1, "w3": J_W3, "w2": J_W2}[which]
    out_f, in_f = (run.F, run.H) if which in ("w1", "w3") else (run.H, run.F)
    sigma = math.sqrt(run.s / in_f)
    per = out_f * in_f
    seed = tensor_seed(run.run_id, j)
    dt = act_dtype(run)
    if experts is None:
        return normal(seed, run.E * per, sigma, dt).reshape(run.E, out_f, in_f)
    return {int(e): normal(seed, per, sigma, dt, first=int(e) * per).reshape(out_f, in_f) for e in experts}


def gen_shared_weight(run: Run, which: str, Fs: int):
    """Shared-expert weights (one dense FFN of width Fs, same initialisation rule as the
    routed experts): "s1" [1,Fs,H], "s3" (SwiGLU up) [1,Fs,H], "s2" [1,H,Fs]."""
    j = {"s1": J_S1, "s3": J_S3, "s2": J_S2}[which]
    out_f, in_f = (Fs, run.H) if which in ("s1", "s3") else (run.H, Fs)
    return normal(tensor_seed(run.run_id, j), out_f * in_f, math.sqrt(run.s / in_f),
                  act_dtype(run)).reshape(1, out_f, in_f)


def gen_dy(run: Run):
    """Upstream gradient dL/dy of the layer output, N(0, 1) in the activation dtype, [T, H]."""
    return normal(tensor_seed(run.run_id, J_DY), run.T * run.H, 1.0, act_dtype(run)).reshape(run.T, run.H)


def gen_all(run: Run):
    x = gen_x(run)
    wg, bias = gen_router(run)
    w1 = gen_expert_weight(run, "w1")
    w3 = gen_expert_weight(run, "w3") if run.act == SWIGLU else None
    w2 = gen_expert_weight(run, "w2")
    return dict(x=x, wg=wg, bias=bias, w1=w1, w3=w3, w2=w2)
