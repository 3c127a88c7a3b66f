// C ABI of the MoE layer forward: argument validation, capacity, workspace
// sizing and the stream-ordered launch sequence.  Declarations and the
// contract of every entry point are in include/moe.h.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kernels.hpp"
#include "moe.h"

namespace {

constexpr int kBlockTokens = 64;  // tokens per histogram block (one wave in the select kernel)
constexpr size_t kAlign = 256;

thread_local char g_last_error[256] = "";

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status hip_fail(hipError_t err, const char* where) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(err));
  return MOE_ERR_HIP;
}

// Capacity in 64-bit; -1 = dropless.  Plain ceil((T*k/E)*cf), raised to
// min_capacity ("Expert-parallel MoE training" explainer, capacity section;
// DeepSpeed discussion #7508).  Evaluated as one multiply, one divide, ceil.
int64_t capacity_of(const moe_config* c) {
  if (c->dropless) return -1;
  const double v = ceil((double)((int64_t)c->T * c->k) * c->capacity_factor / (double)c->E);
  int64_t C = v > 9.0e18 ? INT64_MAX : (int64_t)v;
  if (C < c->min_capacity) C = c->min_capacity;
  return C;
}

int64_t max_rows_of(const moe_config* c) {
  const int64_t tk = (int64_t)c->T * c->k;
  const int64_t C = capacity_of(c);
  if (C < 0) return tk;
  const int64_t ec = C > tk ? tk : C * c->E;
  return ec < tk ? ec : tk;
}

// Capacity as the kernels use it: an int32 bound that no slot reaches when
// nothing can be dropped.
int effective_capacity(const moe_config* c) {
  const int64_t C = capacity_of(c);
  const int64_t tk = (int64_t)c->T * c->k;
  if (C < 0 || C >= tk) return INT32_MAX;
  return (int)C;
}

// Most rows one expert can hold: the capacity, or every kept row when no
// capacity limits (the expert FFN streams weight rows that one tile covers).
int64_t expert_rows_cap(const moe_config* c, int64_t R_max) {
  const int C = effective_capacity(c);
  return C == INT32_MAX || (int64_t)C > R_max ? R_max : (int64_t)C;
}

struct Layout {
  int nb, Q;
  bool split;  // split-bf16 router buffers present
  size_t hist, logits, wp, wsq, wn, lpart, xsq, pairs, utok, count, lp, lz, lc, lkey, lq, nslot, route_end, h, ffn_end,
      total;
  size_t hs, ys, soff, shared_end;  // shared expert: hidden [T][Fs], output [T][H], offsets {0, T}
};

// The split-bf16 router runs for bf16 activations with H a multiple of 64 and a
// 16-byte aligned x; otherwise the exact router does.
bool split_router_shape(const moe_config* c) { return c->dtype == MOE_BF16 && c->H % 64 == 0; }

Layout layout_of(const moe_config* c) {
  Layout L;
  L.nb = (c->T + kBlockTokens - 1) / kBlockTokens;
  L.Q = c->k * L.nb;
  const size_t eb = c->dtype == MOE_BF16 ? 2 : 4;
  L.hist = 0;
  L.logits = align_up(sizeof(int32_t) * (size_t)c->E * (size_t)L.Q);
  size_t end = L.logits + align_up(sizeof(float) * (size_t)c->T * (size_t)c->E);
  L.split = split_router_shape(c);
  L.wp = L.wsq = L.wn = L.lpart = L.xsq = L.pairs = L.utok = L.count = end;
  if (L.split) {
    const size_t Ep = (size_t)moe::split_router_ep(c->E), HS = (size_t)moe::split_router_hs(c->H);
    const size_t hsplit = (size_t)moe::split_router_hsplit(c->T, c->E, c->H);
    L.wp = end;
    L.wsq = L.wp + align_up(sizeof(uint16_t) * 3 * Ep * (size_t)c->H);
    L.wn = L.wsq + align_up(sizeof(double) * HS * Ep);
    L.lpart = L.wn + align_up(sizeof(double) * Ep);
    L.xsq = L.lpart + (c->E > 64 ? align_up(sizeof(double) * hsplit * (size_t)c->T * Ep) : 0);
    L.pairs = L.xsq + align_up(sizeof(float) * hsplit * (size_t)c->T);
    L.utok = L.pairs + align_up(sizeof(int2) * (size_t)c->T * (size_t)c->E);
    L.count = L.utok + align_up(sizeof(int4) * (size_t)c->T);
    end = L.count + kAlign;
  }
  // router training terms: per-64-token-block partial sums
  L.lp = end;
  L.lz = L.lp + align_up(sizeof(double) * (size_t)L.nb * (size_t)c->E);
  L.lc = L.lz + align_up(sizeof(double) * ((size_t)(L.nb > 0 ? L.nb : 1) + (size_t)c->E + 1));
  end = L.lc + align_up(sizeof(int32_t) * (size_t)L.nb * (size_t)c->E);
  // "probs" drop policy: per-assignment key, position and slot
  const size_t tk = (size_t)c->T * (size_t)c->k;
  L.lkey = end;
  L.lq = L.lkey + align_up(sizeof(uint32_t) * tk);
  L.nslot = L.lq + align_up(sizeof(uint32_t) * tk);
  end = L.nslot + align_up(sizeof(int32_t) * tk);
  L.route_end = end;
  L.h = 0;
  L.ffn_end = align_up(eb * (size_t)max_rows_of(c) * (size_t)c->F);
  L.total = L.route_end > L.ffn_end ? L.route_end : L.ffn_end;
  // the shared expert runs after the routed experts: its buffers reuse the same space
  L.hs = L.ys = L.soff = L.shared_end = 0;
  if (c->shared_F > 0) {
    L.hs = 0;
    L.ys = align_up(eb * (size_t)c->T * (size_t)c->shared_F);
    L.soff = L.ys + align_up(eb * (size_t)c->T * (size_t)c->H);
    L.shared_end = L.soff + kAlign;
    if (L.shared_end > L.total) L.total = L.shared_end;
  }
  if (L.total == 0) L.total = kAlign;
  return L;
}

// The per-assignment arrays may be NULL only when there are no tokens.
moe_status check_plan(const moe_config* c, const moe_plan* p) {
  if (!p || !p->demand || !p->kept || !p->offsets || !p->n_dropped) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && (!p->topk_idx || !p->topk_gate || !p->dst_row || !p->row_token)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Argument checks shared by the two route entry points (workspace checked apart).
moe_status check_route_args(const moe_config* c, const void* x, const float* Wg, const moe_plan* plan);
moe_status route_body(const moe_config* c, const void* x, const float* Wg, const float* bias, const moe_plan* plan,
                      void* ws, void* stream);

// Route scratch of moe_route_noalloc: one array per device (each GPU that runs
// the library holds its own copy until the process ends), shared by every call
// on that device.  Host code uses only the device address taken from the symbol
// (per device, once), never the array's name.
constexpr size_t kStaticScratchBytes = (size_t)96 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[moe::kMaxDevices] = {};

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= moe::kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_validate(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->H < 1 || c->F < 1) return MOE_ERR_INVALID_ARG;
  if (c->E < 1 || c->E > 1024) return MOE_ERR_INVALID_ARG;
  if (c->k < 1 || c->k > 16 || c->k > c->E) return MOE_ERR_INVALID_ARG;
  if ((int64_t)c->T * c->k >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->gate_mode < MOE_SOFTMAX_TOPK || c->gate_mode > MOE_TOPK_SOFTMAX) return MOE_ERR_INVALID_ARG;
  if (c->act < MOE_RELU || c->act > MOE_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (c->dropless != 0 && c->dropless != 1) return MOE_ERR_INVALID_ARG;
  if (c->min_capacity < 0) return MOE_ERR_INVALID_ARG;
  if (!c->dropless && !(c->capacity_factor > 0.0 && isfinite(c->capacity_factor))) return MOE_ERR_INVALID_ARG;
  if (c->aux_mode != MOE_AUX_ALL_CHOICES && c->aux_mode != MOE_AUX_FIRST_CHOICE) return MOE_ERR_INVALID_ARG;
  if (!isfinite(c->aux_coeff) || !isfinite(c->z_coeff)) return MOE_ERR_INVALID_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->drop_policy != MOE_DROP_POSITION && c->drop_policy != MOE_DROP_PROBS) return MOE_ERR_INVALID_ARG;
  if (c->second_policy != MOE_SECOND_ALWAYS && c->second_policy != MOE_SECOND_RANDOM) return MOE_ERR_INVALID_ARG;
  if (c->second_policy == MOE_SECOND_RANDOM && c->k != 2) return MOE_ERR_INVALID_ARG;
  if (c->shared_F < 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int64_t moe_capacity(const moe_config* c) {
  if (moe_validate(c) != MOE_OK) return -2;
  return capacity_of(c);
}

int64_t moe_max_rows(const moe_config* c) {
  if (moe_validate(c) != MOE_OK) return -1;
  return max_rows_of(c);
}

size_t moe_workspace_bytes(const moe_config* c) {
  if (moe_validate(c) != MOE_OK) return 0;
  return layout_of(c).total;
}

size_t moe_backward_workspace_bytes(const moe_config* c) {
  if (moe_validate(c) != MOE_OK) return 0;
  return moe::backward_workspace_bytes(c->T, c->H, c->E, c->k, c->F, max_rows_of(c), c->dtype == MOE_BF16, c->act);
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error; }

moe_status moe_route(const moe_config* c, const void* x, const float* Wg, const float* bias, const moe_plan* plan,
                     void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_route_args(c, x, Wg, plan);
  if (s != MOE_OK) return s;
  if (!ws || ws_bytes < layout_of(c).total) return MOE_ERR_WORKSPACE;
  return route_body(c, x, Wg, bias, plan, ws, stream);
}

moe_status moe_route_noalloc(const moe_config* c, const void* x, const float* Wg, const float* bias,
                             const moe_plan* plan, void* stream) {
  moe_status s = check_route_args(c, x, Wg, plan);
  if (s != MOE_OK) return s;
  const size_t need = layout_of(c).route_end;
  if (need > kStaticScratchBytes) {
    snprintf(g_last_error, sizeof g_last_error,
             "moe_route_noalloc: this configuration needs %zu bytes of route scratch, more than the %zu of the "
             "static scratch",
             need, kStaticScratchBytes);
    return MOE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "moe_route_noalloc: static scratch address");
  return route_body(c, x, Wg, bias, plan, ws, stream);
}

}  // extern "C"

namespace {

moe_status check_route_args(const moe_config* c, const void* x, const float* Wg, const moe_plan* plan) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if ((s = check_plan(c, plan)) != MOE_OK) return s;
  if ((c->T > 0 && !x) || !Wg) return MOE_ERR_INVALID_ARG;
  if (c->second_policy == MOE_SECOND_RANDOM && c->T > 0 && !plan->second_u) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Route into the workspace `ws` (at least layout_of(c).route_end bytes; checked by
// the caller together with the arguments).
moe_status route_body(const moe_config* c, const void* x, const float* Wg, const float* bias, const moe_plan* plan,
                      void* ws, void* stream) {
  const float* su = c->second_policy == MOE_SECOND_RANDOM ? plan->second_u : nullptr;
  const Layout L = layout_of(c);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(w + L.hist);
  float* logits = plan->logits ? plan->logits : reinterpret_cast<float*>(w + L.logits);
  const bool bf16 = c->dtype == MOE_BF16;
  const int C = effective_capacity(c);
  const int gm = c->gate_mode | (c->score_fn == MOE_SCORE_SIGMOID ? moe::kSigmoidFlag : 0);
  hipError_t e;
  int fused = 0;  // work the split router's epilogue took over (1: ranks, 2: loss partials)
  // Where gate values decide the plan (the "probs" policy under a limiting
  // capacity, GShard's random second choice) every logit and gate is computed
  // exactly as defined (exact path); elsewhere the split-bf16 router certifies
  // the choices where its shape allows.
  const bool gate_decides = c->second_policy == MOE_SECOND_RANDOM || (c->drop_policy == MOE_DROP_PROBS && C != INT32_MAX);
  if (L.split && aligned16(x) && !gate_decides) {
    moe::SplitScratch sc;
    sc.wp = w + L.wp;
    sc.wsq = reinterpret_cast<double*>(w + L.wsq);
    sc.wn = reinterpret_cast<double*>(w + L.wn);
    sc.lpart = reinterpret_cast<double*>(w + L.lpart);
    sc.xsq = reinterpret_cast<float*>(w + L.xsq);
    sc.pairs = reinterpret_cast<int2*>(w + L.pairs);
    sc.utok = reinterpret_cast<int4*>(w + L.utok);
    sc.count = reinterpret_cast<int*>(w + L.count);
    const moe::SplitEpilogue ep{plan->dst_row,
                                hist,
                                plan->losses ? reinterpret_cast<double*>(w + L.lp) : nullptr,
                                reinterpret_cast<double*>(w + L.lz),
                                reinterpret_cast<int32_t*>(w + L.lc),
                                c->score_fn};
    if ((e = moe::launch_router_split(x, Wg, bias, logits, c->T, c->H, c->E, c->k, gm, plan->topk_idx,
                                      plan->topk_gate, sc, ep, &fused, st)) != hipSuccess)
      return hip_fail(e, "router_split");
    if (!(fused & 1) &&
        (e = moe::launch_router_rank(plan->topk_idx, c->T, c->E, c->k, L.nb, plan->dst_row, hist, st)) != hipSuccess)
      return hip_fail(e, "router_rank");
  } else {
    if ((e = moe::launch_router_exact(x, bf16, Wg, bias, logits, c->T, c->H, c->E, aligned16(x) && c->H % 4 == 0, st)) !=
        hipSuccess)
      return hip_fail(e, "router_exact");
    if ((e = moe::launch_router_select(logits, c->T, c->E, c->k, gm, su, L.nb, plan->topk_idx,
                                       plan->topk_gate, plan->dst_row, hist, st)) != hipSuccess)
      return hip_fail(e, "router_select");
  }
  if ((e = moe::launch_slot_scan(hist, L.Q, c->E, C, plan->demand, plan->kept, st)) != hipSuccess)
    return hip_fail(e, "slot_scan");
  if (c->drop_policy == MOE_DROP_PROBS && C != INT32_MAX) {
    if ((e = moe::launch_slot_probs(hist, L.Q, L.nb, c->T, c->E, c->k, C, plan->topk_idx, plan->topk_gate,
                                    plan->demand, plan->kept, plan->dst_row, plan->row_token, plan->offsets,
                                    plan->n_dropped, (int)max_rows_of(c), reinterpret_cast<uint32_t*>(w + L.lkey),
                                    reinterpret_cast<uint32_t*>(w + L.lq), reinterpret_cast<int32_t*>(w + L.nslot),
                                    st)) != hipSuccess)
      return hip_fail(e, "slot_probs");
  } else if ((e = moe::launch_slot_finalize(hist, L.Q, L.nb, c->T, c->E, c->k, C, plan->topk_idx, plan->kept,
                                            plan->dst_row, plan->row_token, plan->offsets, plan->n_dropped,
                                            (int)max_rows_of(c), st)) != hipSuccess) {
    return hip_fail(e, "slot_finalize");
  }
  if (plan->losses &&
      (e = moe::launch_router_losses(logits, plan->topk_idx, plan->demand, c->T, c->E, c->k, c->score_fn, c->aux_mode,
                                     c->aux_coeff, c->z_coeff, reinterpret_cast<double*>(w + L.lp),
                                     reinterpret_cast<double*>(w + L.lz), reinterpret_cast<int32_t*>(w + L.lc),
                                     plan->losses, (fused & 2) != 0, st)) != hipSuccess)
    return hip_fail(e, "router_losses");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_dispatch(const moe_config* c, const void* x, const moe_plan* plan, void* X, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if (!plan || (c->T > 0 && (!plan->dst_row || !x || !X))) return MOE_ERR_INVALID_ARG;
  const bool bf16 = c->dtype == MOE_BF16;
  hipError_t e = moe::launch_dispatch(x, plan->dst_row, X, c->T, c->H, c->k, (int)max_rows_of(c), bf16,
                                      aligned16(x) && aligned16(X), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "dispatch");
}

moe_status moe_expert_ffn(const moe_config* c, const void* X, const moe_plan* plan, const void* W1, const void* W3,
                          const void* W2, void* Y, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if (!plan || !plan->offsets) return MOE_ERR_INVALID_ARG;
  if (!W1 || !W2 || (c->act == MOE_SWIGLU) != (W3 != nullptr)) return MOE_ERR_INVALID_ARG;
  const int64_t R_max = max_rows_of(c);
  if (R_max > 0 && (!X || !Y)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(c);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  void* h = static_cast<char*>(ws) + L.h;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool vec = c->H % 8 == 0 && c->F % 8 == 0 && aligned16(X) && aligned16(Y) && aligned16(W1) &&
                   aligned16(W3) && aligned16(W2) && aligned16(h);
  hipError_t e = moe::launch_expert_ffn(X, W1, W3, W2, h, Y, plan->offsets, c->E, c->H, c->F, c->act, bf16, vec, R_max,
                                        expert_rows_cap(c, R_max), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "expert_ffn");
}

moe_status moe_combine(const moe_config* c, const void* Y, const moe_plan* plan, const void* residual, void* y,
                       void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if (!plan || (c->T > 0 && (!plan->dst_row || !plan->topk_gate || !y))) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && !Y && max_rows_of(c) > 0) return MOE_ERR_INVALID_ARG;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool vec = c->H % 8 == 0 && aligned16(Y) && aligned16(y) && aligned16(residual);
  hipError_t e = moe::launch_combine(Y, plan->dst_row, plan->topk_gate, residual, y, c->T, c->H, c->k,
                                     (int)max_rows_of(c), bf16, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "combine");
}

}  // extern "C"

namespace {

// moe_forward, and with act != nullptr moe_forward_save (the first GEMM's
// pre-activations kept, tiled bf16 path only).
moe_status forward_impl(const moe_config* c, const void* x, const float* Wg, const float* bias, const void* W1,
                        const void* W3, const void* W2, const void* residual, void* y, const moe_plan* plan, void* X,
                        void* Y, void* act, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if ((s = check_plan(c, plan)) != MOE_OK) return s;
  if (!W1 || !W2 || (c->act == MOE_SWIGLU) != (W3 != nullptr) || !Wg) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && (!x || !y || !X || !Y)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < layout_of(c).total) return MOE_ERR_WORKSPACE;
  // Where the tiled bf16 GEMMs run, the first one reads the token rows of x
  // through plan->row_token itself and the dispatch copy is skipped (X unused).
  const int64_t R_max = max_rows_of(c);
  void* h = static_cast<char*>(ws) + layout_of(c).h;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool vec = c->H % 8 == 0 && c->F % 8 == 0 && aligned16(x) && aligned16(Y) && aligned16(W1) &&
                   aligned16(W3) && aligned16(W2) && aligned16(h);
  const bool tiled = moe::expert_ffn_gathers(bf16, vec, c->H);
  if (act && (!tiled || !moe::expert_ffn_saves(bf16, vec, c->H, c->F) || !aligned16(act))) return MOE_ERR_UNSUPPORTED;
  if ((s = moe_route(c, x, Wg, bias, plan, ws, ws_bytes, stream)) != MOE_OK) return s;
  if (R_max > 0 && c->T > 0 && tiled) {
    // Top-1 on the same path: the second GEMM writes y itself (Y unused).
    const bool fuse = c->k == 1 && moe::expert_ffn_combines(bf16, vec, c->H, c->F) && aligned16(residual) &&
                      aligned16(y);
    const moe::Combine1 cmb{plan->row_token, plan->dst_row, plan->topk_gate,
                            static_cast<const uint16_t*>(residual), c->T};
    hipError_t e = moe::launch_expert_ffn(x, W1, W3, W2, h, fuse ? y : Y, plan->offsets, c->E, c->H, c->F, c->act,
                                          bf16, vec, R_max, expert_rows_cap(c, R_max),
                                          static_cast<hipStream_t>(stream), plan->row_token, c->T,
                                          fuse ? &cmb : nullptr, act);
    if (e != hipSuccess) return hip_fail(e, "expert_ffn");
    if (fuse) return MOE_OK;
  } else {
    if ((s = moe_dispatch(c, x, plan, X, stream)) != MOE_OK) return s;
    if ((s = moe_expert_ffn(c, X, plan, W1, W3, W2, Y, ws, ws_bytes, stream)) != MOE_OK) return s;
  }
  return moe_combine(c, Y, plan, residual, y, stream);
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_config* c, const void* x, const float* Wg, const float* bias, const void* W1,
                       const void* W3, const void* W2, const void* residual, void* y, const moe_plan* plan, void* X,
                       void* Y, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(c, x, Wg, bias, W1, W3, W2, residual, y, plan, X, Y, nullptr, ws, ws_bytes, stream);
}

size_t moe_saved_act_bytes(const moe_config* c) {
  if (moe_validate(c) != MOE_OK) return 0;
  return (c->act == MOE_SWIGLU ? 2 : 1) * (size_t)max_rows_of(c) * (size_t)c->F * 2;
}

moe_status moe_forward_save(const moe_config* c, const void* x, const float* Wg, const float* bias, const void* W1,
                            const void* W3, const void* W2, const void* residual, void* y, const moe_plan* plan,
                            void* X, void* Y, void* act, void* ws, size_t ws_bytes, void* stream) {
  if (!act) return MOE_ERR_INVALID_ARG;
  return forward_impl(c, x, Wg, bias, W1, W3, W2, residual, y, plan, X, Y, act, ws, ws_bytes, stream);
}

moe_status moe_shared_expert(const moe_config* c, const void* x, const void* Ws1, const void* Ws3, const void* Ws2,
                             void* Ys, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if (c->shared_F < 1 || !Ws1 || !Ws2 || (c->act == MOE_SWIGLU) != (Ws3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && (!x || !Ys)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(c);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (c->T == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  void* hs = w + L.hs;
  int32_t* off = reinterpret_cast<int32_t*>(w + L.soff);
  const bool bf16 = c->dtype == MOE_BF16;
  const bool vec = c->H % 8 == 0 && c->shared_F % 8 == 0 && aligned16(x) && aligned16(Ys) && aligned16(Ws1) &&
                   aligned16(Ws3) && aligned16(Ws2) && aligned16(hs);
  // one expert holding every token: rows [0, T)
  hipError_t e = moe::launch_dense_offsets(off, c->T, st);
  if (e == hipSuccess)
    e = moe::launch_expert_ffn(x, Ws1, Ws3, Ws2, hs, Ys, off, 1, c->H, c->shared_F, c->act, bf16, vec, c->T, c->T,
                               st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "shared_expert");
}

moe_status moe_combine_shared(const moe_config* c, const void* Y, const moe_plan* plan, const void* residual,
                              const void* Ys, void* y, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if (!plan || (c->T > 0 && (!plan->dst_row || !plan->topk_gate || !y || !Ys))) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && !Y && max_rows_of(c) > 0) return MOE_ERR_INVALID_ARG;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool vec = c->H % 8 == 0 && aligned16(Y) && aligned16(residual) && aligned16(y) && aligned16(Ys);
  hipError_t e = moe::launch_combine(Y, plan->dst_row, plan->topk_gate, residual, y, c->T, c->H, c->k,
                                     (int)max_rows_of(c), bf16, vec, static_cast<hipStream_t>(stream), Ys);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "combine_shared");
}

moe_status moe_forward_shared(const moe_config* c, const void* x, const float* Wg, const float* bias, const void* W1,
                              const void* W3, const void* W2, const void* Ws1, const void* Ws3, const void* Ws2,
                              const void* residual, void* y, const moe_plan* plan, void* X, void* Y, void* ws,
                              size_t ws_bytes, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if ((s = check_plan(c, plan)) != MOE_OK) return s;
  if (c->shared_F < 1 || !Ws1 || !Ws2 || (c->act == MOE_SWIGLU) != (Ws3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!W1 || !W2 || (c->act == MOE_SWIGLU) != (W3 != nullptr) || !Wg) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && (!x || !y || !X || !Y)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(c);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if ((s = moe_route(c, x, Wg, bias, plan, ws, ws_bytes, stream)) != MOE_OK) return s;
  const int64_t R_max = max_rows_of(c);
  void* h = static_cast<char*>(ws) + L.h;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool vec = c->H % 8 == 0 && c->F % 8 == 0 && aligned16(x) && aligned16(Y) && aligned16(W1) &&
                   aligned16(W3) && aligned16(W2) && aligned16(h);
  if (R_max > 0 && c->T > 0 && moe::expert_ffn_gathers(bf16, vec, c->H)) {
    hipError_t e = moe::launch_expert_ffn(x, W1, W3, W2, h, Y, plan->offsets, c->E, c->H, c->F, c->act, bf16, vec,
                                          R_max, expert_rows_cap(c, R_max), static_cast<hipStream_t>(stream),
                                          plan->row_token, c->T);
    if (e != hipSuccess) return hip_fail(e, "expert_ffn");
  } else {
    if ((s = moe_dispatch(c, x, plan, X, stream)) != MOE_OK) return s;
    if ((s = moe_expert_ffn(c, X, plan, W1, W3, W2, Y, ws, ws_bytes, stream)) != MOE_OK) return s;
  }
  void* Ys = static_cast<char*>(ws) + L.ys;
  if ((s = moe_shared_expert(c, x, Ws1, Ws3, Ws2, Ys, ws, ws_bytes, stream)) != MOE_OK) return s;
  return moe_combine_shared(c, Y, plan, residual, Ys, y, stream);
}

moe_status moe_backward(const moe_config* c, const void* x, const float* Wg, const void* W1, const void* W3,
                        const void* W2, const moe_plan* plan, const void* dy, const void* act, const moe_grads* g,
                        void* ws, size_t ws_bytes, void* stream) {
  moe_status s = moe_validate(c);
  if (s != MOE_OK) return s;
  if (!g || !plan || !Wg || !W1 || !W2 || (c->act == MOE_SWIGLU) != (W3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!g->dWg || !g->dW1 || !g->dW2 || (c->act == MOE_SWIGLU && !g->dW3)) return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && (!x || !dy || !g->dx || !plan->topk_idx || !plan->topk_gate || !plan->dst_row || !plan->demand ||
                   !plan->offsets || !plan->row_token || !plan->logits))
    return MOE_ERR_INVALID_ARG;
  if (!plan->offsets) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_backward_workspace_bytes(c);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  moe::BackwardArgs a{};
  a.T = c->T, a.H = c->H, a.E = c->E, a.k = c->k, a.F = c->F;
  a.act = c->act, a.gate_mode = c->gate_mode, a.score_fn = c->score_fn, a.aux_mode = c->aux_mode;
  a.R_max = max_rows_of(c);
  a.rows_cap = expert_rows_cap(c, a.R_max);
  a.bf16 = c->dtype == MOE_BF16;
  // the matrix-core path reads x, the weights and its workspace 16 bytes at a time
  a.fast = moe::backward_fast_shape(a.bf16, c->H, c->F) && aligned16(x) && aligned16(dy) && aligned16(W1) &&
           aligned16(W3) && aligned16(W2) && aligned16(ws);
  a.with_losses = plan->losses != nullptr;
  a.aux_coeff = c->aux_coeff, a.z_coeff = c->z_coeff;
  a.x = x, a.Wg = Wg, a.W1 = W1, a.W3 = W3, a.W2 = W2;
  a.topk_idx = plan->topk_idx, a.dst_row = plan->dst_row, a.offsets = plan->offsets, a.row_token = plan->row_token;
  a.demand = plan->demand, a.topk_gate = plan->topk_gate, a.logits = plan->logits;
  a.dy = dy;
  a.saved = a.fast && aligned16(act) ? act : nullptr;  // the generic path recomputes in fp32
  a.dx = g->dx, a.dWg = g->dWg, a.dbias = g->dbias, a.dW1 = g->dW1, a.dW3 = g->dW3, a.dW2 = g->dW2, a.dg = g->dg;
  a.ws = ws;
  hipError_t e = moe::launch_backward(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "backward");
}

}  // extern "C"
