// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Compute units of the current device, queried once per device.
hipError_t device_cus(int* cus);

// Raises kernel Kern's dynamic LDS limit to `bytes` (the most any of its
// launches uses) once per device; the attribute persists for the process, so
// launches carry no attribute call.
constexpr int kMaxDevices = 64;
template <auto Kern>
hipError_t lds_limit_once(int bytes) {
  static unsigned long long done = 0;  // bit d: set on device d
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (__atomic_load_n(&done, __ATOMIC_ACQUIRE) >> dev & 1ull) return hipSuccess;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               bytes)) != hipSuccess)
    return e;
  __atomic_fetch_or(&done, 1ull << dev, __ATOMIC_ACQ_REL);
  return hipSuccess;
}

// Added to a moe_gate_mode passed to the router launchers: sigmoid scores
// instead of softmax (the choices are the same; the gates differ).
constexpr int kSigmoidFlag = 16;

// dst_row value the rank step leaves for an absent choice (GShard's second
// choice not taken); the finalize steps turn it into -1.
constexpr int32_t kAbsentChoice = INT32_MIN;

// Logits in their defining order (binary64 sums over h ascending, rounded once
// to fp32: the exact values), any shape.
hipError_t launch_router_exact(const void* x, bool bf16, const float* Wg, const float* bias, float* logits, int T,
                               int H, int E, bool vec_ok, hipStream_t st);
// Split-bf16 router (bf16 x, H % 64 == 0, 16-byte aligned x): logits with a
// certified radius, choices and gates per token, exact recomputation of the
// undecided tokens.
struct SplitScratch {
  void* wp;       // [3][Ep][H] bf16 weight pieces
  double* wsq;    // [H/64][Ep] partial sums of w^2
  double* wn;     // [Ep] ||w_e||
  double* lpart;  // [HS][T][Ep] binary64 partial logit sums (E > 64; HS = split_router_hsplit)
  float* xsq;     // [HS][T] partial sums of x^2 (HS = 1 for E <= 64)
  int2* pairs;    // [T*E] candidate (token, expert)
  int4* utok;     // [T] queued tokens (token, first pair, pair count)
  int* count;     // [2] pairs, queued tokens
};
int split_router_ep(int E);
int split_router_hs(int H);
int split_router_hsplit(int T, int E, int H);
// Work the router's last kernel may take over (null pointers: not wanted):
// the ranks and block histogram of launch_router_rank, and the per-block
// partials of launch_router_losses.  *fused reports what was done (1: ranks,
// 2: loss partials); the caller launches the rest.
struct SplitEpilogue {
  int32_t* dst_rank;
  int32_t* hist;
  double* Ppart;
  double* Zpart;
  int32_t* Cpart;
  int score_fn;
};
hipError_t launch_router_split(const void* x, const float* Wg, const float* bias, float* logits, int T, int H, int E,
                               int k, int gate_mode, int32_t* topk_idx, float* topk_gate, const SplitScratch& sc,
                               const SplitEpilogue& ep, int* fused, hipStream_t st);
hipError_t launch_router_rank(const int32_t* topk_idx, int T, int E, int k, int nb, int32_t* dst_rank, int32_t* hist,
                              hipStream_t st);
// Choices, gates (binary64, rounded once), ranks and block histograms from
// exact logits; second_u (k = 2, or null): GShard's random second choice.
hipError_t launch_router_select(const float* logits, int T, int E, int k, int gate_mode, const float* second_u,
                                int nb, int32_t* topk_idx, float* topk_gate, int32_t* dst_rank, int32_t* hist,
                                hipStream_t st);
// Router training terms from the final logits and choices (see router_losses.hip).
// Workspace: Ppart [E][ceil(T/64)] f64, Zpart [ceil(T/64)] + fP [E+1] f64, Cpart [E][ceil(T/64)] int32.
// partials_done: Ppart, Zpart and Cpart are already filled (by the split router).
hipError_t launch_router_losses(const float* logits, const int32_t* topk_idx, const int32_t* demand, int T, int E,
                                int k, int score_fn, int aux_mode, double aux_coeff, double z_coeff, double* Ppart,
                                double* Zpart, int32_t* Cpart, double* losses, bool partials_done, hipStream_t st);
// "probs" drop policy: replaces launch_slot_finalize when a capacity limits.
// Workspace: lkey, lq, newslot, each [T*k].
hipError_t launch_slot_probs(const int32_t* base, int Q, int nb, int T, int E, int k, int C, const int32_t* topk_idx,
                             const float* topk_gate, const int32_t* demand, const int32_t* kept, int32_t* dst_row,
                             int32_t* row_token, int32_t* offsets, int32_t* n_dropped, int rmax, uint32_t* lkey,
                             uint32_t* lq, int32_t* newslot, hipStream_t st);
hipError_t launch_slot_scan(int32_t* hist, int Q, int E, int C, int32_t* demand, int32_t* kept, hipStream_t st);
hipError_t launch_slot_finalize(const int32_t* base, int Q, int nb, int T, int E, int k, int C,
                                const int32_t* topk_idx, const int32_t* kept, int32_t* dst_row, int32_t* row_token,
                                int32_t* offsets, int32_t* n_dropped, int rmax, hipStream_t st);
hipError_t launch_dispatch(const void* x, const int32_t* dst_row, void* X, int T, int H, int k, int rmax, bool bf16,
                           bool vec_ok, hipStream_t st);
// gather (optional, when expert_ffn_gathers): X is the token rows x [xrows][H]
// and packed row r of the first GEMM reads x[gather[r]] (the dispatch folded
// into the GEMM's loads).
bool expert_ffn_gathers(bool bf16, bool vec, int H);
// Top-1 combine folded into the second GEMM (one choice per token, so packed
// row r is the only term of token row_token[r]): y[t] = fma(gate[t], Y, res[t])
// with Y rounded to bf16 first, as the combine would read it, then rounded once;
// tokens with dst_row[t] outside [0, R_max) get y[t] = res[t] (0 without one).
struct Combine1 {
  const int32_t* row_token;  // [R_max]
  const int32_t* dst_row;    // [T]
  const float* gate;         // [T]
  const uint16_t* res;       // [T][H] bf16 or null
  int T;
};
// rows_cap: most rows any one expert can hold (the capacity, or R_max when
// nothing caps it); at most one m-tile per expert lets the weight loads stream.
// cmb (optional, bf16 tiled path only, see expert_ffn_combines): Y is then the
// layer output y [T][H] instead of the expert rows.  save (optional, tiled path
// only, see expert_ffn_saves): the first GEMM's pre-activations are also kept,
// [m1][R_max][F] bf16 (u, then v for SwiGLU).
hipError_t launch_expert_ffn(const void* X, const void* W1, const void* W3, const void* W2, void* h, void* Y,
                             const int32_t* offsets, int E, int H, int F, int act, bool bf16, bool vec,
                             int64_t R_max, int64_t rows_cap, hipStream_t st, const int32_t* gather = nullptr,
                             int xrows = 0, const Combine1* cmb = nullptr, void* save = nullptr);
// whether launch_expert_ffn can keep the pre-activations for these shapes
bool expert_ffn_saves(bool bf16, bool vec, int H, int F);
// whether launch_expert_ffn can take cmb for these shapes
bool expert_ffn_combines(bool bf16, bool vec, int H, int F);
// shared (optional): the shared expert's output [T][H], added after the routed terms.
hipError_t launch_combine(const void* Y, const int32_t* dst_row, const float* gate, const void* residual, void* y,
                          int T, int H, int k, int rmax, bool bf16, bool vec_ok, hipStream_t st,
                          const void* shared = nullptr);
// off[0] = 0, off[1] = T: the offsets of one expert holding every token.
hipError_t launch_dense_offsets(int32_t* off, int T, hipStream_t st);

// ---- backward ----------------------------------------------------------------
// Strided GEMM over groups (backward.hip): C (+)= A B with A(m, k) = A[row(m) *
// sam + k * sak], B(k, n) = B[krow(k) * sbk + n * sbn], C(m, n) = C[m * scm + n *
// scn]; group g adds a_g, b_g, c_g elements.  ragged 0: group g owns rows
// offs[g] .. offs[g+1]-1 (A's row through gather when given); ragged 1: group g
// owns reduction indices offs[g] .. offs[g+1]-1 (B's row through gather).
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  int M, N, K;
  int64_t sam, sak, sbk, sbn, scm, scn;
  int64_t a_g, b_g, c_g;
  const int32_t* offs;
  int ragged;
  const int32_t* gather;
  int accumulate;
  int ksplit;  // with no offs: group g takes the reduction indices g*ksplit .. (g+1)*ksplit-1
};

struct BackwardArgs {
  int T, H, E, k, F, act, gate_mode, score_fn, aux_mode;
  int64_t R_max, rows_cap;
  bool bf16;
  bool fast;  // matrix-core path (backward_fast_shape and 16-byte aligned buffers)
  bool with_losses;
  double aux_coeff, z_coeff;
  const void* x;
  const float* Wg;
  const void *W1, *W3, *W2;
  const int32_t *topk_idx, *dst_row, *offsets, *row_token, *demand;
  const float *topk_gate, *logits;
  const void* dy;
  const void* saved;  // the forward's pre-activations [m1][R_max][F] bf16, or null (recomputed)
  float *dx, *dWg, *dbias, *dW1, *dW3, *dW2, *dg;  // dbias, dg optional
  void* ws;
};
// C[r] = A[r] . B_e^T for the rows r of expert e (B_e = B + e*N*K, [N][K] row-major),
// bf16 in and out, fp32 accumulation: the grouped GEMM of the expert FFN with no
// epilogue (A's row through gather when given: then A has xrows rows).
hipError_t launch_grouped_gemm_bf16(const void* A, const void* B, void* C, const int32_t* offsets, int E, int N, int K,
                                    int64_t R_max, int64_t rows_cap, bool vec, hipStream_t st,
                                    const int32_t* gather = nullptr, int xrows = 0);
// The same with the second operand k-major: C[r] = A[r] . B_e for the rows r of
// expert e, B_e = B + e*k1*N ([k1][N] row-major) for k < k1 and, when B2 is given
// (K = 2 k1), B2 + e*k1*N for k >= k1.  K % 64 == 0, N % 8 == 0, k1 % 64 == 0.
hipError_t launch_grouped_gemm_bf16_kn(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets,
                                       int E, int N, int K, int k1, int64_t R_max, int64_t rows_cap, hipStream_t st,
                                       const int32_t* gather = nullptr, int xrows = 0);
// the matrix-core path of the backward: bf16, H and F multiples of 64
bool backward_fast_shape(bool bf16, int H, int F);
size_t backward_workspace_bytes(int64_t T, int H, int E, int k, int F, int64_t R_max, bool bf16, int act);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t st);

}  // namespace moe
