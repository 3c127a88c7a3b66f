// Backward of the MoE layer: the gradient of L = sum(dy * y) (+ the router
// training terms) in x, the router weights and bias, and the expert weights,
// with the routing decision held fixed.
//
// The chain is the layer walk-through of the "Expert-parallel MoE training"
// explainer run backwards, and its all-to-all paragraph gives the two
// transposes: the combine's backward has the dispatch's shape (each kept
// choice's row receives g * dy of its token) and the dispatch's backward the
// combine's (each token sums the input gradients of its kept rows).  The same
// explainer's router section: the load-balancing term reaches the router only
// through P_e (f_e comes from the top-k selection), the z-loss acts on the
// logits.  Roundings are taken as the identity; a dropped or absent choice
// gets no gradient from the output but still enters the other gates' Jacobian.
//
// The forward's hidden activations and expert outputs are recomputed from x
// and the plan (activation checkpointing): u = x W1^T (and v = x W3^T), z =
// act(u) (or silu(u) * v), Y = z W2^T; on the matrix-core path u and v may
// instead come from the forward, which can keep them (no recomputation, the
// same values).  Then
//   dY = g * dy (kept rows), dg = <Y, dy>;
//   dz = dY W2;  du = dz * act'(u)  (SwiGLU: du = dz v silu'(u), dv = dz silu(u));
//   dX = du W1 (+ dv W3);  dx = sum of the token's kept rows of dX;
//   dW2_e = dY_e^T z_e;  dW1_e = du_e^T X_e;  dW3_e = dv_e^T X_e;
//   dl = gate Jacobian^T dg (+ training terms);  dWg = x^T dl;  dbias = sum_t dl;
//   dx += dl Wg^T.
// Generic path (any dtype and shape): every product is a tiled fp32-accumulate
// GEMM with arbitrary strides, over groups of rows (one per expert: ragged M) or
// of reduction indices (ragged K), so that no operand needs a transposed copy,
// and every intermediate is fp32.  Matrix-core path (bf16, H and F multiples of
// 64): the recomputation of u and v and the two data-gradient products run on
// the expert FFN's grouped bf16 GEMM (fp32 accumulation, bf16 intermediates);
// the data-gradient products use its k-major form, which reads W2 and W1, W3
// as stored (no transposed copies).  There the first product takes the
// tokens' dy rows unscaled, dzr = dy W2, so that dg = <Y, dy> = <z, dzr> needs
// no Y, and the gate enters du, dv and (through g z) dW2 = sum dy^T (g z).  The
// weight gradients run on a grouped MFMA kernel over each expert's rows that
// reads the activations as stored as well.  The order of every sum is fixed:
// results are deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void sto(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void sto(uint16_t* p, int64_t i, float v) { p[i] = (uint16_t)f32_to_bf16_bits(v); }

// ---------------------------------------------------------------------------
// C (+)= A B per group g (blockIdx.z), fp32 accumulation in k order:
//   A(m, k) = A[row(m) * sam + k * sak],  B(k, n) = B[krow(k) * sbk + n * sbn],
//   C(m, n) = C[m * scm + n * scn]  (+ the group's offsets a_g, b_g, c_g).
// ragged 0: group g owns the rows offs[g] .. offs[g+1]-1 (global row indices for
// A and C; A's row goes through `gather` when given); ragged 1: group g owns the
// reduction indices offs[g] .. offs[g+1]-1 (B's row goes through `gather`).
// With no offs and ksplit > 0, group g owns the reduction indices g*ksplit ..
// (g+1)*ksplit-1 (a split reduction into per-group partial sums).  An empty
// reduction writes zeros (or leaves C unchanged when accumulating).
// ---------------------------------------------------------------------------
template <typename TA, typename TB>
__global__ void __launch_bounds__(256) gemm_generic_kernel(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4], Bs[BK][BN + 4];
  const int g = blockIdx.z;
  int64_t m_lo = 0, k_lo = 0;
  int m_n = p.M, k_n = p.K;
  if (p.offs) {
    const int lo = p.offs[g], hi = p.offs[g + 1];
    if (p.ragged == 0) {
      m_lo = lo;
      m_n = hi - lo;
    } else {
      k_lo = lo;
      k_n = hi - lo;
    }
  } else if (p.ksplit > 0) {
    k_lo = (int64_t)g * p.ksplit;
    k_n = (int)(p.K - k_lo < p.ksplit ? p.K - k_lo : p.ksplit);
  }
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (m0 >= m_n || n0 >= p.N) return;
  const TA* A = static_cast<const TA*>(p.A) + (int64_t)g * p.a_g;
  const TB* B = static_cast<const TB*>(p.B) + (int64_t)g * p.b_g;
  float* C = p.C + (int64_t)g * p.c_g;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < k_n; k0 += BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int mm = e % BM, kk = e / BM;
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.0f;
      if (m < m_n && k < k_n) {
        int64_t row = m_lo + m;
        if (p.ragged == 0 && p.gather) row = p.gather[row];
        v = ld(A, row * p.sam + (k_lo + k) * p.sak);
      }
      As[kk][mm] = v;
      const int nn = e % BN;
      const int n = n0 + nn;
      float w = 0.0f;
      if (n < p.N && k < k_n) {
        int64_t kr = k_lo + k;
        if (p.ragged == 1 && p.gather) kr = p.gather[kr];
        w = ld(B, kr * p.sbk + n * p.sbn);
      }
      Bs[kk][nn] = w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < m_n && n < p.N) {
        float* c = C + (m_lo + m) * p.scm + (int64_t)n * p.scn;
        *c = p.accumulate ? *c + acc[i][j] : acc[i][j];
      }
    }
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ float gelu_f(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

// d/du of the exact-erf GELU: Phi(u) + u phi(u)
__device__ __forceinline__ float gelu_grad_f(float u) {
  return 0.5f * (1.0f + erff(u * 0.70710678118654752f)) + u * __expf(-0.5f * u * u) * 0.39894228040143268f;
}

// z = act(u), or silu(u) * v; rows of the kept range only (R read on the device)
template <typename T>
__global__ void act_fwd_kernel(const T* __restrict__ u, const T* __restrict__ v, T* __restrict__ z,
                               const int32_t* __restrict__ offsets, int E, int F, int act) {
  const int64_t n = (int64_t)offsets[E] * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float a = ld(u, i);
    sto(z, i, act == 2 ? silu_f(a) * ld(v, i) : (act == 0 ? (a > 0.0f ? a : 0.0f) : gelu_f(a)));
  }
}

// du = dz * act'(u); SwiGLU: du = dz * v * silu'(u), dv = dz * silu(u).  du and
// dv rows have stride ldd (du, dv side by side in one [R][2F] buffer on the
// matrix-core path).
template <typename T>
__global__ void act_bwd_kernel(const T* __restrict__ dz, const T* __restrict__ u, const T* __restrict__ v,
                               T* __restrict__ du, T* __restrict__ dv, const int32_t* __restrict__ offsets, int E,
                               int F, int64_t ldd, int act) {
  const int64_t n = (int64_t)offsets[E] * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / F, c = i - r * F, o = r * ldd + c;
    const float a = ld(u, i), d = ld(dz, i);
    if (act == 2) {
      const float s = 1.0f / (1.0f + __expf(-a));
      sto(du, o, d * ld(v, i) * (s * (1.0f + a * (1.0f - s))));
      sto(dv, o, d * (a * s));
    } else {
      sto(du, o, d * (act == 0 ? (a > 0.0f ? 1.0f : 0.0f) : gelu_grad_f(a)));
    }
  }
}

// Block sum of one float per thread (256 threads), in a fixed order.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Combine backward, one block per token: dY[dst_row] = g * dy[t] for each kept
// choice, dg[t][r] = <Y[dst_row], dy[t]> (0 for a dropped or absent choice).
template <typename TD, typename TY>
__global__ void __launch_bounds__(256) combine_bwd_kernel(const TD* __restrict__ dy, const TY* __restrict__ Y,
                                                          const float* __restrict__ gate,
                                                          const int32_t* __restrict__ dst, TY* __restrict__ dY,
                                                          float* __restrict__ dg, int H, int k) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  for (int r = 0; r < k; ++r) {
    const int row = dst[(int64_t)t * k + r];
    if (row < 0) {
      if (threadIdx.x == 0) dg[(int64_t)t * k + r] = 0.0f;
      continue;
    }
    const float g = gate[(int64_t)t * k + r];
    float part = 0.0f;
    for (int h = threadIdx.x; h < H; h += 256) {
      const float d = ld(dy, (int64_t)t * H + h);
      part = __builtin_fmaf(ld(Y, (int64_t)row * H + h), d, part);
      sto(dY, (int64_t)row * H + h, g * d);
    }
    const float s = block_sum256(part, red);
    if (threadIdx.x == 0) dg[(int64_t)t * k + r] = s;
  }
}

// Dispatch backward: dx[t] = sum over r ascending of the kept rows of dX.
template <typename T>
__global__ void __launch_bounds__(256) gather_sum_kernel(const T* __restrict__ dX, const int32_t* __restrict__ dst,
                                                         float* __restrict__ dx, int H, int k) {
  const int t = blockIdx.x;
  for (int h = threadIdx.x; h < H; h += 256) {
    float acc = 0.0f;
    for (int r = 0; r < k; ++r) {
      const int row = dst[(int64_t)t * k + r];
      if (row >= 0) acc += ld(dX, (int64_t)row * H + h);
    }
    dx[(int64_t)t * H + h] = acc;
  }
}

// Matrix-core path, one block per token, for each kept choice (row = its packed
// row, g = its gate), from dzr = dy[t] W2_e (the rows of the dz product taken on
// the token's unscaled dy) and the pre-activations u (and v):
//   z = act(u) (SwiGLU: silu(u) v), in fp32;
//   dg = <Y[row], dy[t]> = <z, dzr>  (Y = z W2_e^T, so no Y is formed);
//   du = g dzr act'(u)  (SwiGLU: du = g dzr v silu'(u), dv = g dzr silu(u));
//   zg[row] = g z, rounded to bf16 (the operand of dW2 = sum dy^T (g z)).
// Eight features per thread and step: 16-byte loads and stores (F % 8 == 0,
// every row 16-byte aligned).  A dropped or absent choice gets dg = 0.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ void __launch_bounds__(256) token_bwd_kernel(const uint16_t* __restrict__ dzr,
                                                        const uint16_t* __restrict__ u,
                                                        const uint16_t* __restrict__ v, uint16_t* __restrict__ zg,
                                                        const float* __restrict__ gate, const int32_t* __restrict__ dst,
                                                        uint16_t* __restrict__ du, uint16_t* __restrict__ dv,
                                                        int64_t ldd, float* __restrict__ dg, int F, int k, int act) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  for (int c = 0; c < k; ++c) {
    const int row = dst[(int64_t)t * k + c];
    if (row < 0) {
      if (threadIdx.x == 0) dg[(int64_t)t * k + c] = 0.0f;
      continue;
    }
    const float g = gate[(int64_t)t * k + c];
    const int64_t rb = (int64_t)row * F, ob = (int64_t)row * ldd;
    float part = 0.0f;
    for (int f = threadIdx.x * 8; f < F; f += 256 * 8) {
      const u32x4_t dq = *reinterpret_cast<const u32x4_t*>(dzr + rb + f);
      const u32x4_t uq = *reinterpret_cast<const u32x4_t*>(u + rb + f);
      const u32x4_t vq = act == 2 ? *reinterpret_cast<const u32x4_t*>(v + rb + f) : u32x4_t{0, 0, 0, 0};
      u32x4_t zo, duo, dvo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float zz[2], gu[2], gv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float d = h ? bf16_hi(dq[j]) : bf16_lo(dq[j]), a = h ? bf16_hi(uq[j]) : bf16_lo(uq[j]);
          if (act == 2) {
            const float b = h ? bf16_hi(vq[j]) : bf16_lo(vq[j]);
            const float sg = 1.0f / (1.0f + __expf(-a));
            zz[h] = a * sg * b;
            gu[h] = g * d * b * (sg * (1.0f + a * (1.0f - sg)));
            gv[h] = g * d * (a * sg);
          } else {
            zz[h] = act == 0 ? (a > 0.0f ? a : 0.0f) : gelu_f(a);
            gu[h] = g * d * (act == 0 ? (a > 0.0f ? 1.0f : 0.0f) : gelu_grad_f(a));
            gv[h] = 0.0f;
          }
          part = __builtin_fmaf(zz[h], d, part);
        }
        zo[j] = pack_bf16x2(g * zz[0], g * zz[1]);
        duo[j] = pack_bf16x2(gu[0], gu[1]);
        dvo[j] = pack_bf16x2(gv[0], gv[1]);
      }
      *reinterpret_cast<u32x4_t*>(zg + rb + f) = zo;
      *reinterpret_cast<u32x4_t*>(du + ob + f) = duo;
      if (act == 2) *reinterpret_cast<u32x4_t*>(dv + ob + f) = dvo;
    }
    const float sum = block_sum256(part, red);
    if (threadIdx.x == 0) dg[(int64_t)t * k + c] = sum;
  }
}

// Dispatch backward on the matrix-core path: dx[t] = sum over r ascending of the
// token's kept rows of dX (bf16), eight features per thread (16-byte loads,
// 32-byte stores; H % 8 == 0, dx 16-byte aligned); the same sums as
// gather_sum_kernel.
__global__ void __launch_bounds__(256) gather_sum_vec_kernel(const uint16_t* __restrict__ dX,
                                                             const int32_t* __restrict__ dst, float* __restrict__ dx,
                                                             int H, int k) {
  const int t = blockIdx.x;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int r = 0; r < k; ++r) {
      const int row = dst[(int64_t)t * k + r];
      if (row < 0) continue;
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(dX + (int64_t)row * H + h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf16_lo(q[j]);
        acc[2 * j + 1] += bf16_hi(q[j]);
      }
    }
    float* o = dx + (int64_t)t * H + h;
    *reinterpret_cast<f32x4_t*>(o) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(o + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
}

// f_e of the load-balancing term: demand / (T k) (every choice) or the first
// choices / T; one block.
__global__ void __launch_bounds__(1024) aux_f_kernel(const int32_t* __restrict__ demand,
                                                     const int32_t* __restrict__ topk_idx, int T, int E, int k,
                                                     int aux_mode, double* __restrict__ f) {
  __shared__ int cnt[1024];
  for (int e = threadIdx.x; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  if (aux_mode == 1)
    for (int t = threadIdx.x; t < T; t += 1024) {
      const int e = topk_idx[(int64_t)t * k];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024)
    f[e] = aux_mode == 1 ? (double)cnt[e] / (double)T : (double)demand[e] / ((double)T * (double)k);
}

// dL/dlogits of one token (one wave), binary64 sums: the gate Jacobian applied
// to dg, plus the load-balancing term through P_e and the z-loss when asked.
constexpr int kMaxJE = 16;  // E <= 1024 = 64 lanes x 16
__global__ void __launch_bounds__(64) gate_bwd_kernel(const float* __restrict__ logits, const int32_t* __restrict__ idx,
                                                      const float* __restrict__ dg, const double* __restrict__ f,
                                                      float* __restrict__ dl, int T, int E, int k, int gate_mode,
                                                      int score_fn, double aux_coeff, double z_coeff) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const float* l = logits + (int64_t)t * E;
  const int je = (E + 63) / 64;
  double lv[kMaxJE], acc[kMaxJE];
  double m = -INFINITY;
  for (int j = 0; j < je; ++j) {
    const int e = lane + 64 * j;
    lv[j] = e < E ? (double)l[e] : -INFINITY;
    acc[j] = 0.0;
    m = lv[j] > m ? lv[j] : m;
  }
  for (int d = 32; d > 0; d >>= 1) {
    const double o = __shfl_xor(m, d, 64);
    m = o > m ? o : m;
  }
  double den = 0.0;
  for (int j = 0; j < je; ++j) den += lane + 64 * j < E ? exp(lv[j] - m) : 0.0;
  for (int d = 32; d > 0; d >>= 1) den += __shfl_xor(den, d, 64);
  auto p_of = [&](double x) { return exp(x - m) / den; };
  // the chosen experts' logits and upstream gradients (every lane holds all k)
  double lc[16], dgc[16];
  int ic[16];
  for (int r = 0; r < k; ++r) {
    ic[r] = idx[(int64_t)t * k + r];
    lc[r] = (double)l[ic[r]];
    dgc[r] = (double)dg[(int64_t)t * k + r];
  }
  auto add_at = [&](int e, double v) {
    if ((e & 63) == lane) acc[e >> 6] += v;
  };
  if (score_fn == 1 && gate_mode != 2) {  // sigmoid scores
    double s[16], S = 0.0, sgd = 0.0;
    for (int r = 0; r < k; ++r) {
      s[r] = 1.0 / (1.0 + exp(-lc[r]));
      S += s[r];
    }
    for (int r = 0; r < k; ++r) sgd += s[r] / S * dgc[r];
    for (int r = 0; r < k; ++r) {
      const double dsc = gate_mode == 0 ? dgc[r] : (dgc[r] - sgd) / S;
      add_at(ic[r], dsc * s[r] * (1.0 - s[r]));
    }
  } else if (gate_mode == 0) {  // softmax over all E, the chosen p
    double sgd = 0.0;
    for (int r = 0; r < k; ++r) sgd += p_of(lc[r]) * dgc[r];
    for (int j = 0; j < je; ++j)
      if (lane + 64 * j < E) acc[j] -= p_of(lv[j]) * sgd;
    for (int r = 0; r < k; ++r) add_at(ic[r], p_of(lc[r]) * dgc[r]);
  } else {  // renormalised or softmax over the chosen: softmax over the chosen logits
    double mc = lc[0], dc = 0.0, sgd = 0.0;
    for (int r = 1; r < k; ++r) mc = lc[r] > mc ? lc[r] : mc;
    for (int r = 0; r < k; ++r) dc += exp(lc[r] - mc);
    for (int r = 0; r < k; ++r) sgd += exp(lc[r] - mc) / dc * dgc[r];
    for (int r = 0; r < k; ++r) add_at(ic[r], exp(lc[r] - mc) / dc * (dgc[r] - sgd));
  }
  if (f && aux_coeff != 0.0) {
    const double scale = aux_coeff * (double)E / (double)T;  // dL/dq_e(t) = scale * f_e
    if (score_fn == 1) {
      double S = 0.0, cs = 0.0;
      for (int j = 0; j < je; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
          const double s = 1.0 / (1.0 + exp(-lv[j]));
          S += s;
          cs += scale * f[e] * s;
        }
      }
      for (int d = 32; d > 0; d >>= 1) {
        S += __shfl_xor(S, d, 64);
        cs += __shfl_xor(cs, d, 64);
      }
      for (int j = 0; j < je; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
          const double s = 1.0 / (1.0 + exp(-lv[j]));
          acc[j] += s * (1.0 - s) / S * (scale * f[e] - cs / S);
        }
      }
    } else {
      double cp = 0.0;
      for (int j = 0; j < je; ++j) {
        const int e = lane + 64 * j;
        if (e < E) cp += scale * f[e] * p_of(lv[j]);
      }
      for (int d = 32; d > 0; d >>= 1) cp += __shfl_xor(cp, d, 64);
      for (int j = 0; j < je; ++j) {
        const int e = lane + 64 * j;
        if (e < E) acc[j] += p_of(lv[j]) * (scale * f[e] - cp);
      }
    }
  }
  if (z_coeff != 0.0) {
    const double lse = m + log(den);
    for (int j = 0; j < je; ++j)
      if (lane + 64 * j < E) acc[j] += z_coeff * 2.0 / (double)T * lse * p_of(lv[j]);
  }
  for (int j = 0; j < je; ++j) {
    const int e = lane + 64 * j;
    if (e < E) dl[(int64_t)t * E + e] = (float)acc[j];
  }
}

// dbias[e] = sum over t of dl[t][e] in two passes of fixed order.  Pass one:
// block (x, c) sums rows c * rows .. of 64 experts in four token phases into
// part[c][e]; pass two adds the chunks, in four phases per expert.
__global__ void __launch_bounds__(256) col_sum_part_kernel(const float* __restrict__ dl, float* __restrict__ part,
                                                          int T, int E, int rows) {
  __shared__ float red[4][64];
  const int el = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el, c = blockIdx.y;
  const int t1 = min(T, (c + 1) * rows);
  float s = 0.0f;
  if (e < E)
    for (int t = c * rows + ph; t < t1; t += 4) s += dl[(int64_t)t * E + e];
  red[ph][el] = s;
  __syncthreads();
  if (ph == 0 && e < E) part[(int64_t)c * E + e] = (red[0][el] + red[1][el]) + (red[2][el] + red[3][el]);
}

// dx[t][h] += sum over e ascending of dl[t][e] Wg[h][e]: fp32 fma from zero, then
// one add into dx (the arithmetic of gemm_generic_kernel, so the same bits).
// 128 x 128 tiles of (t, h), 256 threads of 8 x 8 outputs, 16-wide e stages
// stored e-major in LDS so that a thread's 8 t and 8 h values of one e are two
// 32-byte reads.  E % 4 == 0, H % 4 == 0, dl, Wg and dx 16-byte aligned.
__global__ void __launch_bounds__(256) router_dx_kernel(const float* __restrict__ dl, const float* __restrict__ Wg,
                                                        float* __restrict__ dx, int T, int H, int E) {
  constexpr int BT = 128, BH = 128, BK = 16;
  __shared__ __align__(16) float As[BK][BT + 4], Bs[BK][BH + 4];
  const int t0 = blockIdx.y * BT, h0 = blockIdx.x * BH, tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // the thread's h block tx * 8 and t block ty * 8
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  for (int e0 = 0; e0 < E; e0 += BK) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // 128 rows x 4 groups of 4 e, per operand
      const int p = tid + 256 * q, row = p >> 2, c4 = (p & 3) * 4, e = e0 + c4;
      const int t = t0 + row, h = h0 + row;
      const bool ein = e < E;  // E % 4 == 0: a group is whole or past the end
      const f32x4_t a = (t < T && ein) ? *reinterpret_cast<const f32x4_t*>(dl + (int64_t)t * E + e)
                                       : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4_t b = (h < H && ein) ? *reinterpret_cast<const f32x4_t*>(Wg + (int64_t)h * E + e)
                                       : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        As[c4 + j][row] = a[j];
        Bs[c4 + j][row] = b[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(&As[kk][ty * 8]);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(&As[kk][ty * 8 + 4]);
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(&Bs[kk][tx * 8]);
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(&Bs[kk][tx * 8 + 4]);
      const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + ty * 8 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j4 = 0; j4 < 8; j4 += 4) {
      const int h = h0 + tx * 8 + j4;
      if (h >= H) continue;  // H % 4 == 0: a group of 4 is whole or past the end
      f32x4_t* o = reinterpret_cast<f32x4_t*>(dx + (int64_t)t * H + h);
      f32x4_t c = *o;
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = c[j] + acc[i][j4 + j];
      *o = c;
    }
  }
}

// out[i] = sum over g < parts of part[g * n + i], in g order.
__global__ void __launch_bounds__(256) sum_parts_kernel(const float* __restrict__ part, int parts, int64_t n,
                                                       float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int g = 0; g < parts; ++g) s += part[(int64_t)g * n + i];
    out[i] = s;
  }
}

__global__ void __launch_bounds__(256) col_sum_final_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                           int chunks, int E) {
  __shared__ float red[4][64];
  const int el = threadIdx.x & 63, ph = threadIdx.x >> 6, e = blockIdx.x * 64 + el;
  float s = 0.0f;
  if (e < E)
    for (int c = ph; c < chunks; c += 4) s += part[(int64_t)c * E + e];
  red[ph][el] = s;
  __syncthreads();
  if (ph == 0 && e < E) out[e] = (red[0][el] + red[1][el]) + (red[2][el] + red[3][el]);
}

// ---------------------------------------------------------------------------
// Weight gradients on the matrix cores: dW_e = A_e^T B_e over the expert's
// packed rows, both operands read as stored (rows of features, the k-major
// form of the expert GEMMs' data-gradient products), so that no activation is
// transposed or padded.
// ---------------------------------------------------------------------------

// Zeros that the weight-gradient loads read for rows past an expert's end (a
// direct-to-LDS load cannot substitute a value); never written.
__device__ __align__(16) uint16_t g_wgrad_zero[8];

// C_e[m][n] = sum over the packed rows r of expert e, in row order, of
// A(r)[m] B(r)[n] (fp32 accumulation, fp32 out, C_e = C + e * M * N), where A(r)
// is row ga[r] of A (row r when ga is null; lda elements per row), likewise B;
// the expert's rows are offsets[e] .. offsets[e+1]-1, clamped to rmax.
// 128 x 128 tiles, 4 waves as 2 x 2, each 2 x 2 fragments of
// v_mfma_f32_32x32x16_bf16.  A stage holds 32 rows of each operand's 128
// features of the tile (256 B per row), filled by direct-to-LDS loads: slot ch
// of stage row kr holds chunk ch ^ 4 (kr & 3), and a fragment (feature l % 32,
// rows 8 (l / 32) .. +7 of lane l) is two transposing LDS reads, as in the
// k-major grouped GEMM (the 4 rows x 4 chunks of a 32-lane read phase fall in
// 16 distinct bank groups).  The gathered operand's source rows are fetched one
// stage ahead.  The kernel is bound by its fp32 stores (the reduction per
// expert is short): each wave stages its 64 x 64 block through LDS, 32 rows at
// a time ([32][68] fp32, the padding puts rows 4 apart in different banks), and
// writes whole 256-byte row pieces with 16-byte non-temporal stores (the
// gradient is not read again here).  Features past M or N read the last whole
// chunk and are not stored; M, N multiples of 8, N % 4 == 0.
__global__ void __launch_bounds__(256) wgrad_kn_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                       const int32_t* __restrict__ ga, const uint16_t* __restrict__ B,
                                                       int64_t ldb, const int32_t* __restrict__ gb,
                                                       float* __restrict__ C, const int32_t* __restrict__ offsets,
                                                       int64_t rmax, int xrows, int M, int N) {
  constexpr int BM = 128, BN = 128, BK = 32, RS = BK * BM, STAGE = 2 * RS;  // operand A rows, then B rows
  constexpr int PAD = 68, EPI = 4 * 32 * PAD * 2;  // epilogue staging, in bf16 units
  static_assert(BM == BN && BM / 8 == 16, "16 chunks per stage row");
  __shared__ __align__(16) uint16_t smem[2 * STAGE > EPI ? 2 * STAGE : EPI];
  const int e = blockIdx.z, m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int64_t r1 = min((int64_t)offsets[e + 1], rmax), r0 = min((int64_t)offsets[e], r1);
  const int nk = (int)((r1 - r0 + BK - 1) / BK);
  // this thread's 4 pieces per stage: piece p = q * 256 + tid of operand q / 2,
  // stage row kr0 + 16 (q % 2), slot tid % 16 (LDS element p * 8)
  const int kr0 = tid >> 4, ch = (tid & 15) ^ (4 * (kr0 & 3));
  const int fa = min(m0 + ch * 8, M - 8), fb = min(n0 + ch * 8, N - 8);
  int src[2][2];  // source rows of the next stage to load, [operand][half]; -1: past the expert's end
  auto fetch_rows = [&](int j) {
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t r = r0 + (int64_t)j * BK + kr0 + 16 * h;
        const int32_t* g = op ? gb : ga;
        int s = -1;
        if (r < r1) {
          s = g ? g[r] : (int)r;
          if (g) s = s < 0 ? 0 : (s < xrows ? s : xrows - 1);
        }
        src[op][h] = s;
      }
  };
  auto issue = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int op = q >> 1, s = src[op][q & 1];
      const uint16_t* p = s < 0 ? g_wgrad_zero : (op ? B + (int64_t)s * ldb + fb : A + (int64_t)s * lda + fa);
      __builtin_amdgcn_global_load_lds(p, smem + buf * STAGE + (q * 4 + w) * 512, 16, 0, 0);
    }
  };
  auto frag = [&](const uint16_t* region, int f0, int kk) {
    const int f = f0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int kr = kk * 16 + 8 * (lane >> 5) + ((lane >> 2) & 3);
    const uint16_t* p = region + kr * BM + (((f >> 3) ^ (4 * (kr & 3))) << 3) + (f & 7);
    const s16x4_t lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * BM);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  if (nk > 0) {
    fetch_rows(0);
    issue(0);
    if (nk > 1) fetch_rows(1);
  }
  for (int j = 0; j < nk; ++j) {
    wait_vmcnt<0>();
    __syncthreads();  // stage j is in LDS, every wave is done with stage j - 1, the rows of stage j + 1 are in
    if (j + 1 < nk) {
      issue((j + 1) & 1);
      if (j + 2 < nk) fetch_rows(j + 2);
    }
    const uint16_t* st = smem + (j & 1) * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = frag(st, wm * 64 + i * 32, kk);
        b[i] = frag(st + RS, wn * 64 + i * 32, kk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[jj], acc[i][jj], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done reading the stages: their space stages the stores
  // accumulator element 4g + q of lane l: row 8g + 4(l / 32) + q of the A fragment, column l % 32
  float* sw = reinterpret_cast<float*>(smem) + w * 32 * PAD;
  float* Ce = C + (int64_t)e * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sw[(8 * g + 4 * (lane >> 5) + q) * PAD + jj * 32 + (lane & 31)] = acc[i][jj][4 * g + q];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < 8; ++s) {  // 4 rows x 64 columns per store instruction
      const int r = s * 4 + (lane >> 4), c = (lane & 15) * 4;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(sw + r * PAD + c);
      const int m = m0 + wm * 64 + i * 32 + r, n = n0 + wn * 64 + c;
      if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(Ce + (int64_t)m * N + n));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next half overwrites
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

int grid_1d(int64_t n, int bs) {
  const int64_t b = (n + bs - 1) / bs;
  return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

template <typename TA, typename TB>
hipError_t launch_gemm_generic(const GemmArgs& p, int groups, int max_m, hipStream_t st) {
  if (groups <= 0 || max_m <= 0 || p.N <= 0) return hipSuccess;
  dim3 grid((p.N + 63) / 64, (max_m + 63) / 64, groups);
  gemm_generic_kernel<TA, TB><<<grid, dim3(256), 0, st>>>(p);
  return hipGetLastError();
}

static hipError_t gemm(bool a_bf16, bool b_bf16, const GemmArgs& p, int groups, int max_m, hipStream_t st) {
  if (a_bf16 && b_bf16) return launch_gemm_generic<uint16_t, uint16_t>(p, groups, max_m, st);
  if (a_bf16) return launch_gemm_generic<uint16_t, float>(p, groups, max_m, st);
  if (b_bf16) return launch_gemm_generic<float, uint16_t>(p, groups, max_m, st);
  return launch_gemm_generic<float, float>(p, groups, max_m, st);
}

namespace {

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace of the two paths.  Generic: u, v, z, dz, du, dv [R][F] and Y, dY,
// dX [R][H], fp32.  Matrix-core: u, v, z, dz [R][F], [du | dv] [R][2F] and dX
// [R][H] in bf16 (no Y, dY).  Both end with dl [T][E] fp32, f [E] binary64, dg
// [T][k] fp32, the bias gradient's chunk sums [64][E] fp32 and the router
// weight gradient's partial sums [router_splits][H][E] fp32.

// Chunks of tokens the router weight gradient's reduction is split into: the
// grid of its output tiles times the chunks should fill the GPU (2048
// workgroups), each chunk keeping at least 256 tokens, at most 64 chunks.
int router_splits(int64_t T, int H, int E) {
  const int64_t tiles = (int64_t)((E + 63) / 64) * ((H + 63) / 64);
  int S = 1;
  while (S < 64 && tiles * S < 2048 && T / (2 * S) >= 256) S *= 2;
  return S;
}
struct BwdLayout {
  size_t u, v, z, dz, du, Y, dY, dX, dl, f, dg, cs, rp, total;
};

BwdLayout bwd_layout(int64_t T, int H, int E, int k, int F, int64_t R_max, bool fast) {
  BwdLayout L{};
  const size_t eb = fast ? 2 : 4;
  const size_t RF = al256(eb * (size_t)R_max * (size_t)F), RH = al256(eb * (size_t)R_max * (size_t)H);
  size_t o = 0;
  L.u = o, o += RF;
  L.v = o, o += RF;
  L.z = o, o += RF;
  L.dz = o, o += RF;
  L.du = o, o += 2 * RF;  // generic: du then dv; matrix-core: [R][2F] rows
  L.Y = o, o += fast ? 0 : RH;
  L.dY = o, o += fast ? 0 : RH;
  L.dX = o, o += RH;
  L.dl = o, o += al256(sizeof(float) * (size_t)T * (size_t)E);
  L.f = o, o += al256(sizeof(double) * (size_t)E);
  L.dg = o, o += al256(sizeof(float) * (size_t)T * (size_t)k);
  L.cs = o, o += al256(sizeof(float) * 64 * (size_t)E);
  const int S = router_splits(T, H, E);
  L.rp = o, o += S > 1 ? al256(sizeof(float) * S * (size_t)H * (size_t)E) : 0;
  L.total = o + 256;
  return L;
}

// Router part, common to both paths: dl from dg (+ training terms), dWg, dbias,
// dx += dl Wg^T.
hipError_t router_backward(const BackwardArgs& a, const BwdLayout& L, const float* dg, hipStream_t st) {
  char* w = static_cast<char*>(a.ws);
  float* dl = reinterpret_cast<float*>(w + L.dl);
  double* f = reinterpret_cast<double*>(w + L.f);
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  hipError_t err;
  const bool aux = a.with_losses && a.aux_coeff != 0.0;
  const bool zl = a.with_losses && a.z_coeff != 0.0;
  if (aux) {
    aux_f_kernel<<<1, 1024, 0, st>>>(a.demand, a.topk_idx, T, E, k, a.aux_mode, f);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  gate_bwd_kernel<<<T, 64, 0, st>>>(a.logits, a.topk_idx, dg, aux ? f : nullptr, dl, T, E, k, a.gate_mode, a.score_fn,
                                    aux ? a.aux_coeff : 0.0, zl ? a.z_coeff : 0.0);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  GemmArgs g{};  // dWg[h][e] = sum_t x[t][h] dl[t][e]
  g.A = a.x, g.sam = 1, g.sak = H;
  g.B = dl, g.sbk = E, g.sbn = 1;
  g.C = a.dWg, g.scm = E, g.scn = 1;
  g.M = H, g.N = E, g.K = T;
  // a long reduction over few output tiles: split it into S chunks of tokens
  // (partial sums, then summed in chunk order) so that the grid fills the GPU
  const int S = router_splits(T, H, E);
  if (S > 1) {
    float* part = reinterpret_cast<float*>(w + L.rp);
    g.C = part, g.c_g = (int64_t)H * E;
    g.ksplit = (T + S - 1) / S;
    if ((err = gemm(a.bf16, false, g, S, H, st)) != hipSuccess) return err;
    sum_parts_kernel<<<grid_1d((int64_t)H * E, 256), 256, 0, st>>>(part, S, (int64_t)H * E, a.dWg);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else if ((err = gemm(a.bf16, false, g, 1, H, st)) != hipSuccess) {
    return err;
  }
  if (a.dbias) {
    float* part = reinterpret_cast<float*>(w + L.cs);
    const int rows = T > 64 * 64 ? (T + 63) / 64 : 64, chunks = (T + rows - 1) / rows;  // chunks <= 64
    col_sum_part_kernel<<<dim3((E + 63) / 64, chunks), 256, 0, st>>>(dl, part, T, E, rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    col_sum_final_kernel<<<(E + 63) / 64, 256, 0, st>>>(part, a.dbias, chunks, E);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const bool a16 = ((reinterpret_cast<uintptr_t>(a.Wg) | reinterpret_cast<uintptr_t>(a.dx)) & 15) == 0;
  if (E % 4 == 0 && H % 4 == 0 && a16) {  // dl is 256-byte aligned in the workspace
    router_dx_kernel<<<dim3((H + 127) / 128, (T + 127) / 128), 256, 0, st>>>(dl, a.Wg, a.dx, T, H, E);
    return hipGetLastError();
  }
  GemmArgs x{};  // dx[t][h] += sum_e dl[t][e] Wg[h][e]
  x.A = dl, x.sam = E, x.sak = 1;
  x.B = a.Wg, x.sbk = 1, x.sbn = E;
  x.C = a.dx, x.scm = H, x.scn = 1;
  x.M = T, x.N = H, x.K = E;
  x.accumulate = 1;
  return gemm(false, false, x, 1, T, st);
}

// Weight gradients on the strided GEMM, ragged over each expert's rows:
// dW2[e][h][f] = sum_r dY[r][h] z[r][f]; dW1[e][f][h] = sum_r du[r][f] x[row_token[r]][h]
// (dW3 with dv).  du / dv rows have stride ldd.
template <typename T>
hipError_t weight_grads(const BackwardArgs& a, const T* dY, const T* z, const T* du, const T* dv, int64_t ldd,
                        hipStream_t st) {
  const int H = a.H, E = a.E, F = a.F;
  constexpr bool kb = sizeof(T) == 2;
  hipError_t err;
  GemmArgs g{};
  g.M = H, g.N = F;
  g.offs = a.offsets, g.ragged = 1;
  g.A = dY, g.sam = 1, g.sak = H;
  g.B = z, g.sbk = F, g.sbn = 1;
  g.C = a.dW2, g.scm = F, g.scn = 1, g.c_g = (int64_t)H * F;
  if ((err = gemm(kb, kb, g, E, H, st)) != hipSuccess) return err;
  GemmArgs w{};
  w.M = F, w.N = H;
  w.offs = a.offsets, w.ragged = 1, w.gather = a.row_token;
  w.A = du, w.sam = 1, w.sak = ldd;
  w.B = a.x, w.sbk = H, w.sbn = 1;
  w.C = a.dW1, w.scm = H, w.scn = 1, w.c_g = (int64_t)F * H;
  if ((err = gemm(kb, a.bf16, w, E, F, st)) != hipSuccess) return err;
  if (a.act == 2) {
    w.A = dv;
    w.C = a.dW3;
    if ((err = gemm(kb, a.bf16, w, E, F, st)) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

bool backward_fast_shape(bool bf16, int H, int F) { return bf16 && H % 64 == 0 && F % 64 == 0; }

size_t backward_workspace_bytes(int64_t T, int H, int E, int k, int F, int64_t R_max, bool bf16, int act) {
  const size_t g = bwd_layout(T, H, E, k, F, R_max, false).total;
  if (!backward_fast_shape(bf16, H, F)) return g;
  const size_t f = bwd_layout(T, H, E, k, F, R_max, true).total;
  return f > g ? f : g;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  const int T = a.T, H = a.H, E = a.E, k = a.k, F = a.F;
  const int64_t R_max = a.R_max;
  const bool bf = a.bf16, gated = a.act == 2;
  hipError_t err = hipSuccess;
#define MOE_BW(call)                              \
  do {                                            \
    if ((err = (call)) != hipSuccess) return err; \
  } while (0)
  if (T == 0) {  // no tokens: every gradient is zero
    auto zero = [&](float* q, int64_t n) {
      if (q && n > 0) zero_f32_kernel<<<grid_1d(n, 256), 256, 0, st>>>(q, n);
      return hipGetLastError();
    };
    MOE_BW(zero(a.dWg, (int64_t)H * E));
    MOE_BW(zero(a.dbias, E));
    MOE_BW(zero(a.dW1, (int64_t)E * F * H));
    if (gated) MOE_BW(zero(a.dW3, (int64_t)E * F * H));
    MOE_BW(zero(a.dW2, (int64_t)E * H * F));
    return hipSuccess;
  }
  const BwdLayout L = bwd_layout(T, H, E, k, F, R_max, a.fast);
  char* w = static_cast<char*>(a.ws);
  float* dgw = reinterpret_cast<float*>(w + L.dg);
  float* dg = a.dg ? a.dg : dgw;
  const int mr = (int)(R_max < INT32_MAX ? R_max : INT32_MAX);  // rows bound of the ragged-M grids

  if (a.fast) {
    uint16_t* u_ws = reinterpret_cast<uint16_t*>(w + L.u);  // recomputed u, v
    uint16_t* v_ws = reinterpret_cast<uint16_t*>(w + L.v);
    // u and v as read below: the recomputed ones, or those the forward kept
    const uint16_t* u = a.saved ? static_cast<const uint16_t*>(a.saved) : u_ws;
    const uint16_t* v = a.saved ? u + (size_t)R_max * F : v_ws;
    uint16_t* z = reinterpret_cast<uint16_t*>(w + L.z);
    uint16_t* dz = reinterpret_cast<uint16_t*>(w + L.dz);
    uint16_t* dcat = reinterpret_cast<uint16_t*>(w + L.du);  // [R][2F]: du | dv (or [R][F])
    uint16_t* dX = reinterpret_cast<uint16_t*>(w + L.dX);
    const int KC = gated ? 2 * F : F;  // reduction length of dX = [du | dv] [W1; W3]
    const int64_t rc = a.rows_cap;
    if (R_max > 0) {
      // recompute: u = x[row_token] W1^T, v = x[row_token] W3^T (unless kept; z is
      // formed from them in token_bwd_kernel)
      if (!a.saved) {
        MOE_BW(launch_grouped_gemm_bf16(a.x, a.W1, u_ws, a.offsets, E, F, H, R_max, rc, true, st, a.row_token, T));
        if (gated)
          MOE_BW(launch_grouped_gemm_bf16(a.x, a.W3, v_ws, a.offsets, E, F, H, R_max, rc, true, st, a.row_token, T));
      }
    }
    if (R_max > 0) {
      // dzr = dy[row_token] W2 per kept row (the gate is applied in token_bwd_kernel);
      // W2_e [H][F] is the k-major second operand as stored
      MOE_BW(launch_grouped_gemm_bf16_kn(a.dy, a.W2, nullptr, dz, a.offsets, E, F, H, H, R_max, rc, st, a.row_token,
                                         T));
    }
    token_bwd_kernel<<<T, 256, 0, st>>>(dz, u, v, z, a.topk_gate, a.dst_row, dcat, dcat + F, KC, dg, F, k, a.act);
    MOE_BW(hipGetLastError());
    if (R_max > 0) {
      // dX = du W1 (+ dv W3): W1_e, W3_e [F][H] are the two k-major halves
      MOE_BW(launch_grouped_gemm_bf16_kn(dcat, a.W1, gated ? a.W3 : nullptr, dX, a.offsets, E, H, KC, F, R_max, rc,
                                         st));
      if ((reinterpret_cast<uintptr_t>(a.dx) & 15) == 0)
        gather_sum_vec_kernel<<<T, 256, 0, st>>>(dX, a.dst_row, a.dx, H, k);
      else
        gather_sum_kernel<uint16_t><<<T, 256, 0, st>>>(dX, a.dst_row, a.dx, H, k);
      MOE_BW(hipGetLastError());
    } else {
      zero_f32_kernel<<<grid_1d((int64_t)T * H, 256), 256, 0, st>>>(a.dx, (int64_t)T * H);
      MOE_BW(hipGetLastError());
    }
    // weight gradients on the matrix cores, over each expert's packed rows:
    // dW2 = dy[row_token]^T (g z), dW1 = du^T x[row_token], dW3 = dv^T x[row_token]
    const uint16_t* dy16 = static_cast<const uint16_t*>(a.dy);
    const uint16_t* x16 = static_cast<const uint16_t*>(a.x);
    wgrad_kn_kernel<<<dim3((F + 127) / 128, (H + 127) / 128, E), 256, 0, st>>>(dy16, H, a.row_token, z, F, nullptr,
                                                                               a.dW2, a.offsets, R_max, T, H, F);
    MOE_BW(hipGetLastError());
    wgrad_kn_kernel<<<dim3((H + 127) / 128, (F + 127) / 128, E), 256, 0, st>>>(dcat, KC, nullptr, x16, H, a.row_token,
                                                                               a.dW1, a.offsets, R_max, T, F, H);
    MOE_BW(hipGetLastError());
    if (gated) {
      wgrad_kn_kernel<<<dim3((H + 127) / 128, (F + 127) / 128, E), 256, 0, st>>>(
          dcat + F, KC, nullptr, x16, H, a.row_token, a.dW3, a.offsets, R_max, T, F, H);
      MOE_BW(hipGetLastError());
    }
    MOE_BW(router_backward(a, L, dg, st));
    return hipSuccess;
  }

  float* u = reinterpret_cast<float*>(w + L.u);
  float* v = reinterpret_cast<float*>(w + L.v);
  float* z = reinterpret_cast<float*>(w + L.z);
  float* dz = reinterpret_cast<float*>(w + L.dz);
  float* du = reinterpret_cast<float*>(w + L.du);
  float* dv = du + (size_t)R_max * F;
  float* Y = reinterpret_cast<float*>(w + L.Y);
  float* dY = reinterpret_cast<float*>(w + L.dY);
  float* dX = reinterpret_cast<float*>(w + L.dX);
  if (R_max > 0) {
    // 1. u = x[row_token] W1^T, v = x[row_token] W3^T (per expert, the kept rows)
    GemmArgs g{};
    g.A = a.x;
    g.sam = H, g.sak = 1;
    g.B = a.W1;
    g.sbk = 1, g.sbn = H, g.b_g = (int64_t)F * H;
    g.C = u;
    g.scm = F, g.scn = 1;
    g.M = mr, g.N = F, g.K = H;
    g.offs = a.offsets, g.ragged = 0, g.gather = a.row_token;
    MOE_BW(gemm(bf, bf, g, E, mr, st));
    if (gated) {
      g.B = a.W3;
      g.C = v;
      MOE_BW(gemm(bf, bf, g, E, mr, st));
    }
    // 2. z = act(u) (or silu(u) v)
    act_fwd_kernel<float><<<grid_1d(R_max * F, 256), 256, 0, st>>>(u, v, z, a.offsets, E, F, a.act);
    MOE_BW(hipGetLastError());
    // 3. Y = z W2^T
    GemmArgs y{};
    y.A = z;
    y.sam = F, y.sak = 1;
    y.B = a.W2;
    y.sbk = 1, y.sbn = F, y.b_g = (int64_t)H * F;
    y.C = Y;
    y.scm = H, y.scn = 1;
    y.M = mr, y.N = H, y.K = F;
    y.offs = a.offsets, y.ragged = 0;
    MOE_BW(gemm(false, bf, y, E, mr, st));
  }
  // 4. combine backward: dY (kept rows), dg
  if (bf)
    combine_bwd_kernel<uint16_t, float><<<T, 256, 0, st>>>(static_cast<const uint16_t*>(a.dy), Y, a.topk_gate,
                                                           a.dst_row, dY, dg, H, k);
  else
    combine_bwd_kernel<float, float><<<T, 256, 0, st>>>(static_cast<const float*>(a.dy), Y, a.topk_gate, a.dst_row,
                                                        dY, dg, H, k);
  MOE_BW(hipGetLastError());
  if (R_max > 0) {
    // 5. dz = dY W2 (W2 [E][H][F]: B(k = h, n = f))
    GemmArgs g{};
    g.A = dY;
    g.sam = H, g.sak = 1;
    g.B = a.W2;
    g.sbk = F, g.sbn = 1, g.b_g = (int64_t)H * F;
    g.C = dz;
    g.scm = F, g.scn = 1;
    g.M = mr, g.N = F, g.K = H;
    g.offs = a.offsets, g.ragged = 0;
    MOE_BW(gemm(false, bf, g, E, mr, st));
    // 6. du (, dv)
    act_bwd_kernel<float><<<grid_1d(R_max * F, 256), 256, 0, st>>>(dz, u, v, du, dv, a.offsets, E, F, F, a.act);
    MOE_BW(hipGetLastError());
    // 7. dX = du W1 (+ dv W3)  (W1 [E][F][H]: B(k = f, n = h))
    GemmArgs x{};
    x.A = du;
    x.sam = F, x.sak = 1;
    x.B = a.W1;
    x.sbk = H, x.sbn = 1, x.b_g = (int64_t)F * H;
    x.C = dX;
    x.scm = H, x.scn = 1;
    x.M = mr, x.N = H, x.K = F;
    x.offs = a.offsets, x.ragged = 0;
    MOE_BW(gemm(false, bf, x, E, mr, st));
    if (gated) {
      x.A = dv;
      x.B = a.W3;
      x.accumulate = 1;
      MOE_BW(gemm(false, bf, x, E, mr, st));
    }
    // 8. dx = sum of the token's kept rows of dX
    gather_sum_kernel<float><<<T, 256, 0, st>>>(dX, a.dst_row, a.dx, H, k);
  } else {
    zero_f32_kernel<<<grid_1d((int64_t)T * H, 256), 256, 0, st>>>(a.dx, (int64_t)T * H);
  }
  MOE_BW(hipGetLastError());
  // 9. weight gradients; 10-11. router
  MOE_BW(weight_grads<float>(a, dY, z, du, dv, F, st));
  MOE_BW(router_backward(a, L, dg, st));
#undef MOE_BW
  return hipSuccess;
}

}  // namespace moe
