// Router training terms: the load-balancing loss alpha * E * sum_e f_e P_e and
// the z-loss beta * mean_t logsumexp(l_t)^2 ("Expert-parallel MoE training"
// explainer, router section: the auxiliary-loss and z-loss paragraphs; Switch
// Transformers explainer, "Load balance & capacity").
//
// P_e is the mean over tokens of softmax(l_t)_e (sigmoid scoring: the token's
// sigmoid scores over their sum); f_e is demand_e / (T k)
// (aux_mode 0: every choice counts, k in the denominator) or the fraction of
// tokens whose first choice is e (aux_mode 1, DeepSpeed's top-2 path).  Both are
// computed from the routing's fp32 logits after the choices are final.
//
// Three kernels, fixed summation orders throughout (deterministic):
//   partial: one block per 64-token block, one wave per 16 tokens, lane l
//            holding experts l + 64 j; per-token softmax and logsumexp in fp32,
//            sums over tokens in binary64, waves combined in wave order;
//   expert:  one wave per expert: the sum over the blocks and f_e P_e (one more
//            wave sums the logsumexp^2 partials);
//   final:   one block: sum_e f_e P_e through a fixed-shape tree, the scalars.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Partial sums per 64-token block.  Each wave takes 16 tokens, four at a time
// with all four rows loaded before any is used, and accumulates in token order;
// the layout Ppart[e][blk] lets one wave per expert read its partials
// contiguously afterwards.
template <int JE>
__global__ void __launch_bounds__(256) router_loss_partial_kernel(const float* __restrict__ logits,
                                                                  const int32_t* __restrict__ topk_idx, int T, int E,
                                                                  int k, int score_fn, int nb,
                                                                  double* __restrict__ Ppart,
                                                                  double* __restrict__ Zpart,
                                                                  int32_t* __restrict__ Cpart) {
  constexpr int TB = 4;  // tokens in flight per wave
  __shared__ double s_p[4][64 * JE];
  __shared__ int s_c[4][64 * JE];
  __shared__ double s_z[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int blk = blockIdx.x;
  double acc[JE], z = 0.0;
  int cnt[JE];
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    acc[j] = 0.0;
    cnt[j] = 0;
  }
  for (int t0 = 0; t0 < 16; t0 += TB) {
    float v[TB][JE];
    int first[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = blk * 64 + w * 16 + t0 + u;
      const bool ok = t < T;
      const float* row = logits + (size_t)(ok ? t : 0) * E;
#pragma unroll
      for (int j = 0; j < JE; ++j) {
        const int e = lane + 64 * j;
        v[u][j] = (ok && e < E) ? row[e] : -__builtin_inff();
      }
      first[u] = ok ? topk_idx[(size_t)t * k] : -1;
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      if (first[u] < 0) break;  // past the last token (tokens are in order)
      float m = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < JE; ++j) m = fmaxf(m, v[u][j]);
#pragma unroll
      for (int d = 32; d > 0; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      float ex[JE], den = 0.0f;
#pragma unroll
      for (int j = 0; j < JE; ++j) {
        ex[j] = lane + 64 * j < E ? expf(v[u][j] - m) : 0.0f;
        den += ex[j];
      }
#pragma unroll
      for (int d = 32; d > 0; d >>= 1) den += __shfl_xor(den, d, 64);
      if (score_fn) {  // sigmoid scores over their sum
        float sc[JE], ssum = 0.0f;
#pragma unroll
        for (int j = 0; j < JE; ++j) {
          sc[j] = lane + 64 * j < E ? 1.0f / (1.0f + expf(-v[u][j])) : 0.0f;
          ssum += sc[j];
        }
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) ssum += __shfl_xor(ssum, d, 64);
#pragma unroll
        for (int j = 0; j < JE; ++j) acc[j] += (double)(sc[j] / ssum);
      } else {
#pragma unroll
        for (int j = 0; j < JE; ++j) acc[j] += (double)(ex[j] / den);
      }
      const double lse = (double)m + (double)logf(den);
      z += lse * lse;
#pragma unroll
      for (int j = 0; j < JE; ++j) cnt[j] += (lane + 64 * j == first[u]);
    }
  }
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    s_p[w][lane + 64 * j] = acc[j];
    s_c[w][lane + 64 * j] = cnt[j];
  }
  if (lane == 0) s_z[w] = z;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    Ppart[(size_t)e * nb + blk] = ((s_p[0][e] + s_p[1][e]) + s_p[2][e]) + s_p[3][e];
    Cpart[(size_t)e * nb + blk] = s_c[0][e] + s_c[1][e] + s_c[2][e] + s_c[3][e];
  }
  if (threadIdx.x == 0) Zpart[blk] = ((s_z[0] + s_z[1]) + s_z[2]) + s_z[3];
}

// One wave per expert (and one more for the z-loss): lanes sum the block
// partials with stride 64 in order, then a fixed butterfly.  Writes
// fP[e] = f_e * P_e and, from the extra wave, zsum.
__global__ void __launch_bounds__(256) router_loss_expert_kernel(const double* __restrict__ Ppart,
                                                                 const double* __restrict__ Zpart,
                                                                 const int32_t* __restrict__ Cpart,
                                                                 const int32_t* __restrict__ demand, int nb, int T,
                                                                 int E, int k, int aux_mode,
                                                                 double* __restrict__ fP) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e > E) return;
  double P = 0.0;
  int64_t first = 0;
  if (e < E) {
    for (int b = lane; b < nb; b += 64) {
      P += Ppart[(size_t)e * nb + b];
      first += Cpart[(size_t)e * nb + b];
    }
  } else {
    for (int b = lane; b < nb; b += 64) P += Zpart[b];
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    P += __shfl_xor(P, d, 64);
    first += __shfl_xor(first, d, 64);
  }
  if (lane != 0) return;
  if (e == E) {
    fP[E] = P;  // sum over tokens of logsumexp^2
    return;
  }
  const double f = aux_mode == 0 ? (double)demand[e] / ((double)T * (double)k) : (double)first / (double)T;
  fP[e] = f * (P / (double)T);
}

// Sum of one double per thread over the 256 threads, fixed tree; result in s[0].
__device__ __forceinline__ double block_sum_256(double v, double* s) {
  s[threadIdx.x] = v;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if ((int)threadIdx.x < d) s[threadIdx.x] += s[threadIdx.x + d];
    __syncthreads();
  }
  const double r = s[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(256) router_loss_final_kernel(const double* __restrict__ fP, int T, int E,
                                                                double aux_coeff, double z_coeff,
                                                                double* __restrict__ losses) {
  __shared__ double s[256];
  double dot = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) dot += fP[e];
  dot = block_sum_256(dot, s);
  if (threadIdx.x == 0) {
    losses[0] = T > 0 ? aux_coeff * (double)E * dot : 0.0;
    losses[1] = T > 0 ? z_coeff * fP[E] / (double)T : 0.0;
  }
}

hipError_t launch_router_losses(const float* logits, const int32_t* topk_idx, const int32_t* demand, int T, int E,
                                int k, int score_fn, int aux_mode, double aux_coeff, double z_coeff, double* Ppart,
                                double* Zpart, int32_t* Cpart, double* losses, bool partials_done,
                                hipStream_t st) {
  const int nb = (T + 63) / 64;
  double* fP = Zpart + (nb > 0 ? nb : 1);  // [E + 1] after the z partials
  if (nb > 0) {
    const int je = (E + 63) / 64;
    if (!partials_done) {
#define MOE_LP(J)                                                                                                \
  router_loss_partial_kernel<J><<<dim3(nb), dim3(256), 0, st>>>(logits, topk_idx, T, E, k, score_fn, nb, Ppart, \
                                                                Zpart, Cpart)
    if (je <= 1) MOE_LP(1);
    else if (je <= 2) MOE_LP(2);
    else if (je <= 4) MOE_LP(4);
    else if (je <= 8) MOE_LP(8);
    else MOE_LP(16);
#undef MOE_LP
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    router_loss_expert_kernel<<<dim3((E + 1 + 3) / 4), dim3(256), 0, st>>>(Ppart, Zpart, Cpart, demand, nb, T, E,
                                                                           k, aux_mode, fP);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  router_loss_final_kernel<<<dim3(1), dim3(256), 0, st>>>(fP, T, E, aux_coeff, z_coeff, losses);
  return hipGetLastError();
}

}  // namespace moe
