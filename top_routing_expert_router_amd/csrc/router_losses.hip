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
// Two kernels, fixed summation orders throughout (deterministic):
//   partial: one block per 64-token block, one wave per 16 tokens, lane l
//            holding experts l + 64 j; per-token softmax and logsumexp in fp32,
//            sums over tokens in binary64, waves combined in wave order;
//   final:   one block: per-expert sums over the blocks, f_e P_e, and the two
//            scalars through a fixed-shape tree.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <int JE>
__global__ void __launch_bounds__(256) router_loss_partial_kernel(const float* __restrict__ logits,
                                                                  const int32_t* __restrict__ topk_idx, int T, int E,
                                                                  int k, int score_fn, double* __restrict__ Ppart,
                                                                  double* __restrict__ Zpart,
                                                                  int32_t* __restrict__ Cpart) {
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
  for (int tt = 0; tt < 16; ++tt) {
    const int t = blk * 64 + w * 16 + tt;
    if (t >= T) break;
    const float* row = logits + (size_t)t * E;
    float v[JE];
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < JE; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? row[e] : -__builtin_inff();
      m = fmaxf(m, v[j]);
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    float ex[JE], den = 0.0f;
#pragma unroll
    for (int j = 0; j < JE; ++j) {
      ex[j] = lane + 64 * j < E ? expf(v[j] - m) : 0.0f;
      den += ex[j];
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) den += __shfl_xor(den, d, 64);
    if (score_fn) {  // sigmoid scores over their sum
      float sc[JE], ssum = 0.0f;
#pragma unroll
      for (int j = 0; j < JE; ++j) {
        sc[j] = lane + 64 * j < E ? 1.0f / (1.0f + expf(-v[j])) : 0.0f;
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
    const int first = topk_idx[(size_t)t * k];
#pragma unroll
    for (int j = 0; j < JE; ++j) cnt[j] += (lane + 64 * j == first);
  }
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    s_p[w][lane + 64 * j] = acc[j];
    s_c[w][lane + 64 * j] = cnt[j];
  }
  if (lane == 0) s_z[w] = z;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    Ppart[(size_t)blk * E + e] = ((s_p[0][e] + s_p[1][e]) + s_p[2][e]) + s_p[3][e];
    Cpart[(size_t)blk * E + e] = s_c[0][e] + s_c[1][e] + s_c[2][e] + s_c[3][e];
  }
  if (threadIdx.x == 0) Zpart[blk] = ((s_z[0] + s_z[1]) + s_z[2]) + s_z[3];
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

__global__ void __launch_bounds__(256) router_loss_final_kernel(const double* __restrict__ Ppart,
                                                                const double* __restrict__ Zpart,
                                                                const int32_t* __restrict__ Cpart,
                                                                const int32_t* __restrict__ demand, int nb, int T,
                                                                int E, int k, int aux_mode, double aux_coeff,
                                                                double z_coeff, double* __restrict__ losses) {
  __shared__ double s[256];
  double dot = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) {
    double P = 0.0;
    int64_t first = 0;
    for (int b = 0; b < nb; ++b) {
      P += Ppart[(size_t)b * E + e];
      first += Cpart[(size_t)b * E + e];
    }
    const double f = aux_mode == 0 ? (double)demand[e] / ((double)T * (double)k) : (double)first / (double)T;
    dot += f * (P / (double)T);
  }
  dot = block_sum_256(dot, s);
  double zs = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) zs += Zpart[b];
  zs = block_sum_256(zs, s);
  if (threadIdx.x == 0) {
    losses[0] = T > 0 ? aux_coeff * (double)E * dot : 0.0;
    losses[1] = T > 0 ? z_coeff * zs / (double)T : 0.0;
  }
}

hipError_t launch_router_losses(const float* logits, const int32_t* topk_idx, const int32_t* demand, int T, int E,
                                int k, int score_fn, int aux_mode, double aux_coeff, double z_coeff, double* Ppart,
                                double* Zpart, int32_t* Cpart, double* losses, hipStream_t st) {
  const int nb = (T + 63) / 64;
  if (nb > 0) {
    const int je = (E + 63) / 64;
#define MOE_LP(J) \
  router_loss_partial_kernel<J><<<dim3(nb), dim3(256), 0, st>>>(logits, topk_idx, T, E, k, score_fn, Ppart, Zpart, \
                                                                Cpart)
    if (je <= 1) MOE_LP(1);
    else if (je <= 2) MOE_LP(2);
    else if (je <= 4) MOE_LP(4);
    else if (je <= 8) MOE_LP(8);
    else MOE_LP(16);
#undef MOE_LP
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  router_loss_final_kernel<<<dim3(1), dim3(256), 0, st>>>(Ppart, Zpart, Cpart, demand, nb, T, E, k, aux_mode,
                                                          aux_coeff, z_coeff, losses);
  return hipGetLastError();
}

}  // namespace moe
