// Router: logits GEMM (fp64-accumulated, rounded once to fp32) and the
// per-token selection / gate / in-block rank kernel.
//
// Switch Transformers explainer §1.1 (logits = router weight times x, softmax,
// argmax) and §2.1 (router input, logits and softmax in fp32); "Expert-parallel
// MoE training" explainer, router part (Wg in R^{HxE}, softmax then top-k, or
// top-k then normalise over the selected).
//
// Logits: each product x*Wg (bf16 or fp32 times fp32) is exact in binary64 and
// the sum is accumulated in binary64 on the fp64 matrix cores, then rounded once
// to fp32 with the bias added in binary64.  The result is the correctly rounded
// fp32 logit except when the binary64 sum sits within ~1e-14 (relative) of an
// fp32 rounding boundary, so the discrete routing downstream does not depend on
// the summation order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// K1a: logits[t][e] = fl32( sum_h x[t][h] * Wg[h][e] + bias[e] )
//
// Workgroup: 4 waves; wave w owns 16 tokens; the workgroup owns 64 tokens and
// 16*WN experts.  v_mfma_f64_16x16x4f64 per step: lane (i = l%16, q = l/16)
// supplies A[i][q] = x[t0+i][kv] and B[q][i] = Wg[kv][e0+16n+i] where the virtual
// k index kv = h0 + 8q + s runs over the 32-wide h chunk as s = 0..7 (every lane
// keeps its own 8 consecutive x values in registers; the same kv is used for A
// and B, so the sum covers each h exactly once).  The Wg chunk [32][16*WN] is
// staged through LDS (row stride 16*WN + 2 floats keeps the four q rows of one
// read in distinct banks) and shared by the four waves.
// ---------------------------------------------------------------------------
template <bool kBF16, int WN>
__global__ void __launch_bounds__(256) router_logits_kernel(const void* __restrict__ x, const float* __restrict__ Wg,
                                                            const float* __restrict__ bias, float* __restrict__ logits,
                                                            int T, int H, int E, int vec_ok) {
  constexpr int BE = 16 * WN;
  constexpr int S = BE + 2;
  constexpr int KC = 32;
  __shared__ float s_w[2][KC * S];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int t0 = blockIdx.x * 64 + 16 * w;
  const int e0 = blockIdx.y * BE;
  const int t_lane = t0 + i;
  const size_t eb = kBF16 ? 2 : 4;
  const char* xrow = static_cast<const char*>(x) + (size_t)(t_lane < T ? t_lane : 0) * H * eb;

  f64x4_t acc[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) acc[n] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  const int nchunks = (H + KC - 1) / KC;
  constexpr int WPER = (KC * BE) / 256;  // Wg elements per thread per chunk (2*WN)
  float wreg[WPER];
  float xv[8];

  auto load_w = [&](int c) {
#pragma unroll
    for (int j = 0; j < WPER; ++j) {
      int idx = tid + 256 * j;
      int row = idx / BE, col = idx % BE;
      int h = c * KC + row, e = e0 + col;
      wreg[j] = (h < H && e < E) ? Wg[(size_t)h * E + e] : 0.0f;
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int j = 0; j < WPER; ++j) {
      int idx = tid + 256 * j;
      int row = idx / BE, col = idx % BE;
      s_w[buf][row * S + col] = wreg[j];
    }
  };
  auto load_x = [&](int c, float (&v)[8]) {
    if (t_lane < T) {
      load8_f32<kBF16>(xrow, (int64_t)c * KC + 8 * q, H, vec_ok, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
  };

  load_w(0);
  load_x(0, xv);
  store_w(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    float xn[8];
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(c + 1);
      load_x(c + 1, xn);
    }
    const float* sw = s_w[buf];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const double a = (double)xv[s];
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const double b = (double)sw[(8 * q + s) * S + 16 * n + i];
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[n], 0, 0, 0);
      }
    }
    if (more) {
      store_w(buf ^ 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = xn[j];
    }
    __syncthreads();
  }

  // D layout of the f64 16x16x4 MFMA: lane (i, q) holds D[q + 4j][i], j = 0..3.
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    const int e = e0 + 16 * n + i;
    if (e >= E) continue;
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + q + 4 * j;
      if (t < T) logits[(size_t)t * E + e] = (float)(acc[n][j] + b);
    }
  }
}

// ---------------------------------------------------------------------------
// K1b: per token (one lane per token, one wave per block of 64 tokens):
//   top-k over the E fp32 logits — larger first, ties to the lower index —
//   the k gates, and, for every choice r, the token's rank among the block's
//   tokens that chose the same expert at the same r (ballot peeling over the
//   expert id bits; no atomics) plus the block histogram hist[e][r*nb + blk].
// The rank is parked in dst_row, which the finalise kernel overwrites.
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ void __launch_bounds__(64) router_select_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           int gate_mode, int nbits, int nb,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_gate,
                                                           int32_t* __restrict__ dst_rank,
                                                           int32_t* __restrict__ hist) {
  extern __shared__ int s_cnt[];  // [E]
  const int lane = threadIdx.x;
  const int blk = blockIdx.x;
  const int t = blk * 64 + lane;
  const bool valid = t < T;
  const float* l = logits + (size_t)(valid ? t : 0) * E;
  const bool vec = (E % 4) == 0;

  float tv[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    tv[j] = -__builtin_inff();
    ti[j] = 0;
  }
  auto consider = [&](float v, int e) {
    if (v > tv[KMAX - 1]) {
      tv[KMAX - 1] = v;
      ti[KMAX - 1] = e;
#pragma unroll
      for (int j = KMAX - 1; j > 0; --j) {
        if (tv[j] > tv[j - 1]) {
          float a = tv[j];
          tv[j] = tv[j - 1];
          tv[j - 1] = a;
          int b = ti[j];
          ti[j] = ti[j - 1];
          ti[j - 1] = b;
        }
      }
    }
  };
  if (valid) {
    if (vec) {
      for (int e = 0; e < E; e += 4) {
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(l + e);
        consider(v[0], e);
        consider(v[1], e + 1);
        consider(v[2], e + 2);
        consider(v[3], e + 3);
      }
    } else {
      for (int e = 0; e < E; ++e) consider(l[e], e);
    }
  }

  // gates (fp32)
  const float m = tv[0];
  float den = 0.0f;
  if (valid) {
    if (gate_mode == 0) {  // softmax over all E, no renormalisation
      if (vec) {
        for (int e = 0; e < E; e += 4) {
          f32x4_t v = *reinterpret_cast<const f32x4_t*>(l + e);
          den += expf(v[0] - m);
          den += expf(v[1] - m);
          den += expf(v[2] - m);
          den += expf(v[3] - m);
        }
      } else {
        for (int e = 0; e < E; ++e) den += expf(l[e] - m);
      }
    } else {  // normalised over the k chosen (renormalised softmax == softmax over the chosen)
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) den += expf(tv[j] - m);
    }
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r < k) {
        topk_idx[(size_t)t * k + r] = ti[r];
        topk_gate[(size_t)t * k + r] = expf(tv[r] - m) / den;
      }
    }
  }

  // ranks + block histogram, one choice index r at a time
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const uint64_t valid_mask = __ballot(valid);
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r < k) {
      for (int e = lane; e < E; e += 64) s_cnt[e] = 0;
      __syncthreads();
      const int my_e = ti[r];
      uint64_t same = valid_mask;
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (my_e >> b) & 1;
        const uint64_t mb = __ballot(bit);
        same &= bit ? mb : ~mb;
      }
      if (valid) {
        const int rank = __popcll(same & lt_mask);
        dst_rank[(size_t)t * k + r] = rank;
        if (rank == 0) s_cnt[my_e] = __popcll(same);
      }
      __syncthreads();
      const int Q = k * nb;
      for (int e = lane; e < E; e += 64) hist[(size_t)e * Q + r * nb + blk] = s_cnt[e];
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const void* x, bool bf16, const float* Wg, const float* bias, float* logits, int T,
                                int H, int E, bool vec_ok, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 block(256);
  const int gx = (T + 63) / 64;
  if (E <= 16) {
    dim3 grid(gx, 1);
    if (bf16) router_logits_kernel<true, 1><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok);
    else router_logits_kernel<false, 1><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok);
  } else if (E <= 32) {
    dim3 grid(gx, 1);
    if (bf16) router_logits_kernel<true, 2><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok);
    else router_logits_kernel<false, 2><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok);
  } else {
    dim3 grid(gx, (E + 63) / 64);
    if (bf16) router_logits_kernel<true, 4><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok);
    else router_logits_kernel<false, 4><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok);
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const float* logits, int T, int E, int k, int gate_mode, int nb, int32_t* topk_idx,
                                float* topk_gate, int32_t* dst_rank, int32_t* hist, hipStream_t st) {
  if (T == 0) return hipSuccess;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  dim3 grid(nb), block(64);
  size_t shm = sizeof(int) * (size_t)E;
#define MOE_SEL(KM)                                                                                              \
  router_select_kernel<KM><<<grid, block, shm, st>>>(logits, T, E, k, gate_mode, nbits, nb, topk_idx, topk_gate, \
                                                     dst_rank, hist)
  if (k <= 1) MOE_SEL(1);
  else if (k <= 2) MOE_SEL(2);
  else if (k <= 4) MOE_SEL(4);
  else if (k <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

}  // namespace moe
