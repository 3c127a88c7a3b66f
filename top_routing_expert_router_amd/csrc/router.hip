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
// Workgroup: 4 waves as TW token groups (16 tokens each) x KW = 4 / TW slices
// of the h range; the workgroup owns 16*TW tokens and 16*WN experts.
// v_mfma_f64_16x16x4f64 per step: lane (i = l%16, q = l/16) supplies
// A[i][q] = x[t0+i][kv] and B[q][i] = Wg[kv][e0+16n+i] where the virtual k
// index kv = h0 + 4q + s runs over a 16-wide h chunk as s = 0..3 (each lane
// keeps its own 4 consecutive x values in registers, prefetched two chunks
// ahead; A and B use the same kv, so every h is covered once).  The Wg chunk
// [16][16*WN] of a slice is staged through LDS (double-buffered, row stride
// 16*WN + 2 floats) and shared by the slice's TW waves.  The KW partial sums of
// a token / expert pair are added in slice order through LDS, so the result
// does not depend on scheduling.
// ---------------------------------------------------------------------------
template <bool kBF16, int WN, int TW>
__global__ void __launch_bounds__(256) router_logits_kernel(const void* __restrict__ x, const float* __restrict__ Wg,
                                                            const float* __restrict__ bias, float* __restrict__ logits,
                                                            int T, int H, int E, int vec_ok) {
  constexpr int KW = 4 / TW;
  constexpr int BE = 16 * WN;
  constexpr int S = BE + 2;
  constexpr int KC = 16;
  constexpr int CH = KC * S;                        // floats per staged chunk
  constexpr int WPER = KC * BE / (64 * TW);         // Wg floats per lane per chunk
  constexpr int RED = KW > 1 ? KW * 16 * TW * BE * 2 : 0;  // floats of the partial-sum exchange (doubles)
  constexpr int SMEM = (KW * 2 * CH > RED ? KW * 2 * CH : RED);
  __shared__ __align__(16) float smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int tg = w % TW, kg = w / TW;
  const int gl = tg * 64 + lane;  // lane index inside the slice group
  const int i = lane & 15;
  const int q = lane >> 4;
  const int t0 = blockIdx.x * (16 * TW) + 16 * tg;
  const int e0 = blockIdx.y * BE;
  const int t_lane = t0 + i;
  const size_t eb = kBF16 ? 2 : 4;
  const char* xrow = static_cast<const char*>(x) + (size_t)(t_lane < T ? t_lane : 0) * H * eb;

  const int nchunks = (H + KC - 1) / KC;
  const int per = (nchunks + KW - 1) / KW;  // chunks per slice (all slices iterate `per` times)
  const int c_begin = kg * per;

  f64x4_t acc[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) acc[n] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  float wreg[WPER];
  auto load_w = [&](int c) {
#pragma unroll
    for (int j = 0; j < WPER; ++j) {
      const int idx = gl + 64 * TW * j;
      const int row = idx / BE, col = idx % BE;
      const int h = c * KC + row, e = e0 + col;
      wreg[j] = (c < nchunks && h < H && e < E) ? Wg[(size_t)h * E + e] : 0.0f;
    }
  };
  auto store_w = [&](int buf) {
    float* sw = smem + (kg * 2 + buf) * CH;
#pragma unroll
    for (int j = 0; j < WPER; ++j) {
      const int idx = gl + 64 * TW * j;
      sw[(idx / BE) * S + idx % BE] = wreg[j];
    }
  };
  auto load_x = [&](int c, float (&v)[4]) {
    if (t_lane < T && c < nchunks) {
      const int64_t h = (int64_t)c * KC + 4 * q;
      if (kBF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(xrow);
        if (vec_ok && h + 4 <= H) {
          const uint2 u = *reinterpret_cast<const uint2*>(p + h);
          v[0] = __uint_as_float(u.x << 16);
          v[1] = __uint_as_float(u.x & 0xFFFF0000u);
          v[2] = __uint_as_float(u.y << 16);
          v[3] = __uint_as_float(u.y & 0xFFFF0000u);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = h + j < H ? bf16_bits_to_f32(p[h + j]) : 0.0f;
        }
      } else {
        const float* p = reinterpret_cast<const float*>(xrow);
        if (vec_ok && h + 4 <= H) {
          const f32x4_t u = *reinterpret_cast<const f32x4_t*>(p + h);
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = u[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = h + j < H ? p[h + j] : 0.0f;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = 0.0f;
    }
  };

  float x0[4], x1[4], x2[4];  // chunks c, c+1, c+2
  load_w(c_begin);
  load_x(c_begin, x0);
  load_x(c_begin + 1, x1);
  store_w(0);
  __syncthreads();
  for (int cl = 0; cl < per; ++cl) {
    const int c = c_begin + cl;
    const bool more = cl + 1 < per;
    if (more) load_w(c + 1);
    load_x(c + 2, x2);
    const float* sw = smem + (kg * 2 + (cl & 1)) * CH;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const double a = (double)x0[s2];
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const double b = (double)sw[(4 * q + s2) * S + 16 * n + i];
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[n], 0, 0, 0);
      }
    }
    if (more) store_w((cl + 1) & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x0[j] = x1[j];
      x1[j] = x2[j];
    }
    __syncthreads();
  }

  // D layout of the f64 16x16x4 MFMA: lane (i, q) holds D[q + 4j][i], j = 0..3.
  // Partial sums: red[kg][tg][token 0..15][expert 0..BE), then slice 0's waves add them up.
  double* red = reinterpret_cast<double*>(smem);
  if (KW > 1) {
#pragma unroll
    for (int n = 0; n < WN; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[((kg * TW + tg) * 16 + q + 4 * j) * BE + 16 * n + i] = acc[n][j];
    __syncthreads();
  }
  if (kg == 0) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int e = e0 + 16 * n + i;
      const double b = (bias && e < E) ? (double)bias[e] : 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tr = q + 4 * j;
        double v = acc[n][j];
#pragma unroll
        for (int k2 = 1; k2 < KW; ++k2) v += red[((k2 * TW + tg) * 16 + tr) * BE + 16 * n + i];
        const int t = t0 + tr;
        if (t < T && e < E) logits[(size_t)t * E + e] = (float)(v + b);
      }
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
// For every choice r: the token's rank among the block's 64 tokens that chose
// the same expert at the same r (ballot peeling over the expert id bits; no
// atomics), parked in dst_rank, and the block histogram hist[e][r*nb + blk].
// An absent choice (GShard's random second choice not taken) ranks under the
// virtual expert E, which has no histogram row, and gets kAbsentChoice in dst_rank.
template <int KMAX>
__device__ __forceinline__ void block_ranks(const int (&ti)[KMAX], const bool (&absent)[KMAX], bool valid, int k,
                                            int E, int nbits, int nb, int t, int32_t* __restrict__ dst_rank,
                                            int32_t* __restrict__ hist, int* s_cnt) {
  const int lane = threadIdx.x;
  const int blk = blockIdx.x;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const uint64_t valid_mask = __ballot(valid);
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r < k) {
      for (int e = lane; e <= E; e += 64) s_cnt[e] = 0;
      __syncthreads();
      const int my_e = absent[r] ? E : ti[r];
      uint64_t same = valid_mask;
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (my_e >> b) & 1;
        const uint64_t mb = __ballot(bit);
        same &= bit ? mb : ~mb;
      }
      if (valid) {
        const int rank = __popcll(same & lt_mask);
        dst_rank[(size_t)t * k + r] = absent[r] ? kAbsentChoice : rank;
        if (rank == 0) s_cnt[my_e] = __popcll(same);
      }
      __syncthreads();
      const int Q = k * nb;
      for (int e = lane; e < E; e += 64) hist[(size_t)e * Q + r * nb + blk] = s_cnt[e];
      __syncthreads();
    }
  }
}

template <int KMAX>
__global__ void __launch_bounds__(64) router_select_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           int gate_mode, const float* __restrict__ second_u,
                                                           int nbits, int nb,
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
  float gv[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) gv[r] = 0.0f;
  if (valid) {
    if (gate_mode == 0) {  // softmax scores over all E, no renormalisation
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
        gv[r] = gate_value<KMAX>(gate_mode, k, tv, den, r);
        topk_idx[(size_t)t * k + r] = ti[r];
        topk_gate[(size_t)t * k + r] = gv[r];
      }
    }
  }

  bool absent[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) absent[r] = false;
  if (KMAX >= 2 && second_u && valid) absent[1] = !second_choice_taken(second_u[t], gv[0], gv[1]);
  block_ranks<KMAX>(ti, absent, valid, k, E, nbits, nb, t, dst_rank, hist, s_cnt);
}

// Ranks and block histogram from a finished topk_idx (the split router writes
// the choices itself): the rank part of the kernel above, with one wave per
// (64-token block, choice r) since the choices are ranked independently.
__global__ void __launch_bounds__(64) router_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                         const float* __restrict__ topk_gate,
                                                         const float* __restrict__ second_u, int T, int E, int k,
                                                         int nbits, int nb, int32_t* __restrict__ dst_rank,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int s_cnt[];  // [E + 1]
  const int lane = threadIdx.x, blk = blockIdx.x, r = blockIdx.y;
  const int t = blk * 64 + lane;
  const bool valid = t < T;
  const bool absent = r == 1 && second_u && valid &&
                      !second_choice_taken(second_u[t], topk_gate[(size_t)t * k], topk_gate[(size_t)t * k + 1]);
  const int my_e = absent ? E : (valid ? topk_idx[(size_t)t * k + r] : 0);
  for (int e = lane; e <= E; e += 64) s_cnt[e] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (my_e >> b) & 1;
    const uint64_t mb = __ballot(bit);
    same &= bit ? mb : ~mb;
  }
  if (valid) {
    const int rank = __popcll(same & lt_mask);
    dst_rank[(size_t)t * k + r] = absent ? kAbsentChoice : rank;
    if (rank == 0) s_cnt[my_e] = __popcll(same);
  }
  __syncthreads();
  const int Q = k * nb;
  for (int e = lane; e < E; e += 64) hist[(size_t)e * Q + r * nb + blk] = s_cnt[e];
}

// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const void* x, bool bf16, const float* Wg, const float* bias, float* logits, int T,
                                int H, int E, bool vec_ok, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int WN = E <= 16 ? 1 : (E <= 32 ? 2 : 4);
  const int gy = (E + 16 * WN - 1) / (16 * WN);
  // enough workgroups for four waves per SIMD: split the h range when tokens are few
  int TW = 4;
  while (TW > 1 && (int64_t)((T + 16 * TW - 1) / (16 * TW)) * gy < 1024) TW /= 2;
  dim3 block(256), grid((T + 16 * TW - 1) / (16 * TW), gy);
#define MOE_RL(B, N, W) router_logits_kernel<B, N, W><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok)
#define MOE_RL_TW(B, N) \
  if (TW == 4) MOE_RL(B, N, 4); \
  else if (TW == 2) MOE_RL(B, N, 2); \
  else MOE_RL(B, N, 1)
#define MOE_RL_WN(B) \
  if (WN == 1) { MOE_RL_TW(B, 1); } \
  else if (WN == 2) { MOE_RL_TW(B, 2); } \
  else { MOE_RL_TW(B, 4); }
  if (bf16) {
    MOE_RL_WN(true);
  } else {
    MOE_RL_WN(false);
  }
#undef MOE_RL_WN
#undef MOE_RL_TW
#undef MOE_RL
  return hipGetLastError();
}

hipError_t launch_router_select(const float* logits, int T, int E, int k, int gate_mode, const float* second_u,
                                int nb, int32_t* topk_idx, float* topk_gate, int32_t* dst_rank, int32_t* hist,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;  // expert ids 0 .. E (E: an absent choice)
  dim3 grid(nb), block(64);
  size_t shm = sizeof(int) * (size_t)(E + 1);
#define MOE_SEL(KM)                                                                                            \
  router_select_kernel<KM><<<grid, block, shm, st>>>(logits, T, E, k, gate_mode, second_u, nbits, nb, topk_idx, \
                                                     topk_gate, dst_rank, hist)
  if (k <= 1) MOE_SEL(1);
  else if (k <= 2) MOE_SEL(2);
  else if (k <= 4) MOE_SEL(4);
  else if (k <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

hipError_t launch_router_rank(const int32_t* topk_idx, const float* topk_gate, const float* second_u, int T, int E,
                              int k, int nb, int32_t* dst_rank, int32_t* hist, hipStream_t st) {
  if (T == 0) return hipSuccess;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;  // expert ids 0 .. E (E: an absent choice)
  dim3 grid(nb, k), block(64);
  size_t shm = sizeof(int) * (size_t)(E + 1);
  router_rank_kernel<<<grid, block, shm, st>>>(topk_idx, topk_gate, second_u, T, E, k, nbits, nb, dst_rank, hist);
  return hipGetLastError();
}

}  // namespace moe
