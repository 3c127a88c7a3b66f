// Router: exact logits in their defining order, and the per-token selection /
// gate / in-block rank kernel.
//
// Switch Transformers explainer §1.1 (logits = router weight times x, softmax,
// argmax) and §2.1 (router input, logits and softmax in fp32); "Expert-parallel
// MoE training" explainer, router part (Wg in R^{HxE}, softmax then top-k, or
// top-k then normalise over the selected).
//
// Logits: l[t][e] = fl32(acc + b_e) with acc = 0 and, for h = 0, 1, ..., H-1,
// acc = acc + x[t][h]*Wg[h][e] in binary64.  A bf16 or fp32 activation times an
// fp32 weight has at most 48 significant bits, so the product is exact and
// fma(x, w, acc) rounds exactly once, like the add: computed here with the same
// operations in the same order, the logits are those bits, not an
// approximation of them.  The gates are taken in binary64 from those logits in
// the same fixed order and rounded once to fp32.  This path serves every shape
// the split-bf16 router does not take, and the routing variants whose plan the
// gate values decide (the "probs" drop policy under a limiting capacity,
// GShard's random second choice).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// K1a: exact logits.  256 threads as TG token groups x EG expert groups; a
// thread owns 4 tokens x 8 experts (32 binary64 accumulators), a workgroup
// TB = 4 TG tokens x BE = 8 EG experts.  Per chunk of KC h values the token
// rows (transposed, fp32: bf16 widens exactly) and the weight rows are staged
// in LDS, double-buffered, the next chunk's global loads in flight while the
// current one is multiplied.  Each accumulator's chain runs over h in
// ascending order.
// ---------------------------------------------------------------------------
template <bool kBF16, int EG>
__global__ void __launch_bounds__(256) router_exact_kernel(const void* __restrict__ x, const float* __restrict__ Wg,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits, int T, int H, int E,
                                                           int vec_ok /* 16-byte aligned x, H % 4 == 0 */) {
  constexpr int TG = 256 / EG, TB = 4 * TG, BE = 8 * EG;
  constexpr int KC = 4096 / TB;           // h per chunk: TB * KC = 4096 staged activations
  constexpr int XS = TB + 4, WS = BE + 4;  // padded LDS row strides (floats; 16-byte aligned rows)
  constexpr int NXV = TB * KC / 4 / 256;  // 4-element activation groups per thread per chunk
  constexpr int NW = (BE * KC + 255) / 256;
  static_assert(KC % 4 == 0 && NXV >= 1, "chunk shape");
  __shared__ __align__(16) float xs[2][KC * XS];
  __shared__ __align__(16) float wsm[2][KC * WS];

  const int tid = threadIdx.x;
  const int tg = tid / EG, eg = tid % EG;
  const int t0 = blockIdx.x * TB, e0 = blockIdx.y * BE;
  const int nchunks = (H + KC - 1) / KC;

  float xr[NXV][4], wr[NW];
  auto load = [&](int c) {
    const int h0 = c * KC;
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + 256 * i;
      const int tok = v / (KC / 4), hv = (v % (KC / 4)) * 4;
      const int t = t0 + tok;
      const int64_t h = (int64_t)h0 + hv;
      if (t < T) {
        if (kBF16) {
          const uint16_t* p = static_cast<const uint16_t*>(x) + (size_t)t * H;
          if (vec_ok && h + 4 <= H) {
            const uint2 u = *reinterpret_cast<const uint2*>(p + h);
            xr[i][0] = __uint_as_float(u.x << 16);
            xr[i][1] = __uint_as_float(u.x & 0xFFFF0000u);
            xr[i][2] = __uint_as_float(u.y << 16);
            xr[i][3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[i][j] = h + j < H ? bf16_bits_to_f32(p[h + j]) : 0.0f;
          }
        } else {
          const float* p = static_cast<const float*>(x) + (size_t)t * H;
          if (vec_ok && h + 4 <= H) {
            const f32x4_t u = *reinterpret_cast<const f32x4_t*>(p + h);
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[i][j] = u[j];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[i][j] = h + j < H ? p[h + j] : 0.0f;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[i][j] = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int j = tid + 256 * i;
      const int hh = j / BE, e = e0 + j % BE;
      wr[i] = (j < BE * KC && h0 + hh < H && e < E) ? Wg[(size_t)(h0 + hh) * E + e] : 0.0f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + 256 * i;
      const int tok = v / (KC / 4), hv = (v % (KC / 4)) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[buf][(hv + j) * XS + tok] = xr[i][j];
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int j = tid + 256 * i;
      if (j < BE * KC) wsm[buf][(j / BE) * WS + j % BE] = wr[i];
    }
  };

  double acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;

  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) load(c + 1);
    const int buf = c & 1;
    auto step = [&](int hh) {  // one h: 32 products added in order
      const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(&xs[buf][hh * XS + 4 * tg]);
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(&wsm[buf][hh * WS + 8 * eg]);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(&wsm[buf][hh * WS + 8 * eg + 4]);
      double xd[4], wd[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xd[i] = (double)xv[i];
        wd[i] = (double)w0[i];
        wd[4 + i] = (double)w1[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fma(xd[i], wd[j], acc[i][j]);
    };
    const int hn = H - c * KC;  // h of this chunk, ascending
    if (hn >= KC) {
#pragma unroll
      for (int hh = 0; hh < KC; ++hh) step(hh);
    } else {
      for (int hh = 0; hh < hn; ++hh) step(hh);
    }
    if (more) store((c + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = e0 + 8 * eg + j;
    if (e >= E) continue;
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * tg + i;
      if (t < T) logits[(size_t)t * E + e] = (float)(bias ? acc[i][j] + b : acc[i][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// K1b: per token (one lane per token, one wave per block of 64 tokens): top-k
// over the E fp32 logits (larger first, ties to the lower index), the k gates
// in binary64, and the ranks below.
//
// For every choice r: the token's rank among the block's 64 tokens that chose
// the same expert at the same r (ballot peeling over the expert id bits; no
// atomics), parked in dst_rank (the finalise kernels overwrite it), and the
// block histogram hist[e][r*nb + blk].  An absent choice (GShard's random
// second choice not taken) ranks under the virtual expert E, which has no
// histogram row, and gets kAbsentChoice in dst_rank.
// ---------------------------------------------------------------------------
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

  // Gates in binary64 from the fp32 logits, each rounded once to fp32, with the
  // operations of their definition in its order: m = the largest logit;
  // softmax denominators summed over e ascending (all E) or over the choices
  // in order (the k chosen); the renormalised gates p_r over the sum of the
  // chosen p in choice order; sigmoid scores 1 / (1 + exp(-l)).
  float gv[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) gv[r] = 0.0f;
  if (valid) {
    const int gm = gate_mode & (kSigmoidFlag - 1);
    double gd[KMAX];
    if ((gate_mode & kSigmoidFlag) && gm != 2) {
      double sum = 0.0;
#pragma unroll
      for (int r = 0; r < KMAX; ++r)
        if (r < k) {
          gd[r] = 1.0 / (1.0 + exp(-(double)tv[r]));
          sum += gd[r];
        }
      if (gm != 0)
#pragma unroll
        for (int r = 0; r < KMAX; ++r)
          if (r < k) gd[r] = gd[r] / sum;
    } else {
      const double m = (double)tv[0];
      double den = 0.0;
      if (gm == 2) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k) den += exp((double)tv[j] - m);
      } else {
        for (int e = 0; e < E; ++e) den += exp((double)l[e] - m);
      }
#pragma unroll
      for (int r = 0; r < KMAX; ++r)
        if (r < k) gd[r] = exp((double)tv[r] - m) / den;
      if (gm == 1) {
        double ps = 0.0;
#pragma unroll
        for (int r = 0; r < KMAX; ++r)
          if (r < k) ps += gd[r];
#pragma unroll
        for (int r = 0; r < KMAX; ++r)
          if (r < k) gd[r] = gd[r] / ps;
      }
    }
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r < k) {
        gv[r] = (float)gd[r];
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
__global__ void __launch_bounds__(64) router_rank_kernel(const int32_t* __restrict__ topk_idx, int T, int E, int k,
                                                         int nbits, int nb, int32_t* __restrict__ dst_rank,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int s_cnt[];  // [E]
  const int lane = threadIdx.x, blk = blockIdx.x, r = blockIdx.y;
  const int t = blk * 64 + lane;
  const bool valid = t < T;
  const int my_e = valid ? topk_idx[(size_t)t * k + r] : 0;
  for (int e = lane; e < E; e += 64) s_cnt[e] = 0;
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
    dst_rank[(size_t)t * k + r] = rank;
    if (rank == 0) s_cnt[my_e] = __popcll(same);
  }
  __syncthreads();
  const int Q = k * nb;
  for (int e = lane; e < E; e += 64) hist[(size_t)e * Q + r * nb + blk] = s_cnt[e];
}

// ---------------------------------------------------------------------------
hipError_t launch_router_exact(const void* x, bool bf16, const float* Wg, const float* bias, float* logits, int T,
                               int H, int E, bool vec_ok, hipStream_t st) {
  if (T == 0) return hipSuccess;
  // experts per workgroup: the smallest of 8, 16, 32, 64 that holds E (more
  // tokens per workgroup when there are few experts)
  const int EG = E <= 8 ? 1 : E <= 16 ? 2 : E <= 32 ? 4 : 8;
  const int TB = 1024 / EG, BE = 8 * EG;
  const dim3 grid((T + TB - 1) / TB, (E + BE - 1) / BE), block(256);
#define MOE_RX(B, G) router_exact_kernel<B, G><<<grid, block, 0, st>>>(x, Wg, bias, logits, T, H, E, vec_ok ? 1 : 0)
#define MOE_RX_EG(B)               \
  if (EG == 1) MOE_RX(B, 1);       \
  else if (EG == 2) MOE_RX(B, 2);  \
  else if (EG == 4) MOE_RX(B, 4);  \
  else MOE_RX(B, 8)
  if (bf16) {
    MOE_RX_EG(true);
  } else {
    MOE_RX_EG(false);
  }
#undef MOE_RX_EG
#undef MOE_RX
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

hipError_t launch_router_rank(const int32_t* topk_idx, int T, int E, int k, int nb, int32_t* dst_rank, int32_t* hist,
                              hipStream_t st) {
  if (T == 0) return hipSuccess;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;  // expert ids 0 .. E-1
  dim3 grid(nb, k), block(64);
  size_t shm = sizeof(int) * (size_t)E;
  router_rank_kernel<<<grid, block, shm, st>>>(topk_idx, T, E, k, nbits, nb, dst_rank, hist);
  return hipGetLastError();
}

}  // namespace moe
