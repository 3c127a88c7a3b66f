// Router logits on the bf16 matrix cores with a certified error radius, and an
// exact recomputation of the logits whose ordering the radius cannot settle.
//
// The routing decision (the k experts of a token and their order; Switch
// Transformers explainer §1.1, "Expert-parallel MoE training" explainer, router
// part) is defined on fp32 logits l = fl32(bias + sum_h x*Wg), the sum taken in
// binary64 (§2.1 of the Switch explainer keeps the router in fp32).  Here:
//
//  1. prep:    Wg [H][E] fp32 is split per element into three bf16 values,
//              w = hi + mid + lo exactly (each residual of an RNE rounding to 8
//              significant bits has at most 16, then 8 bits left), stored
//              expert-major [3][Ep][H]; partial sums of w^2 per 64 h.
//  2. approx:  v = fl32(bias + sum over 64-wide h chunks of two fp32 MFMA
//              chains, one over the 64 exact products x*hi and one over the
//              128 products x*mid, x*lo; per chunk the two chain sums are
//              added in fp32, and the chunk sums in binary64).  A sum of n
//              terms whose every addition errs by at most 2^-23 of the running
//              magnitude (round-to-nearest or truncation alike) is off by at
//              most ~n 2^-23 sum|terms|; |hi| <= (1 + 2^-8)|w| and |mid| + |lo|
//              <= 2^-7 |w|; the fp32 addition of the two chain sums errs by at
//              most 2^-24 of their magnitude; Cauchy-Schwarz gives sum|x*w| <=
//              ||x|| ||w_e||.  Hence
//                |v - l_exact| <= rho = c1 ||x|| ||w_e|| + c2 |v| + c3 |bias|.
//  3. certify: per token (one wave), the top k by (v desc, index asc) and its
//              gates.  The decision is certain when fl32(v - rho) of each
//              selected expert exceeds fl32(v + rho) of the next one and of
//              every unselected expert (fp32 rounding is monotone, so the exact
//              fp32 logits keep that order strictly).  Otherwise every expert
//              whose interval reaches the lowest selected lower bound is a
//              candidate and the token is queued.
//  4. refine:  per queued token, each candidate's logit is recomputed exactly
//              (binary64 sum of x * (hi + mid + lo), rounded once to fp32) in
//              place, then the token's top k and gates are taken again.
//
// Non-candidates keep their approximate logit, which is strictly below every
// selected exact logit, so the selection over the patched row equals the one
// over the exact logits; their gates differ from exact ones by about 1e-7
// (relative).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kChunk = 64;  // h per pipeline stage and per fp32 accumulation chain
constexpr f32x4_t kZero4 = {0.f, 0.f, 0.f, 0.f};

__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(w);
  const float r1 = w - bf16_bits_to_f32(hi);  // exact
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);  // exact, at most 8 significant bits
  lo = f32_to_bf16_bits(r2);                    // exact
}

}  // namespace

// ---------------------------------------------------------------------------
// Prep: one block per 64 experts x 64 h.  wp[p][e][h] (zero rows past E) and
// wsq[h / 64][e] = sum over the block's 64 h of w^2 (binary64, fixed order).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) router_split_prep_kernel(const float* __restrict__ Wg, int H, int E, int Ep,
                                                                uint16_t* __restrict__ wp, double* __restrict__ wsq,
                                                                int* __restrict__ count) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * 64;
  const int h0 = blockIdx.y * kChunk;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid < 2) count[tid] = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = (tid >> 6) + 4 * j;
    const int e = e0 + (tid & 63);
    tile[r][tid & 63] = e < E ? Wg[(size_t)(h0 + r) * E + e] : 0.0f;
  }
  __syncthreads();
  const int el = tid >> 2, hq = tid & 3;  // expert e0 + el, h sub-range 16*hq
  const int e = e0 + el;
  double sq = 0.0;
  uint32_t pk[3][8];
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    uint32_t h0b, m0, l0, h1b, m1, l1;
    const float a = tile[16 * hq + j][el], b = tile[16 * hq + j + 1][el];
    sq = __builtin_fma((double)a, (double)a, sq);
    sq = __builtin_fma((double)b, (double)b, sq);
    split3(a, h0b, m0, l0);
    split3(b, h1b, m1, l1);
    pk[0][j / 2] = h0b | (h1b << 16);
    pk[1][j / 2] = m0 | (m1 << 16);
    pk[2][j / 2] = l0 | (l1 << 16);
  }
  if (e < Ep) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      uint16_t* dst = wp + ((size_t)p * Ep + e) * H + h0 + 16 * hq;
      *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
      *reinterpret_cast<u32x4_t*>(dst + 8) = u32x4_t{pk[p][4], pk[p][5], pk[p][6], pk[p][7]};
    }
  }
  sq += __shfl_xor(sq, 1, 64);
  sq += __shfl_xor(sq, 2, 64);
  if (hq == 0 && e < Ep) wsq[(size_t)blockIdx.y * Ep + e] = sq;
}

// ---------------------------------------------------------------------------
// Selection on one token's logit row by a group of G lanes (G = 16, 32 or 64;
// lane g of the group holds experts g + G*j): k rounds of a group-wide maximum
// of (value desc, index asc).  All lanes of the group end with the chosen
// experts, their values and (if kIv) their interval bounds; `taken` marks the
// chosen entries in their owner lanes.
// ---------------------------------------------------------------------------
template <int G, int JE, int KMAX, bool kIv>
__device__ __forceinline__ void group_topk(const float (&v)[JE], const float (&lo)[JE], const float (&hi)[JE],
                                           bool (&taken)[JE], int k, int (&se)[KMAX], float (&sv)[KMAX],
                                           float (&slo)[KMAX], float (&shi)[KMAX]) {
  const int lg = threadIdx.x & (G - 1);
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r >= k) break;
    float bv = -__builtin_inff(), blo = 0.f, bhi = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < JE; ++j)
      if (!taken[j] && (v[j] > bv || (v[j] == bv && lg + G * j < be))) {
        bv = v[j];
        be = lg + G * j;
        if (kIv) {
          blo = lo[j];
          bhi = hi[j];
        }
      }
#pragma unroll
    for (int d = G / 2; d > 0; d >>= 1) {
      const float ov = __shfl_xor(bv, d, 64);
      const int oe = __shfl_xor(be, d, 64);
      float olo = 0.f, ohi = 0.f;
      if (kIv) {
        olo = __shfl_xor(blo, d, 64);
        ohi = __shfl_xor(bhi, d, 64);
      }
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
        if (kIv) {
          blo = olo;
          bhi = ohi;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < JE; ++j)
      if (lg + G * j == be) taken[j] = true;
    se[r] = be;
    sv[r] = bv;
    slo[r] = blo;
    shi[r] = bhi;
  }
}

// Gates of the chosen experts (gate_mode 0: softmax over all E; otherwise the
// softmax over the k chosen; kSigmoidFlag: sigmoid scores, see gate_value);
// choice r is written by lane r % G of the group.
template <int G, int JE, int KMAX>
__device__ __forceinline__ void group_gates(const float (&v)[JE], int E, int k, int gate_mode, const int (&se)[KMAX],
                                            const float (&sv)[KMAX], int t, bool active,
                                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                                            int* m_idx = nullptr, float* m_gate = nullptr) {
  const int lg = threadIdx.x & (G - 1);
  const float m = sv[0];
  float den = 0.0f;
  if (gate_mode == 0) {  // softmax scores, no renormalisation
#pragma unroll
    for (int j = 0; j < JE; ++j)
      if (lg + G * j < E) den += expf(v[j] - m);
#pragma unroll
    for (int d = G / 2; d > 0; d >>= 1) den += __shfl_xor(den, d, 64);
  } else {
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
      if (r < k) den += expf(sv[r] - m);
  }
  if (!active) return;
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    if (r < k && (r & (G - 1)) == lg) {  // every choice r < k has a writer, also when G < k
      const float g = gate_value<KMAX>(gate_mode, k, sv, den, r);
      topk_idx[(size_t)t * k + r] = se[r];
      topk_gate[(size_t)t * k + r] = g;
      if (m_idx) {  // the token's row of a workgroup-local copy
        m_idx[r] = se[r];
        m_gate[r] = g;
      }
    }
}

// Choices, gates and certification of one token held by a group of G lanes
// (v: approximate logits; wne: ||w_e|| rounded up; be: bias; xn: bound on
// ||x||; all radius arithmetic in fp32 rounded up by a 2^-20 margin).  An
// undecided token is queued with the experts whose exact logit is needed: the
// chosen ones whose interval meets another chosen one's or an unchosen one's,
// and the unchosen ones whose interval reaches the lowest chosen lower bound.
// Every other expert's interval is disjoint from all intervals that matter, so
// its approximate logit sorts where its exact one would.
template <int G, int JE, int KMAX>
__device__ __forceinline__ void certify_token(const float (&v)[JE], const float (&wne)[JE], const float (&be)[JE],
                                              int E, int H, int k, int gate_mode, float c1, bool active, int t,
                                              float xn, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_gate, int2* __restrict__ pairs,
                                              int4* __restrict__ utok, int* __restrict__ count,
                                              int* m_idx = nullptr, float* m_gate = nullptr) {
  const int lane = threadIdx.x & 63, lg = lane & (G - 1);
  constexpr float up = 1.0f + 0x1p-20f;
  const float c2 = 0x1p-24f + 0x1p-44f;
  const float c3 = (float)H * 0x1p-52f;
  float lo[JE], hi[JE];
  bool taken[JE];
  bool bad = !(xn <= 1e30f);
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    if (lg + G * j < E) {
      const float rho = (c1 * xn * wne[j] + c2 * fabsf(v[j]) + c3 * fabsf(be[j])) * up + 1e-30f;
      lo[j] = v[j] - rho;
      hi[j] = v[j] + rho;
      bad |= !(fabsf(v[j]) <= 3.0e38f) || !(rho <= 1e30f);
      taken[j] = false;
    } else {
      lo[j] = hi[j] = -__builtin_inff();
      taken[j] = true;
    }
  }
  int se[KMAX];
  float sv[KMAX], slo[KMAX], shi[KMAX];
  group_topk<G, JE, KMAX, true>(v, lo, hi, taken, k, se, sv, slo, shi);
  group_gates<G, JE, KMAX>(v, E, k, gate_mode, se, sv, t, active, topk_idx, topk_gate, m_idx, m_gate);

  float tau = slo[0];
  bool ordered = true;
#pragma unroll
  for (int r = 1; r < KMAX; ++r)
    if (r < k) {
      ordered &= slo[r - 1] > shi[r];
      tau = fminf(tau, slo[r]);
    }
  float rest = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < JE; ++j)
    if (!taken[j] && lg + G * j < E) rest = fmaxf(rest, hi[j]);
#pragma unroll
  for (int d = G / 2; d > 0; d >>= 1) rest = fmaxf(rest, __shfl_xor(rest, d, 64));
  const uint64_t gmask = (G == 64 ? ~0ull : ((1ull << (G & 63)) - 1)) << (lane & ~(G - 1));
  bad = (__ballot(bad) & gmask) != 0;
  const bool queue = active && (bad || !ordered || !(tau > rest));

  bool cand[JE];
  uint64_t bj[JE];
  int total = 0;
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    const int e = lg + G * j;
    bool need = false;
    if (queue && e < E) {
      if (bad) {
        need = true;
      } else if (taken[j]) {
        need = lo[j] <= rest;
#pragma unroll
        for (int r = 0; r < KMAX; ++r)
          if (r < k && se[r] != e && slo[r] <= hi[j] && shi[r] >= lo[j]) need = true;
      } else {
        need = hi[j] >= tau;
      }
    }
    cand[j] = need;
    bj[j] = __ballot(need) & gmask;
    total += __popcll(bj[j]);
  }
  int base = 0;
  if (queue && lg == 0) {
    base = atomicAdd(&count[0], total);
    const int slot = atomicAdd(&count[1], 1);
    utok[slot] = int4{t, base, total, 0};
  }
  base = __shfl(base, lane & ~(G - 1), 64);
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int off = 0;
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    if (cand[j]) pairs[base + off + __popcll(bj[j] & lt)] = int2{t, lg + G * j};
    off += __popcll(bj[j]);
  }
}

// sum_h x[h] * (hi + mid + lo)[e][h] in binary64 over one wave (lanes over h);
// every lane returns the sum.
__device__ __forceinline__ double exact_dot(const uint16_t* __restrict__ xr, const uint16_t* __restrict__ wp, int e,
                                            int H, int Ep) {
  const int lane = threadIdx.x & 63;
  const uint16_t* w0 = wp + (size_t)e * H;
  const uint16_t* w1 = wp + ((size_t)Ep + e) * H;
  const uint16_t* w2 = wp + ((size_t)2 * Ep + e) * H;
  double s = 0.0;
  for (int h = 8 * lane; h < H; h += 512) {
    const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + h);
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(w0 + h);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(w1 + h);
    const u32x4_t cc = *reinterpret_cast<const u32x4_t*>(w2 + h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int sh = half ? 0 : 16;
        const uint32_t m = half ? 0xFFFF0000u : 0xFFFFFFFFu;
        const double xd = (double)__uint_as_float((xv[q] << sh) & m);
        const double wd = (double)__uint_as_float((a[q] << sh) & m) + (double)__uint_as_float((b[q] << sh) & m) +
                          (double)__uint_as_float((cc[q] << sh) & m);
        s = __builtin_fma(xd, wd, s);
      }
    }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d, 64);
  return s;
}

// The same sum over the fp32 weights Wg [H][E] directly (w = hi + mid + lo, so
// the binary64 result is the same).
__device__ __forceinline__ double exact_dot_raw(const uint16_t* __restrict__ xr, const float* __restrict__ Wg, int e,
                                                int H, int E) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int h = 8 * lane; h < H; h += 512) {
    const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t bits = half ? (xv[q] & 0xFFFF0000u) : (xv[q] << 16);
        s = __builtin_fma((double)__uint_as_float(bits), (double)Wg[(size_t)(h + 2 * q + half) * E + e], s);
      }
    }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d, 64);
  return s;
}

// Bound on ||x|| from an fp32 sum of squares of bf16 values, in any order
// (each of the <= 2H roundings errs by at most 2^-23 relative, or by at most
// 2^-126 absolute where the matrix cores flush a tiny product or partial sum
// to zero), and on the rounding of the square root.
__device__ __forceinline__ float xnorm_bound(float sq, int H) {
  return sqrtf((sq + (float)(2 * H) * 0x1p-126f) * (1.0f + (float)H * 0x1p-22f + 0x1p-20f)) * (1.0f + 0x1p-20f);
}

// Work the fused epilogue takes over from later kernels when its token tile
// is a whole number of 64-token blocks: the ranks and per-block expert counts
// (dst_rank non-null) and the per-block loss partials (Ppart non-null).
struct SplitTail {
  int32_t* dst_rank;      // [T][k] rank among the block's tokens with the same choice
  int32_t* hist;          // [E][k][nb] choices per expert, choice and block
  int nbits, nb;          // bits of an expert id 0..E-1; 64-token blocks
  double* Ppart;          // [E][nb] sum over the block of P(e | t)
  double* Zpart;          // [nb] sum over the block of logsumexp^2
  int32_t* Cpart;         // [E][nb] first choices per expert
  int score_fn;           // 0: softmax, 1: sigmoid over their sum
};

// ---------------------------------------------------------------------------
// Approximate logits: v_mfma_f32_16x16x32_bf16 on x (bf16, exact) times the
// weight pieces.  8 waves as TG token groups x EG expert groups x KS h slices;
// a wave owns 16*MF tokens x 16*WN experts of its slice.  A stage holds, per
// slice, BM x-rows and 3*BN piece rows of 64 h (128 B per row, chunk c of row r
// at slot c ^ ((r >> 1) & 7), so the 16 rows a 16-lane LDS read phase touches
// hit distinct banks), filled by direct-to-LDS loads; S stages in a ring.
// After every stage both fp32 chains are added into binary64 accumulators and
// cleared.  Slices are combined through LDS in slice order.  Also writes
// sum_h x^2 per token (fp32), and the blocks of the first token tile write the
// norms ||w_e|| of their experts.
// ---------------------------------------------------------------------------
template <int TG, int EG, int KS, int MF, int WN, int S, bool FUSE, int KMAX, bool RAW>
__global__ void __launch_bounds__(512) router_split_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wp, const float* __restrict__ Wg,
    const float* __restrict__ bias,
    const double* __restrict__ wsq, float* __restrict__ logits, double* __restrict__ lpart, float* __restrict__ xsq,
    double* __restrict__ wn, int T, int H, int E, int Ep, int k, int gate_mode, double c1,
    int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, int2* __restrict__ pairs, int4* __restrict__ utok, int* __restrict__ count,
    SplitTail tail) {
  static_assert(TG * EG * KS == 8, "8 waves");
  constexpr int BM = 16 * MF * TG, BN = 16 * WN * EG;
  static_assert(!RAW || (FUSE && KS == 1 && BN == 64), "fp32 weights in the stage: one slice of 64 experts");
  constexpr int SR = BM + 3 * BN;  // rows per slice per stage
  constexpr int ROWS = KS * SR;
  // 64-lane load instructions per stage: 8 rows of 64 h each; with RAW the
  // weight block (64 h x 64 experts fp32, 16 KB) takes 16 more
  constexpr int NIX = BM / 8;
  constexpr int NI = RAW ? NIX + 16 : ROWS / 8;
  constexpr int L = (NI + 7) / 8;
  constexpr int STAGE = RAW ? BM * kChunk + 64 * 64 * 2 : ROWS * kChunk;  // bf16 elements
  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tg = w % TG, eg = (w / TG) % EG, ks = w / (TG * EG);
  const int t0 = blockIdx.x * BM, e0 = blockIdx.y * BN;
  const int nk = H / kChunk;
  // Unfused (the experts span several workgroups): the h chunks are also
  // split over gridDim.z workgroups, each writing the binary64 sums of its
  // own chunks; they are added in z order when the logits are certified.
  const int nkw = FUSE ? nk : nk / (int)gridDim.z;   // chunks of this workgroup
  const int kc0 = FUSE ? 0 : (int)blockIdx.z * nkw;  // its first chunk
  const int nks = nkw / KS;                          // stages (chunks per slice)

  auto lds_pos = [](int r, int c) { return (r * 8 + (c ^ ((r >> 1) & 7))) * 8; };

  // Operands of the fused epilogue, loaded now so that their latency overlaps
  // the main loop: the bias of expert tid, and the squared weight norms of two
  // h chunks per thread (thread tid: expert tid % BN, chunks tid / BN + 8 q).
  constexpr int NG = 512 / BN;
  __shared__ float s_bias[BN];
  float bpre = 0.0f;
  double wpre[2] = {0.0, 0.0};
  if constexpr (FUSE) {
    if (bias && tid < BN && e0 + tid < E) bpre = bias[e0 + tid];
    if constexpr (!RAW) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int hb = tid / BN + q * NG;
        if (hb < nk) wpre[q] = wsq[(size_t)hb * Ep + e0 + tid % BN];
      }
    }
  }

  // Each load instruction's address at the first stage, computed once: a stage
  // adds 128 bytes (the next 64 h of a bf16 row) or, for the fp32 weight block,
  // 64 rows of E floats.
  uintptr_t lbase[L];
  bool lraw[L];
#pragma unroll
  for (int q = 0; q < L; ++q) {
    int g = q * 8 + w;
    if (g >= NI) g = NI - 1;  // waves without a group of their own repeat the last one
    lraw[q] = RAW && g >= NIX;
    if (RAW && g >= NIX) {
      // weight block: 16-byte slot s of row h holds experts 4 (s ^ 4((h >> 3) & 3)) .. +3,
      // so the four 8-h groups a fragment read spans fall on different banks
      const int q2 = (g - NIX) * 64 + lane;
      const int hr = q2 >> 4;
      int c4 = ((q2 & 15) ^ (((hr >> 3) & 3) << 2)) * 4;
      if (e0 + c4 >= E) c4 = 0;  // columns past E: any valid address (never used)
      lbase[q] = reinterpret_cast<uintptr_t>(Wg + (size_t)hr * E + e0 + c4);
      continue;
    }
    const int p = g * 64 + lane;
    const int r = p >> 3;
    const int c = (p & 7) ^ ((r >> 1) & 7);
    const int sl = r / SR, rr = r % SR;
    const int h = (kc0 + sl * nks) * kChunk + c * 8;
    const uint16_t* src;
    if (rr < BM) {
      const int t = t0 + rr < T ? t0 + rr : T - 1;
      src = x + (size_t)t * H + h;
    } else {
      const int q2 = rr - BM;
      src = wp + ((size_t)(q2 / BN) * Ep + e0 + q2 % BN) * H + h;
    }
    lbase[q] = reinterpret_cast<uintptr_t>(src);
  }
  const size_t wstep = (size_t)kChunk * E * sizeof(float);
  auto issue = [&](int buf, int j) {
    uint16_t* st = smem + buf * STAGE;
#pragma unroll
    for (int q = 0; q < L; ++q) {
      const int g = q * 8 + w < NI ? q * 8 + w : NI - 1;
      const uintptr_t a = lbase[q] + (size_t)j * (lraw[q] ? wstep : (size_t)kChunk * sizeof(uint16_t));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(a), st + g * 512, 16, 0, 0);
    }
  };

  f32x4_t acc_hi[MF][WN], acc_ml[MF][WN];
  double acc64[MF][WN][4];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      acc_hi[i][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc_ml[i][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc64[i][n][j] = 0.0;
    }
  // sum_h x^2 of the wave's token rows (waves of expert group 0): the diagonal
  // of x x^T, accumulated on the matrix cores from the x fragments themselves
  f32x4_t acc_sq[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) acc_sq[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float sq[MF];
  float wsum[WN];  // RAW: sum of w^2 over this lane's fragments (waves of token group 0)
#pragma unroll
  for (int n = 0; n < WN; ++n) wsum[n] = 0.0f;

  int issued = 0;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (issued < nks) issue(issued % S, issued), ++issued;

  const int rbase = ks * SR;
  for (int j = 0; j < nks; ++j) {
    wait_stages<L>(issued - j - 1);
    lds_barrier();
    if (issued < nks) issue(issued % S, issued), ++issued;
    const uint16_t* st = smem + (j % S) * STAGE;
    // RAW: both k-steps' fp32 weights read up front, so the reads of the second
    // overlap the splitting and MFMAs of the first
    float wraw[RAW ? 2 : 1][WN][8];
    if constexpr (RAW) {
      const float* wb = reinterpret_cast<const float*>(st + BM * kChunk);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k0 = kk * 32 + 8 * (lane >> 4);
        const int sw = ((k0 >> 3) & 3) << 2;
#pragma unroll
        for (int n = 0; n < WN; ++n) {
          const int e = (eg * WN + n) * 16 + (lane & 15);
          const int col = (((e >> 2) ^ sw) << 2) | (e & 3);
#pragma unroll
          for (int i = 0; i < 8; ++i) wraw[kk][n][i] = wb[(k0 + i) * 64 + col];
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8_t a[MF];
#pragma unroll
      for (int i = 0; i < MF; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(st + lds_pos(rbase + (tg * MF + i) * 16 + (lane & 15), c));
      if constexpr (RAW) {
        // the 8 fp32 weights of this lane's fragment (expert e, h = k0 .. k0+7), split
        // here into bf16 hi + mid + lo by truncation (w = hi + mid + lo exactly)
#pragma unroll
        for (int n = 0; n < WN; ++n) {
          u32x4_t ph, pm, pl;
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            uint32_t hb2[2], mb2[2], lb2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float wv = wraw[kk][n][i + u];
              const float hf = __uint_as_float(__float_as_uint(wv) & 0xFFFF0000u);
              const float r1 = wv - hf;
              const float mf = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
              const float r2 = r1 - mf;
              hb2[u] = __float_as_uint(hf) >> 16;
              mb2[u] = __float_as_uint(mf) >> 16;
              lb2[u] = __float_as_uint(r2) >> 16;
              if (tg == 0) wsum[n] = __builtin_fmaf(wv, wv, wsum[n]);
            }
            ph[i / 2] = hb2[0] | (hb2[1] << 16);
            pm[i / 2] = mb2[0] | (mb2[1] << 16);
            pl[i / 2] = lb2[0] | (lb2[1] << 16);
          }
          const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, ph), bm = __builtin_bit_cast(bf16x8_t, pm),
                         bl = __builtin_bit_cast(bf16x8_t, pl);
#pragma unroll
          for (int i = 0; i < MF; ++i) {
            // each stage's chains start from a zero C operand (no clearing)
            acc_hi[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bh, kk == 0 ? kZero4 : acc_hi[i][n], 0, 0, 0);
            acc_ml[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bm, kk == 0 ? kZero4 : acc_ml[i][n], 0, 0, 0);
            acc_ml[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bl, acc_ml[i][n], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int n = 0; n < WN; ++n) {
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(
                st + lds_pos(rbase + BM + p * BN + (eg * WN + n) * 16 + (lane & 15), c));
#pragma unroll
            for (int i = 0; i < MF; ++i) {
              // each stage's chains start from a zero C operand (no clearing)
              if (p == 0)
                acc_hi[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, kk == 0 ? kZero4 : acc_hi[i][n], 0, 0, 0);
              else
                acc_ml[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a[i], b, kk == 0 && p == 1 ? kZero4 : acc_ml[i][n], 0, 0, 0);
            }
          }
      }
      if (eg == 0) {
#pragma unroll
        for (int i = 0; i < MF; ++i) acc_sq[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], a[i], acc_sq[i], 0, 0, 0);
      }
    }
    // the two chain sums are added in fp32 (one more rounding, at most 2^-24
    // of their magnitude), then into the binary64 accumulators
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int n = 0; n < WN; ++n)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc64[i][n][jj] += (double)(acc_hi[i][n][jj] + acc_ml[i][n][jj]);
  }

  // row sums of x^2 to every lane l of row l%16: entry (t, t) of the 16 x 16
  // block is element t%4 of lane 16 (t/4) + t
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int t = lane & 15, q = lane & 3;
    const float d = q == 0 ? acc_sq[i][0] : q == 1 ? acc_sq[i][1] : q == 2 ? acc_sq[i][2] : acc_sq[i][3];
    sq[i] = __shfl(d, 16 * (t >> 2) + t, 64);
  }

  // slices > 0 hand their partial sums to slice 0 through LDS
  if (KS > 1) {
    wait_vmcnt<0>();
    __syncthreads();
    double* red = reinterpret_cast<double*>(smem);
    float* rsq = reinterpret_cast<float*>(red + (size_t)(KS - 1) * TG * EG * MF * WN * 4 * 64);
    const int wi = tg + TG * eg;
    if (ks > 0) {
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int n = 0; n < WN; ++n)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            red[((((size_t)(ks - 1) * TG * EG + wi) * MF + i) * WN * 4 + n * 4 + jj) * 64 + lane] = acc64[i][n][jj];
      if (eg == 0)
#pragma unroll
        for (int i = 0; i < MF; ++i) rsq[(((ks - 1) * TG + tg) * MF + i) * 64 + lane] = sq[i];
    }
    __syncthreads();
    if (ks == 0) {
      for (int k2 = 1; k2 < KS; ++k2) {
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int n = 0; n < WN; ++n)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              acc64[i][n][jj] +=
                  red[((((size_t)(k2 - 1) * TG * EG + wi) * MF + i) * WN * 4 + n * 4 + jj) * 64 + lane];
        if (eg == 0)
#pragma unroll
          for (int i = 0; i < MF; ++i) sq[i] += rsq[(((k2 - 1) * TG + tg) * MF + i) * 64 + lane];
      }
    }
  }

  if (!FUSE) {
    if (blockIdx.x == 0 && blockIdx.z == 0 && tid < BN && e0 + tid < E) {
      double s = 0.0;
      for (int hb = 0; hb < nk; ++hb) s += wsq[(size_t)hb * Ep + e0 + tid];
      wn[e0 + tid] = sqrt(s * (1.0 + 0x1p-40));
    }
    if (ks != 0) return;
  }

  // accumulator lane l: tokens 4*(l/16) + jj, expert l%16 of the fragment
  constexpr int SV = BN + 1;  // row stride of the staged logits
  float* s_v = reinterpret_cast<float*>(smem);
  float* s_x = s_v + BM * SV;
  if (FUSE) {
    if (KS == 1) wait_vmcnt<0>();
    if (tid < BN) s_bias[tid] = bpre;
    __syncthreads();  // every wave is done with the stage buffers (and slice partials)
  }
  if (ks == 0) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int el = (eg * WN + n) * 16 + (lane & 15);
      const int e = e0 + el;
      if (e >= E) continue;
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int tl = (tg * MF + i) * 16 + 4 * (lane >> 4) + jj;
          if constexpr (FUSE) {
            const float v = (float)(acc64[i][n][jj] + (double)s_bias[el]);
            if (t0 + tl < T) logits[(size_t)(t0 + tl) * E + e] = v;
            s_v[tl * SV + el] = v;
          } else if (t0 + tl < T) {
            lpart[((size_t)blockIdx.z * T + t0 + tl) * Ep + e] = acc64[i][n][jj];
          }
        }
    }
    if (eg == 0 && lane < 16) {
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const int tl = (tg * MF + i) * 16 + lane;
        if (!FUSE && t0 + tl < T) xsq[(size_t)blockIdx.z * T + t0 + tl] = sq[i];
        if (FUSE) s_x[tl] = sq[i];
      }
    }
  }
  if constexpr (FUSE) {
    // the workgroup holds all E logits of its BM tokens: choices, gates and
    // certification here in one pass, G lanes per token, JE experts per lane
    static_assert(BN <= 64, "all experts in one tile");
    constexpr int G0 = 512 / BM < BN ? 512 / BM : BN;
    constexpr int G = G0 >= 64 ? 64 : G0;
    constexpr int JE = BN / G;
    const int lg = lane & (G - 1);
    const int tl = tid / G;  // token of this group
    __shared__ float s_wn[BN];  // ||w_e||, rounded up
    double* s_wpart = reinterpret_cast<double*>(s_x + BM);  // [NG][BN] partial sums
    if constexpr (RAW) {
      // the four k groups of a fragment (lanes l, l^16, l^32, l^48) hold one expert's sums
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        float sn = wsum[n];
        sn += __shfl_xor(sn, 16, 64);
        sn += __shfl_xor(sn, 32, 64);
        const int e = (eg * WN + n) * 16 + lane;
        if (tg == 0 && lane < 16) s_wn[e] = e0 + e < E ? xnorm_bound(sn, H) : 0.0f;
      }
    } else {
      double sw = wpre[0] + wpre[1];
      for (int hb = tid / BN + 2 * NG; hb < nk; hb += NG) sw += wsq[(size_t)hb * Ep + tid % BN];
      s_wpart[tid] = sw;
      __syncthreads();
      if (tid < BN) {
        double sw2 = 0.0;
#pragma unroll
        for (int g = 0; g < NG; ++g) sw2 += s_wpart[g * BN + tid];
        s_wn[tid] = tid < E ? (float)sqrt(sw2 * (1.0 + 0x1p-40)) * (1.0f + 0x1p-20f) : 0.0f;
      }
    }
    __shared__ int s_cnt[2];  // candidate pairs, queued tokens of this workgroup
    if (tid < 2) s_cnt[tid] = 0;
    __syncthreads();
    float wne[JE], be[JE], v[JE];
#pragma unroll
    for (int j = 0; j < JE; ++j) {
      const int e = lg + G * j;
      wne[j] = e < E ? s_wn[e] : 0.0f;
      be[j] = e < E ? s_bias[e] : 0.0f;
    }
    const int t = t0 + tl;
    const bool active = tl < BM && t < T;
#pragma unroll
    for (int j = 0; j < JE; ++j) {
      const int e = lg + G * j;
      v[j] = (active && e < E) ? s_v[tl * SV + e] : -__builtin_inff();
    }
    const float xn = active ? xnorm_bound(s_x[tl], H) : 0.0f;
    int4* s_utok = reinterpret_cast<int4*>(s_wpart + 512);  // [BM]
    int2* s_pairs = reinterpret_cast<int2*>(s_utok + BM);     // [BM * BN]
    double* s_lp = reinterpret_cast<double*>(s_pairs + BM * BN);  // [8][64] loss partials
    int* s_lc = reinterpret_cast<int*>(s_lp + 512);               // [8][64]
    double* s_lz = reinterpret_cast<double*>(s_lc + 512);         // [8]
    int* s_idx = reinterpret_cast<int*>(s_lz + 8);                // [BM][k] final choices
    float* s_gt = reinterpret_cast<float*>(s_idx + BM * KMAX);    // [BM][k] their gates
    int* s_rc = reinterpret_cast<int*>(s_gt + BM * KMAX);         // [BM / 64][64 + 1] expert counts
    const bool mirror = tail.dst_rank != nullptr || tail.Ppart != nullptr;
    certify_token<G, JE, KMAX>(v, wne, be, E, H, k, gate_mode, (float)c1 * (1.0f + 0x1p-20f), active,
                               active ? t : 0, xn, topk_idx, topk_gate, s_pairs, s_utok, s_cnt,
                               mirror && active ? s_idx + tl * k : nullptr, s_gt + tl * k);
    __syncthreads();
    // refine the queued tokens here: exact logits of the candidates (a wave
    // per pair), then the selection again over the patched rows (a wave per token)
    const int npairs = s_cnt[0], ntok = s_cnt[1];
    if (ntok > 0) {
      for (int c = w; c < npairs; c += 8) {
        const int2 pr = s_pairs[c];
        const double sx = RAW ? exact_dot_raw(x + (size_t)pr.x * H, Wg, pr.y, H, E)
                              : exact_dot(x + (size_t)pr.x * H, wp, pr.y, H, Ep);
        if (lane == 0) {
          const float lv = (float)(sx + (double)s_bias[pr.y]);
          logits[(size_t)pr.x * E + pr.y] = lv;
          s_v[(pr.x - t0) * SV + pr.y] = lv;
        }
      }
      __syncthreads();
      for (int u = w; u < ntok; u += 8) {
        const int tq = s_utok[u].x;
        float rv[1], dummy[1];
        bool taken[1];
        rv[0] = lane < E ? s_v[(tq - t0) * SV + lane] : -__builtin_inff();
        dummy[0] = 0.f;
        taken[0] = lane >= E;
        int se[KMAX];
        float sv[KMAX], s1[KMAX], s2[KMAX];
        group_topk<64, 1, KMAX, false>(rv, dummy, dummy, taken, k, se, sv, s1, s2);
        group_gates<64, 1, KMAX>(rv, E, k, gate_mode, se, sv, tq, true, topk_idx, topk_gate,
                                 mirror ? s_idx + (tq - t0) * k : nullptr, s_gt + (tq - t0) * k);
      }
    }
    if (tail.dst_rank || tail.Ppart) {
      __syncthreads();  // every token's final choices are written
      constexpr int RB = BM / 64 > 0 ? BM / 64 : 1;  // 64-token blocks of this workgroup
      const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
      if (tail.dst_rank && w < RB && (blockIdx.x * RB + w) * 64 < T) {
        // ranks: position among the block's earlier tokens with the same choice;
        // counts per expert
        const int b = blockIdx.x * RB + w, tr = b * 64 + lane;
        const bool valid = tr < T;
        const int Q = k * tail.nb;
        const uint64_t vmask = __ballot(valid);
        int ti[KMAX];
#pragma unroll
        for (int r = 0; r < KMAX; ++r) ti[r] = (valid && r < k) ? s_idx[(w * 64 + lane) * k + r] : 0;
        int* cnt_e = s_rc + w * 65;  // this wave's counts
#pragma unroll
        for (int r = 0; r < KMAX; ++r) {
          if (r >= k) break;
          const int my_e = ti[r];
          uint64_t same = vmask;
          for (int bit = 0; bit < tail.nbits; ++bit) {
            const uint64_t mb = __ballot((my_e >> bit) & 1);
            same &= ((my_e >> bit) & 1) ? mb : ~mb;
          }
          if (valid) tail.dst_rank[(size_t)tr * k + r] = __popcll(same & lt);
          // the first lane of each choice group writes the group's size (the
          // wave's LDS operations complete in order)
          cnt_e[lane] = 0;
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          __builtin_amdgcn_wave_barrier();
          if (valid && (same & lt) == 0) cnt_e[my_e] = __popcll(same);
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          __builtin_amdgcn_wave_barrier();
          if (lane < E) tail.hist[(size_t)lane * Q + r * tail.nb + b] = cnt_e[lane];
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      }
      if (tail.Ppart) {
        // loss partials: P(e | t) (softmax, or sigmoid scores over their sum),
        // logsumexp^2 and first choices, lane = expert; each wave sums its
        // tokens in order, the waves of a block are added in wave order
        constexpr int WPB = 8 / RB, TPW = 64 / WPB;
        const int rb = w / WPB;
        double acc = 0.0, z = 0.0;
        int cnt = 0;
        // the TPW tokens' reductions side by side (independent shuffle chains);
        // tokens past T contribute nothing
        constexpr int TU = TPW < 8 ? TPW : 8;
        for (int u0 = 0; u0 < TPW; u0 += TU) {
          float vv[TU], m[TU], den[TU];
          bool ok[TU];
#pragma unroll
          for (int u = 0; u < TU; ++u) {
            const int tl = rb * 64 + (w % WPB) * TPW + u0 + u;
            ok[u] = t0 + tl < T;
            vv[u] = (ok[u] && lane < E) ? s_v[tl * SV + lane] : -__builtin_inff();
            m[u] = vv[u];
          }
#pragma unroll
          for (int d = 32; d > 0; d >>= 1)
#pragma unroll
            for (int u = 0; u < TU; ++u) m[u] = fmaxf(m[u], __shfl_xor(m[u], d, 64));
#pragma unroll
          for (int u = 0; u < TU; ++u) den[u] = (ok[u] && lane < E) ? expf(vv[u] - m[u]) : 0.0f;
          float ex[TU];
#pragma unroll
          for (int u = 0; u < TU; ++u) ex[u] = den[u];
#pragma unroll
          for (int d = 32; d > 0; d >>= 1)
#pragma unroll
            for (int u = 0; u < TU; ++u) den[u] += __shfl_xor(den[u], d, 64);
          if (tail.score_fn) {
            float sc[TU], ss[TU];
#pragma unroll
            for (int u = 0; u < TU; ++u) ss[u] = sc[u] = (ok[u] && lane < E) ? 1.0f / (1.0f + expf(-vv[u])) : 0.0f;
#pragma unroll
            for (int d = 32; d > 0; d >>= 1)
#pragma unroll
              for (int u = 0; u < TU; ++u) ss[u] += __shfl_xor(ss[u], d, 64);
#pragma unroll
            for (int u = 0; u < TU; ++u)
              if (ok[u]) acc += (double)(sc[u] / ss[u]);
          } else {
#pragma unroll
            for (int u = 0; u < TU; ++u)
              if (ok[u]) acc += (double)(ex[u] / den[u]);
          }
#pragma unroll
          for (int u = 0; u < TU; ++u) {
            if (!ok[u]) continue;
            const int tl = rb * 64 + (w % WPB) * TPW + u0 + u;
            const double lse = (double)m[u] + (double)logf(den[u]);
            z += lse * lse;
            cnt += lane == s_idx[tl * k];
          }
        }
        s_lp[w * 64 + lane] = acc;
        s_lc[w * 64 + lane] = cnt;
        if (lane == 0) s_lz[w] = z;
        __syncthreads();
        if (tid < RB * 64) {
          const int rb2 = tid / 64, e = tid % 64, b = blockIdx.x * RB + rb2;
          if (b * 64 < T) {
            double ps = 0.0, zs = 0.0;
            int cs = 0;
            for (int q = 0; q < WPB; ++q) {
              ps += s_lp[(rb2 * WPB + q) * 64 + e];
              cs += s_lc[(rb2 * WPB + q) * 64 + e];
              zs += s_lz[rb2 * WPB + q];
            }
            if (e < E) {
              tail.Ppart[(size_t)e * tail.nb + b] = ps;
              tail.Cpart[(size_t)e * tail.nb + b] = cs;
            }
            if (e == 0) tail.Zpart[b] = zs;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Certify + select (experts beyond one workgroup's tile): one wave per token.
// The approximate logit is the binary64 sum of the HS partial sums (in their
// order) plus the bias, rounded once to fp32; sum_h x^2 the fp32 sum of its
// HS parts.
// ---------------------------------------------------------------------------
template <int JE, int KMAX>
__global__ void __launch_bounds__(256) router_certify_kernel(const double* __restrict__ lpart, int HS,
                                                             float* __restrict__ logits,
                                                             const float* __restrict__ xsq,
                                                             const double* __restrict__ wn,
                                                             const float* __restrict__ bias, int T, int H, int E,
                                                             int Ep, int k, int gate_mode, double c1,
                                                             int32_t* __restrict__ topk_idx,
                                                             float* __restrict__ topk_gate, int2* __restrict__ pairs,
                                                             int4* __restrict__ utok, int* __restrict__ count) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float* row = logits + (size_t)t * E;
  float sq = 0.0f;
  for (int z = 0; z < HS; ++z) sq += xsq[(size_t)z * T + t];
  const float xn = xnorm_bound(sq, H);
  float v[JE], be[JE], wne[JE];
#pragma unroll
  for (int j = 0; j < JE; ++j) {
    const int e = lane + 64 * j;
    wne[j] = e < E ? (float)wn[e] * (1.0f + 0x1p-20f) : 0.0f;
    be[j] = (bias && e < E) ? bias[e] : 0.0f;
    v[j] = -__builtin_inff();
    if (e < E) {
      double s = 0.0;
      for (int z = 0; z < HS; ++z) s += lpart[((size_t)z * T + t) * Ep + e];
      v[j] = (float)(s + (double)be[j]);
      row[e] = v[j];
    }
  }
  certify_token<64, JE, KMAX>(v, wne, be, E, H, k, gate_mode, (float)c1 * (1.0f + 0x1p-20f), true, t, xn, topk_idx,
                              topk_gate, pairs, utok,
                              count);
}

// ---------------------------------------------------------------------------
// Refine: one block (4 waves) per queued token.  Each wave recomputes whole
// candidates: binary64 sum of x[t][h] * (hi+mid+lo), lane-strided over h in
// 8-element groups, a fixed butterfly across the wave, plus the bias, rounded
// once to fp32.  Then wave 0 takes the token's top k and gates again.
// ---------------------------------------------------------------------------
template <int JE, int KMAX>
__global__ void __launch_bounds__(256) router_refine_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wp,
                                                            const float* __restrict__ bias,
                                                            const int2* __restrict__ pairs,
                                                            const int4* __restrict__ utok,
                                                            const int* __restrict__ count, float* __restrict__ logits,
                                                            int H, int E, int Ep, int k, int gate_mode,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ntok = count[1];
  for (int u = blockIdx.x; u < ntok; u += gridDim.x) {
    const int4 rec = utok[u];
    const int t = rec.x;
    const uint16_t* xr = x + (size_t)t * H;
    for (int c = w; c < rec.z; c += 4) {
      const int e = pairs[rec.y + c].y;
      const double s = exact_dot(xr, wp, e, H, Ep);
      if (lane == 0) logits[(size_t)t * E + e] = (float)(s + (bias ? (double)bias[e] : 0.0));
    }
    __syncthreads();
    if (w == 0) {
      const float* row = logits + (size_t)t * E;
      float v[JE], dummy[JE];
      bool taken[JE];
#pragma unroll
      for (int j = 0; j < JE; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < E ? row[e] : -__builtin_inff();
        dummy[j] = 0.f;
        taken[j] = e >= E;
      }
      int se[KMAX];
      float sv[KMAX], s1[KMAX], s2[KMAX];
      group_topk<64, JE, KMAX, false>(v, dummy, dummy, taken, k, se, sv, s1, s2);
      group_gates<64, JE, KMAX>(v, E, k, gate_mode, se, sv, t, true, topk_idx, topk_gate);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
int split_router_bn(int E) { return E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : 128; }

int split_router_ep(int E) {
  const int bn = split_router_bn(E);
  return (E + bn - 1) / bn * bn;
}

int split_router_hs(int H) { return H / kChunk; }

// Workgroups the unfused logits split h over (a divisor of the chunk count):
// the largest power of two up to 8 that keeps the grid of 256-token x
// 64-expert tiles within 256 workgroups.
int split_router_hsplit(int T, int E, int H) {
  if (E <= 64) return 1;
  const int64_t tiles = (int64_t)((T + 255) / 256) * (split_router_ep(E) / 64);
  const int nk = H / kChunk;
  int hs = 1;
  while (hs < 8 && tiles * hs * 2 <= 256 && nk % (hs * 2) == 0) hs *= 2;
  return hs;
}

struct SplitArgs {
  const uint16_t* x;
  const uint16_t* wp;
  const float* Wg;
  const float* bias;
  float* logits;
  int32_t* topk_idx;
  float* topk_gate;
  const SplitScratch* sc;
  int T, H, E, Ep, k, gate_mode;
  int hs;  // h split over workgroups (unfused form)
  double c1;
  SplitTail tail;  // requested epilogue work (null pointers: none)
  int* fused;      // out: 1 ranks done, 2 loss partials done
};

template <int TG, int EG, int KS, int MF, int WN, int S, bool FUSE, int KMAX, bool RAW = false>
static hipError_t launch_split_logits(const SplitArgs& a, hipStream_t st) {
  constexpr int BM = 16 * MF * TG, BN = 16 * WN * EG;
  constexpr int ROWS = KS * (BM + 3 * BN);
  size_t shm = sizeof(uint16_t) * (size_t)S * (RAW ? BM * kChunk + 64 * 64 * 2 : ROWS * kChunk);
  const size_t red = (KS > 1) ? (sizeof(double) * (size_t)(KS - 1) * TG * EG * MF * WN * 4 * 64 +
                                 sizeof(float) * (size_t)(KS - 1) * TG * MF * 64)
                              : 0;
  // fused epilogue: staged logits and x norms, norm partials, local queue
  const size_t fz = FUSE ? sizeof(float) * (size_t)BM * (BN + 2) + sizeof(double) * 512 + 16 * (size_t)BM +
                               8 * (size_t)BM * BN + 8 * 512 + 4 * 512 + 8 * 8 + 8 * (size_t)BM * KMAX +
                               4 * (size_t)(BM / 64 + 1) * 65
                         : 0;
  // the epilogue ranks and loss partials need whole 64-token blocks
  constexpr bool kTail = FUSE && BM % 64 == 0;
  SplitTail tail{};
  if (kTail) tail = a.tail;
  *a.fused = kTail ? ((tail.dst_rank ? 1 : 0) | (tail.Ppart ? 2 : 0)) : 0;
  if (red > shm) shm = red;
  if (fz > shm) shm = fz;
  auto kern = router_split_logits_kernel<TG, EG, KS, MF, WN, S, FUSE, KMAX, RAW>;
  hipError_t err = lds_limit_once<router_split_logits_kernel<TG, EG, KS, MF, WN, S, FUSE, KMAX, RAW>>((int)shm);
  if (err != hipSuccess) return err;
  dim3 grid((a.T + BM - 1) / BM, a.Ep / BN, FUSE ? 1 : a.hs);
  kern<<<grid, dim3(512), shm, st>>>(a.x, a.wp, a.Wg, a.bias, a.sc->wsq, a.logits, a.sc->lpart, a.sc->xsq, a.sc->wn,
                                     a.T, a.H, a.E, a.Ep,
                                     a.k, a.gate_mode, a.c1, a.topk_idx, a.topk_gate, a.sc->pairs, a.sc->utok,
                                     a.sc->count, tail);
  return hipGetLastError();
}

// fused selection: one instantiation per bound on k
template <int TG, int EG, int KS, int MF, int WN, int S, bool RAW = false>
static hipError_t launch_split_fused(const SplitArgs& a, hipStream_t st) {
  if (a.k <= 1) return launch_split_logits<TG, EG, KS, MF, WN, S, true, 1, RAW>(a, st);
  if (a.k <= 2) return launch_split_logits<TG, EG, KS, MF, WN, S, true, 2, RAW>(a, st);
  if (a.k <= 4) return launch_split_logits<TG, EG, KS, MF, WN, S, true, 4, RAW>(a, st);
  if (a.k <= 8) return launch_split_logits<TG, EG, KS, MF, WN, S, true, 8, RAW>(a, st);
  return launch_split_logits<TG, EG, KS, MF, WN, S, true, 16, RAW>(a, st);
}

hipError_t launch_router_split(const void* x, const float* Wg, const float* bias, float* logits, int T, int H, int E,
                               int k, int gate_mode, int32_t* topk_idx, float* topk_gate, const SplitScratch& sc,
                               const SplitEpilogue& ep, int* fused, hipStream_t st) {
  *fused = 0;
  if (T == 0) return hipSuccess;
  const int Ep = split_router_ep(E), nk = H / kChunk;
  uint16_t* wp = static_cast<uint16_t*>(sc.wp);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  // 33..64 experts (a multiple of 4, 16-byte aligned Wg): the fused kernel loads
  // the fp32 weights itself and splits them as it reads its fragments, so no
  // prep pass; otherwise the pieces are prepared once per call
  const bool raw = E > 32 && E <= 64 && E % 4 == 0 && (reinterpret_cast<uintptr_t>(Wg) & 15u) == 0;
  hipError_t err = hipSuccess;
  if (!raw) {
    router_split_prep_kernel<<<dim3((Ep + 63) / 64, nk), dim3(256), 0, st>>>(Wg, H, E, Ep, wp, sc.wsq, sc.count);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }

  // hi chain: 64 products (+ the running sum), |hi| <= (1 + 2^-7)|w|; mid/lo
  // chain: 128 products, |mid| + |lo| <= 2^-7 |w|; 2^-23 per addition; the
  // fp32 sum of the two chains, 2^-24 of at most (1 + 2^-6) sum|x*w|; 1%
  // slack; binary64 sums (here and in the exact definition) add at most
  // 4 H 2^-53 relative to sum|x*w|.
  const double c1 = 1.01 * ((65.0 * (1.0 + 0x1p-7) + 129.0 * 0x1p-7) * 0x1p-23 + (1.0 + 0x1p-6) * 0x1p-24) +
                    4.0 * (double)H * 0x1p-53;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;  // expert ids 0 .. E-1
  const SplitTail tail{ep.dst_rank, ep.hist, nbits, (T + 63) / 64, ep.Ppart, ep.Zpart, ep.Cpart, ep.score_fn};
  SplitArgs a{xb,  wp, Wg, bias,      logits, topk_idx, topk_gate, &sc, T,    H,
              E,   Ep, k,  gate_mode, split_router_hsplit(T, E, H),   c1,        tail, fused};

  if (E <= 16) {
    // 16 experts per wave; split h across waves when there are few tokens
    if ((int64_t)T >= 128 * 256 || nk % 2) err = launch_split_fused<8, 1, 1, 1, 1, 4>(a, st);
    else if ((int64_t)T >= 64 * 256 || nk % 4) err = launch_split_fused<4, 1, 2, 1, 1, 3>(a, st);
    else err = launch_split_fused<2, 1, 4, 1, 1, 3>(a, st);
  } else if (E <= 32) {
    err = launch_split_fused<8, 1, 1, 1, 2, 4>(a, st);
  } else if (E <= 64) {
    err = raw ? launch_split_fused<2, 4, 1, 2, 1, 4, true>(a, st) : launch_split_fused<2, 4, 1, 2, 1, 4>(a, st);
  } else {
    // 256 tokens x 64 experts per workgroup, h split over a.hs workgroups
    err = launch_split_logits<4, 2, 1, 4, 2, 2, false, 1>(a, st);
  }
  if (err != hipSuccess) return err;

  const int je = (E + 63) / 64;
  // refine: one block per queued token, grid-strided; four blocks per CU keep
  // enough tokens in flight when many are undecided (k = 8 of 256 experts)
  const dim3 cgrid((T + 3) / 4), rgrid(T < 1024 ? T : 1024);
  const bool fused_tile = E <= 64;
#define MOE_CR(J, K)                                                                                               \
  do {                                                                                                             \
    if (!fused_tile) {                                                                                             \
      router_certify_kernel<J, K><<<cgrid, dim3(256), 0, st>>>(sc.lpart, a.hs, logits, sc.xsq, sc.wn, bias, T, H, \
                                                               E, Ep, k, gate_mode, c1, topk_idx, topk_gate,      \
                                                               sc.pairs, sc.utok, sc.count);                       \
      if ((err = hipGetLastError()) != hipSuccess) return err;                                                     \
      router_refine_kernel<J, K><<<rgrid, dim3(256), 0, st>>>(xb, wp, bias, sc.pairs, sc.utok, sc.count, logits,  \
                                                              H, E, Ep, k, gate_mode, topk_idx, topk_gate);        \
    }                                                                                                              \
  } while (0)
#define MOE_CR_K(J)              \
  if (k <= 1) MOE_CR(J, 1);      \
  else if (k <= 2) MOE_CR(J, 2); \
  else if (k <= 4) MOE_CR(J, 4); \
  else if (k <= 8) MOE_CR(J, 8); \
  else MOE_CR(J, 16)
  if (je <= 1) { MOE_CR_K(1); }
  else if (je <= 2) { MOE_CR_K(2); }
  else if (je <= 4) { MOE_CR_K(4); }
  else if (je <= 8) { MOE_CR_K(8); }
  else { MOE_CR_K(16); }
#undef MOE_CR_K
#undef MOE_CR
  return hipGetLastError();
}

}  // namespace moe
