// Expert FFN as a ragged grouped GEMM over expert-contiguous packed rows.
//
// "Expert-parallel MoE training" explainer: experts are FFNs (gated ones with
// gate / up / down matrices, memory calculator); DeepSpeed discussion #7508: run
// the experts on the actual tokens per expert instead of a fixed [E, C, H]
// buffer.  Each expert's rows are padded only to the tile, never to a capacity.
//
//   GEMM1: h = act(X W1_e^T)  or  silu(X W1_e^T) * (X W3_e^T)   [rows x F]
//   GEMM2: Y = h W2_e^T                                          [rows x H]
// W1/W3 are [E][F][H] and W2 is [E][H][F] (each matrix [out][in]), so both GEMMs
// read A and B along the contraction dimension (K-contiguous "TN" form).
//
// The tile schedule is derived on the device from offsets[E+1]: workgroup id ->
// (global m-tile, n-tile); a block-wide scan of ceil(kept_e / BM) maps the
// m-tile to its expert.  No host synchronisation, no tile straddles experts.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

enum { EPI_NONE = 0, EPI_RELU = 1, EPI_GELU = 2, EPI_SWIGLU = 3, EPI_COMBINE1 = 4 };

// GELU x Phi(x) = x/2 + |x|/2 (1 - erfc(|x| / sqrt 2)) with
// erfc(z) ~ (a1 t + ... + an t^n) e^(-z^2), t = 1 / (1 + p z), from Abramowitz &
// Stegun, Handbook of Mathematical Functions, written in m = x/2 so that the
// last step is one fma (one reciprocal and one exp2 per element).
//   fp32 outputs: formula 7.1.26, n = 5 (|error| <= 1.5e-7); the GELU is then
//     within 5e-7 over [-12, 12] in fp32.
//   bf16 outputs: formula 7.1.25, n = 3 (|error| <= 2.5e-5): within 2.6e-5 and
//     1.1e-5 |x|, far below the bf16 rounding of the stored activation (2^-9
//     relative), for two operations less per element.
template <bool kBF16>
__device__ __forceinline__ float gelu_erf(float a) {
  const float m = 0.5f * a;
  float t, p;
  if (kBF16) {
    t = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(m), 0.66534505468967010f, 1.0f));  // z = sqrt 2 |m|
    p = __builtin_fmaf(t, 0.7478556f, -0.0958798f);
    p = __builtin_fmaf(t, p, 0.3480242f);
  } else {
    t = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(m), 0.46328377653272080f, 1.0f));
    p = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
    p = __builtin_fmaf(t, p, 1.421413741f);
    p = __builtin_fmaf(t, p, -0.284496736f);
    p = __builtin_fmaf(t, p, 0.254829592f);
  }
  p *= t;
  const float e = __builtin_amdgcn_exp2f(m * m * -2.8853900817779268f);  // e^(-z^2) = e^(-2 m^2)
  return __builtin_fmaf(fabsf(m), __builtin_fmaf(-p, e, 1.0f), m);
}

// Activation of an output element: a from the first (gate) weights, b from the
// second (up) ones for SwiGLU; kBF16: the result is stored as bf16.
template <int EPI, bool kBF16 = true>
__device__ __forceinline__ float epilogue(float a, float b) {
  if (EPI == EPI_RELU) return a > 0.0f ? a : 0.0f;
  if (EPI == EPI_GELU) return gelu_erf<kBF16>(a);
  if (EPI == EPI_SWIGLU)  // silu(a) * b = a / (1 + e^-a) * b
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f)) * b;
  return a;
}

// Maps m-tile `mt` to (expert, row offset inside the expert) from offsets.
// Returns false (uniformly over the block) when mt is past the last tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int mt, int* s_scan,
                                          int* s_info) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per = (E + nthr - 1) / nthr;
  const int e_begin = tid * per;
  int cnt = 0;
  for (int j = 0; j < per; ++j) {
    const int e = e_begin + j;
    if (e < E) cnt += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  }
  int total;
  int run = block_exclusive_scan(cnt, s_scan, &total);
  if (mt >= total) return false;
  for (int j = 0; j < per; ++j) {
    const int e = e_begin + j;
    if (e < E) {
      const int c = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
      if (mt >= run && mt < run + c) {
        s_info[0] = e;
        s_info[1] = (mt - run) * BM;
      }
      run += c;
    }
  }
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM.  Workgroup tile 128 x 128 x 64, 4 waves as 2 x 2, each
// wave 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators.
// A / B tiles are staged through LDS (row stride 72 elements = 144 B), double
// buffered: the next K tile is fetched into registers while the current one is
// multiplied.  MFMA operand layout: lane l supplies row (l % 32) and the eight
// consecutive k at 8 * (l / 32) of the 16-wide k step; accumulator element
// 4g + j of lane l is row 8g + 4(l / 32) + j, column l % 32.
// ---------------------------------------------------------------------------
constexpr int GB_BM = 128, GB_BN = 128, GB_BK = 64, GB_LDK = GB_BK + 8;
constexpr int GB_TILE = GB_BM * GB_LDK;  // elements per staged tile

template <int EPI>
__global__ void __launch_bounds__(256) grouped_gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ B,
                                                                const uint16_t* __restrict__ B2,
                                                                uint16_t* __restrict__ C,
                                                                const int32_t* __restrict__ offsets, int E, int N,
                                                                int K, int ntn, int rmax) {
  constexpr bool kGated = EPI == EPI_SWIGLU;
  constexpr int NB = kGated ? 2 : 1;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s_a = smem;                  // [2][GB_TILE]
  uint16_t* s_b = smem + 2 * GB_TILE;    // [NB][2][GB_TILE]
  __shared__ int s_scan[256 / 64 + 1];
  __shared__ int s_info[2];

  const int tid = threadIdx.x;
  const int mt = blockIdx.x / ntn;
  const int nt = blockIdx.x - mt * ntn;
  if (!find_tile<GB_BM>(offsets, E, mt, s_scan, s_info)) return;
  const int e = s_info[0];
  const int mloc = s_info[1];
  const int row0 = offsets[e] + mloc;
  // rows of this tile; clamped to the row buffers' size whatever offsets holds
  const int rows = min(min(GB_BM, offsets[e + 1] - offsets[e] - mloc), rmax - row0);
  if (rows <= 0) return;
  const int n0 = nt * GB_BN;

  const uint16_t* Ab = A + (size_t)row0 * K;
  const uint16_t* Bb = B + ((size_t)e * N + n0) * K;
  const uint16_t* B2b = kGated ? B2 + ((size_t)e * N + n0) * K : nullptr;

  // global -> register staging: 4 chunks of 8 elements per thread per tile
  u32x4_t ra[4], rb[NB][4];
  auto fetch = [&](int kt) {
    const int k0 = kt * GB_BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      const int row = c >> 3, kc = (c & 7) * 8;
      const bool kin = k0 + kc < K;
      ra[j] = (row < rows && kin) ? *reinterpret_cast<const u32x4_t*>(Ab + (size_t)row * K + k0 + kc)
                                  : u32x4_t{0, 0, 0, 0};
      const bool nin = n0 + row < N && kin;
      rb[0][j] = nin ? *reinterpret_cast<const u32x4_t*>(Bb + (size_t)row * K + k0 + kc) : u32x4_t{0, 0, 0, 0};
      if (kGated)
        rb[NB - 1][j] = nin ? *reinterpret_cast<const u32x4_t*>(B2b + (size_t)row * K + k0 + kc)
                            : u32x4_t{0, 0, 0, 0};
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      const int row = c >> 3, kc = (c & 7) * 8;
      const int off = buf * GB_TILE + row * GB_LDK + kc;
      *reinterpret_cast<u32x4_t*>(s_a + off) = ra[j];
#pragma unroll
      for (int b = 0; b < NB; ++b) *reinterpret_cast<u32x4_t*>(s_b + b * 2 * GB_TILE + off) = rb[b][j];
    }
  };

  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 31;
  const int lk = (lane >> 5) * 8;

  f32x16_t acc[NB][2][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][mi][ni][v] = 0.0f;

  const int nk = (K + GB_BK - 1) / GB_BK;
  fetch(0);
  stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) fetch(kt + 1);
    const uint16_t* sa = s_a + buf * GB_TILE;
#pragma unroll
    for (int kk = 0; kk < GB_BK; kk += 16) {
      bf16x8_t af[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(sa + (wm * 64 + mi * 32 + lr) * GB_LDK + kk + lk);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint16_t* sb = s_b + b * 2 * GB_TILE + buf * GB_TILE;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t*>(sb + (wn * 64 + ni * 32 + lr) * GB_LDK + kk + lk);
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            acc[b][mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr, acc[b][mi][ni], 0, 0, 0);
        }
      }
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
  }

  // epilogue: activation, round to bf16, store the valid rows / columns
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + wn * 64 + ni * 32 + lr;
      if (col >= N) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wm * 64 + mi * 32 + 8 * g + (lane >> 5) * 4 + j;
          if (row < rows) {
            const float v = epilogue<EPI>(acc[0][mi][ni][4 * g + j], acc[NB - 1][mi][ni][4 * g + j]);
            C[(size_t)(row0 + row) * N + col] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
    }
}

// ---------------------------------------------------------------------------
// Scalar grouped GEMM (fp32 runs and shapes the vector path does not take):
// one thread per output element, fp32 accumulation in k order.
// ---------------------------------------------------------------------------
template <bool kBF16, int EPI>
__global__ void __launch_bounds__(64) grouped_gemm_scalar_kernel(const void* __restrict__ A,
                                                                 const void* __restrict__ B,
                                                                 const void* __restrict__ B2, void* __restrict__ C,
                                                                 const int32_t* __restrict__ offsets, int E, int N,
                                                                 int K, int nbx) {
  const int row = blockIdx.x / nbx;  // grid covers exactly R_max rows
  const int n = (blockIdx.x - row * nbx) * 64 + threadIdx.x;
  const int R = offsets[E];
  if (row >= R || n >= N) return;
  int lo = 0, hi = E;  // largest e with offsets[e] <= row (and a non-empty range)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  const int e = lo;
  const size_t a0 = (size_t)row * K;
  const size_t b0 = ((size_t)e * N + n) * K;
  float s1 = 0.0f, s2 = 0.0f;
  for (int kk = 0; kk < K; ++kk) {
    float a, b, b2 = 0.0f;
    if (kBF16) {
      a = bf16_bits_to_f32(static_cast<const uint16_t*>(A)[a0 + kk]);
      b = bf16_bits_to_f32(static_cast<const uint16_t*>(B)[b0 + kk]);
      if (EPI == EPI_SWIGLU) b2 = bf16_bits_to_f32(static_cast<const uint16_t*>(B2)[b0 + kk]);
    } else {
      a = static_cast<const float*>(A)[a0 + kk];
      b = static_cast<const float*>(B)[b0 + kk];
      if (EPI == EPI_SWIGLU) b2 = static_cast<const float*>(B2)[b0 + kk];
    }
    s1 = __builtin_fmaf(a, b, s1);
    if (EPI == EPI_SWIGLU) s2 = __builtin_fmaf(a, b2, s2);
  }
  const float v = epilogue<EPI, kBF16>(s1, s2);
  if (kBF16) static_cast<uint16_t*>(C)[(size_t)row * N + n] = (uint16_t)f32_to_bf16_bits(v);
  else static_cast<float*>(C)[(size_t)row * N + n] = v;
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM, LDS-tiled: a 256-thread block computes 64 rows x 64
// columns of one expert (each thread 4 x 4), staging 16 k of the A rows and
// of the weight rows (both of them for SwiGLU) in LDS, k-major so that a
// thread's four rows and four columns are two 16-byte LDS reads (fp32
// layers, which the bf16 tiles do not take).  Every
// output is one fp32 fma chain in k order, as in the scalar kernel, so the
// two give the same bits.  Block (mt, nt): m-tile mt of the expert list
// (ceil(kept_e / 64) per expert), n-tile nt.
// ---------------------------------------------------------------------------
constexpr int F32_T = 64, F32_BK = 16;

template <int EPI>
__global__ void __launch_bounds__(256) grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                               const float* __restrict__ B,
                                                               const float* __restrict__ B2, float* __restrict__ C,
                                                               const int32_t* __restrict__ offsets, int E, int N,
                                                               int K) {
  constexpr bool kGated = EPI == EPI_SWIGLU;
  // rows of 68: the 16 k of one row land in distinct banks when stored
  __shared__ __align__(16) float sa[F32_BK][F32_T + 4];
  __shared__ __align__(16) float sb[kGated ? 2 : 1][F32_BK][F32_T + 4];
  __shared__ int s_scan[5];
  __shared__ int s_info[2];
  if (!find_tile<F32_T>(offsets, E, blockIdx.x, s_scan, s_info)) return;
  const int e = s_info[0];
  const int row0 = offsets[e] + s_info[1];
  const int rows = min(F32_T, offsets[e + 1] - row0);
  const int n0 = blockIdx.y * F32_T;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  // loads: thread tid brings k = tid % 16 of row tid / 16 + 16 i (i < 4)
  const int lk = tid & 15, lr = tid >> 4;
  float acc[2][4][4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[g][i][j] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += F32_BK) {
    const int k = k0 + lk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 16 * i;
      sa[lk][r] = (r < rows && k < K) ? A[(size_t)(row0 + r) * K + k] : 0.0f;
      const int n = n0 + r;
      sb[0][lk][r] = (n < N && k < K) ? B[((size_t)e * N + n) * K + k] : 0.0f;
      if constexpr (kGated) sb[1][lk][r] = (n < N && k < K) ? B2[((size_t)e * N + n) * K + k] : 0.0f;
    }
    __syncthreads();
    const int kn = K - k0 < F32_BK ? K - k0 : F32_BK;
    for (int kk = 0; kk < kn; ++kk) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sa[kk][4 * ty]);
#pragma unroll
      for (int g = 0; g < (kGated ? 2 : 1); ++g) {
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&sb[g][kk][4 * tx]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[g][i][j] = __builtin_fmaf(a[i], b[j], acc[g][i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * ty + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n < N) C[(size_t)(row0 + r) * N + n] = epilogue<EPI, false>(acc[0][i][j], acc[1][i][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined persistent grouped GEMM (the bf16 path when K % 32 == 0).
//
// Roles: the MFMA's first operand is a weight fragment (rows n), the second a
// token fragment (rows m), so each lane ends with four consecutive output
// columns of one token row and writes them as one 8-byte store.
//
// Workgroup tile: BM token rows x WR weight rows (WR output columns, or for
// SwiGLU WR/2 gate + WR/2 up rows = WR/2 output columns), NW waves as WGM
// (token direction) x NW/WGM (weight direction); a wave owns MF x NF
// v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators.  Shapes in use:
// 256 x 256 (2 x 4 waves), 256 x 192 (4 x 2 waves, for N where it fills the
// CUs in whole waves of tiles) and 128 x 256 (2 x 4 waves, small experts).
//
// Data movement: global_load_lds_dwordx4 moves 16-byte chunks straight into
// LDS (no VGPR staging).  A stage holds BM + WR rows of BK = 64 k (128 B per
// row); chunk c of row r sits at slot c ^ ((r >> 1) & 7) of its row.  The LDS
// has 64 four-byte banks and serves a 16-byte-per-lane read 16 lanes at a
// time, so the 16 rows such a phase touches land in distinct bank groups.  S
// stages form a ring: the loads of stage j + S - 1 are issued right after the
// barrier of step j and waited for S - 1 steps later with an explicit vmcnt
// (vector memory operations complete in issue order; stores issued in between
// only make a wait stricter).  Within a stage, the fragment reads of k-step
// kk + 1 are interleaved one by one with the MFMAs of k-step kk.
//
// Persistent: at most one workgroup per CU; workgroup b takes every G-th tile
// of the device-side tile list (expert-major, then n-tile, then m-tile).  The
// stage ring runs on across tile boundaries, so the next tile's first loads
// are in flight while the current tile's epilogue runs.
//
// BT (k-major weights, plain products only): the weight operand is stored
// [E][K][N] (N contiguous), as W2 is for dY W2 and W1, W3 for du W1 + dv W3,
// and a stage holds BK k-rows of WR columns instead of WR rows of BK k.  Slot
// ch of k-row kr holds the columns of chunk ch ^ 4 (kr & 3).  The weight
// fragment (column l % 32, k 8 (l / 32) .. +7 of lane l) comes from two
// transposing LDS reads (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// s addresses 4 columns 4 (s % 4) .. +3 of k-row s / 4, and lane i receives
// column i of those 16 for the 4 k-rows.  The 32 lanes of a read phase touch 4
// k-rows x 4 chunks, which the swizzle puts in 16 distinct bank groups.  W2 is
// then an optional second weight tensor that continues the contraction: k < k1
// from W ([E][k1][N]), k >= k1 from W2 (same shape, K = 2 k1).
//
// SAVE (first GEMM only): the pre-activations of every output element are also
// stored as bf16 for the backward, u = X W_e^T at save[row][n] and, for
// SwiGLU, v = X W3_e^T at save[rmax + row][n] (rows of N), with the same lane
// swaps and 16-byte stores as the activation.
// ---------------------------------------------------------------------------
struct PipeTile {
  int e, row0, rows, n0;
};

// Top-1 combine of 8 output columns: o holds the bf16 expert outputs (as the
// second GEMM would store them), r the bf16 residual; fp32 fma, one rounding.
__device__ __forceinline__ u32x4_t combine1_8(u32x4_t o, u32x4_t r, float g) {
  u32x4_t out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = __builtin_fmaf(g, __uint_as_float(o[j] << 16), __uint_as_float(r[j] << 16));
    const float hi = __builtin_fmaf(g, __uint_as_float(o[j] & 0xffff0000u), __uint_as_float(r[j] & 0xffff0000u));
    out[j] = pack_bf16x2(lo, hi);
  }
  return out;
}

// Top-1 combine, tokens that no packed row holds: y[t] = res[t] (or 0).  Part
// `part` of `parts`, nthr threads, 16 bytes per thread-iteration.
__device__ __forceinline__ void combine1_dropped(const Combine1& cmb, uint16_t* __restrict__ y, int H, int rmax,
                                                 int part, int parts, int tid, int nthr) {
  const int nch = H / 8;
  const int64_t total = (int64_t)cmb.T * nch;
  for (int64_t i = (int64_t)part * nthr + tid; i < total; i += (int64_t)parts * nthr) {
    const int t = (int)(i / nch);
    const int c = (int)(i - (int64_t)t * nch) * 8;
    const int d = cmb.dst_row[t];
    if (d >= 0 && d < rmax) continue;
    const u32x4_t v = cmb.res ? *reinterpret_cast<const u32x4_t*>(cmb.res + (size_t)t * H + c) : u32x4_t{0, 0, 0, 0};
    *reinterpret_cast<u32x4_t*>(y + (size_t)t * H + c) = v;
  }
}

// A row of zeros (zero-initialised at load, never written) that the token-row
// loads of a tile's padding rows read instead of a real row: their products
// are discarded either way, and zero operands cost the matrix cores less
// power, which the clock of a power-limited GEMM turns into speed.
constexpr int kZeroRowElems = 32768;
__device__ __align__(16) uint16_t g_zero_row[kZeroRowElems];

// Cache policy of a direct-to-LDS load: 0, or non-temporal (kLoadNT) for
// weight rows that no other tile reads (NTW: every expert fits one m-tile), so
// that the streamed weights do not push the token rows and the hidden
// activations, which other tiles and the next GEMM read again, out of L2.
constexpr int kLoadNT = 2;

// Gathered A (A = the token rows x, gather = row_token): a wave's A loads of a
// tile cover NA groups of RPL packed rows (group q: rows RPL (q NW + w) .. +RPL-1).  One
// direct-to-LDS load of 4 bytes per lane brings their row_token entries into
// the wave's slot of an LDS table, issued a tile ahead, so that when the tile
// starts its entries are there (every stage wait since covers that load);
// rows past the tile's `rows` take the tile's first row.
template <int NA, int NW, int RPL>
__device__ __forceinline__ void fetch_gather_rows(const int32_t* __restrict__ gather, const PipeTile& t, int w,
                                                  int lane, int* slot) {
  static_assert(NA * RPL <= 64, "one load instruction");
  const int l = lane % (NA * RPL);
  const int r = ((l / RPL) * NW + w) * RPL + l % RPL;
  const int row = t.row0 + (r < t.rows ? r : 0);
  __builtin_amdgcn_global_load_lds(gather + row, slot, 4, 0, 0);
}

__device__ __forceinline__ int clamp_row(int tok, int xrows) { return tok < 0 ? 0 : (tok < xrows ? tok : xrows - 1); }


// BM token rows x WR weight rows per tile, BK k per stage, S stages, NW waves
// as WGM (token direction) x NW / WGM (weight direction); at most 256 registers
// per wave (two waves per SIMD: one workgroup of 8 waves or two of 4 per CU).
template <int BM, int WR, int BK, int S, int WGM, int EPI, int NW, bool NTW, bool BT = false, bool SAVE = false>
__global__ void __launch_bounds__(64 * NW, 2) grouped_gemm_pipe_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ W,
                                                                   const uint16_t* __restrict__ W2,
                                                                   uint16_t* __restrict__ C,
                                                                   const int32_t* __restrict__ offsets, int E,
                                                                   int N, int K, int rmax,
                                                                   const int32_t* __restrict__ gather, int xrows,
                                                                   Combine1 cmb, int rlo, int rhi, int k1,
                                                                   uint16_t* __restrict__ save) {
  constexpr bool kGated = EPI == EPI_SWIGLU;
  constexpr int BN = kGated ? WR / 2 : WR;                // output columns per tile
  constexpr int ROWS = BM + WR;                           // rows per stage
  constexpr int CPR = BK / 8;                             // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;                           // rows per 16-byte-per-lane load
  constexpr int RSH = CPR == 8 ? 1 : (CPR == 4 ? 2 : 3);  // rows per 256-byte LDS phase = 1 << RSH
  constexpr int STAGE = ROWS * BK;                        // bf16 elements per stage
  constexpr int L = ROWS * CPR / (64 * NW);         // 16-byte loads per wave per stage
  constexpr int WGN = NW / WGM;
  constexpr int MF = BM / WGM / 32;                       // token fragments per wave
  constexpr int NF = WR / WGN / 32;                       // weight fragments per wave
  constexpr int HF = kGated ? NF / 2 : NF;                // output column fragments per wave
  constexpr int KS = BK / 16;                             // MFMA k-steps per stage
  static_assert(ROWS * CPR % (64 * NW) == 0 && BM % 64 == 0 && (CPR == 4 || CPR == 8 || CPR == 2), "tile");
  static_assert(MF >= 1 && NF >= 1 && (!kGated || NF % 2 == 0), "SwiGLU waves pair gate and up fragments");
  static_assert(!BT || (EPI == EPI_NONE && WR % 128 == 0), "k-major weights: plain products, 16+ chunks per k-row");
  static_assert(!SAVE || EPI == EPI_RELU || EPI == EPI_GELU || EPI == EPI_SWIGLU, "pre-activations of the first GEMM");
  static_assert(S >= 2 && S - 2 <= 4 && (S - 1) * L < 64 && KS % 2 == 0, "stages");
  extern __shared__ __align__(16) uint16_t smem[];
  int* s_ts = reinterpret_cast<int*>(smem + S * STAGE);  // [E+1] first tile of each expert
  int* s_off = s_ts + (E + 1);                             // [E+1] offsets
  __shared__ int s_scan[NW + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int ntn = (N + BN - 1) / BN;
  constexpr int NA = BM * CPR / (64 * NW);  // this wave's load instructions of A rows per stage
  __shared__ int s_gidx[2][NW][64];          // gathered row indices, two tiles
  int gbuf = 0;                              // table of the tile being loaded

  {  // tile list: ceil(kept_e / BM) * ntn tiles per expert whose row count
     // lies in (rlo, rhi] (the other experts belong to another launch)
    const int per = (E + 64 * NW - 1) / (64 * NW);
    const int e0 = tid * per;
    auto tiles_of = [&](int e) {
      const int rows = offsets[e + 1] - offsets[e];
      return rows > rlo && rows <= rhi ? (rows + BM - 1) / BM * ntn : 0;
    };
    int cnt = 0;
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) cnt += tiles_of(e);
    }
    int total;
    int run = block_exclusive_scan(cnt, s_scan, &total);
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) {
        s_ts[e] = run;
        s_off[e] = offsets[e];
        run += tiles_of(e);
      }
    }
    if (tid == 0) {
      s_ts[E] = total;
      s_off[E] = offsets[E];
    }
    __syncthreads();
  }
  const int G = gridDim.x;
  const int total_tiles = s_ts[E];
  // Workgroups are dealt to the 8 XCDs round-robin (b % 8).  Round i gives XCD
  // x the contiguous tile range [i*G + x*G/8, i*G + (x+1)*G/8), so tiles that
  // share a weight tile or a block of token rows meet in the same L2.
  const int slot = (G % 8 == 0) ? ((int)blockIdx.x % 8) * (G / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;
  const int my_tiles = total_tiles > slot ? (total_tiles - 1 - slot) / G + 1 : 0;
  const int nk = K / BK;
  const int total_steps = my_tiles * nk;
  if (total_steps == 0) {
    if constexpr (EPI == EPI_COMBINE1) combine1_dropped(cmb, C, N, rmax, slot, G, tid, 64 * NW);
    return;
  }

  auto decode = [&](int i) {  // i-th tile of this workgroup
    const int g = slot + i * G;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_ts[mid] <= g) lo = mid;
      else hi = mid;
    }
    const int mt_e = (s_off[lo + 1] - s_off[lo] + BM - 1) / BM;
    const int local = g - s_ts[lo];
    const int nt = local / mt_e;
    PipeTile t;
    t.e = lo;
    t.row0 = s_off[lo] + (local - nt * mt_e) * BM;
    t.rows = min(min(BM, s_off[lo + 1] - t.row0), rmax - t.row0);
    if (t.rows <= 0) {  // only for offsets inconsistent with the row buffers
      t.rows = 0;
      t.row0 = 0;
    }
    t.n0 = nt * BN;
    return t;
  };

  // chunk c of stage row r -> LDS element offset.  A 16-byte-per-lane read is
  // served 16 lanes (256 B, all 64 banks) at a time; rows that share a phase
  // get different chunk slots.
  auto lds_pos = [](int r, int c) { return (r * CPR + (c ^ ((r >> RSH) & (CPR - 1)))) * 8; };

  // Row pointers of this wave's L loads for the tile being loaded, fixed for
  // the whole tile; a stage only adds its k offset.
  uintptr_t rowp[L];
  auto set_rows = [&](const PipeTile& t) {
#pragma unroll
    for (int q = 0; q < L; ++q) {
      const int blk = q * NW + w;  // 64 lanes = 64 / CPR rows; never straddles the two regions
      const int p = blk * 64 + lane;
      const int r = p / CPR;
      const int c = (p % CPR) ^ ((r >> RSH) & (CPR - 1));
      if (r < BM) {
        const int rr = r < t.rows ? r : 0;
        const int src = gather ? clamp_row(s_gidx[gbuf][w][q * RPL + lane / CPR], xrows) : t.row0 + rr;
        rowp[q] = (r >= t.rows && K <= kZeroRowElems) ? reinterpret_cast<uintptr_t>(g_zero_row + c * 8)
                                                      : reinterpret_cast<uintptr_t>(A + (size_t)src * K + c * 8);
      } else if constexpr (BT) {
        const int pw = p - BM * CPR, kr = pw / (WR / 8), ch = (pw % (WR / 8)) ^ (4 * (kr & 3));
        int n = t.n0 + ch * 8;
        n = n < N - 8 ? n : N - 8;  // chunks past N: whole chunks, never stored
        rowp[q] = reinterpret_cast<uintptr_t>(W + ((size_t)t.e * k1 + kr) * N + n);
      } else {
        const int wr = r - BM;
        const uint16_t* base = (kGated && wr >= WR / 2) ? W2 : W;
        int n = t.n0 + (kGated ? (wr & (WR / 2 - 1)) : wr);
        n = n < N ? n : N - 1;
        rowp[q] = reinterpret_cast<uintptr_t>(base + ((size_t)t.e * N + n) * K + c * 8);
      }
    }
  };
  // k-major weights: byte distance from W to W2 (the k >= k1 half)
  const uintptr_t wdelta = BT ? reinterpret_cast<uintptr_t>(W2) - reinterpret_cast<uintptr_t>(W) : 0;
  auto issue = [&](int buf, int kstep) {
    uint16_t* st = smem + buf * STAGE;
    const int k0 = kstep * BK;
    uintptr_t woff = 0;  // k-major weights: byte offset of the stage's first k-row
    if constexpr (BT) woff = k0 < k1 ? (uintptr_t)k0 * N * 2 : wdelta + (uintptr_t)(k0 - k1) * N * 2;
#pragma unroll
    for (int q = 0; q < L; ++q) {
      const uint16_t* src = (BT && q >= NA) ? reinterpret_cast<const uint16_t*>(rowp[q] + woff)
                                            : reinterpret_cast<const uint16_t*>(rowp[q]) + k0;
      if (NTW && q >= NA) __builtin_amdgcn_global_load_lds(src, st + (q * NW + w) * 512, 16, 0, kLoadNT);
      else __builtin_amdgcn_global_load_lds(src, st + (q * NW + w) * 512, 16, 0, 0);
    }
  };

  f32x16_t acc[NF][MF];
  auto zero = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[f][i][v] = 0.0f;
  };

  struct Frags {
    bf16x8_t w[NF], x[MF];
  };
  // V (0 .. MF): the wave's token fragments that hold rows of the tile; the
  // others are neither read nor multiplied (their rows are never stored)
  auto read_frags = [&](auto vc, int buf, int kk, Frags& fr) {
    constexpr int V = decltype(vc)::value;
    if constexpr (V == 0) return;
    // more reads than MFMAs per k-step: the extra reads go first, and they are
    // the token fragments, so that the first MFMAs of the next k-step wait
    // only for reads issued early in this one
    constexpr bool kXFirst = V + (BT ? 2 : 1) * NF > V * NF;
    const uint16_t* st = smem + buf * STAGE;
    const int c = kk * 2 + (lane >> 5);
    if constexpr (kXFirst) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int r = wm * (MF * 32) + i * 32 + (lane & 31);
        fr.x[i] = *reinterpret_cast<const bf16x8_t*>(st + lds_pos(r, c));
      }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if constexpr (BT) {
        const int n = wn * (NF * 32) + f * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int kr = kk * 16 + 8 * (lane >> 5) + ((lane >> 2) & 3);
        const uint16_t* wp = st + BM * BK + kr * WR + (((n >> 3) ^ (4 * (kr & 3))) << 3) + (n & 7);
        const s16x4_t lo = lds_read_tr16(wp), hi = lds_read_tr16(wp + 4 * WR);
        fr.w[f] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        const int r = BM + (kGated ? (f / HF) * (WR / 2) + wn * (HF * 32) + (f % HF) * 32 : wn * (NF * 32) + f * 32) +
                      (lane & 31);
        fr.w[f] = *reinterpret_cast<const bf16x8_t*>(st + lds_pos(r, c));
      }
    }
    if constexpr (!kXFirst) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int r = wm * (MF * 32) + i * 32 + (lane & 31);
        fr.x[i] = *reinterpret_cast<const bf16x8_t*>(st + lds_pos(r, c));
      }
    }
  };
  auto mfma = [&](auto vc, const Frags& fr) {
    constexpr int V = decltype(vc)::value;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < V; ++i)
        acc[f][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.w[f], fr.x[i], acc[f][i], 0, 0, 0);
  };

  // accumulator element 4g + jj of lane l: weight row 8g + 4(l / 32) + jj, token row l % 32
  auto store = [&](const PipeTile& t) {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int m = wm * (MF * 32) + i * 32 + (lane & 31);
      int crow_i = t.row0 + m;  // output row: the packed row, or its token (top-1 combine)
      bool ok = m < t.rows;
      float gt = 0.0f;
      if constexpr (EPI == EPI_COMBINE1) {
        const int tok = ok ? cmb.row_token[crow_i] : -1;
        ok = tok >= 0 && tok < cmb.T;
        crow_i = ok ? tok : 0;
        gt = cmb.gate[crow_i];
      }
      if (ok) {
        uint16_t* crow = C + (size_t)crow_i * N;
        u32x4_t rv[HF][2];  // top-1 combine: this lane's residual groups of the row, loaded first
        if constexpr (EPI == EPI_COMBINE1) {
#pragma unroll
          for (int f = 0; f < HF; ++f)
#pragma unroll
            for (int g = 0; g < 4; g += 2) {
              const int n = t.n0 + wn * (HF * 32) + f * 32 + 8 * (g + (lane >> 5));
              rv[f][g / 2] = (cmb.res && n < N) ? *reinterpret_cast<const u32x4_t*>(cmb.res + (size_t)crow_i * N + n)
                                                : u32x4_t{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int f = 0; f < HF; ++f)
#pragma unroll
          for (int g = 0; g < 4; g += 2) {
            uint32_t pk[2][2];  // [group g, g + 1][packed column pair]
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float v[4];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj)
                v[jj] = kGated ? epilogue<EPI>(acc[f][i][4 * (g + h) + jj], acc[HF + f][i][4 * (g + h) + jj])
                               : epilogue<EPI>(acc[f][i][4 * (g + h) + jj], 0.0f);
              pk[h][0] = pack_bf16x2(v[0], v[1]);
              pk[h][1] = pack_bf16x2(v[2], v[3]);
            }
            // lanes l and l + 32 hold the two column halves of the 8-column
            // groups of one row: after swapping lanes 32..63 of group g's
            // words with lanes 0..31 of group g + 1's, lane l holds all of
            // group g and lane l + 32 all of group g + 1 (16-byte stores)
            const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
            const int n = t.n0 + wn * (HF * 32) + f * 32 + 8 * (g + (lane >> 5));
            u32x4_t o = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
            if constexpr (EPI == EPI_COMBINE1) o = combine1_8(o, rv[f][g / 2], gt);
            if (n < N) *reinterpret_cast<u32x4_t*>(crow + n) = o;
            if constexpr (SAVE) {
              {  // the pre-activations, rounded to bf16 (the same swaps as above)
#pragma unroll
                for (int part = 0; part < (kGated ? 2 : 1); ++part) {
                  const int fa = part ? HF + f : f;
                  uint32_t pa[2][2];
#pragma unroll
                  for (int h = 0; h < 2; ++h) {
                    pa[h][0] = pack_bf16x2(acc[fa][i][4 * (g + h)], acc[fa][i][4 * (g + h) + 1]);
                    pa[h][1] = pack_bf16x2(acc[fa][i][4 * (g + h) + 2], acc[fa][i][4 * (g + h) + 3]);
                  }
                  const auto a0 = __builtin_amdgcn_permlane32_swap(pa[0][0], pa[1][0], false, false);
                  const auto a1 = __builtin_amdgcn_permlane32_swap(pa[0][1], pa[1][1], false, false);
                  if (n < N)
                    *reinterpret_cast<u32x4_t*>(save + ((size_t)part * rmax + crow_i) * N + n) =
                        u32x4_t{a0[0], a1[0], a0[1], a1[1]};
                }
              }
            }
          }
      }
    }
  };

  if (gather) {
    fetch_gather_rows<NA, NW, RPL>(gather, decode(0), w, lane, &s_gidx[0][w][0]);
    wait_vmcnt<0>();
  }
  set_rows(decode(0));  // rows of the tile of the next stage to load
  if (gather && my_tiles > 1) fetch_gather_rows<NA, NW, RPL>(gather, decode(1), w, lane, &s_gidx[1][w][0]);

  int lt_i = 0, lt_k = 0, issued = 0;
  auto issue_next = [&]() {
    issue(issued % S, lt_k);
    ++issued;
    if (++lt_k == nk) {
      lt_k = 0;
      if (++lt_i < my_tiles) {
        if (gather) {
          gbuf ^= 1;
          if (nk < S) wait_vmcnt<0>();  // fewer stages per tile than in flight: the table may not be in yet
        }
        set_rows(decode(lt_i));
        if (gather && lt_i + 1 < my_tiles)
          fetch_gather_rows<NA, NW, RPL>(gather, decode(lt_i + 1), w, lane, &s_gidx[gbuf ^ 1][w][0]);
      }
    }
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (issued < total_steps) issue_next();

  // Step j: (loads of stage j + S - 1 into the buffer stage j - 1 used) ->
  // MFMAs of stage j, reading k-step kk + 1 while k-step kk multiplies ->
  // wait for stage j + 1, barrier, read its first k-step while the last MFMAs
  // of stage j drain.  A buffer is overwritten only after the barrier that
  // follows every wave's last read of it.  The nk steps of a tile run in the
  // instance of `tile_steps` for the wave's count of valid token fragments;
  // every instance issues the same loads and barriers.
  Frags fr[2];
  auto tile_steps = [&](auto vc, int j0) {
    constexpr int V = decltype(vc)::value;
    constexpr int NRD = V == 0 ? 0 : V + (BT ? 2 : 1) * NF;  // LDS reads per k-step
    constexpr int NMF = V * NF;                              // MFMAs per k-step
    constexpr int NIL = NMF < NRD ? NMF : NRD;               // reads interleaved one by one with MFMAs
    read_frags(vc, j0 % S, 0, fr[0]);
    for (int j = j0; j < j0 + nk; ++j) {
      if (issued < total_steps) issue_next();
      const int buf = j % S;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) read_frags(vc, buf, kk + 1, fr[(kk + 1) & 1]);
        mfma(vc, fr[kk & 1]);
        if (NMF > 0 && kk + 1 < KS) {
          // one fragment read of the next k-step between consecutive MFMAs, so
          // the LDS latency hides behind the matrix pipe instead of a full drain
          if constexpr (NRD > NIL) __builtin_amdgcn_sched_group_barrier(0x100, NRD - NIL, 0);
#pragma unroll
          for (int q = 0; q < NIL; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (NMF > NIL) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NIL, 0);
        }
      }
      if (j + 1 < total_steps) {
        wait_stages<L>(issued - j - 2);  // stage j + 1 complete
        lds_barrier();
        if (j + 1 < j0 + nk) read_frags(vc, (j + 1) % S, 0, fr[0]);
      }
    }
  };
  wait_stages<L>(issued - 1);
  lds_barrier();
  for (int ti = 0; ti < my_tiles; ++ti) {
    const PipeTile ct = decode(ti);  // tile being computed
    zero();
    int nv = (ct.rows - wm * (MF * 32) + 31) / 32;
    nv = nv < 0 ? 0 : (nv > MF ? MF : nv);
    nv = __builtin_amdgcn_readfirstlane(nv);
    const int j0 = ti * nk;
    if (nv >= MF) tile_steps(std::integral_constant<int, MF>{}, j0);
    else if (MF > 3 && nv == 3) tile_steps(std::integral_constant<int, (MF > 3 ? 3 : 0)>{}, j0);
    else if (MF > 2 && nv == 2) tile_steps(std::integral_constant<int, (MF > 2 ? 2 : 0)>{}, j0);
    else if (nv == 1) tile_steps(std::integral_constant<int, 1>{}, j0);
    else tile_steps(std::integral_constant<int, 0>{}, j0);
    store(ct);
  }
  if constexpr (EPI == EPI_COMBINE1) combine1_dropped(cmb, C, N, rmax, slot, G, tid, 64 * NW);
}

// ---------------------------------------------------------------------------
// The same tiles with separate LDS rings for the two operands: token rows in a
// ring of 2 stages, weight rows in a ring of SW >= 3.  Per step j the loads go
// out token group first (stage j + 1), then weight group (stage j + SW - 1), so
// that waiting for the token stage j + 1 leaves the newest weight group in
// flight (vector memory operations complete in issue order): the weight rows,
// streamed from HBM once per tile, get SW - 1 steps to arrive, the token rows
// (shared by the tiles of one expert, mostly L2 hits) one step.  BK = 64, 8
// waves.
// ---------------------------------------------------------------------------
template <int BM, int WR, int SW, int WGM, int EPI, bool NTW>
__global__ void __launch_bounds__(512, 1) grouped_gemm_ring_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ W,
                                                                   const uint16_t* __restrict__ W2,
                                                                   uint16_t* __restrict__ C,
                                                                   const int32_t* __restrict__ offsets, int E,
                                                                   int N, int K, int rmax,
                                                                   const int32_t* __restrict__ gather, int xrows,
                                                                   Combine1 cmb) {
  constexpr int NW = 8, BK = 64, CPR = 8, RSH = 1;
  constexpr bool kGated = EPI == EPI_SWIGLU;
  constexpr int BN = kGated ? WR / 2 : WR;
  constexpr int ASTAGE = BM * BK, WSTAGE = WR * BK;  // bf16 elements per stage of each ring
  constexpr int LA = BM * CPR / (64 * NW), LW = WR * CPR / (64 * NW);  // loads per wave per stage
  constexpr int WGN = NW / WGM;
  constexpr int MF = BM / WGM / 32, NF = WR / WGN / 32;
  constexpr int HF = kGated ? NF / 2 : NF;
  constexpr int KS = BK / 16;
  static_assert(BM * CPR % (64 * NW) == 0 && WR * CPR % (64 * NW) == 0, "whole load groups");
  static_assert(MF >= 1 && NF >= 1 && (!kGated || NF % 2 == 0), "SwiGLU waves pair gate and up fragments");
  static_assert(MF * NF >= MF + NF, "enough MFMAs to interleave the next k-step's reads");
  static_assert(SW >= 3 && LA + (SW - 2) * LW < 64, "rings");
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s_a = smem;                                     // [2][BM][BK]
  uint16_t* s_w = smem + 2 * ASTAGE;                        // [SW][WR][BK]
  int* s_ts = reinterpret_cast<int*>(s_w + SW * WSTAGE);   // [E+1]
  int* s_off = s_ts + (E + 1);                              // [E+1]
  __shared__ int s_scan[NW + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int ntn = (N + BN - 1) / BN;
  __shared__ int s_gidx[2][NW][64];  // gathered row indices, two tiles
  int gbuf = 0;
  {
    const int per = (E + 64 * NW - 1) / (64 * NW);
    const int e0 = tid * per;
    int cnt = 0;
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) cnt += (offsets[e + 1] - offsets[e] + BM - 1) / BM * ntn;
    }
    int total;
    int run = block_exclusive_scan(cnt, s_scan, &total);
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) {
        s_ts[e] = run;
        s_off[e] = offsets[e];
        run += (offsets[e + 1] - offsets[e] + BM - 1) / BM * ntn;
      }
    }
    if (tid == 0) {
      s_ts[E] = total;
      s_off[E] = offsets[E];
    }
    __syncthreads();
  }
  const int G = gridDim.x;
  const int total_tiles = s_ts[E];
  const int slot = (G % 8 == 0) ? ((int)blockIdx.x % 8) * (G / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;
  const int my_tiles = total_tiles > slot ? (total_tiles - 1 - slot) / G + 1 : 0;
  const int nk = K / BK;
  const int total_steps = my_tiles * nk;
  if (total_steps == 0) {
    if constexpr (EPI == EPI_COMBINE1) combine1_dropped(cmb, C, N, rmax, slot, G, tid, 64 * NW);
    return;
  }

  auto decode = [&](int i) {
    const int g = slot + i * G;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_ts[mid] <= g) lo = mid;
      else hi = mid;
    }
    const int mt_e = (s_off[lo + 1] - s_off[lo] + BM - 1) / BM;
    const int local = g - s_ts[lo];
    const int nt = local / mt_e;
    PipeTile t;
    t.e = lo;
    t.row0 = s_off[lo] + (local - nt * mt_e) * BM;
    t.rows = min(min(BM, s_off[lo + 1] - t.row0), rmax - t.row0);
    if (t.rows <= 0) {
      t.rows = 0;
      t.row0 = 0;
    }
    t.n0 = nt * BN;
    return t;
  };
  auto lds_pos = [](int r, int c) { return (r * CPR + (c ^ ((r >> RSH) & (CPR - 1)))) * 8; };

  // per-tile row addresses of this wave's loads (integers: see the pipe kernel)
  uintptr_t rowA[LA], rowW[LW];
  auto set_rows_a = [&](const PipeTile& t) {
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int p = (q * NW + w) * 64 + lane;
      const int r = p / CPR, c = (p % CPR) ^ ((r >> RSH) & (CPR - 1));
      const int rr = r < t.rows ? r : 0;
      const int src = gather ? clamp_row(s_gidx[gbuf][w][q * 8 + lane / CPR], xrows) : t.row0 + rr;
      rowA[q] = (r >= t.rows && K <= kZeroRowElems) ? reinterpret_cast<uintptr_t>(g_zero_row + c * 8)
                                                    : reinterpret_cast<uintptr_t>(A + (size_t)src * K + c * 8);
    }
  };
  auto set_rows_w = [&](const PipeTile& t) {
#pragma unroll
    for (int q = 0; q < LW; ++q) {
      const int p = (q * NW + w) * 64 + lane;
      const int r = p / CPR, c = (p % CPR) ^ ((r >> RSH) & (CPR - 1));
      const uint16_t* base = (kGated && r >= WR / 2) ? W2 : W;
      int n = t.n0 + (kGated ? (r & (WR / 2 - 1)) : r);
      n = n < N ? n : N - 1;
      rowW[q] = reinterpret_cast<uintptr_t>(base + ((size_t)t.e * N + n) * K + c * 8);
    }
  };
  // load trackers: next stage index, its tile and k-step, per operand
  int a_next = 0, a_tile = 0, a_k = 0;
  int w_next = 0, w_tile = 0, w_k = 0;
  if (gather) {
    fetch_gather_rows<LA, NW, 8>(gather, decode(0), w, lane, &s_gidx[0][w][0]);
    wait_vmcnt<0>();
  }
  set_rows_a(decode(0));
  if (gather && my_tiles > 1) fetch_gather_rows<LA, NW, 8>(gather, decode(1), w, lane, &s_gidx[1][w][0]);
  set_rows_w(decode(0));
  auto issue_a = [&]() {
    uint16_t* st = s_a + (a_next & 1) * ASTAGE;
#pragma unroll
    for (int q = 0; q < LA; ++q)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(rowA[q]) + a_k * BK,
                                       st + (q * NW + w) * 512, 16, 0, 0);
    ++a_next;
    if (++a_k == nk) {
      a_k = 0;
      if (++a_tile < my_tiles) {
        // the table of this tile came in with a load issued a tile earlier, before
        // at least one weight group that every step's wait covers
        gbuf ^= 1;
        set_rows_a(decode(a_tile));
        if (gather && a_tile + 1 < my_tiles)
          fetch_gather_rows<LA, NW, 8>(gather, decode(a_tile + 1), w, lane, &s_gidx[gbuf ^ 1][w][0]);
      }
    }
  };
  auto issue_w = [&]() {
    uint16_t* st = s_w + (w_next % SW) * WSTAGE;
#pragma unroll
    for (int q = 0; q < LW; ++q) {
      const uint16_t* src = reinterpret_cast<const uint16_t*>(rowW[q]) + w_k * BK;
      if (NTW) __builtin_amdgcn_global_load_lds(src, st + (q * NW + w) * 512, 16, 0, kLoadNT);
      else __builtin_amdgcn_global_load_lds(src, st + (q * NW + w) * 512, 16, 0, 0);
    }
    ++w_next;
    if (++w_k == nk) {
      w_k = 0;
      if (++w_tile < my_tiles) set_rows_w(decode(w_tile));
    }
  };

  f32x16_t acc[NF][MF];
  auto zero = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[f][i][v] = 0.0f;
  };
  struct Frags {
    bf16x8_t w[NF], x[MF];
  };
  auto read_frags = [&](int j, int kk, Frags& fr) {
    const uint16_t* sa = s_a + (j & 1) * ASTAGE;
    const uint16_t* sw = s_w + (j % SW) * WSTAGE;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int r = (kGated ? (f / HF) * (WR / 2) + wn * (HF * 32) + (f % HF) * 32 : wn * (NF * 32) + f * 32) +
                    (lane & 31);
      fr.w[f] = *reinterpret_cast<const bf16x8_t*>(sw + lds_pos(r, c));
    }
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int r = wm * (MF * 32) + i * 32 + (lane & 31);
      fr.x[i] = *reinterpret_cast<const bf16x8_t*>(sa + lds_pos(r, c));
    }
  };
  auto mfma = [&](const Frags& fr) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < MF; ++i)
        acc[f][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.w[f], fr.x[i], acc[f][i], 0, 0, 0);
  };
  auto store = [&](const PipeTile& t) {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int m = wm * (MF * 32) + i * 32 + (lane & 31);
      int crow_i = t.row0 + m;  // output row: the packed row, or its token (top-1 combine)
      bool ok = m < t.rows;
      float gt = 0.0f;
      if constexpr (EPI == EPI_COMBINE1) {
        const int tok = ok ? cmb.row_token[crow_i] : -1;
        ok = tok >= 0 && tok < cmb.T;
        crow_i = ok ? tok : 0;
        gt = cmb.gate[crow_i];
      }
      if (ok) {
        uint16_t* crow = C + (size_t)crow_i * N;
        u32x4_t rv[HF][2];  // top-1 combine: this lane's residual groups of the row, loaded first
        if constexpr (EPI == EPI_COMBINE1) {
#pragma unroll
          for (int f = 0; f < HF; ++f)
#pragma unroll
            for (int g = 0; g < 4; g += 2) {
              const int n = t.n0 + wn * (HF * 32) + f * 32 + 8 * (g + (lane >> 5));
              rv[f][g / 2] = (cmb.res && n < N) ? *reinterpret_cast<const u32x4_t*>(cmb.res + (size_t)crow_i * N + n)
                                                : u32x4_t{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int f = 0; f < HF; ++f)
#pragma unroll
          for (int g = 0; g < 4; g += 2) {
            uint32_t pk[2][2];  // [group g, g + 1][packed column pair]
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float v[4];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj)
                v[jj] = kGated ? epilogue<EPI>(acc[f][i][4 * (g + h) + jj], acc[HF + f][i][4 * (g + h) + jj])
                               : epilogue<EPI>(acc[f][i][4 * (g + h) + jj], 0.0f);
              pk[h][0] = pack_bf16x2(v[0], v[1]);
              pk[h][1] = pack_bf16x2(v[2], v[3]);
            }
            // lanes l and l + 32 hold the two column halves of the 8-column
            // groups of one row: after swapping lanes 32..63 of group g's
            // words with lanes 0..31 of group g + 1's, lane l holds all of
            // group g and lane l + 32 all of group g + 1 (16-byte stores)
            const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
            const int n = t.n0 + wn * (HF * 32) + f * 32 + 8 * (g + (lane >> 5));
            u32x4_t o = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
            if constexpr (EPI == EPI_COMBINE1) o = combine1_8(o, rv[f][g / 2], gt);
            if (n < N) *reinterpret_cast<u32x4_t*>(crow + n) = o;
          }
      }
    }
  };

  // prologue: weight stages 0 .. SW-2, then token stage 0 (so that waiting for
  // a token stage covers the older weight stage of the same index)
#pragma unroll
  for (int s2 = 0; s2 < SW - 1; ++s2)
    if (w_next < total_steps) issue_w();
  issue_a();
  wait_vmcnt<0>();
  lds_barrier();

  PipeTile ct = decode(0);
  zero();
  Frags fr[2];
  read_frags(0, 0, fr[0]);
  for (int j = 0; j < total_steps; ++j) {
    // buffers (j+1) & 1 and (j + SW - 1) % SW were last read in step j - 1
    const bool more_a = a_next < total_steps;
    if (more_a) issue_a();  // stage j + 1
    const bool more_w = w_next < total_steps;
    if (more_w) issue_w();  // stage j + SW - 1
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 1 < KS) read_frags(j, kk + 1, fr[(kk + 1) & 1]);
      mfma(fr[kk & 1]);
      if (kk + 1 < KS) {
#pragma unroll
        for (int q = 0; q < MF + NF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MF * NF - (MF + NF), 0);
      }
    }
    if (j + 1 < total_steps) {
      // token stage j+1 (issued this step, before the weight group) and weight
      // stage j+1 (issued SW - 2 steps ago) complete; the weight group of this
      // step may stay in flight
      if (more_a && more_w) wait_vmcnt<LW>();
      else wait_vmcnt<0>();
      lds_barrier();
      read_frags(j + 1, 0, fr[0]);
    }
    if ((j + 1) % nk == 0) {
      store(ct);
      zero();
      if (j + 1 < total_steps) ct = decode((j + 1) / nk);
    }
  }
  if constexpr (EPI == EPI_COMBINE1) combine1_dropped(cmb, C, N, rmax, slot, G, tid, 64 * NW);
}

template <int BM, int WR, int SW, int WGM, int EPI, bool NTW>
static hipError_t launch_ring(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets, int E,
                              int N, int K, int64_t R_max, int cus, const int32_t* gather, int xrows,
                              const Combine1& cmb, hipStream_t st) {
  constexpr int BN = EPI == EPI_SWIGLU ? WR / 2 : WR;
  const int ntn = (N + BN - 1) / BN;
  const int64_t tiles = ((R_max + BM - 1) / BM + (R_max < E ? R_max : E)) * ntn;
  if (tiles <= 0) return hipSuccess;
  const int grid = (int)(tiles < cus ? tiles : cus);
  const size_t shm = sizeof(uint16_t) * ((size_t)2 * BM + (size_t)SW * WR) * 64 + sizeof(int) * 2 * (size_t)(E + 1);
  constexpr int kMaxShm = sizeof(uint16_t) * (2 * BM + SW * WR) * 64 + sizeof(int) * 2 * (1024 + 1);  // E <= 1024
  hipError_t err = lds_limit_once<grouped_gemm_ring_kernel<BM, WR, SW, WGM, EPI, NTW>>(kMaxShm);
  if (err != hipSuccess) return err;
  grouped_gemm_ring_kernel<BM, WR, SW, WGM, EPI, NTW><<<dim3(grid), dim3(512), shm, st>>>(
      static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(B2),
      static_cast<uint16_t*>(C), offsets, E, N, K, (int)R_max, gather, xrows, cmb);
  return hipGetLastError();
}

// rlo, rhi: only the experts with rlo < rows <= rhi
template <int BM, int WR, int BK, int S, int WGM, int EPI, bool NTW, int NW = 8, bool BT = false, bool SAVE = false>
static hipError_t launch_pipe(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets, int E,
                              int N, int K, int64_t R_max, int cus, const int32_t* gather, int xrows,
                              const Combine1& cmb, hipStream_t st, int rlo = -1, int rhi = INT32_MAX, int k1 = 0,
                              uint16_t* save = nullptr) {
  constexpr int BN = EPI == EPI_SWIGLU ? WR / 2 : WR;
  const int ntn = (N + BN - 1) / BN;
  const int64_t tiles = ((R_max + BM - 1) / BM + (R_max < E ? R_max : E)) * ntn;
  if (tiles <= 0) return hipSuccess;
  const int64_t slots = (int64_t)cus * (8 / NW);  // resident workgroups
  const int grid = (int)(tiles < slots ? tiles : slots);
  const size_t shm = sizeof(uint16_t) * (size_t)S * (BM + WR) * BK + sizeof(int) * 2 * (size_t)(E + 1);
  constexpr int kMaxShm = sizeof(uint16_t) * S * (BM + WR) * BK + sizeof(int) * 2 * (1024 + 1);  // E <= 1024
  hipError_t err = lds_limit_once<grouped_gemm_pipe_kernel<BM, WR, BK, S, WGM, EPI, NW, NTW, BT, SAVE>>(kMaxShm);
  if (err != hipSuccess) return err;
  grouped_gemm_pipe_kernel<BM, WR, BK, S, WGM, EPI, NW, NTW, BT, SAVE><<<dim3(grid), dim3(64 * NW), shm, st>>>(
      static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(B2),
      static_cast<uint16_t*>(C), offsets, E, N, K, (int)R_max, gather, xrows, cmb, rlo, rhi, k1, save);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_bf16(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets, int E,
                              int N, int K, int64_t R_max, hipStream_t st) {
  const int ntn = (N + GB_BN - 1) / GB_BN;
  const int64_t mtiles = (R_max + GB_BM - 1) / GB_BM + (R_max < E ? R_max : E);
  const int64_t grid = mtiles * ntn;
  if (grid <= 0) return hipSuccess;
  const size_t shm = sizeof(uint16_t) * (size_t)GB_TILE * 2 * (1 + (EPI == EPI_SWIGLU ? 2 : 1));
  hipError_t err = lds_limit_once<grouped_gemm_bf16_kernel<EPI>>((int)shm);
  if (err != hipSuccess) return err;
  grouped_gemm_bf16_kernel<EPI><<<dim3((unsigned)grid), dim3(256), shm, st>>>(
      static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(B2),
      static_cast<uint16_t*>(C), offsets, E, N, K, ntn, (int)R_max);
  return hipGetLastError();
}

template <bool kBF16, int EPI>
static hipError_t launch_scalar(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets, int E,
                                int N, int K, int64_t R_max, hipStream_t st) {
  const int nbx = (N + 63) / 64;
  const int64_t grid = R_max * nbx;
  if (grid <= 0) return hipSuccess;
  grouped_gemm_scalar_kernel<kBF16, EPI><<<dim3((unsigned)grid), dim3(64), 0, st>>>(A, B, B2, C, offsets, E, N, K,
                                                                                      nbx);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_f32(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets, int E,
                             int N, int K, int64_t R_max, hipStream_t st) {
  // m-tiles: at most ceil(R_max / 64) + one partial tile per expert
  const int64_t mtiles = (R_max + F32_T - 1) / F32_T + (R_max < E ? R_max : E);
  const int ntn = (N + F32_T - 1) / F32_T;
  if (mtiles <= 0 || ntn <= 0) return hipSuccess;
  if (mtiles > INT32_MAX || ntn > 65535) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_COMBINE1) return hipErrorInvalidValue;
  grouped_gemm_f32_kernel<EPI><<<dim3((unsigned)mtiles, (unsigned)ntn), dim3(256), 0, st>>>(
      static_cast<const float*>(A), static_cast<const float*>(B), static_cast<const float*>(B2),
      static_cast<float*>(C), offsets, E, N, K);
  return hipGetLastError();
}

template <int EPI, bool SAVE = false>
static hipError_t launch_one(bool vec, bool bf16, const void* A, const void* B, const void* B2, void* C,
                             const int32_t* offsets, int E, int N, int K, int64_t R_max, int64_t rows_cap,
                             hipStream_t st, const int32_t* gather = nullptr, int xrows = 0,
                             const Combine1& cmb = Combine1{}, uint16_t* save = nullptr) {
  if (vec && bf16 && K % 64 == 0) {
    int cus = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    // Experts with more than 128 rows on average take 256-row tiles: 256 x 256
    // (two stages of 512 rows), or, where 192 weight rows per tile fill the
    // CUs more evenly in whole waves of tiles, 256 x 192 with split rings (two
    // token stages, three weight stages).  Otherwise 128 x 256 tiles (three
    // 48 KB stages).
    constexpr bool kGated = EPI == EPI_SWIGLU;
    // the pipe tiles: BM x 256 with three 48 KB stages (BM = 128) or two 64 KB
    // stages (BM = 256); ntw: weight loads non-temporal (one m-tile per expert)
    auto pipe128 = [&](bool ntw, int rlo, int rhi) {
      return ntw ? launch_pipe<128, 256, 64, 3, 2, EPI, true, 8, false, SAVE>(A, B, B2, C, offsets, E, N, K, R_max, cus,
                                                                              gather, xrows, cmb, st, rlo, rhi, 0, save)
                 : launch_pipe<128, 256, 64, 3, 2, EPI, false, 8, false, SAVE>(
                       A, B, B2, C, offsets, E, N, K, R_max, cus, gather, xrows, cmb, st, rlo, rhi, 0, save);
    };
    auto pipe256 = [&](bool ntw, int rlo) {
      return ntw ? launch_pipe<256, 256, 64, 2, 2, EPI, true, 8, false, SAVE>(
                       A, B, B2, C, offsets, E, N, K, R_max, cus, gather, xrows, cmb, st, rlo, INT32_MAX, 0, save)
                 : launch_pipe<256, 256, 64, 2, 2, EPI, false, 8, false, SAVE>(
                       A, B, B2, C, offsets, E, N, K, R_max, cus, gather, xrows, cmb, st, rlo, INT32_MAX, 0, save);
    };
    if (R_max / E > 128) {
      auto fill = [&](int bn) {
        const int64_t tiles = (R_max / 256) * ((N + bn - 1) / bn);
        const int64_t waves = (tiles + cus - 1) / cus;
        return waves > 0 ? (double)tiles / (double)(waves * cus) : 0.0;
      };
      if constexpr (!kGated)
        if (fill(192) > fill(256) + 0.05 && !SAVE)
          return rows_cap <= 256 ? launch_ring<256, 192, 3, 4, EPI, true>(A, B, B2, C, offsets, E, N, K, R_max, cus,
                                                                           gather, xrows, cmb, st)
                                 : launch_ring<256, 192, 3, 4, EPI, false>(A, B, B2, C, offsets, E, N, K, R_max, cus,
                                                                            gather, xrows, cmb, st);
      return pipe256(rows_cap <= 256, -1);
    }
    // With experts of more than 128 rows possible, those take 256 x 256 tiles
    // (a CU's loads per stage carry twice the MFMA work) in a launch of their
    // own after the 128 x 256 tiles of the others.  (The top-1 combine epilogue
    // also handles the dropped tokens once per launch: kept in one launch.)
    if constexpr (EPI != EPI_COMBINE1) {
      if (rows_cap > 128) {
        hipError_t e1 = pipe128(true, -1, 128);
        if (e1 != hipSuccess) return e1;
        return pipe256(rows_cap <= 256, 128);
      }
    }
    return pipe128(rows_cap <= 128, -1, INT32_MAX);
  }
  // only the tiled kernels read gathered rows, combine or keep pre-activations
  if (gather || EPI == EPI_COMBINE1 || SAVE) return hipErrorInvalidValue;
  if (vec && bf16) return launch_bf16<EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
  if (bf16) return launch_scalar<true, EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
  // fp32: the LDS tiles once there is work to fill them (below about 2^26
  // multiply-adds the one-thread-per-output kernel has less fixed latency)
  if (R_max * (int64_t)N * K >= ((int64_t)1 << 26)) return launch_f32<EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
  return launch_scalar<false, EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
}

hipError_t device_cus(int* cus) {
  static int cached[kMaxDevices] = {};  // 0: not queried yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int v = __atomic_load_n(&cached[dev], __ATOMIC_ACQUIRE);
  if (v == 0) {
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELEASE);
  }
  *cus = v;
  return hipSuccess;
}

bool expert_ffn_gathers(bool bf16, bool vec, int H) { return bf16 && vec && H % 64 == 0; }
bool expert_ffn_combines(bool bf16, bool vec, int H, int F) { return bf16 && vec && H % 8 == 0 && F % 64 == 0; }
bool expert_ffn_saves(bool bf16, bool vec, int H, int F) { return bf16 && vec && H % 64 == 0 && F % 8 == 0; }

hipError_t launch_expert_ffn(const void* X, const void* W1, const void* W3, const void* W2, void* h, void* Y,
                             const int32_t* offsets, int E, int H, int F, int act, bool bf16, bool vec,
                             int64_t R_max, int64_t rows_cap, hipStream_t st, const int32_t* gather, int xrows,
                             const Combine1* cmb, void* saved) {
  if (R_max == 0) return cmb ? hipErrorInvalidValue : hipSuccess;  // the combine needs a launch to run in
  if (gather && !expert_ffn_gathers(bf16, vec, H)) return hipErrorInvalidValue;
  if (saved && !expert_ffn_saves(bf16, vec, H, F)) return hipErrorInvalidValue;
  uint16_t* save = static_cast<uint16_t*>(saved);
  if (cmb && !expert_ffn_combines(bf16, vec, H, F)) return hipErrorInvalidValue;
  hipError_t err;
  switch (act) {
    case 0:
      err = save ? launch_one<EPI_RELU, true>(vec, bf16, X, W1, nullptr, h, offsets, E, F, H, R_max, rows_cap, st,
                                              gather, xrows, Combine1{}, save)
                 : launch_one<EPI_RELU>(vec, bf16, X, W1, nullptr, h, offsets, E, F, H, R_max, rows_cap, st, gather,
                                        xrows);
      break;
    case 1:
      err = save ? launch_one<EPI_GELU, true>(vec, bf16, X, W1, nullptr, h, offsets, E, F, H, R_max, rows_cap, st,
                                              gather, xrows, Combine1{}, save)
                 : launch_one<EPI_GELU>(vec, bf16, X, W1, nullptr, h, offsets, E, F, H, R_max, rows_cap, st, gather,
                                        xrows);
      break;
    default:
      err = save ? launch_one<EPI_SWIGLU, true>(vec, bf16, X, W1, W3, h, offsets, E, F, H, R_max, rows_cap, st,
                                                gather, xrows, Combine1{}, save)
                 : launch_one<EPI_SWIGLU>(vec, bf16, X, W1, W3, h, offsets, E, F, H, R_max, rows_cap, st, gather,
                                          xrows);
      break;
  }
  if (err != hipSuccess) return err;
  if (cmb)
    return launch_one<EPI_COMBINE1>(vec, bf16, h, W2, nullptr, Y, offsets, E, H, F, R_max, rows_cap, st, nullptr, 0,
                                    *cmb);
  return launch_one<EPI_NONE>(vec, bf16, h, W2, nullptr, Y, offsets, E, H, F, R_max, rows_cap, st);
}

hipError_t launch_grouped_gemm_bf16(const void* A, const void* B, void* C, const int32_t* offsets, int E, int N, int K,
                                    int64_t R_max, int64_t rows_cap, bool vec, hipStream_t st, const int32_t* gather,
                                    int xrows) {
  if (R_max == 0) return hipSuccess;
  return launch_one<EPI_NONE>(vec, true, A, B, nullptr, C, offsets, E, N, K, R_max, rows_cap, st, gather, xrows);
}

hipError_t launch_grouped_gemm_bf16_kn(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets,
                                       int E, int N, int K, int k1, int64_t R_max, int64_t rows_cap, hipStream_t st,
                                       const int32_t* gather, int xrows) {
  if (R_max == 0) return hipSuccess;
  if (K % 64 != 0 || N % 8 != 0 || N < 8 || (B2 ? (2 * k1 != K || k1 % 64 != 0) : k1 != K))
    return hipErrorInvalidValue;
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  const Combine1 cmb{};
  // the row-major form's tile choice, pipe tiles only: 128 x 256 for experts of
  // at most 128 rows, 256 x 256 for the larger ones
  if (R_max / E > 128 || rows_cap > 128) {
    if (R_max / E <= 128) {
      err = launch_pipe<128, 256, 64, 3, 2, EPI_NONE, true, 8, true>(A, B, B2, C, offsets, E, N, K, R_max, cus, gather,
                                                                     xrows, cmb, st, -1, 128, k1);
      if (err != hipSuccess) return err;
    }
    const int rlo = R_max / E > 128 ? -1 : 128;
    return rows_cap <= 256 ? launch_pipe<256, 256, 64, 2, 2, EPI_NONE, true, 8, true>(
                                 A, B, B2, C, offsets, E, N, K, R_max, cus, gather, xrows, cmb, st, rlo, INT32_MAX, k1)
                           : launch_pipe<256, 256, 64, 2, 2, EPI_NONE, false, 8, true>(
                                 A, B, B2, C, offsets, E, N, K, R_max, cus, gather, xrows, cmb, st, rlo, INT32_MAX, k1);
  }
  return launch_pipe<128, 256, 64, 3, 2, EPI_NONE, true, 8, true>(A, B, B2, C, offsets, E, N, K, R_max, cus, gather,
                                                                  xrows, cmb, st, -1, INT32_MAX, k1);
}

}  // namespace moe
