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
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

enum { EPI_NONE = 0, EPI_RELU = 1, EPI_GELU = 2, EPI_SWIGLU = 3 };

template <int EPI>
__device__ __forceinline__ float epilogue(float a, float b) {
  if (EPI == EPI_RELU) return a > 0.0f ? a : 0.0f;
  if (EPI == EPI_GELU) return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
  if (EPI == EPI_SWIGLU) return (a / (1.0f + expf(-a))) * b;
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
  const float v = epilogue<EPI>(s1, s2);
  if (kBF16) static_cast<uint16_t*>(C)[(size_t)row * N + n] = (uint16_t)f32_to_bf16_bits(v);
  else static_cast<float*>(C)[(size_t)row * N + n] = v;
}

template <int EPI>
static hipError_t launch_bf16(const void* A, const void* B, const void* B2, void* C, const int32_t* offsets, int E,
                              int N, int K, int64_t R_max, hipStream_t st) {
  const int ntn = (N + GB_BN - 1) / GB_BN;
  const int64_t mtiles = (R_max + GB_BM - 1) / GB_BM + (R_max < E ? R_max : E);
  const int64_t grid = mtiles * ntn;
  if (grid <= 0) return hipSuccess;
  const size_t shm = sizeof(uint16_t) * (size_t)GB_TILE * 2 * (1 + (EPI == EPI_SWIGLU ? 2 : 1));
  hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_bf16_kernel<EPI>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
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
static hipError_t launch_one(bool vec, bool bf16, const void* A, const void* B, const void* B2, void* C,
                             const int32_t* offsets, int E, int N, int K, int64_t R_max, hipStream_t st) {
  if (vec && bf16) return launch_bf16<EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
  if (bf16) return launch_scalar<true, EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
  return launch_scalar<false, EPI>(A, B, B2, C, offsets, E, N, K, R_max, st);
}

hipError_t launch_expert_ffn(const void* X, const void* W1, const void* W3, const void* W2, void* h, void* Y,
                             const int32_t* offsets, int E, int H, int F, int act, bool bf16, bool vec,
                             int64_t R_max, hipStream_t st) {
  if (R_max == 0) return hipSuccess;
  hipError_t err;
  switch (act) {
    case 0: err = launch_one<EPI_RELU>(vec, bf16, X, W1, nullptr, h, offsets, E, F, H, R_max, st); break;
    case 1: err = launch_one<EPI_GELU>(vec, bf16, X, W1, nullptr, h, offsets, E, F, H, R_max, st); break;
    default: err = launch_one<EPI_SWIGLU>(vec, bf16, X, W1, W3, h, offsets, E, F, H, R_max, st); break;
  }
  if (err != hipSuccess) return err;
  return launch_one<EPI_NONE>(vec, bf16, h, W2, nullptr, Y, offsets, E, H, F, R_max, st);
}

}  // namespace moe
