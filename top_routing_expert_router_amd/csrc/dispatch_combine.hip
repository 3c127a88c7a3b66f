// Dispatch (gather into expert-contiguous rows) and combine (gate-weighted sum
// plus residual): the two bandwidth kernels around the expert FFN.
//
// "Expert-parallel MoE training" explainer, walk through one MoE layer: tokens
// are grouped by target expert; afterwards the outputs are unpermuted, multiplied
// by the gate probabilities, summed, and the residual is added.  Switch
// Transformers explainer §1.2: an overflowed token skips the expert and passes
// through the residual.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// K3 (vector path): token-major; every 16-byte piece of x[t] is read once and
// written to each of the token's kept rows.
__global__ void __launch_bounds__(256) dispatch_vec_kernel(const u32x4_t* __restrict__ x,
                                                           const int32_t* __restrict__ dst_row,
                                                           u32x4_t* __restrict__ X, int64_t total, int nvec, int k,
                                                           int rmax) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / nvec;
    const int c = (int)(i - t * nvec);
    const u32x4_t v = x[i];
    for (int r = 0; r < k; ++r) {
      const int d = dst_row[t * k + r];
      if (d >= 0 && d < rmax) X[(int64_t)d * nvec + c] = v;
    }
  }
}

// K3 (scalar path): one element (2 or 4 bytes) per thread-iteration.
template <typename U>
__global__ void __launch_bounds__(256) dispatch_scalar_kernel(const U* __restrict__ x,
                                                              const int32_t* __restrict__ dst_row, U* __restrict__ X,
                                                              int64_t total, int H, int k, int rmax) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H;
    const int c = (int)(i - t * H);
    const U v = x[i];
    for (int r = 0; r < k; ++r) {
      const int d = dst_row[t * k + r];
      if (d >= 0 && d < rmax) X[(int64_t)d * H + c] = v;
    }
  }
}

// K5: y[t][c..c+8) = residual + sum_r g[t][r] * Y[dst_row[t][r]] (r ascending,
// fp32 fused multiply-add), rounded once to the output dtype.
template <bool kBF16>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ Y, const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ gate,
                                                      const void* __restrict__ residual, void* __restrict__ y,
                                                      int64_t total, int nch, int H, int k, int rmax,
                                                      int vec_ok, const void* __restrict__ shared) {
  const size_t eb = kBF16 ? 2 : 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / nch;
    const int64_t c = (i - t * nch) * 8;
    float acc[8];
    if (residual) {
      load8_f32<kBF16>(static_cast<const char*>(residual) + (size_t)t * H * eb, c, H, vec_ok, acc);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    }
    for (int r = 0; r < k; ++r) {
      const int d = dst_row[t * k + r];
      if (d < 0 || d >= rmax) continue;
      const float g = gate[t * k + r];
      float v[8];
      load8_f32<kBF16>(static_cast<const char*>(Y) + (size_t)d * H * eb, c, H, vec_ok, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(g, v[j], acc[j]);
    }
    if (shared) {  // the shared expert's output, added last
      float v[8];
      load8_f32<kBF16>(static_cast<const char*>(shared) + (size_t)t * H * eb, c, H, vec_ok, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
    if (kBF16) {
      uint16_t* out = static_cast<uint16_t*>(y) + (size_t)t * H;
      if (vec_ok && c + 8 <= H) {
        u32x4_t o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_bits(acc[2 * j]) | (f32_to_bf16_bits(acc[2 * j + 1]) << 16);
        *reinterpret_cast<u32x4_t*>(out + c) = o;
      } else {
        for (int j = 0; j < 8; ++j)
          if (c + j < H) out[c + j] = (uint16_t)f32_to_bf16_bits(acc[j]);
      }
    } else {
      float* out = static_cast<float*>(y) + (size_t)t * H;
      if (vec_ok && c + 8 <= H) {
        *reinterpret_cast<f32x4_t*>(out + c) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4_t*>(out + c + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
      } else {
        for (int j = 0; j < 8; ++j)
          if (c + j < H) out[c + j] = acc[j];
      }
    }
  }
}

// K5 for bf16 rows in 16-byte groups and k <= KU: the same sum in the same
// order, with the token's choices and all of its expert rows loaded before the
// first multiply-add (KU rows in flight per thread instead of one at a time).
template <int KU>
__global__ void __launch_bounds__(256) combine_bf16_kernel(const uint16_t* __restrict__ Y,
                                                           const int32_t* __restrict__ dst_row,
                                                           const float* __restrict__ gate,
                                                           const uint16_t* __restrict__ residual,
                                                           uint16_t* __restrict__ y, int64_t total, int nch, int H,
                                                           int k, int rmax, const uint16_t* __restrict__ shared) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / nch;
    const int64_t c = (i - t * nch) * 8;
    int d[KU];
    float g[KU];
#pragma unroll
    for (int r = 0; r < KU; ++r) {
      d[r] = r < k ? dst_row[t * k + r] : -1;
      g[r] = r < k ? gate[t * k + r] : 0.0f;
    }
    u32x4_t q[KU];
#pragma unroll
    for (int r = 0; r < KU; ++r)
      q[r] = (d[r] >= 0 && d[r] < rmax) ? *reinterpret_cast<const u32x4_t*>(Y + (size_t)d[r] * H + c)
                                        : u32x4_t{0, 0, 0, 0};
    const u32x4_t rq = residual ? *reinterpret_cast<const u32x4_t*>(residual + (size_t)t * H + c)
                                : u32x4_t{0, 0, 0, 0};
    float acc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = __uint_as_float(rq[j] << 16);
      acc[2 * j + 1] = __uint_as_float(rq[j] & 0xFFFF0000u);
    }
#pragma unroll
    for (int r = 0; r < KU; ++r) {
      if (d[r] < 0 || d[r] >= rmax) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = __builtin_fmaf(g[r], __uint_as_float(q[r][j] << 16), acc[2 * j]);
        acc[2 * j + 1] = __builtin_fmaf(g[r], __uint_as_float(q[r][j] & 0xFFFF0000u), acc[2 * j + 1]);
      }
    }
    if (shared) {  // the shared expert's output, added last
      const u32x4_t sq = *reinterpret_cast<const u32x4_t*>(shared + (size_t)t * H + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(sq[j] << 16);
        acc[2 * j + 1] += __uint_as_float(sq[j] & 0xFFFF0000u);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_bits(acc[2 * j]) | (f32_to_bf16_bits(acc[2 * j + 1]) << 16);
    *reinterpret_cast<u32x4_t*>(y + (size_t)t * H + c) = o;
  }
}

static int grid_for(int64_t total, int block) {
  int64_t g = (total + block - 1) / block;
  const int64_t cap = 256 * 64;  // enough resident waves for 256 CUs; the loop strides the rest
  if (g > cap) g = cap;
  return (int)(g > 0 ? g : 1);
}

hipError_t launch_dispatch(const void* x, const int32_t* dst_row, void* X, int T, int H, int k, int rmax, bool bf16,
                           bool vec_ok, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int eb = bf16 ? 2 : 4;
  if (vec_ok && ((int64_t)H * eb) % 16 == 0) {
    const int nvec = (int)((int64_t)H * eb / 16);
    const int64_t total = (int64_t)T * nvec;
    dispatch_vec_kernel<<<grid_for(total, 256), 256, 0, st>>>(static_cast<const u32x4_t*>(x), dst_row,
                                                               static_cast<u32x4_t*>(X), total, nvec, k, rmax);
  } else {
    const int64_t total = (int64_t)T * H;
    if (bf16)
      dispatch_scalar_kernel<uint16_t><<<grid_for(total, 256), 256, 0, st>>>(
          static_cast<const uint16_t*>(x), dst_row, static_cast<uint16_t*>(X), total, H, k, rmax);
    else
      dispatch_scalar_kernel<uint32_t><<<grid_for(total, 256), 256, 0, st>>>(
          static_cast<const uint32_t*>(x), dst_row, static_cast<uint32_t*>(X), total, H, k, rmax);
  }
  return hipGetLastError();
}

__global__ void dense_offsets_kernel(int32_t* off, int T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

hipError_t launch_dense_offsets(int32_t* off, int T, hipStream_t st) {
  dense_offsets_kernel<<<1, 64, 0, st>>>(off, T);
  return hipGetLastError();
}

hipError_t launch_combine(const void* Y, const int32_t* dst_row, const float* gate, const void* residual, void* y,
                          int T, int H, int k, int rmax, bool bf16, bool vec_ok, hipStream_t st, const void* shared) {
  if (T == 0) return hipSuccess;
  const int nch = (H + 7) / 8;
  const int64_t total = (int64_t)T * nch;
  if (bf16 && vec_ok && H % 8 == 0 && k <= 16) {
    const uint16_t *Yb = static_cast<const uint16_t*>(Y), *rb = static_cast<const uint16_t*>(residual),
                   *sb = static_cast<const uint16_t*>(shared);
    uint16_t* yb = static_cast<uint16_t*>(y);
    const int g = grid_for(total, 256);
    if (k <= 1) combine_bf16_kernel<1><<<g, 256, 0, st>>>(Yb, dst_row, gate, rb, yb, total, nch, H, k, rmax, sb);
    else if (k <= 2) combine_bf16_kernel<2><<<g, 256, 0, st>>>(Yb, dst_row, gate, rb, yb, total, nch, H, k, rmax, sb);
    else if (k <= 4) combine_bf16_kernel<4><<<g, 256, 0, st>>>(Yb, dst_row, gate, rb, yb, total, nch, H, k, rmax, sb);
    else if (k <= 8) combine_bf16_kernel<8><<<g, 256, 0, st>>>(Yb, dst_row, gate, rb, yb, total, nch, H, k, rmax, sb);
    else combine_bf16_kernel<16><<<g, 256, 0, st>>>(Yb, dst_row, gate, rb, yb, total, nch, H, k, rmax, sb);
    return hipGetLastError();
  }
  if (bf16)
    combine_kernel<true><<<grid_for(total, 256), 256, 0, st>>>(Y, dst_row, gate, residual, y, total, nch, H, k,
                                                                rmax, vec_ok, shared);
  else
    combine_kernel<false><<<grid_for(total, 256), 256, 0, st>>>(Y, dst_row, gate, residual, y, total, nch, H, k,
                                                                 rmax, vec_ok, shared);
  return hipGetLastError();
}

}  // namespace moe
