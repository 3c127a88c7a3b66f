// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32.  A bf16 value is the upper half of a binary32, so widening is
// a shift; narrowing rounds to nearest, ties to even (inputs are finite).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values rounded to nearest, ties to even, as bf16 packed into one word
// (lo in bits 0..15): one hardware conversion for the pair.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// Loads 8 consecutive elements [i, i+8) of a row of `n` elements as fp32,
// zero-filling past the end.  `vec_ok` promises 16-byte alignment of every
// vector access (the row base and i are multiples of the vector width).
template <bool kBF16>
__device__ __forceinline__ void load8_f32(const void* row, int64_t i, int64_t n, bool vec_ok, float (&v)[8]) {
  if (kBF16) {
    const uint16_t* p = static_cast<const uint16_t*>(row);
    if (vec_ok && i + 8 <= n) {
      u32x4_t q = *reinterpret_cast<const u32x4_t*>(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(q[j] << 16);
        v[2 * j + 1] = __uint_as_float(q[j] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (i + j < n) ? bf16_bits_to_f32(p[i + j]) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(row);
    if (vec_ok && i + 8 <= n) {
      f32x4_t a = *reinterpret_cast<const f32x4_t*>(p + i);
      f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + i + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[4 + j] = b[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (i + j < n) ? p[i + j] : 0.0f;
    }
  }
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Block-wide exclusive scan of one int per thread (blockDim.x a multiple of 64,
// at most 1024).  `tmp` must hold blockDim.x / 64 + 1 ints.  Returns the exclusive
// prefix and writes the block total into *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < nw; ++i) {
      int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[nw] = run;
  }
  __syncthreads();
  int ex = tmp[w] + inc - v;
  *total = tmp[nw];
  __syncthreads();
  return ex;
}

// Gate value of choice r from the chosen logits sv[0..k) (sv[0] the largest) and
// den: the softmax denominator over all E relative to sv[0] (gate mode 0) or over
// the chosen (other modes).  With sigmoid scores (kSigmoidFlag in the mode) the
// gate is the chosen score itself (mode 0) or the score over the chosen scores'
// sum (mode 1); mode 2 is the softmax over the chosen either way.
template <int KMAX>
__device__ __forceinline__ float gate_value(int gate_mode, int k, const float (&sv)[KMAX], float den, int r) {
  const int gm = gate_mode & (kSigmoidFlag - 1);
  if ((gate_mode & kSigmoidFlag) && gm != 2) {
    const float sc = 1.0f / (1.0f + expf(-sv[r]));
    if (gm == 0) return sc;
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) sum += 1.0f / (1.0f + expf(-sv[j]));
    return sc / sum;
  }
  return expf(sv[r] - sv[0]) / den;
}

// GShard's random second choice ("Expert-parallel MoE training" explainer,
// router: top-2 with the second expert taken at random by its weight): taken iff
// u * (g1 + g2) < 2 * g2, in binary64 on the fp32 gates.
__device__ __forceinline__ bool second_choice_taken(float u, float g1, float g2) {
  return (double)u * ((double)g1 + (double)g2) < 2.0 * (double)g2;
}

// Explicit waits for direct-to-LDS loads (vector memory operations complete in
// issue order, so `vmcnt <= N` means all but the last N issued have landed).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Transposing LDS read (ds_read_b64_tr_b16) of the 8 bytes at p, an LDS
// address: in each group of 16 lanes, lane i receives element i % 4 of the
// reads of lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12, in that order.
__device__ __forceinline__ s16x4_t lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

// Workgroup barrier ordering LDS accesses for the compiler, without the
// vmcnt(0) that a memory fence would add (direct-to-LDS loads are waited on
// explicitly before it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Waits until at most `after` stages of L loads are outstanding (a count past
// the counter's range of 63 waits for more, never less).
template <int L>
__device__ __forceinline__ void wait_stages(int after) {
  constexpr int c1 = L < 63 ? L : 63, c2 = 2 * L < 63 ? 2 * L : 63, c3 = 3 * L < 63 ? 3 * L : 63,
                c4 = 4 * L < 63 ? 4 * L : 63;
  switch (after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<c1>(); break;
    case 2: wait_vmcnt<c2>(); break;
    case 3: wait_vmcnt<c3>(); break;
    default: wait_vmcnt<c4>(); break;
  }
}

}  // namespace moe
