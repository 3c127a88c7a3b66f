// Capacity-limited slot assignment and packing, from the per-block histograms
// and in-block ranks that the select kernel produced.
//
// "Expert-parallel MoE training" explainer, router/capacity section:
// capacity = ceil((T*k/E)*cf); assignments past an expert's capacity are dropped
// ("position" policy: the ones at the end of the batch), or nothing is dropped
// (dropless).  DeepSpeed discussion #7508: an index permutation replaces the dense
// one-hot [T,E,C] dispatch mask.
//
// Priority: choice-major, then token order (every token's first choice before
// any second choice).  With blocks of 64 tokens and hist[e][r*nb + blk] = number
// of tokens of block blk whose choice r is expert e, the slot of (t, r) at
// expert e is  base[e][r*nb + blk] + rank(t, r)  where base is the exclusive
// prefix sum of hist[e][.] in (r, blk) order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// K2a: one workgroup per expert scans its k*nb histogram entries in place
// (-> base), and writes demand[e] and kept[e] = min(demand, C).
__global__ void __launch_bounds__(256) slot_scan_kernel(int32_t* __restrict__ hist, int Q, int C,
                                                        int32_t* __restrict__ demand, int32_t* __restrict__ kept) {
  __shared__ int tmp[256 / 64 + 1];
  const int e = blockIdx.x;
  int32_t* h = hist + (size_t)e * Q;
  const int per = (Q + 255) / 256;
  const int start = threadIdx.x * per;
  const int end = min(start + per, Q);
  int s = 0;
  for (int q = start; q < end; ++q) s += h[q];
  int total;
  int run = block_exclusive_scan(s, tmp, &total);
  for (int q = start; q < end; ++q) {
    int v = h[q];
    h[q] = run;
    run += v;
  }
  if (threadIdx.x == 0) {
    demand[e] = total;
    kept[e] = total < C ? total : C;
  }
}

// K2b: one wave per block of 64 tokens.  Every workgroup derives offsets (the
// exclusive prefix sum of kept) in LDS; workgroup 0 also publishes offsets[0..E]
// and n_dropped.  Then each lane resolves its token's k assignments.
__global__ void __launch_bounds__(64) slot_finalize_kernel(const int32_t* __restrict__ base, int Q, int nb, int T,
                                                           int E, int k, int C, const int32_t* __restrict__ topk_idx,
                                                           const int32_t* __restrict__ kept,
                                                           int32_t* __restrict__ dst_row,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ n_dropped, int rmax) {
  extern __shared__ int s_off[];  // [E+1]
  const int lane = threadIdx.x;
  const int per = (E + 63) / 64;
  const int e_begin = lane * per;
  int s = 0;
  for (int j = 0; j < per; ++j) {
    int e = e_begin + j;
    if (e < E) s += kept[e];
  }
  int inc = wave_inclusive_scan(s);
  int run = inc - s;
  for (int j = 0; j < per; ++j) {
    int e = e_begin + j;
    if (e < E) {
      s_off[e] = run;
      run += kept[e];
    }
  }
  const int R = __shfl(inc, 63, 64);
  if (lane == 0) s_off[E] = R;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = lane; e <= E; e += 64) offsets[e] = s_off[e];
    if (lane == 0) *n_dropped = T * k - R;
  }
  const int blk = blockIdx.x;
  const int t = blk * 64 + lane;
  if (t >= T) return;
  for (int r = 0; r < k; ++r) {
    const size_t i = (size_t)t * k + r;
    const int e = topk_idx[i];
    const int slot = base[(size_t)e * Q + r * nb + blk] + dst_row[i];
    const int d = s_off[e] + slot;
    if (slot < C && d < rmax) {  // d < R <= rmax for any plan this kernel derives
      dst_row[i] = d;
      row_token[d] = t;
    } else {
      dst_row[i] = -1;
    }
  }
}

hipError_t launch_slot_scan(int32_t* hist, int Q, int E, int C, int32_t* demand, int32_t* kept, hipStream_t st) {
  slot_scan_kernel<<<dim3(E), dim3(256), 0, st>>>(hist, Q, C, demand, kept);
  return hipGetLastError();
}

hipError_t launch_slot_finalize(const int32_t* base, int Q, int nb, int T, int E, int k, int C,
                                const int32_t* topk_idx, const int32_t* kept, int32_t* dst_row, int32_t* row_token,
                                int32_t* offsets, int32_t* n_dropped, int rmax, hipStream_t st) {
  const int grid = nb > 0 ? nb : 1;
  slot_finalize_kernel<<<dim3(grid), dim3(64), sizeof(int) * (size_t)(E + 1), st>>>(
      base, Q, nb, T, E, k, C, topk_idx, kept, dst_row, row_token, offsets, n_dropped, rmax);
  return hipGetLastError();
}

}  // namespace moe
