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

// K2b: one wave per (block of 64 tokens, choice r): the assignments are
// resolved independently.  Every workgroup derives offsets (the exclusive
// prefix sum of kept) in LDS; workgroup (0, 0) also publishes offsets[0..E] and
// n_dropped.  Then each lane resolves its token's choice r.
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
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int e = lane; e <= E; e += 64) offsets[e] = s_off[e];
    if (lane == 0) *n_dropped = T * k - R;
  }
  const int blk = blockIdx.x, r = blockIdx.y;
  const int t = blk * 64 + lane;
  if (t >= T) return;
  const size_t i = (size_t)t * k + r;
  if (dst_row[i] == kAbsentChoice) {
    dst_row[i] = -1;
    return;
  }
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

hipError_t launch_slot_scan(int32_t* hist, int Q, int E, int C, int32_t* demand, int32_t* kept, hipStream_t st) {
  slot_scan_kernel<<<dim3(E), dim3(256), 0, st>>>(hist, Q, C, demand, kept);
  return hipGetLastError();
}

hipError_t launch_slot_finalize(const int32_t* base, int Q, int nb, int T, int E, int k, int C,
                                const int32_t* topk_idx, const int32_t* kept, int32_t* dst_row, int32_t* row_token,
                                int32_t* offsets, int32_t* n_dropped, int rmax, hipStream_t st) {
  const dim3 grid(nb > 0 ? nb : 1, k);
  slot_finalize_kernel<<<grid, dim3(64), sizeof(int) * (size_t)(E + 1), st>>>(
      base, Q, nb, T, E, k, C, topk_idx, kept, dst_row, row_token, offsets, n_dropped, rmax);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// "probs" drop policy ("Expert-parallel MoE training" explainer, capacity / drop
// section: drop the lowest-probability assignments instead of the last ones).
// Per expert, the C assignments with the largest gate are kept (equal gates:
// the earlier choice-major position q = r*T + t first) and packed in position
// order.  As 64-bit keys (gate bits << 32) | ~q, all distinct and ordered like
// (gate desc, q asc), the kept set is {key >= the C-th largest key}.
//
// P1 (one wave per 64-token block): each assignment's position among its
//    expert's assignments -> list index off_all[e] + pos (off_all = exclusive
//    prefix sum of demand); key and q stored there; dst_row holds the index.
// P2 (one workgroup per expert): radix select of the C-th largest key (8 passes
//    of 8 bits, most significant first), then the kept flags' exclusive prefix
//    sum in list (= position) order gives each kept assignment its slot.
// P3 (one wave per 64-token block): dst_row = offsets[e] + slot, row_token.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void offsets_in_lds(const int32_t* __restrict__ cnt, int E, int* s_off) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int e_begin = lane * per;
  int s = 0;
  for (int j = 0; j < per; ++j) {
    const int e = e_begin + j;
    if (e < E) s += cnt[e];
  }
  const int inc = wave_inclusive_scan(s);
  int run = inc - s;
  for (int j = 0; j < per; ++j) {
    const int e = e_begin + j;
    if (e < E) {
      s_off[e] = run;
      run += cnt[e];
    }
  }
  if (lane == 63) s_off[E] = inc;
}

__global__ void __launch_bounds__(64) slot_list_kernel(const int32_t* __restrict__ base, int Q, int nb, int T, int E,
                                                       int k, const int32_t* __restrict__ topk_idx,
                                                       const float* __restrict__ topk_gate,
                                                       const int32_t* __restrict__ demand,
                                                       int32_t* __restrict__ dst_row, uint32_t* __restrict__ lkey,
                                                       uint32_t* __restrict__ lq) {
  extern __shared__ int s_off[];  // [E+1]
  offsets_in_lds(demand, E, s_off);
  __syncthreads();
  const int blk = blockIdx.x;
  const int t = blk * 64 + threadIdx.x;
  if (t >= T) return;
  for (int r = 0; r < k; ++r) {
    const size_t i = (size_t)t * k + r;
    if (dst_row[i] == kAbsentChoice) continue;
    const int e = topk_idx[i];
    const int L = s_off[e] + base[(size_t)e * Q + r * nb + blk] + dst_row[i];
    dst_row[i] = L;
    lkey[L] = __float_as_uint(topk_gate[i]);
    lq[L] = (uint32_t)r * (uint32_t)T + (uint32_t)t;
  }
}

__global__ void __launch_bounds__(256) slot_probs_kernel(const int32_t* __restrict__ demand, int E, int C,
                                                         const uint32_t* __restrict__ lkey,
                                                         const uint32_t* __restrict__ lq,
                                                         int32_t* __restrict__ newslot) {
  __shared__ int s_hist[256];
  __shared__ int s_tmp[256 / 64 + 1];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  const int e = blockIdx.x, tid = threadIdx.x;
  // off_all[e] = sum of demand over the experts before e (fixed-shape block sum)
  int part = 0;
  for (int j = tid; j < e; j += 256) part += demand[j];
  int total;
  (void)block_exclusive_scan(part, s_tmp, &total);
  const int off = total;
  const int n = demand[e];
  if (n <= C) {
    for (int j = tid; j < n; j += 256) newslot[off + j] = j;
    return;
  }
  auto key = [&](int j) -> uint64_t {
    return ((uint64_t)lkey[off + j] << 32) | (uint64_t)(0xFFFFFFFFu - lq[off + j]);
  };
  if (tid == 0) {
    s_prefix = 0;
    s_need = C;
  }
  uint64_t mask = 0;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    s_hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    for (int j = tid; j < n; j += 256) {
      const uint64_t kj = key(j);
      if ((kj & mask) == prefix) atomicAdd(&s_hist[(kj >> shift) & 0xFF], 1);
    }
    __syncthreads();
    {  // bucket holding the need-th largest among the candidates: counts from the
       // top (thread i holds bucket 255 - i); exactly one bucket brackets need
      const int b = 255 - tid;
      const int h = s_hist[b];
      int above_total;
      const int above = block_exclusive_scan(h, s_tmp, &above_total);  // candidates in buckets > b
      const int need = s_need;
      __syncthreads();
      if (above < need && above + h >= need) {
        s_need = need - above;
        s_prefix = prefix | ((uint64_t)b << shift);
      }
    }
    mask |= (uint64_t)0xFF << shift;
    __syncthreads();
  }
  const uint64_t thr = s_prefix;  // the C-th largest key
  int run = 0;
  for (int j0 = 0; j0 < n; j0 += 256) {
    const int j = j0 + tid;
    const int f = (j < n && key(j) >= thr) ? 1 : 0;
    int chunk;
    const int ex = block_exclusive_scan(f, s_tmp, &chunk);
    if (j < n) newslot[off + j] = f ? run + ex : -1;
    run += chunk;
  }
}

__global__ void __launch_bounds__(64) slot_finalize_probs_kernel(int T, int E, int k,
                                                                 const int32_t* __restrict__ topk_idx,
                                                                 const int32_t* __restrict__ kept,
                                                                 const int32_t* __restrict__ newslot,
                                                                 int32_t* __restrict__ dst_row,
                                                                 int32_t* __restrict__ row_token,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ n_dropped, int rmax) {
  extern __shared__ int s_off[];  // [E+1]
  offsets_in_lds(kept, E, s_off);
  __syncthreads();
  const int lane = threadIdx.x;
  if (blockIdx.x == 0) {
    for (int e = lane; e <= E; e += 64) offsets[e] = s_off[e];
    if (lane == 0) *n_dropped = T * k - s_off[E];
  }
  const int t = blockIdx.x * 64 + lane;
  if (t >= T) return;
  for (int r = 0; r < k; ++r) {
    const size_t i = (size_t)t * k + r;
    if (dst_row[i] == kAbsentChoice) {
      dst_row[i] = -1;
      continue;
    }
    const int e = topk_idx[i];
    const int slot = newslot[dst_row[i]];
    const int d = s_off[e] + slot;
    if (slot >= 0 && d < rmax) {  // d < R <= rmax for any plan this path derives
      dst_row[i] = d;
      row_token[d] = t;
    } else {
      dst_row[i] = -1;
    }
  }
}

hipError_t launch_slot_probs(const int32_t* base, int Q, int nb, int T, int E, int k, int C, const int32_t* topk_idx,
                             const float* topk_gate, const int32_t* demand, const int32_t* kept, int32_t* dst_row,
                             int32_t* row_token, int32_t* offsets, int32_t* n_dropped, int rmax, uint32_t* lkey,
                             uint32_t* lq, int32_t* newslot, hipStream_t st) {
  const int grid = nb > 0 ? nb : 1;
  const size_t shm = sizeof(int) * (size_t)(E + 1);
  if (T > 0) {
    slot_list_kernel<<<dim3(grid), dim3(64), shm, st>>>(base, Q, nb, T, E, k, topk_idx, topk_gate, demand, dst_row,
                                                         lkey, lq);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    slot_probs_kernel<<<dim3(E), dim3(256), 0, st>>>(demand, E, C, lkey, lq, newslot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  slot_finalize_probs_kernel<<<dim3(grid), dim3(64), shm, st>>>(T, E, k, topk_idx, kept, newslot, dst_row,
                                                                 row_token, offsets, n_dropped, rmax);
  return hipGetLastError();
}

}  // namespace moe
