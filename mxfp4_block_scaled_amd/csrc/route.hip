// Top-k routing and the expert-grouped (stable) permutation.
//
// Each token picks the top-k of E experts [page "【DeepSeek V4】Triton FP4 优化实战",
// "FP4 MoE GEMM 是什么？": 6 of 256], ordered by (logit descending, index
// ascending); the gates are the softmax over the selected logits. The pairs
// p = t*k + j are then grouped by expert, ascending p inside an expert (the
// on-GPU half of MoE dispatch, page "Domestic GPUs are awesome! Moore thread
// full-link adaptation DeepSeek-V4").
//
// The stable rank of pair (t, j) inside expert e is the number of tokens
// t' < t that chose e (a token never picks an expert twice). Inside a wave it
// is a popcount over a 64-bit ballot-style mask of the tokens that chose e
// (built with LDS atomic ORs); across waves and blocks it is a prefix count.
//
// Small T (<= 256): one workgroup does everything in one launch.
// Larger T: four launches - per-block top-k + per-block expert counts,
// per-expert scan over blocks, ranks -> pair_row, and the inversion
// pair_row -> sorted_pair. The per-block counts live in sorted_pair (used as
// scratch) until the last launch overwrites it with the result, so the call
// needs no workspace: this requires (nblocks + 1) * E <= T * k.
#include "launch.hpp"

namespace mxf {

constexpr int kRouteThreads = 256;
constexpr int kSmallT = 256;

__device__ __forceinline__ bool beats(float x, int i, float y, int j) {
  // does candidate (x, i) rank before (y, j)? an empty candidate (i < 0) never does
  return i >= 0 && (j < 0 || x > y || (x == y && i < j));
}

// top-S of one logits row, sorted; slots past the real ones keep id -1
template <int S, bool kVec>
__device__ __forceinline__ void topk_scan(const float* __restrict__ row, int E, float (&v)[S], int (&id)[S]) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    v[s] = 0.0f;
    id[s] = -1;
  }
  auto insert = [&](float x, int i) {
    float c = x;
    int ci = i;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bool b = beats(c, ci, v[s], id[s]);
      const float tv = v[s];
      const int ti = id[s];
      v[s] = b ? c : tv;
      id[s] = b ? ci : ti;
      c = b ? tv : c;
      ci = b ? ti : ci;
    }
  };
  if (kVec) {
    for (int e = 0; e < E; e += 4) {
      const float4 f = *reinterpret_cast<const float4*>(row + e);
      insert(f.x, e);
      insert(f.y, e + 1);
      insert(f.z, e + 2);
      insert(f.w, e + 3);
    }
  } else {
    for (int e = 0; e < E; ++e) insert(row[e], e);
  }
}

template <int S>
__device__ __forceinline__ void write_route(int64_t t, int topk, const float (&v)[S], const int (&id)[S],
                                            int32_t* __restrict__ topk_ids, float* __restrict__ gates) {
  float z[S];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    if (j < topk) {
      z[j] = expf(v[j] - v[0]);
      sum += z[j];
    }
  }
#pragma unroll
  for (int j = 0; j < S; ++j) {
    if (j < topk) {
      topk_ids[t * topk + j] = id[j];
      gates[t * topk + j] = z[j] / sum;
    }
  }
}

// exclusive scan over the 256 threads of a block; tmp: 4 ints of LDS
__device__ __forceinline__ int block_exclusive_scan(int x, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    base += (i < w) ? tmp[i] : 0;
    tot += tmp[i];
  }
  *total = tot;
  return base + incl - x;
}

__device__ __forceinline__ int wave_rank(const unsigned long long* bits, int E, int e) {
  // tokens of earlier waves in the block, plus lower lanes of this wave, that chose e
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int r = 0;
  for (int i = 0; i < w; ++i) r += __popcll(bits[i * E + e]);
  return r + __popcll(bits[w * E + e] & ((1ull << lane) - 1ull));
}

template <int S, bool kVec>
__global__ void __launch_bounds__(kRouteThreads) route_small_kernel(
    const float* __restrict__ logits, int T, int E, int topk, int32_t* __restrict__ topk_ids,
    float* __restrict__ gates, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row) {
  extern __shared__ unsigned long long bits[];  // [4][E]
  __shared__ int offs[1025];
  __shared__ int tmp[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * E; i += kRouteThreads) bits[i] = 0ull;
  __syncthreads();
  float v[S];
  int id[S];
  const bool valid = tid < T;
  if (valid) {
    topk_scan<S, kVec>(logits + (int64_t)tid * E, E, v, id);
    write_route<S>(tid, topk, v, id, topk_ids, gates);
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < topk) atomicOr(&bits[w * E + id[j]], 1ull << lane);
  }
  __syncthreads();
  // per-expert totals and their exclusive scan (thread owns experts [tid*C, tid*C+C))
  const int C = (E + kRouteThreads - 1) / kRouteThreads;
  int local = 0;
  for (int i = 0; i < C; ++i) {
    const int e = tid * C + i;
    if (e < E) {
      int c = 0;
      for (int ww = 0; ww < 4; ++ww) c += __popcll(bits[ww * E + e]);
      local += c;
    }
  }
  int total;
  int base = block_exclusive_scan(local, tmp, &total);
  for (int i = 0; i < C; ++i) {
    const int e = tid * C + i;
    if (e < E) {
      int c = 0;
      for (int ww = 0; ww < 4; ++ww) c += __popcll(bits[ww * E + e]);
      offs[e] = base;
      expert_offsets[e] = base;
      base += c;
    }
  }
  if (tid == 0) {
    offs[E] = total;
    expert_offsets[E] = total;
  }
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      if (j < topk) {
        const int e = id[j];
        const int r = offs[e] + wave_rank(bits, E, e);
        const int p = tid * topk + j;
        pair_row[p] = r;
        sorted_pair[r] = p;
      }
    }
  }
}

// large T, launch 1: top-k of 256 tokens per block + the block's expert counts
template <int S, bool kVec>
__global__ void __launch_bounds__(kRouteThreads) route_count_kernel(
    const float* __restrict__ logits, int64_t T, int E, int topk, int32_t* __restrict__ topk_ids,
    float* __restrict__ gates, int32_t* __restrict__ scratch) {
  extern __shared__ int cnt[];  // [E]
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kRouteThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kRouteThreads + tid;
  if (t < T) {
    float v[S];
    int id[S];
    topk_scan<S, kVec>(logits + t * E, E, v, id);
    write_route<S>(t, topk, v, id, topk_ids, gates);
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < topk) atomicAdd(&cnt[id[j]], 1);
  }
  __syncthreads();
  for (int i = tid; i < E; i += kRouteThreads) scratch[(int64_t)blockIdx.x * E + i] = cnt[i];
}

// large T, launch 2: block e turns column e of the counts into exclusive prefixes
// over blocks and stores the expert total in row nblk
__global__ void __launch_bounds__(kRouteThreads) route_scan_kernel(int32_t* __restrict__ scratch, int nblk, int E) {
  __shared__ int tmp[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int J = (nblk + kRouteThreads - 1) / kRouteThreads;
  int local = 0;
  for (int i = 0; i < J; ++i) {
    const int b = tid * J + i;
    if (b < nblk) local += scratch[(int64_t)b * E + e];
  }
  int total;
  int base = block_exclusive_scan(local, tmp, &total);
  for (int i = 0; i < J; ++i) {
    const int b = tid * J + i;
    if (b < nblk) {
      const int c = scratch[(int64_t)b * E + e];
      scratch[(int64_t)b * E + e] = base;
      base += c;
    }
  }
  if (tid == 0) scratch[(int64_t)nblk * E + e] = total;
}

// large T, launch 3: expert offsets (every block rescans the E totals) and ranks
__global__ void __launch_bounds__(kRouteThreads) route_rank_kernel(
    const int32_t* __restrict__ topk_ids, int64_t T, int E, int topk, int nblk,
    const int32_t* __restrict__ scratch, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ pair_row) {
  extern __shared__ unsigned long long bits[];  // [4][E]
  __shared__ int offs[1025];
  __shared__ int tmp[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * E; i += kRouteThreads) bits[i] = 0ull;
  const int C = (E + kRouteThreads - 1) / kRouteThreads;
  const int32_t* totals = scratch + (int64_t)nblk * E;
  int local = 0;
  for (int i = 0; i < C; ++i) {
    const int e = tid * C + i;
    if (e < E) local += totals[e];
  }
  int total;
  int base = block_exclusive_scan(local, tmp, &total);  // contains a barrier
  for (int i = 0; i < C; ++i) {
    const int e = tid * C + i;
    if (e < E) {
      offs[e] = base;
      if (blockIdx.x == 0) expert_offsets[e] = base;
      base += totals[e];
    }
  }
  if (tid == 0 && blockIdx.x == 0) expert_offsets[E] = total;
  const int64_t t = (int64_t)blockIdx.x * kRouteThreads + tid;
  int ids[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ids[j] = 0;
  if (t < T) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < topk) ids[j] = topk_ids[t * topk + j];
  }
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < topk) atomicOr(&bits[w * E + ids[j]], 1ull << lane);
  }
  __syncthreads();
  if (t < T) {
    const int32_t* blk = scratch + (int64_t)blockIdx.x * E;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < topk) {
        const int e = ids[j];
        pair_row[t * topk + j] = offs[e] + blk[e] + wave_rank(bits, E, e);
      }
    }
  }
}

// large T, launch 4: sorted_pair = inverse of pair_row (overwrites the scratch)
__global__ void __launch_bounds__(kRouteThreads) invert_kernel(const int32_t* __restrict__ pair_row, int64_t n,
                                                               int32_t* __restrict__ sorted_pair) {
  const int64_t p = (int64_t)blockIdx.x * kRouteThreads + threadIdx.x;
  if (p < n) sorted_pair[pair_row[p]] = (int32_t)p;
}

int route_permute_supported(int64_t T, int E, int topk) {
  if (T <= kSmallT) return 1;
  const int64_t nblk = cdiv(T, kRouteThreads);
  return (nblk + 1) * (int64_t)E <= T * topk ? 1 : 0;
}

template <int S>
static void launch_route_s(const float* logits, int64_t T, int E, int topk, int32_t* topk_ids, float* gates,
                           int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row, bool vec,
                           hipStream_t stream) {
  const size_t bits_bytes = sizeof(unsigned long long) * 4 * E;
  if (T <= kSmallT) {
    if (vec)
      route_small_kernel<S, true><<<1, kRouteThreads, bits_bytes, stream>>>(
          logits, (int)T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row);
    else
      route_small_kernel<S, false><<<1, kRouteThreads, bits_bytes, stream>>>(
          logits, (int)T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row);
    return;
  }
  const int nblk = (int)cdiv(T, kRouteThreads);
  int32_t* scratch = sorted_pair;
  if (vec)
    route_count_kernel<S, true><<<nblk, kRouteThreads, sizeof(int) * E, stream>>>(logits, T, E, topk, topk_ids,
                                                                                   gates, scratch);
  else
    route_count_kernel<S, false><<<nblk, kRouteThreads, sizeof(int) * E, stream>>>(logits, T, E, topk, topk_ids,
                                                                                    gates, scratch);
  route_scan_kernel<<<E, kRouteThreads, 0, stream>>>(scratch, nblk, E);
  route_rank_kernel<<<nblk, kRouteThreads, bits_bytes, stream>>>(topk_ids, T, E, topk, nblk, scratch,
                                                                 expert_offsets, pair_row);
  const int64_t n = T * topk;
  invert_kernel<<<(unsigned)cdiv(n, kRouteThreads), kRouteThreads, 0, stream>>>(pair_row, n, sorted_pair);
}

int launch_route_permute(const float* logits, int64_t T, int E, int topk, int32_t* topk_ids, float* gates,
                         int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row,
                         hipStream_t stream) {
  const bool vec = (E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  if (topk <= 6)
    launch_route_s<6>(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row, vec, stream);
  else
    launch_route_s<8>(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row, vec, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf
