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
// Small T (<= 256): one workgroup does everything in one launch (4 waves and one
// token mask per expert for T <= 64, E <= 256).
// Larger T: five launches - top-k (a group of 16 or 64 lanes per token),
// per-block expert counts, per-expert scan over blocks, ranks -> pair_row,
// and the inversion pair_row -> sorted_pair. The per-block counts live in sorted_pair (used as
// scratch) until the last launch overwrites it with the result, so the call
// needs no workspace: this requires (nblocks + 1) * E <= T * k.
#include "launch.hpp"
#include "mx_codec.hpp"

namespace mxf {

constexpr int kRouteThreads = 256;
constexpr int kSmallT = 256;

__device__ __forceinline__ bool beats(float x, int i, float y, int j) {
  // does candidate (x, i) rank before (y, j)? an empty candidate (i < 0) never does
  return i >= 0 && (j < 0 || x > y || (x == y && i < j));
}

// the (value, index) pair of the lane that DPP control kCtrl selects (all lanes active)
template <int kCtrl, typename F>
__device__ __forceinline__ void take_dpp(float bv, int bi, F&& take) {
  const int ov = __builtin_amdgcn_update_dpp(0, __float_as_int(bv), kCtrl, 0xF, 0xF, false);
  const int oi = __builtin_amdgcn_update_dpp(0, bi, kCtrl, 0xF, 0xF, false);
  take(__int_as_float(ov), oi);
}

// Top-k of one logits row by a group of L lanes (L = 16 or 64; 64 / L tokens per
// wave). Lane j of the group holds logits e = j + L*i, i < 16 (E <= 16 L). Each
// of the k rounds takes the group's best not-yet-taken (logit, index) pair with
// a butterfly over the L lanes (higher logit first, then lower index).
// Results are uniform across the group.
template <int L>
__device__ __forceinline__ void group_topk(const float* __restrict__ row, int E, int topk, bool active,
                                           float (&val)[8], int (&id)[8]) {
  const int j = threadIdx.x & (L - 1);
  float v[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = j + L * i;
    v[i] = (active && e < E) ? row[e] : 0.0f;
    if (!(active && e < E)) taken |= 1u << i;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    val[r] = 0.0f;
    id[r] = -1;
    if (r < topk) {
      float bv = 0.0f;
      int bi = -1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = j + L * i;
        const bool ok = !((taken >> i) & 1u);
        if (ok && beats(v[i], e, bv, bi)) {
          bv = v[i];
          bi = e;
        }
      }
      // the group's best pair: a max over a total order, so any exchange pattern that
      // reaches all L lanes will do - within each 16-lane row by DPP on the VALU
      // (swap neighbours, swap pairs, mirror each 8-lane half, mirror the row), across
      // rows (L = 64) by lane permutes
      auto take = [&](float ov, int oi) {
        if (beats(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      };
      take_dpp<0xB1>(bv, bi, take);   // quad_perm [1, 0, 3, 2]
      take_dpp<0x4E>(bv, bi, take);   // quad_perm [2, 3, 0, 1]
      take_dpp<0x141>(bv, bi, take);  // row_half_mirror
      take_dpp<0x140>(bv, bi, take);  // row_mirror
#pragma unroll
      for (int d = 16; d < L; d <<= 1) take(__shfl_xor(bv, d), __shfl_xor(bi, d));
      if (bi >= 0 && (bi & (L - 1)) == j) taken |= 1u << (bi / L);
      val[r] = bv;
      id[r] = bi;
    }
  }
}

__device__ __forceinline__ void write_route(int64_t t, int topk, const float (&v)[8], const int (&id)[8],
                                            int32_t* __restrict__ topk_ids, float* __restrict__ gates) {
  float z[8];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < topk) {
      z[j] = expf(v[j] - v[0]);
      sum += z[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < topk) {
      topk_ids[t * topk + j] = id[j];
      gates[t * topk + j] = z[j] / sum;
    }
  }
}

// exclusive scan over the NW waves of a block; tmp: NW ints of LDS
template <int NW = 4>
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
  for (int i = 0; i < NW; ++i) {
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

constexpr int kSmallThreads = 1024;

// T <= 256: one workgroup of 16 waves. Phase 1: top-k by lane groups; phase 2:
// thread t < T builds the per-wave expert masks; then counts, scan and ranks.
template <int L>
__global__ void __launch_bounds__(kSmallThreads) route_small_kernel(
    const float* __restrict__ logits, int T, int E, int topk, int32_t* __restrict__ topk_ids,
    float* __restrict__ gates, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row) {
  extern __shared__ unsigned long long bits[];  // [4][E]: tokens 0..255 in 4 mask words
  __shared__ int sids[kSmallT * 8];
  __shared__ int offs[1025];
  __shared__ int tmp[16];
  constexpr int TPW = 64 / L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4 * E; i += kSmallThreads) bits[i] = 0ull;
  const int grp = w * TPW + lane / L;
  for (int t0 = 0; t0 < T; t0 += 16 * TPW) {
    const int t = t0 + grp;
    const bool active = t < T;
    float val[8];
    int id[8];
    group_topk<L>(logits + (int64_t)(active ? t : 0) * E, E, topk, active, val, id);
    if (active && (lane & (L - 1)) == 0) {
      write_route(t, topk, val, id, topk_ids, gates);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < topk) sids[t * topk + j] = id[j];
    }
  }
  __syncthreads();
  if (tid < T) {
    for (int j = 0; j < topk; ++j) atomicOr(&bits[(tid >> 6) * E + sids[tid * topk + j]], 1ull << lane);
  }
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int ww = 0; ww < 4; ++ww) c += __popcll(bits[ww * E + tid]);
  int total;
  const int base = block_exclusive_scan<16>(c, tmp, &total);
  if (tid < E) {
    offs[tid] = base;
    expert_offsets[tid] = base;
  }
  if (tid == 0) {
    offs[E] = total;
    expert_offsets[E] = total;
  }
  __syncthreads();
  if (tid < T) {
    for (int j = 0; j < topk; ++j) {
      const int e = sids[tid * topk + j];
      const int r = offs[e] + wave_rank(bits, E, e);
      const int p = tid * topk + j;
      pair_row[p] = r;
      sorted_pair[r] = p;
    }
  }
}

// T <= 64 and E <= 256 (decode): the same steps with 4 waves and one 64-bit token
// mask per expert
constexpr int kTinyT = 64, kTinyE = 256, kTinyThreads = 256;

// the whole routing of T <= 64 tokens over E <= 256 experts by one workgroup of kTinyThreads
__device__ __forceinline__ void route_tiny_body(const float* __restrict__ logits, int T, int E, int topk,
                                                int32_t* __restrict__ topk_ids, float* __restrict__ gates,
                                                int32_t* __restrict__ expert_offsets,
                                                int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row) {
  constexpr int L = 16, TPW = 64 / L, NW = kTinyThreads / 64;
  __shared__ unsigned long long bits[kTinyE];  // bit t: token t chose expert e
  __shared__ int sids[kTinyT * 8];
  __shared__ int offs[kTinyE + 1];
  __shared__ int tmp[NW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < E) bits[tid] = 0ull;
  const int grp = w * TPW + lane / L;
  for (int t0 = 0; t0 < T; t0 += NW * TPW) {
    const int t = t0 + grp;
    const bool active = t < T;
    float val[8];
    int id[8];
    group_topk<L>(logits + (int64_t)(active ? t : 0) * E, E, topk, active, val, id);
    if (active && (lane & (L - 1)) == 0) {
      write_route(t, topk, val, id, topk_ids, gates);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < topk) sids[t * topk + j] = id[j];
    }
  }
  __syncthreads();
  if (tid < T)
    for (int j = 0; j < topk; ++j) atomicOr(&bits[sids[tid * topk + j]], 1ull << tid);
  __syncthreads();
  const int c = tid < E ? __popcll(bits[tid]) : 0;
  int total;
  const int base = block_exclusive_scan<NW>(c, tmp, &total);
  if (tid < E) {
    offs[tid] = base;
    expert_offsets[tid] = base;
  }
  if (tid == 0) {
    offs[E] = total;
    expert_offsets[E] = total;
  }
  __syncthreads();
  if (tid < T) {
    for (int j = 0; j < topk; ++j) {
      const int e = sids[tid * topk + j];
      const int r = offs[e] + __popcll(bits[e] & ((1ull << tid) - 1ull));
      const int p = tid * topk + j;
      pair_row[p] = r;
      sorted_pair[r] = p;
    }
  }
}

__global__ void __launch_bounds__(kTinyThreads) route_tiny_kernel(
    const float* __restrict__ logits, int T, int E, int topk, int32_t* __restrict__ topk_ids,
    float* __restrict__ gates, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row) {
  route_tiny_body(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row);
}

// Quantisation of the layer input and the routing in one launch (T <= 64, E <= 256):
// workgroup 0 routes, workgroups 1.. quantise 256 blocks of 32 elements each. The two
// steps share no data; one launch instead of two saves a launch's fixed cost, which
// at decode sizes is most of either step's time.
template <bool kF32In, bool kFP4>
__global__ void __launch_bounds__(kTinyThreads) quantize_route_kernel(
    const void* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ q, uint8_t* __restrict__ q_scale,
    const float* __restrict__ logits, int T, int E, int topk, int32_t* __restrict__ topk_ids,
    float* __restrict__ gates, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row) {
  static_assert(kTinyThreads == 256, "one quantisation block per thread, 256 per workgroup");
  if (blockIdx.x == 0) {
    route_tiny_body(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row);
    return;
  }
  const int64_t b = (int64_t)(blockIdx.x - 1) * 256 + threadIdx.x;
  if (b < nblocks) quantize_act_block<kF32In, kFP4>(x, b, q, q_scale);
}

int quantize_route_supported(int64_t T, int E) { return T >= 0 && T <= kTinyT && E >= 1 && E <= kTinyE; }

int launch_quantize_route(const void* x, bool f32_in, int64_t H, bool fp4, uint8_t* q, uint8_t* q_scale,
                          const float* logits, int64_t T, int E, int topk, int32_t* topk_ids, float* gates,
                          int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row, hipStream_t stream) {
  if (!quantize_route_supported(T, E)) return -1;
  const int64_t nblocks = T * (H / 32);
  const dim3 grid((unsigned)(1 + cdiv(nblocks, 256))), block(kTinyThreads);
  const int t = (int)T;
  if (f32_in) {
    if (fp4)
      quantize_route_kernel<true, true><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale, logits, t, E, topk,
                                                                    topk_ids, gates, expert_offsets, sorted_pair,
                                                                    pair_row);
    else
      quantize_route_kernel<true, false><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale, logits, t, E, topk,
                                                                     topk_ids, gates, expert_offsets, sorted_pair,
                                                                     pair_row);
  } else {
    if (fp4)
      quantize_route_kernel<false, true><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale, logits, t, E, topk,
                                                                     topk_ids, gates, expert_offsets, sorted_pair,
                                                                     pair_row);
    else
      quantize_route_kernel<false, false><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale, logits, t, E, topk,
                                                                      topk_ids, gates, expert_offsets, sorted_pair,
                                                                      pair_row);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// large T, launch 1: top-k, one token per group of L lanes (64 / L tokens per wave)
template <int L>
__global__ void __launch_bounds__(kRouteThreads) route_topk_kernel(const float* __restrict__ logits, int64_t T,
                                                                   int E, int topk, int32_t* __restrict__ topk_ids,
                                                                   float* __restrict__ gates) {
  constexpr int TPB = kRouteThreads / L;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / L;
  const bool active = t < T;
  float val[8];
  int id[8];
  group_topk<L>(logits + (active ? t : 0) * E, E, topk, active, val, id);
  if (active && (lane & (L - 1)) == 0) write_route(t, topk, val, id, topk_ids, gates);
}

// large T, launch 2: the expert counts of each block of 256 tokens
__global__ void __launch_bounds__(kRouteThreads) route_count_kernel(const int32_t* __restrict__ topk_ids,
                                                                    int64_t T, int E, int topk,
                                                                    int32_t* __restrict__ scratch) {
  extern __shared__ int cnt[];  // [E]
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kRouteThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kRouteThreads + tid;
  if (t < T) {
    for (int j = 0; j < topk; ++j) atomicAdd(&cnt[topk_ids[t * topk + j]], 1);
  }
  __syncthreads();
  for (int i = tid; i < E; i += kRouteThreads) scratch[(int64_t)blockIdx.x * E + i] = cnt[i];
}

// large T, launch 3: block e turns column e of the counts into exclusive prefixes
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

// large T, launch 4: expert offsets (every block rescans the E totals) and ranks
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

// large T, launch 5: sorted_pair = inverse of pair_row (overwrites the scratch)
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

template <int L>
static void launch_route_l(const float* logits, int64_t T, int E, int topk, int32_t* topk_ids, float* gates,
                           int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row, hipStream_t stream) {
  const size_t bits_bytes = sizeof(unsigned long long) * 4 * E;
  if (L == 16 && T <= kTinyT && E <= kTinyE) {
    route_tiny_kernel<<<1, kTinyThreads, 0, stream>>>(logits, (int)T, E, topk, topk_ids, gates, expert_offsets,
                                                      sorted_pair, pair_row);
    return;
  }
  if (T <= kSmallT) {
    route_small_kernel<L><<<1, kSmallThreads, bits_bytes, stream>>>(logits, (int)T, E, topk, topk_ids, gates,
                                                                     expert_offsets, sorted_pair, pair_row);
    return;
  }
  const int nblk = (int)cdiv(T, kRouteThreads);
  int32_t* scratch = sorted_pair;
  constexpr int TPB = kRouteThreads / L;
  route_topk_kernel<L><<<(unsigned)cdiv(T, TPB), kRouteThreads, 0, stream>>>(logits, T, E, topk, topk_ids, gates);
  route_count_kernel<<<nblk, kRouteThreads, sizeof(int) * E, stream>>>(topk_ids, T, E, topk, scratch);
  route_scan_kernel<<<E, kRouteThreads, 0, stream>>>(scratch, nblk, E);
  route_rank_kernel<<<nblk, kRouteThreads, bits_bytes, stream>>>(topk_ids, T, E, topk, nblk, scratch,
                                                                 expert_offsets, pair_row);
  const int64_t n = T * topk;
  invert_kernel<<<(unsigned)cdiv(n, kRouteThreads), kRouteThreads, 0, stream>>>(pair_row, n, sorted_pair);
}

int launch_route_permute(const float* logits, int64_t T, int E, int topk, int32_t* topk_ids, float* gates,
                         int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row,
                         hipStream_t stream) {
  if (E <= 256)
    launch_route_l<16>(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row, stream);
  else
    launch_route_l<64>(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf
