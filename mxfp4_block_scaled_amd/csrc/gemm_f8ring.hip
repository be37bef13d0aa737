// LDS-ring MXFP4 GEMM for E4M3 activations: 256 activation rows x 256 weight rows
// per workgroup, 8 waves of 64 x 128 on the 32x32x64 scaled MFMA (FP8 x FP4).
//
// The FP8 x FP4 instruction runs at half the FP4 x FP4 rate, so a 128-k stage of
// this kernel holds as many matrix-core cycles as a 256-k stage of the FP4 kernel
// (gemm_wide.hip) while moving 50 KB instead of 68 KB: 32 KB of activation codes,
// 16 KB of weight codes and 2 KB of scales, every operand by LDS-DMA in whole
// 128-byte lines (weight tiles are shared by the waves through LDS, so each line is
// fetched once per workgroup). Three 50 KB slots fit the 160 KB of LDS: the copies
// of stage st + 2 are issued at the top of stage st, two stages ahead.
//
// K order: MFMA step s (64 k) of a stage takes hardware block hb from memory block
// 2 s + hb, i.e. the stage's k in memory order. So
//   * a weight lane (row l % 32, block hb = l / 32) reads 16-byte chunk 2 s + hb of its
//     64-byte stage row;
//   * an activation lane (FP8: bytes 0..15 are k [16 g, 16 g + 16) of hardware block 0,
//     bytes 16..31 the same of hardware block 1) reads 16-byte chunks 4 s + g and
//     4 s + 2 + g of its 128-byte stage row;
//   * the scale byte of (row, hardware block hb) is byte 2 s + hb of the row's 4 stage
//     scale bytes: a lane loads that dword, shifts it right by 8 hb and takes byte 2 s
//     (op_sel = 2 s).
// Row groups of 64 that lie wholly past an expert's last row skip their MFMAs and
// LDS reads (the wave still issues its copies and meets every barrier).
#include "tile256.hpp"

namespace mxf {

namespace f8r {
constexpr int BM = 256, BN = 256;
constexpr int KS = 128;                // k per stage
constexpr int S = KS / 64;             // MFMA steps per stage
constexpr int RA = KS;                 // E4M3 activation bytes per row per stage
constexpr int RB = KS / 2;             // E2M1 weight bytes per row per stage
constexpr int CA = RA / 16;            // 16-byte chunks per activation row per stage
constexpr int CB = RB / 16;            // 16-byte chunks per weight row per stage
constexpr int IA = BM * CA / 64 / 8;   // activation copies (16 B per lane) per wave per stage
constexpr int IB = BN * CB / 64 / 8;   // weight copies per wave per stage
constexpr int D = IA + IB + 1;         // + one 4-byte scale copy: vector-memory ops per wave per stage
constexpr int NSLOT = 3;
}  // namespace f8r

struct alignas(16) F8Slot {
  uint8_t A[f8r::BM * f8r::RA];  // activation codes, [row][128], 16-byte chunks XOR-swizzled per row
  uint8_t B[f8r::BN * f8r::RB];  // weight codes, [row][64], swizzled likewise
  uint8_t As[f8r::BM * 4];       // the stage's 4 scale bytes per activation row
  uint8_t Bs[f8r::BN * 4];       // and per weight row
};
static_assert(f8r::NSLOT * sizeof(F8Slot) <= 160 * 1024, "the ring must fit in LDS");
static_assert(kTile256Staging <= (int)(f8r::NSLOT * sizeof(F8Slot)), "the epilogue stages through the ring");

// swizzles of the 16-byte chunk index: with them the 16 lanes that one LDS cycle
// serves (16 consecutive rows, one chunk each) hit 16 different 16-byte bank groups
__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }  // 128-byte rows
__device__ __forceinline__ int swz_b(int r) { return (r >> 2) & 3; }              // 64-byte rows

// NST > 0: K / 128 is a compile-time constant and the ring is fully unrolled;
// NST == 0: any K (multiple of 128) with a runtime loop.
template <int kMode, bool kYBF16, int NST>
__global__ void __launch_bounds__(512) gemm_f8ring_kernel(GemmArgs a) {
  using namespace f8r;
  __shared__ F8Slot ring[NSLOT];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5,
            r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;  // rows [64 wm, 64 wm + 64), column half wn

  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  int e = 0, n_tile;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    // XCD x owns n-tiles [x*nt/8, (x+1)*nt/8) and walks the row units
    const int n_lo = x * ntiles / 8, n_hi = (x + 1) * ntiles / 8, nn = n_hi - n_lo;
    if (nn == 0) return;
    const int m_unit = jb / nn;
    n_tile = n_lo + jb % nn;
    row0 = (int64_t)m_unit * BM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < BM ? a.M - row0 : BM);
  } else {
    int loc;
    grouped_work_item<BM>(a.offsets, a.E, a.split, ntiles, x, jb, e, n_tile, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t arow = K, wrow = K / 2, srow = K / 32;
  const int nst = NST > 0 ? NST : (int)(K / KS);

  auto a_src_row = [&](int r) -> int64_t {  // rows past m read the unit's first row (never stored)
    if (r >= m) r = 0;
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };
  // FC1: weight rows [0, 128) of the tile are gate rows, [128, 256) the matching up rows
  auto b_row = [&](int r) -> int64_t {
    if (kMode == kModeFC1) return (r < BN / 2 ? 0 : a.I - BN / 2) + (int64_t)n_tile * (BN / 2) + r;
    return (int64_t)n_tile * BN + r;
  };

  // range-checked buffer resources (32-bit byte offsets; the host checks the extents)
  const int eu = __builtin_amdgcn_readfirstlane(e);
  const buf_rsrc ra = make_rsrc(a.act, (uint32_t)(a.act_rows * arow));
  const buf_rsrc ras = make_rsrc(a.act_scale, (uint32_t)(a.act_rows * srow));
  const buf_rsrc rb = make_rsrc(a.w + (int64_t)eu * a.N * wrow, (uint32_t)(a.N * wrow));
  const buf_rsrc rbs = make_rsrc(a.w_scale + (int64_t)eu * a.N * srow, (uint32_t)(a.N * srow));

  // per-lane copy sources at stage 0 (the stage adds a scalar offset): LDS chunk c
  // of an operand holds row c / (chunks per row), global chunk (c % cpr) ^ swizzle(row)
  uint32_t va[IA], vb[IB];
#pragma unroll
  for (int q = 0; q < IA; ++q) {
    const int chunk = (wave * IA + q) * 64 + lane;
    const int r = chunk / CA, pc = chunk % CA;
    va[q] = (uint32_t)(a_src_row(r) * arow + 16 * (pc ^ swz_a(r)));
  }
#pragma unroll
  for (int q = 0; q < IB; ++q) {
    const int chunk = (wave * IB + q) * 64 + lane;
    const int r = chunk / CB, pc = chunk % CB;
    vb[q] = (uint32_t)(b_row(r) * wrow + 16 * (pc ^ swz_b(r)));
  }
  // scales: waves 0-3 copy the 4 stage bytes of activation rows [64 w, 64 w + 64),
  // waves 4-7 those of weight rows [64 (w - 4), ...): one 4-byte copy per lane
  const bool sc_a = wave < 4;
  const int sc_row = 64 * (wave & 3) + lane;
  const uint32_t vsc = (uint32_t)((sc_a ? a_src_row(sc_row) : b_row(sc_row)) * srow);

  // copies of stage st into ring slot sl: weight rows first (mostly HBM), then
  // activation rows (mostly L2), then the scales
  auto issue = [&](F8Slot& sl, int st) {
#pragma unroll
    for (int q = 0; q < IB; ++q) buf_dma16(rb, &sl.B[(wave * IB + q) * 1024], vb[q], (uint32_t)st * RB);
#pragma unroll
    for (int q = 0; q < IA; ++q) buf_dma16(ra, &sl.A[(wave * IA + q) * 1024], va[q], (uint32_t)st * RA);
    if (sc_a) buf_dma4(ras, &sl.As[(wave & 3) * 256], vsc, (uint32_t)st * 4);
    else buf_dma4(rbs, &sl.Bs[(wave & 3) * 256], vsc, (uint32_t)st * 4);
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  int arow_l[2], brow_l[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) arow_l[f] = 64 * wm + 32 * f + r32;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    // FC1: fragments 0, 1 are gate columns [64 wn, 64 wn + 64), 2, 3 the matching up columns
    if (kMode == kModeFC1) brow_l[f] = (f < 2 ? 0 : BN / 2) + 64 * wn + 32 * (f & 1) + r32;
    else brow_l[f] = 128 * wn + 32 * f + r32;
  }
  // Byte offsets of this lane's fragment rows in a slot with chunk g applied; step s
  // and the lo/hi half only XOR further chunk bits in (4 s and 2 for A, 2 s for B).
  // They pass through an empty asm at each use, so the compiler recomputes the XOR
  // per read instead of holding an address register per (slot, step, fragment).
  int aoff[2], boff[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) aoff[f] = arow_l[f] * RA + 16 * (g ^ swz_a(arow_l[f]));
#pragma unroll
  for (int f = 0; f < 4; ++f) boff[f] = brow_l[f] * RB + 16 * (g ^ swz_b(brow_l[f]));

  struct Frags {
    v4i lo[2], hi[2], b[4];
  };
  auto load_frags = [&](const F8Slot& sl, auto S_, Frags& F) {
    constexpr int s = decltype(S_)::value;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      int o = aoff[f];
      asm volatile("" : "+v"(o));
      F.lo[f] = *reinterpret_cast<const v4i*>(&sl.A[o ^ (64 * s)]);
      F.hi[f] = *reinterpret_cast<const v4i*>(&sl.A[o ^ (64 * s + 32)]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      int o = boff[f];
      asm volatile("" : "+v"(o));
      F.b[f] = *reinterpret_cast<const v4i*>(&sl.B[o ^ (32 * s)]);
    }
  };
  auto mfma_step = [&](auto S_, const Frags& F, const int* sa, const int* sb) {
    constexpr int s = decltype(S_)::value;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
      const v8i af = v8i{F.lo[fm][0], F.lo[fm][1], F.lo[fm][2], F.lo[fm][3],
                         F.hi[fm][0], F.hi[fm][1], F.hi[fm][2], F.hi[fm][3]};
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        const v8i bf = v8i{F.b[fn][0], F.b[fn][1], F.b[fn][2], F.b[fn][3], 0, 0, 0, 0};
        acc[fm][fn] = mfma32x32x64<kFmtFP4, kFmtFP8, 2 * s>(bf, af, acc[fm][fn], sb[fn], sa[fm]);
      }
    }
  };
  // one stage on slot sl: this lane's scale dwords (shifted so that byte 2 s is the
  // one of its hardware block at step s), the fragments of steps 0 and 1 (the reads
  // of step 1 land under the MFMAs of step 0), then the MFMAs of both steps
  auto compute = [&](auto kActive, const F8Slot& sl) {
    constexpr bool act = decltype(kActive)::value;
    if constexpr (act) {
      int sa[2], sb[4];
#pragma unroll
      for (int f = 0; f < 2; ++f) sa[f] = (int)(*reinterpret_cast<const uint32_t*>(&sl.As[4 * arow_l[f]]) >> (8 * g));
#pragma unroll
      for (int f = 0; f < 4; ++f) sb[f] = (int)(*reinterpret_cast<const uint32_t*>(&sl.Bs[4 * brow_l[f]]) >> (8 * g));
      Frags F0, F1;
      load_frags(sl, std::integral_constant<int, 0>{}, F0);
      __builtin_amdgcn_sched_barrier(0);
      load_frags(sl, std::integral_constant<int, 1>{}, F1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(std::integral_constant<int, 0>{}, F0, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(std::integral_constant<int, 1>{}, F1, sa, sb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ring of three slots: at stage st wait for this wave's copies of st (those of
  // st + 1 may stay in flight), barrier (every wave's part has landed and every wave
  // is done with st - 1, whose slot the copies of st + 2 then overwrite), issue
  // st + 2, compute st
  auto step = [&](auto kActive, auto I, int st) {
    constexpr int i = decltype(I)::value;
    if (st + 1 < nst) wait_vmcnt<D>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (st + 2 < nst) issue(ring[(i + 2) % NSLOT], st + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(kActive, ring[i]);
  };
  auto run = [&](auto kActive) {
    if constexpr (NST > 0) {
      static_for<0, NST>([&](auto X_) {
        constexpr int X = decltype(X_)::value;
        step(kActive, std::integral_constant<int, X % NSLOT>{}, X);
      });
    } else {
      for (int st0 = 0; st0 < nst; st0 += NSLOT) {
        step(kActive, std::integral_constant<int, 0>{}, st0);
        if (st0 + 1 < nst) step(kActive, std::integral_constant<int, 1>{}, st0 + 1);
        if (st0 + 2 < nst) step(kActive, std::integral_constant<int, 2>{}, st0 + 2);
      }
    }
  };
  issue(ring[0], 0);
  if (nst > 1) issue(ring[1], 1);
  if (64 * wm < __builtin_amdgcn_readfirstlane(m)) run(std::true_type{});
  else run(std::false_type{});
  if (kMode != kModeFC1) lds_barrier();  // every wave is done with the ring: it becomes the staging area
  tile256_epilogue<kMode, kYBF16, false>(a, acc, reinterpret_cast<uint8_t*>(&ring[0]), n_tile, row0, m);
}

template <int kMode, bool kYBF16>
static void launch_f8ring_t(const GemmArgs& a, int64_t m_units, hipStream_t stream) {
  const dim3 grid = tile256_grid(kMode, a, m_units, 1);
  // fully unrolled instances for K = 7168 and K = 2048 (the layer's H and I)
  const int64_t nst = a.K / f8r::KS;
  if (nst == 56) gemm_f8ring_kernel<kMode, kYBF16, 56><<<grid, 512, 0, stream>>>(a);
  else if (nst == 16) gemm_f8ring_kernel<kMode, kYBF16, 16><<<grid, 512, 0, stream>>>(a);
  else gemm_f8ring_kernel<kMode, kYBF16, 0><<<grid, 512, 0, stream>>>(a);
}

void launch_f8ring_gemm(int mode, bool y_bf16, const GemmArgs& a, int64_t m_units, hipStream_t stream) {
  if (mode == kModeFC1) launch_f8ring_t<kModeFC1, false>(a, m_units, stream);
  else if (mode == kModeDense) launch_f8ring_t<kModeDense, false>(a, m_units, stream);
  else if (y_bf16) launch_f8ring_t<kModeFC2, true>(a, m_units, stream);
  else launch_f8ring_t<kModeFC2, false>(a, m_units, stream);
}

}  // namespace mxf
