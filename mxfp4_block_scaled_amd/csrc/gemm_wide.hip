// Wide LDS-ring MXFP4 GEMM for E2M1 activations: 256 activation rows x 256 weight
// rows per workgroup, 8 waves of 64 x 128 on the 32x32x64 scaled MFMA.
//
// Why a second ring kernel: with FP4 x FP4 operands a 128 x 256 tile moves 51 KB
// from L2 into LDS per 256-k stage for 128 MFMAs, which at the matrix cores' rate
// asks for about 46 bytes per clock per CU - the measured ceiling of the
// L2 -> LDS copy path. A 256 x 256 tile moves 68 KB for 256 MFMAs (two thirds of
// the bytes per product). Two 68 KB slots fill most of the 160 KB of LDS, so the
// ring is two stages deep: the copies of stage st+1 are issued at the top of stage
// st and land while it is computed. The copy path still sets the pace: on the
// 16384-token FP4 layer FC1's copies alone (no LDS reads, no MFMAs) take 80 % of
// the kernel's time, its MFMAs and LDS reads alone (no copies) 75 %.
//
// Row groups of 64 that lie wholly past an expert's last row skip their MFMAs (the
// wave still issues its share of the copies and meets every barrier), so the
// padding of a 256-row unit costs copy bandwidth but not matrix-core time.
#include "tile256.hpp"

namespace mxf {

namespace wide {
constexpr int BM = 256, BN = 256;
constexpr int KS = 256;                  // k per stage
constexpr int S = KS / 64;               // MFMA steps per stage
constexpr int R = KS / 2;                // bytes per row per stage (E2M1, A and B alike)
constexpr int CH = R / 16;               // 16-byte chunks per row
constexpr int SB = KS / 32;              // scale bytes per row per stage
constexpr int G = 4;                     // stages per scale group
constexpr int SG = G * SB;               // scale bytes per row per group
constexpr int IA = BM * CH / 64 / 8;     // A copies (16 B per lane) per wave per stage
constexpr int IB = BN * CH / 64 / 8;     // B copies per wave per stage
constexpr int D = IA + IB;
}  // namespace wide

struct alignas(16) WideSlot {
  uint8_t A[wide::BM * wide::R];
  uint8_t B[wide::BN * wide::R];
};
// the scales of G stages ([256 rows][32 bytes] per operand), double-buffered
struct alignas(16) WideScales {
  uint8_t A[wide::BM * wide::SG];
  uint8_t B[wide::BN * wide::SG];
};
static_assert(2 * sizeof(WideSlot) + 2 * sizeof(WideScales) <= 160 * 1024, "ring and scale buffers must fit in LDS");
static_assert(kTile256Staging <= (int)sizeof(WideSlot), "eight waves' staging regions must fit one slot");

// NST > 0: K / 256 is a compile-time constant and the ring is fully unrolled;
// NST == 0: any K (multiple of 256) with a runtime loop.

// NTG: consecutive n-tiles per workgroup (grouped GEMMs in the expert-major order;
// 1 for dense), unrolled like the stages
template <int kMode, bool kYBF16, int NST, int NTG>
__global__ void __launch_bounds__(512) gemm_wide_kernel(GemmArgs a) {
  using namespace wide;
  // the scale buffers first: at LDS addresses below 64 KB their offsets fit an
  // LDS instruction's immediate field
  __shared__ WideScales scl0, scl1;
  __shared__ WideSlot slot0, slot1;

  // the wave index through readfirstlane: the compiler then sees it as uniform and
  // forms the LDS-DMA destinations (M0) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5,
            r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;  // rows [64 wm, 64 wm + 64), column half wn

  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  static_assert(NTG == 1 || (NST > 0 && NST % 2 == 0 && kMode != kModeDense), "n-tile groups need an even stage count");
  constexpr int ntg = NTG;
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
    int loc, n_grp;
    grouped_work_item<BM>(a.offsets, a.E, a.split, ntiles / ntg, x, jb, e, n_grp, loc);
    if (e < 0) return;
    n_tile = n_grp * ntg;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow = K / 2, srow = K / 32;

  auto a_src_row = [&](int r) -> int64_t {  // rows past m read the unit's first row (never stored)
    if (r >= m) r = 0;
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };
  // FC1: weight rows [0, 128) of the tile are gate rows, [128, 256) the matching up rows
  auto b_row = [&](int r) -> int64_t {
    if (kMode == kModeFC1) return (r < BN / 2 ? 0 : a.I - BN / 2) + (int64_t)n_tile * (BN / 2) + r;
    return (int64_t)n_tile * BN + r;
  };

  // per-lane copy sources as 32-bit byte offsets into range-checked buffer
  // resources (activations, this expert's weights, their scales); LDS chunk c of a
  // slot holds row c / 8, global chunk (c % 8) ^ swz(row) of that row's 128-byte
  // stage segment. The expert index is wave-uniform; readfirstlane makes the
  // compiler see that, so the resources live in scalar registers.
  const int eu = __builtin_amdgcn_readfirstlane(e);
  const buf_rsrc ra = make_rsrc(a.act, (uint32_t)(a.act_rows * wrow));
  const buf_rsrc ras = make_rsrc(a.act_scale, (uint32_t)(a.act_rows * srow));
  const buf_rsrc rb = make_rsrc(a.w + (int64_t)eu * a.N * wrow, (uint32_t)(a.N * wrow));
  const buf_rsrc rbs = make_rsrc(a.w_scale + (int64_t)eu * a.N * srow, (uint32_t)(a.N * srow));
  uint32_t va[IA], vb[IB];
#pragma unroll
  for (int q = 0; q < IA; ++q) {
    const int chunk = (wave * IA + q) * 64 + lane;
    const int r = chunk / CH, pc = chunk % CH;
    va[q] = (uint32_t)(a_src_row(r) * wrow + 16 * (pc ^ swz<CH>(r)));
  }
#pragma unroll
  for (int q = 0; q < IB; ++q) {
    const int chunk = (wave * IB + q) * 64 + lane;
    const int r = chunk / CH, pc = chunk % CH;
    vb[q] = (uint32_t)(b_row(r) * wrow + 16 * (pc ^ swz<CH>(r)));
  }
  // the weight rows of n-tile n_tile + t sit t * bstep rows further on (FC1: both the
  // gate and the up half move by 128 rows)
  const int64_t bstep = kMode == kModeFC1 ? BN / 2 : BN;
  // Scales move in groups of G stages (32 bytes per row): one 16-byte piece per
  // lane, lane l's piece landing at 16 l, so wave w fills rows [32 w, 32 w + 32) of
  // a [256][32] group buffer with one copy per operand - a quarter of the copy
  // instructions (each touching 32 rows) that per-stage scale copies would take.
  // A group past the end of K reads other rows' bytes or, at the end of the
  // buffer, zeros (range check); those bytes are never used.
  const uint32_t vsa = (uint32_t)(a_src_row(32 * wave + (lane >> 1)) * srow + 16 * (lane & 1));
  const uint32_t vsb = (uint32_t)(b_row(32 * wave + (lane >> 1)) * srow + 16 * (lane & 1));
  auto issue_scales = [&](WideScales& sc, int grp, int t) {
    buf_dma16(ras, &sc.A[wave * 1024], vsa, (uint32_t)grp * SG);
    buf_dma16(rbs, &sc.B[wave * 1024], vsb, (uint32_t)(grp * SG + t * bstep * srow));
  };

  // copy j (0 .. D-1) of stage st of n-tile n_tile + t into slot sl: A chunks, then B chunks
  auto issue_one = [&](WideSlot& sl, int st, int t, int j) {
    if (j < IA) {
      buf_dma16(ra, &sl.A[(wave * IA + j) * 1024], va[j], (uint32_t)st * R);
    } else {
      const int q = j - IA;
      buf_dma16(rb, &sl.B[(wave * IB + q) * 1024], vb[q], (uint32_t)(st * R + t * bstep * wrow));
    }
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

  // MFMA step s of a stage covers, for lane group g, the 32-k block 4 g + s (16-byte
  // chunk 4 g + s of a row; byte s of the lane's scale dword)
  struct Frags {
    v4i a[2], b[4];
  };
  // Byte offset of a fragment row's chunk 4 g + s in a slot: the row's offset with
  // chunk 4 g, XOR 16 s (s only touches bits 4-5). The offsets at s = 0 pass through
  // an empty asm at every use, so the compiler recomputes the XOR per step instead
  // of keeping one address register per (slot, step, fragment).
  int aoff[2], boff[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) aoff[f] = arow_l[f] * R + 16 * ((4 * g) ^ swz<CH>(arow_l[f]));
#pragma unroll
  for (int f = 0; f < 4; ++f) boff[f] = brow_l[f] * R + 16 * ((4 * g) ^ swz<CH>(brow_l[f]));
  auto load_frags = [&](const WideSlot& sl, int s, Frags& F) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      int o = aoff[f];
      asm volatile("" : "+v"(o));
      F.a[f] = *reinterpret_cast<const v4i*>(&sl.A[o ^ (16 * s)]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      int o = boff[f];
      asm volatile("" : "+v"(o));
      F.b[f] = *reinterpret_cast<const v4i*>(&sl.B[o ^ (16 * s)]);
    }
  };
  auto mfma_step = [&](auto S_, const Frags& F, const int* sa, const int* sb) {
    constexpr int s = decltype(S_)::value;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
      const v8i af = v8i{F.a[fm][0], F.a[fm][1], F.a[fm][2], F.a[fm][3], 0, 0, 0, 0};
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        const v8i bf = v8i{F.b[fn][0], F.b[fn][1], F.b[fn][2], F.b[fn][3], 0, 0, 0, 0};
        acc[fm][fn] = mfma32x32x64<kFmtFP4, kFmtFP4, s>(bf, af, acc[fm][fn], sb[fn], sa[fm]);
      }
    }
  };

  // One stage. Step 0 issues every copy of stage nst_ into slot nsl (when `more`),
  // activation rows then weight rows, and the next scale group into nsc (when
  // `more_sc`); then step s reads the fragments of step s + 1 and runs the MFMAs of
  // step s. Full scheduling fences between the steps keep that order, so each step's
  // LDS reads overlap the previous step's MFMAs and the copies have the whole stage to
  // land. The stage's scales are stage `sub` of group buffer csc. (Measured on the
  // 16384-token FP4 layer against copies spread over the four steps: FC1 -2.5 %, FC2
  // -4 %; weight rows first instead runs as fast but fetches 12 % (FC1) and 7 % (FC2)
  // more from HBM.)
  auto stage = [&](auto kActive, const WideSlot& sl, WideSlot& nsl, bool more, int nst_, int t_, const WideScales& csc,
                   WideScales& nsc, bool more_sc, int grp_next, int t_sc, int sub) {
    constexpr bool act = decltype(kActive)::value;
    int sa[2], sb[4];
    Frags F[2];
    if constexpr (act) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        int o = arow_l[f] * SG + 4 * g;
        asm volatile("" : "+v"(o));
        sa[f] = *reinterpret_cast<const int*>(&csc.A[o + SB * sub]);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        int o = brow_l[f] * SG + 4 * g;
        asm volatile("" : "+v"(o));
        sb[f] = *reinterpret_cast<const int*>(&csc.B[o + SB * sub]);
      }
      load_frags(sl, 0, F[0]);
    }
    auto one = [&](auto S_) {
      constexpr int s = decltype(S_)::value;
      if (s == 0 && more) {
#pragma unroll
        for (int j = 0; j < D; ++j) issue_one(nsl, nst_, t_, j);
      }
      if (s == 0 && more_sc) issue_scales(nsc, grp_next, t_sc);
      if constexpr (act) {
        if constexpr (s + 1 < S) load_frags(sl, s + 1, F[(s + 1) & 1]);
        mfma_step(S_, F[s & 1], sa, sb);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    one(std::integral_constant<int, 0>{});
    one(std::integral_constant<int, 1>{});
    one(std::integral_constant<int, 2>{});
    one(std::integral_constant<int, 3>{});
  };
  static_assert(S == 4, "four MFMA steps per stage");

  // ring of two slots: at stage st wait for its copies (the only ones in flight),
  // barrier (every wave's part has landed and every wave is done with st - 1),
  // then compute st while the copies of st + 1 go to the other slot. With several
  // n-tiles per workgroup the ring runs on: the last stage of n-tile t copies stage 0
  // of n-tile t + 1 (K / 256 is even, so every n-tile starts in slot 0), and its
  // first scale group goes to buffer 0 in that stage when the n-tile's last group
  // uses buffer 1, else right after the stage loop.
  const int nst = NST > 0 ? NST : (int)(K / KS);
  const int ngrp = (nst + G - 1) / G;
  auto run = [&](auto kActive, auto T_) {
    constexpr int t = decltype(T_)::value;
    auto step = [&](auto I, int st) {
      constexpr int i = decltype(I)::value;
      wait_vmcnt<0>();
      lds_barrier();
      WideSlot& cur = i == 0 ? slot0 : slot1;
      WideSlot& nxt = i == 0 ? slot1 : slot0;
      const int grp = st / G;
      WideScales& csc = (grp & 1) ? scl1 : scl0;
      WideScales& nsc = (grp & 1) ? scl0 : scl1;
      const bool last = st + 1 == nst, next_tile = last && t + 1 < ntg;
      const bool sc_in_tile = st % G == 0 && grp + 1 < ngrp;
      const bool sc_next_tile = next_tile && ngrp % 2 == 0;
      stage(kActive, cur, nxt, !last || next_tile, last ? 0 : st + 1, last ? t + 1 : t, csc, nsc,
            sc_in_tile || sc_next_tile, sc_in_tile ? grp + 1 : 0, sc_in_tile ? t : t + 1, st % G);
    };
    auto turn = [&](int st0) {
      step(std::integral_constant<int, 0>{}, st0);
      if (st0 + 1 < nst) step(std::integral_constant<int, 1>{}, st0 + 1);
    };
    if constexpr (NST > 0) {
#pragma unroll
      for (int st0 = 0; st0 < NST; st0 += 2) turn(st0);
    } else {
      for (int st0 = 0; st0 < nst; st0 += 2) turn(st0);
    }
  };
#pragma unroll
  for (int j = 0; j < D; ++j) issue_one(slot0, 0, 0, j);
  issue_scales(scl0, 0, 0);
  const bool active = 64 * wm < __builtin_amdgcn_readfirstlane(m);
  static_for<0, NTG>([&](auto T_) {
    constexpr int t = decltype(T_)::value;
    if (t > 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
    }
    if (active) run(std::true_type{}, T_);
    else run(std::false_type{}, T_);
    constexpr bool more_tiles = t + 1 < NTG;
    if (kMode != kModeFC1 || (more_tiles && ngrp % 2 == 1)) lds_barrier();  // every wave is done with the ring
    if (more_tiles && ngrp % 2 == 1) issue_scales(scl0, 0, t + 1);
    // staging (FC2 / dense) in slot 1 only: slot 0 may be receiving the next n-tile's stage 0
    tile256_epilogue<kMode, kYBF16, true>(a, acc, reinterpret_cast<uint8_t*>(&slot1), n_tile + t, row0, m);
  });
}

template <int kMode, bool kYBF16>
static void launch_wide_t(const GemmArgs& a_in, int64_t m_units, hipStream_t stream) {
  // fully unrolled instances for K = 7168 and K = 2048 (the layer's H and I)
  GemmArgs a = a_in;
  const int64_t nst = a.K / wide::KS;
  if constexpr (kMode != kModeDense) {
    if (nst == 8 && a.ngroup == 4) {
      gemm_wide_kernel<kMode, kYBF16, 8, 4><<<tile256_grid(kMode, a, m_units, 4), 512, 0, stream>>>(a);
      return;
    }
    if (nst == 8 && a.ngroup == 2) {
      gemm_wide_kernel<kMode, kYBF16, 8, 2><<<tile256_grid(kMode, a, m_units, 2), 512, 0, stream>>>(a);
      return;
    }
  }
  a.ngroup = 1;
  const dim3 grid = tile256_grid(kMode, a, m_units, 1);
  if (nst == 28) gemm_wide_kernel<kMode, kYBF16, 28, 1><<<grid, 512, 0, stream>>>(a);
  else if (nst == 8) gemm_wide_kernel<kMode, kYBF16, 8, 1><<<grid, 512, 0, stream>>>(a);
  else gemm_wide_kernel<kMode, kYBF16, 0, 1><<<grid, 512, 0, stream>>>(a);
}

// Measured on the 16384-token FP4 layer: four n-tiles per workgroup take FC2 (8
// stages per n-tile) from 1.41 to 1.30 ms (seven: no further change); FC1 (28
// stages) gains nothing from two, so it keeps one.
void launch_wide_gemm(int mode, bool y_bf16, const GemmArgs& a_in, int64_t m_units, hipStream_t stream) {
  // consecutive n-tiles per workgroup for the grouped FC2 at K = 2048: the ring runs
  // on from one n-tile into the next, which needs an even stage count
  GemmArgs a = a_in;
  a.ngroup = 1;
  if (mode == kModeFC2 && a.K / wide::KS == 8) a.ngroup = a.ntiles % 4 == 0 ? 4 : a.ntiles % 2 == 0 ? 2 : 1;
  if (mode == kModeFC1) launch_wide_t<kModeFC1, false>(a, m_units, stream);
  else if (mode == kModeDense) launch_wide_t<kModeDense, false>(a, m_units, stream);
  else if (y_bf16) launch_wide_t<kModeFC2, true>(a, m_units, stream);
  else launch_wide_t<kModeFC2, false>(a, m_units, stream);
}

}  // namespace mxf
