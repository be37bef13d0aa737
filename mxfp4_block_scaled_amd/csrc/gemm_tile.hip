// LDS-ring MXFP4 GEMM for many rows per expert (prefill, dense M > 64) on the
// 32x32x64 scaled MFMA.
#include "gemm_common.hpp"

namespace mxf {

// ---------------------------------------------------------------------------------
// LDS-ring kernel, 32x32x64 scaled MFMA: 128 rows x 256 weight rows per workgroup
// (4 waves of 64 x 128). Operand tiles go HBM -> LDS with global_load_lds_dwordx4
// (no staging registers) into a ring of NS stage slots; the loads of stage st+NS-1
// are issued while stage st is computed, so NS-1 stages are in flight. Each slot is
// its own __shared__ object so the compiler can tell the slot being read from the
// slots being filled; lds_barrier() keeps the loads in flight across the barrier
// and an explicit vmcnt wait (counted in load instructions per wave) marks a
// stage as landed. 16-byte chunks are XOR-swizzled within a row: a lane of a DMA
// instruction writes LDS chunk p (fixed by its lane id) and fetches the global
// chunk that belongs there.
namespace t3 {
constexpr int BM = tile::BM, BN = tile::BN;
}  // namespace t3

template <bool kActFP4>
struct T3Cfg {
  static constexpr int KS = 256;                    // k per stage
  static constexpr int NS = kActFP4 ? 3 : 2;        // ring slots (a 3rd FP8 slot would not fit in LDS)
  static constexpr int S = KS / 64;                 // MFMA steps per stage
  static constexpr int RA = kActFP4 ? KS / 2 : KS;  // A bytes per row per stage
  static constexpr int RB = KS / 2;                 // B bytes per row per stage
  static constexpr int CA = RA / 16, CB = RB / 16;  // 16-byte chunks per row
  static constexpr int SB = KS / 32;                // scale bytes per row per stage
  static constexpr int IA = t3::BM * CA / 64 / 4;   // A DMA instructions per wave
  static constexpr int IB = t3::BN * CB / 64 / 4;   // B DMA instructions per wave
  static constexpr int ISA = t3::BM * SB / 256 / 4; // A-scale DMA instructions (4 B per lane) per wave
  static constexpr int ISB = t3::BN * SB / 256 / 4; // B-scale DMA instructions per wave
  static constexpr int D = IA + IB + ISA + ISB;      // DMA instructions per wave per stage
};

template <bool kActFP4>
struct alignas(16) T3Slot {
  uint8_t A[t3::BM * T3Cfg<kActFP4>::RA];
  uint8_t B[t3::BN * T3Cfg<kActFP4>::RB];
  uint8_t As[t3::BM * T3Cfg<kActFP4>::SB];
  uint8_t Bs[t3::BN * T3Cfg<kActFP4>::SB];
};

// NST > 0: the stage count K / 256 is a compile-time constant and the ring loop is
// fully unrolled (a runtime loop makes the compiler drain all loads once per ring
// turn); NST == 0: any K (multiple of 256) with a runtime loop.
template <bool kActFP4, int kMode, bool kYBF16, int NST>
__global__ void __launch_bounds__(256) gemm_tile3_kernel(GemmArgs a) {
  using namespace t3;
  using C = T3Cfg<kActFP4>;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  struct alignas(16) NoSlot {
    uint8_t pad[16];
  };
  __shared__ T3Slot<kActFP4> slot0, slot1;
  __shared__ typename std::conditional<kActFP4, T3Slot<kActFP4>, NoSlot>::type slot2;  // 3rd slot: FP4 only

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware order (block b runs on XCD b % 8): XCD x owns n-tiles [x*nt/8, (x+1)*nt/8)
  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  const int n_lo = x * ntiles / 8, n_hi = (x + 1) * ntiles / 8, nn = n_hi - n_lo;
  if (nn == 0) return;
  const int m_unit = jb / nn;
  const int n_tile = n_lo + jb % nn;

  int e = 0;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    row0 = (int64_t)m_unit * BM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < BM ? a.M - row0 : BM);
  } else {
    int loc;
    find_unit<BM>(a.offsets, a.E, m_unit, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow = K / 2, srow = K / 32;
  const int64_t arow = kActFP4 ? K / 2 : K;

  // activation row (rows past m read row 0 of the tile's first source; never stored)
  auto a_src_row = [&](int r) -> int64_t {
    if (r >= m) r = 0;
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };
  auto b_row = [&](int r) -> int64_t {
    if (kMode == kModeFC1) return (r < BN / 2 ? 0 : a.I - BN / 2) + (int64_t)n_tile * (BN / 2) + r;
    return (int64_t)n_tile * BN + r;
  };

  // per-lane global sources of this wave's DMA instructions (stage 0)
  const uint8_t* pa[C::IA];
  const uint8_t* pb[C::IB];
  const uint8_t* psa[C::ISA];
  const uint8_t* psb[C::ISB];
#pragma unroll
  for (int q = 0; q < C::IA; ++q) {
    const int chunk = (wave * C::IA + q) * 64 + lane;  // LDS chunk this lane fills
    const int r = chunk / C::CA, pc = chunk % C::CA;
    pa[q] = a.act + a_src_row(r) * arow + 16 * (pc ^ swz<C::CA>(r));
  }
#pragma unroll
  for (int q = 0; q < C::IB; ++q) {
    const int chunk = (wave * C::IB + q) * 64 + lane;
    const int r = chunk / C::CB, pc = chunk % C::CB;
    pb[q] = a.w + ((int64_t)e * a.N + b_row(r)) * wrow + 16 * (pc ^ swz<C::CB>(r));
  }
#pragma unroll
  for (int q = 0; q < C::ISA; ++q) {
    const int dw = (wave * C::ISA + q) * 64 + lane;  // dword of the A-scale slot
    const int r = dw / (C::SB / 4), part = dw % (C::SB / 4);
    psa[q] = a.act_scale + a_src_row(r) * srow + 4 * part;
  }
#pragma unroll
  for (int q = 0; q < C::ISB; ++q) {
    const int dw = (wave * C::ISB + q) * 64 + lane;
    const int r = dw / (C::SB / 4), part = dw % (C::SB / 4);
    psb[q] = a.w_scale + ((int64_t)e * a.N + b_row(r)) * srow + 4 * part;
  }

  // copy j (0 .. D-1) of stage st into slot sl: A chunks, B chunks, A scales, B scales
  auto issue_one = [&](T3Slot<kActFP4>& sl, int st, int j) {
    if (j < C::IA) {
      dma16_to_lds(pa[j] + (int64_t)st * C::RA, &sl.A[(wave * C::IA + j) * 1024]);
    } else if (j < C::IA + C::IB) {
      const int q = j - C::IA;
      dma16_to_lds(pb[q] + (int64_t)st * C::RB, &sl.B[(wave * C::IB + q) * 1024]);
    } else if (j < C::IA + C::IB + C::ISA) {
      const int q = j - C::IA - C::IB;
      dma4_to_lds(psa[q] + (int64_t)st * C::SB, &sl.As[(wave * C::ISA + q) * 256]);
    } else {
      const int q = j - C::IA - C::IB - C::ISA;
      dma4_to_lds(psb[q] + (int64_t)st * C::SB, &sl.Bs[(wave * C::ISB + q) * 256]);
    }
  };
  auto issue = [&](T3Slot<kActFP4>& sl, int st) {
#pragma unroll
    for (int j = 0; j < C::D; ++j) issue_one(sl, st, j);
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = v16f{};

  int arow_l[2], brow_l[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) arow_l[f] = 64 * wm + 32 * f + r32;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if (kMode == kModeFC1) brow_l[f] = (f < 2 ? 0 : BN / 2) + 64 * wn + 32 * (f & 1) + r32;
    else brow_l[f] = 128 * wn + 32 * f + r32;
  }

  // compute one stage; ahead of MFMA step s go copies [s DC, (s + 1) DC) of the
  // next stage (when nsl is given), so the copies spread over the stage instead
  // of stalling the wave in one burst
  constexpr int DC = (C::D + C::S - 1) / C::S;
  auto compute = [&](const T3Slot<kActFP4>& sl, T3Slot<kActFP4>* nsl, int nst_) {
    int sa[2], sb[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (C::SB == 8) sa[f] = *reinterpret_cast<const int*>(&sl.As[arow_l[f] * 8 + 4 * g]);
      else sa[f] = *reinterpret_cast<const uint16_t*>(&sl.As[arow_l[f] * 4 + 2 * g]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (C::SB == 8) sb[f] = *reinterpret_cast<const int*>(&sl.Bs[brow_l[f] * 8 + 4 * g]);
      else sb[f] = *reinterpret_cast<const uint16_t*>(&sl.Bs[brow_l[f] * 4 + 2 * g]);
    }
#pragma unroll
    for (int s = 0; s < C::S; ++s) {
      if (nsl) {
#pragma unroll
        for (int j = s * DC; j < (s + 1) * DC && j < C::D; ++j) issue_one(*nsl, nst_, j);
      }
      __builtin_amdgcn_sched_barrier(0x078F);  // the copies stay in this step; all else may move
      v8i af[2], bf[4];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int r = arow_l[f];
        const uint8_t* rowp = &sl.A[r * C::RA];
        if (kActFP4) {
          const int c = C::S * g + s;
          const v4i x4 = *reinterpret_cast<const v4i*>(rowp + 16 * (c ^ swz<C::CA>(r)));
          af[f] = v8i{x4[0], x4[1], x4[2], x4[3], 0, 0, 0, 0};
        } else {
          const int c1 = 2 * s + g, c2 = 2 * (C::S + s) + g;
          const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c1 ^ swz<C::CA>(r)));
          const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (c2 ^ swz<C::CA>(r)));
          af[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int r = brow_l[f];
        const int c = C::S * g + s;
        const v4i y4 = *reinterpret_cast<const v4i*>(&sl.B[r * C::RB + 16 * (c ^ swz<C::CB>(r))]);
        bf[f] = v8i{y4[0], y4[1], y4[2], y4[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          if (s == 0) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 0>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 1) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 1>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 2) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 2>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 3>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
        }
    }
  };

  // ring pipeline: at stage st, stages st..st+NS-2 have been issued; wait for st
  // (leaving the later ones in flight), barrier, refill the slot freed by st-1, compute st
  constexpr int NS = C::NS, D = C::D;
  const int nst = NST > 0 ? NST : (int)(K / C::KS);
  // every ring step is a compile-time instance, so each DMA and each LDS read names
  // its slot object (the compiler then keeps the loads of other slots in flight)
  auto slot_of = [&](auto I) -> T3Slot<kActFP4>& {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) {
      return slot0;
    } else if constexpr (i == 1) {
      return slot1;
    } else {
      if constexpr (kActFP4) return slot2;  // the 3rd slot exists for FP4 only
      else return slot0;                    // never reached: FP8 runs a 2-slot ring
    }
  };
  auto step = [&](auto I, int st) {
    constexpr int i = decltype(I)::value;
    constexpr int inext = (i + NS - 1) % NS;
    if (NS == 3 && st + 1 < nst) wait_vmcnt<D>();  // stage st+1 may stay in flight
    else wait_vmcnt<0>();
    lds_barrier();
    compute(slot_of(I), st + NS - 1 < nst ? &slot_of(std::integral_constant<int, inext>{}) : nullptr, st + NS - 1);
  };
  issue(slot0, 0);
  if constexpr (NS == 3) {
    if (nst > 1) issue(slot1, 1);
  }
  auto ring_turn = [&](int st0) {
    step(std::integral_constant<int, 0>{}, st0);
    if (st0 + 1 < nst) step(std::integral_constant<int, 1>{}, st0 + 1);
    if constexpr (NS == 3) {
      if (st0 + 2 < nst) step(std::integral_constant<int, 2>{}, st0 + 2);
    }
  };
  if constexpr (NST > 0) {
#pragma unroll
    for (int st0 = 0; st0 < NST; st0 += NS) ring_turn(st0);
  } else {
    for (int st0 = 0; st0 < nst; st0 += NS) ring_turn(st0);
  }
  lds_barrier();  // every wave is done reading the ring; slot0 becomes epilogue staging

  // epilogues, 64-row halves staged in slot0 (the waves with wm == half write)
  uint8_t* stage = slot0.A;
  if (kMode == kModeFC1) {
    float(*hf)[BN / 2 + 4] = reinterpret_cast<float(*)[BN / 2 + 4]>(stage);
    const int64_t i0 = (int64_t)n_tile * (BN / 2);
    const int64_t hrow = kActFP4 ? a.I / 2 : a.I;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rr = 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
              hf[rr][64 * wn + 32 * f + r32] = silu_mul(acc[fm][f][v], acc[fm][f + 2][v]);
            }
      }
      __syncthreads();
      const int rr = tid >> 2, blk = tid & 3;  // 64 rows x 4 blocks of 32 = 256 items
      const int lr = 64 * half + rr;
      if (lr < m) {
        const int64_t R = row0 + lr;
        quantize_store32<kActFP4>(&hf[rr][32 * blk], a.h + R * hrow + (i0 + 32 * blk) / (kActFP4 ? 2 : 1),
                                  a.h_scale + R * (a.I / 32) + i0 / 32 + blk);
      }
      __syncthreads();
    }
  } else if (kYBF16) {
    uint16_t(*ob)[BN + 8] = reinterpret_cast<uint16_t(*)[BN + 8]>(stage);
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int fn = 0; fn < 4; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rr = 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
              ob[rr][128 * wn + 32 * fn + r32] = (uint16_t)bf16_round(acc[fm][fn][v]);
            }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < (64 * BN / 8) / 256; ++q) {
        const int idx = tid + 256 * q;
        const int rr = idx >> 5, cc = (idx & 31) * 8;
        const int lr = 64 * half + rr;
        if (lr < m)
          *reinterpret_cast<uint4*>(out + (row0 + lr) * a.N + (int64_t)n_tile * BN + cc) =
              *reinterpret_cast<const uint4*>(&ob[rr][cc]);
      }
      __syncthreads();
    }
  } else {
    float(*of)[BN + 4] = reinterpret_cast<float(*)[BN + 4]>(stage);
    float* out = static_cast<float*>(a.out);
#pragma unroll
    for (int quarter = 0; quarter < 4; ++quarter) {
      if (wm == (quarter >> 1)) {
        const int fm = quarter & 1;
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rr = 8 * (v >> 2) + 4 * g + (v & 3);
            of[rr][128 * wn + 32 * fn + r32] = acc[fm][fn][v];
          }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < (32 * BN / 4) / 256; ++q) {
        const int idx = tid + 256 * q;
        const int rr = idx >> 6, cc = (idx & 63) * 4;
        const int lr = 32 * quarter + rr;
        if (lr < m)
          *reinterpret_cast<float4*>(out + (row0 + lr) * a.N + (int64_t)n_tile * BN + cc) =
              *reinterpret_cast<const float4*>(&of[rr][cc]);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// Register-streamed weights: 128 activation rows x 256 weight rows per workgroup.
// Wave w owns weight rows [64 w, 64 w + 64) of the tile (FC1: the 32 gate rows of
// I-columns [32 w, 32 w + 32) and the 32 matching up rows) against all 128
// activation rows: 4 x 2 fragments of the 32x32x64 scaled MFMA. A weight row is
// read by exactly one wave, so weights go HBM -> registers directly; the
// activation tile, shared by the 4 waves, goes HBM -> LDS by global_load_lds
// into a ring of NSA slots. Stage st + NSA - 1 (activation slot and weight
// registers alike) is issued right after the barrier of stage st, so NSA - 1
// stages are in flight while one is computed. FC1's SwiGLU pairs sit in one wave
// and the epilogues stage through that wave's own LDS region (no cross-wave
// hand-off after the main loop).
namespace t4 {
constexpr int BM = tile::BM, BN = tile::BN;
constexpr int S = 4;    // MFMA steps per 256-k stage
constexpr int NSA = 4;  // ring slots
}  // namespace t4

template <bool kActFP4>
struct T4Cfg {
  static constexpr int RA = kActFP4 ? 128 : 256;   // activation bytes per row per stage
  static constexpr int CA = RA / 16;               // 16-byte chunks per activation row per stage
  static constexpr int IA = t4::BM * CA / 64 / 4;  // activation DMA instructions per wave per stage
  static constexpr int NB = 2 * t4::S + 2;         // weight loads per wave per stage (data + scales)
  static constexpr int NV = IA + 1 + NB;           // vector-memory instructions per wave per stage
  static_assert(NB + 2 * NV < 64, "in-flight loads must fit the vmcnt counter");
};

template <bool kActFP4>
struct alignas(16) T4Slot {
  uint8_t A[t4::BM * T4Cfg<kActFP4>::RA];  // activation codes, 16-byte chunks XOR-swizzled per row
  uint8_t As[t4::BM * 8];                   // activation scale bytes, [row][8]
};

template <bool kActFP4, int kMode, bool kYBF16, int NST>
__global__ void __launch_bounds__(256) gemm_tile4_kernel(GemmArgs a) {
  using C = T4Cfg<kActFP4>;
  constexpr int BM = t4::BM, BN = t4::BN, S = t4::S, NSA = t4::NSA;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  __shared__ T4Slot<kActFP4> slot0, slot1, slot2, slot3;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;

  // XCD-aware order (block b runs on XCD b % 8): XCD x owns n-tiles [x*nt/8, (x+1)*nt/8)
  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  const int n_lo = x * ntiles / 8, n_hi = (x + 1) * ntiles / 8, nn = n_hi - n_lo;
  if (nn == 0) return;
  const int m_unit = jb / nn;
  const int n_tile = n_lo + jb % nn;

  int e = 0;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    row0 = (int64_t)m_unit * BM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < BM ? a.M - row0 : BM);
  } else {
    int loc;
    find_unit<BM>(a.offsets, a.E, m_unit, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow = K / 2, srow = K / 32;
  const int64_t arow = kActFP4 ? K / 2 : K;
  const int nst = NST > 0 ? NST : (int)(K / 256);

  // activation row r of the tile (rows past m read the tile's first row; never stored)
  auto a_src_row = [&](int r) -> int64_t {
    if (r >= m) r = 0;
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };

  // All loads go through raw buffer resources (32-bit byte offsets; the host
  // routes shapes whose operands exceed 4 GiB elsewhere). Per-lane offsets are
  // fixed; the stage advances a scalar offset.
  const buf_rsrc ra = make_rsrc(a.act, (uint32_t)(a.act_rows * arow));
  const buf_rsrc ras = make_rsrc(a.act_scale, (uint32_t)(a.act_rows * srow));
  // e is the same in every lane (find_unit broadcasts it); say so, so that the
  // weight resources live in scalar registers
  const int eu = __builtin_amdgcn_readfirstlane(e);
  const buf_rsrc rb = make_rsrc(a.w + (int64_t)eu * a.N * wrow, (uint32_t)(a.N * wrow));
  const buf_rsrc rbs = make_rsrc(a.w_scale + (int64_t)eu * a.N * srow, (uint32_t)(a.N * srow));

  // activation DMA offsets of stage 0: this lane fills LDS chunk (wave IA + q) 64 + lane
  uint32_t va[C::IA];
#pragma unroll
  for (int q = 0; q < C::IA; ++q) {
    const int chunk = (wave * C::IA + q) * 64 + lane;
    const int r = chunk / C::CA, pc = chunk % C::CA;
    va[q] = (uint32_t)(a_src_row(r) * arow + 16 * (pc ^ swz<C::CA>(r)));
  }
  // activation-scale DMA offset: dword wave 64 + lane of the [128][8] scale slot
  const int sdw = wave * 64 + lane;
  const uint32_t vas = (uint32_t)(a_src_row(sdw >> 1) * srow + 4 * (sdw & 1));

  // this wave's two weight fragments: offsets of the code and scale rows (stage 0)
  uint32_t vb[2], vbs[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    int64_t n;
    if (kMode == kModeFC1) n = (f == 0 ? 0 : a.I) + (int64_t)n_tile * (BN / 2) + 32 * wave + r32;
    else n = (int64_t)n_tile * BN + 64 * wave + 32 * f + r32;
    vb[f] = (uint32_t)(n * wrow + 64 * g);
    vbs[f] = (uint32_t)(n * srow + 4 * g);
  }

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  v4i bq[NSA][2][S];  // weight codes: lane (r32, g) of step s holds block S g + s of its row
  int bsc[NSA][2];    // weight scale bytes of blocks S g .. S g + 3 (op_sel = s)

  auto slot_of = [&](auto I) -> T4Slot<kActFP4>& {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return slot0;
    else if constexpr (i == 1) return slot1;
    else if constexpr (i == 2) return slot2;
    else return slot3;
  };
  // issue stage st into ring slot / register buffer I: activation DMAs first, then weights
  auto issue = [&](auto I, int st) {
    constexpr int i = decltype(I)::value;
    T4Slot<kActFP4>& sl = slot_of(I);
    const uint32_t sa_off = (uint32_t)st * C::RA, ss_off = (uint32_t)st * 8, sb_off = (uint32_t)st * 128;
#pragma unroll
    for (int q = 0; q < C::IA; ++q) buf_dma16(ra, &sl.A[(wave * C::IA + q) * 1024], va[q], sa_off);
    buf_dma4(ras, &sl.As[wave * 256], vas, ss_off);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int s = 0; s < S; ++s) bq[i][f][s] = buf_load16(rb, vb[f] + 16 * s, sb_off);
#pragma unroll
    for (int f = 0; f < 2; ++f) bsc[i][f] = buf_load4(rbs, vbs[f], ss_off);
  };
  auto compute = [&](auto I) {
    constexpr int i = decltype(I)::value;
    const T4Slot<kActFP4>& sl = slot_of(I);
    int sa[4];
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) sa[fm] = *reinterpret_cast<const int*>(&sl.As[(32 * fm + r32) * 8 + 4 * g]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      v8i af[4];
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) {
        const int r = 32 * fm + r32;
        const uint8_t* rowp = &sl.A[r * C::RA];
        if (kActFP4) {
          const v4i x4 = *reinterpret_cast<const v4i*>(rowp + 16 * ((S * g + s) ^ swz<C::CA>(r)));
          af[fm] = v8i{x4[0], x4[1], x4[2], x4[3], 0, 0, 0, 0};
        } else {
          const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * ((2 * s + g) ^ swz<C::CA>(r)));
          const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * ((2 * (S + s) + g) ^ swz<C::CA>(r)));
          af[fm] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const v4i b4 = bq[i][fn][s];
        const v8i bf = v8i{b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) {
          if (s == 0) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 0>(af[fm], bf, acc[fm][fn], sa[fm], bsc[i][fn]);
          else if (s == 1) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 1>(af[fm], bf, acc[fm][fn], sa[fm], bsc[i][fn]);
          else if (s == 2) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 2>(af[fm], bf, acc[fm][fn], sa[fm], bsc[i][fn]);
          else acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 3>(af[fm], bf, acc[fm][fn], sa[fm], bsc[i][fn]);
        }
      }
    }
  };
  // wait until this wave's activation DMAs of stage st have landed: issued after
  // them are the weight loads of st and every later stage already issued
  auto wait_stage = [&](int st) {
    const int ahead = min(NSA - 2, nst - 1 - st);
    if (ahead >= 2) wait_vmcnt<C::NB + 2 * C::NV>();
    else if (ahead == 1) wait_vmcnt<C::NB + C::NV>();
    else wait_vmcnt<C::NB>();
  };
  auto step = [&](auto I, int st) {
    constexpr int i = decltype(I)::value;
    wait_stage(st);
    lds_barrier();  // every wave's part of stage st has landed; every wave is done with st - 1
    if (st + NSA - 1 < nst) issue(std::integral_constant<int, (i + NSA - 1) % NSA>{}, st + NSA - 1);
    compute(I);
  };
  static_assert(NSA == 4, "the ring below is written for 4 slots");
  issue(std::integral_constant<int, 0>{}, 0);
  if (nst > 1) issue(std::integral_constant<int, 1>{}, 1);
  if (nst > 2) issue(std::integral_constant<int, 2>{}, 2);
  auto ring_turn = [&](int st0) {
    step(std::integral_constant<int, 0>{}, st0);
    if (st0 + 1 < nst) step(std::integral_constant<int, 1>{}, st0 + 1);
    if (st0 + 2 < nst) step(std::integral_constant<int, 2>{}, st0 + 2);
    if (st0 + 3 < nst) step(std::integral_constant<int, 3>{}, st0 + 3);
  };
  if constexpr (NST > 0) {
#pragma unroll
    for (int st0 = 0; st0 < NST; st0 += NSA) ring_turn(st0);
  } else {
    for (int st0 = 0; st0 < nst; st0 += NSA) ring_turn(st0);
  }
  lds_barrier();  // every wave is done reading the ring; slot w becomes wave w's staging area

  uint8_t* const stage = wave == 0 ? slot0.A : wave == 1 ? slot1.A : wave == 2 ? slot2.A : slot3.A;
  // the staging writes and reads below are this wave's own: LDS runs a wave's
  // accesses in order, the asm keeps the compiler from reordering them
  auto lds_wave_fence = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  if (kMode == kModeFC1) {
    // h = silu(gate) * up for this wave's 32 I-columns, 64 rows at a time, then
    // each lane requantises one row's block of 32
    static_assert(64 * 36 * 4 <= (int)sizeof(T4Slot<kActFP4>), "FC1 staging must fit a slot");
    float(*hf)[36] = reinterpret_cast<float(*)[36]>(stage);
    const int64_t icol = (int64_t)n_tile * (BN / 2) + 32 * wave;
    const int64_t hrow = kActFP4 ? a.I / 2 : a.I;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int f2 = 0; f2 < 2; ++f2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          hf[32 * f2 + 8 * (v >> 2) + 4 * g + (v & 3)][r32] = silu_mul(acc[2 * half + f2][0][v], acc[2 * half + f2][1][v]);
      lds_wave_fence();
      const int lr = 64 * half + lane;
      if (lr < m) {
        const int64_t R = row0 + lr;
        quantize_store32<kActFP4>(&hf[lane][0], a.h + R * hrow + icol / (kActFP4 ? 2 : 1),
                                  a.h_scale + R * (a.I / 32) + icol / 32);
      }
      lds_wave_fence();
    }
  } else if (kYBF16) {
    static_assert(32 * 72 * 2 <= (int)sizeof(T4Slot<kActFP4>), "bf16 staging must fit a slot");
    uint16_t(*ob)[72] = reinterpret_cast<uint16_t(*)[72]>(stage);
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int64_t col0 = (int64_t)n_tile * BN + 64 * wave;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          ob[8 * (v >> 2) + 4 * g + (v & 3)][32 * fn + r32] = (uint16_t)bf16_round(acc[fm][fn][v]);
      lds_wave_fence();
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // 32 rows x 64 columns = 256 pieces of 16 bytes
        const int idx = lane + 64 * j;
        const int rr = idx >> 3, c8 = idx & 7;
        const int lr = 32 * fm + rr;
        if (lr < m)
          *reinterpret_cast<uint4*>(out + (row0 + lr) * a.N + col0 + 8 * c8) =
              *reinterpret_cast<const uint4*>(&ob[rr][8 * c8]);
      }
      lds_wave_fence();
    }
  } else {
    static_assert(32 * 68 * 4 <= (int)sizeof(T4Slot<kActFP4>), "fp32 staging must fit a slot");
    float(*of)[68] = reinterpret_cast<float(*)[68]>(stage);
    float* out = static_cast<float*>(a.out);
    const int64_t col0 = (int64_t)n_tile * BN + 64 * wave;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) of[8 * (v >> 2) + 4 * g + (v & 3)][32 * fn + r32] = acc[fm][fn][v];
      lds_wave_fence();
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // 32 rows x 64 columns = 512 pieces of 16 bytes
        const int idx = lane + 64 * j;
        const int rr = idx >> 4, c4 = idx & 15;
        const int lr = 32 * fm + rr;
        if (lr < m)
          *reinterpret_cast<float4*>(out + (row0 + lr) * a.N + col0 + 4 * c4) =
              *reinterpret_cast<const float4*>(&of[rr][4 * c4]);
      }
      lds_wave_fence();
    }
  }
}

template <bool kActFP4, int kMode, bool kYBF16>
static void launch_tile4(const GemmArgs& a, int64_t m_units, hipStream_t stream) {
  const int64_t nn = cdiv(a.ntiles, 8);
  const dim3 grid((unsigned)(8 * nn * m_units));
  const int64_t nst = a.K / 256;
  if (nst == 28) gemm_tile4_kernel<kActFP4, kMode, kYBF16, 28><<<grid, 256, 0, stream>>>(a);
  else if (nst == 8) gemm_tile4_kernel<kActFP4, kMode, kYBF16, 8><<<grid, 256, 0, stream>>>(a);
  else gemm_tile4_kernel<kActFP4, kMode, kYBF16, 0><<<grid, 256, 0, stream>>>(a);
}

#ifndef MXF_TILE4
#define MXF_TILE4 1
#endif

// ---------------------------------------------------------------------------------
// Eight-wave variant of the LDS-ring kernel: the same 128 x 256 tile, ring and
// copies, computed by 8 waves of 64 x 64 (2 x 2 fragments) - two waves per SIMD,
// so one wave's MFMAs run while the other waits at the barrier, on a copy or on
// its LDS reads. FC1: wave (wm, wn) holds the gate rows of I-columns
// [32 wn, 32 wn + 32) and the matching up rows; the epilogues stage through each
// wave's own LDS region.
template <bool kActFP4>
struct T8Cfg {
  using B = T3Cfg<kActFP4>;
  static constexpr int IA = t3::BM * B::CA / 64 / 8;  // A copies per wave per stage (16 B per lane)
  static constexpr int IB = t3::BN * B::CB / 64 / 8;  // B copies per wave per stage
  static constexpr int D = IA + IB + 2;              // + one A-scale and one B-scale copy (4 B per lane)
};

template <bool kActFP4, int kMode, bool kYBF16, int NST>
__global__ void __launch_bounds__(512) gemm_tile8_kernel(GemmArgs a) {
  using namespace t3;
  using C = T3Cfg<kActFP4>;
  using C8 = T8Cfg<kActFP4>;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  struct alignas(16) NoSlot {
    uint8_t pad[16];
  };
  __shared__ T3Slot<kActFP4> slot0, slot1;
  __shared__ typename std::conditional<kActFP4, T3Slot<kActFP4>, NoSlot>::type slot2;  // 3rd slot: FP4 only

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;

  // XCD-aware order (block b runs on XCD b % 8): XCD x owns n-tiles [x*nt/8, (x+1)*nt/8)
  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  const int n_lo = x * ntiles / 8, n_hi = (x + 1) * ntiles / 8, nn = n_hi - n_lo;
  if (nn == 0) return;
  const int m_unit = jb / nn;
  const int n_tile = n_lo + jb % nn;

  int e = 0;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    row0 = (int64_t)m_unit * BM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < BM ? a.M - row0 : BM);
  } else {
    int loc;
    find_unit<BM>(a.offsets, a.E, m_unit, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow = K / 2, srow = K / 32;
  const int64_t arow = kActFP4 ? K / 2 : K;

  auto a_src_row = [&](int r) -> int64_t {  // rows past m read the tile's first row (never stored)
    if (r >= m) r = 0;
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };
  auto b_row = [&](int r) -> int64_t {
    if (kMode == kModeFC1) return (r < BN / 2 ? 0 : a.I - BN / 2) + (int64_t)n_tile * (BN / 2) + r;
    return (int64_t)n_tile * BN + r;
  };

  // per-lane copy sources of stage 0
  const uint8_t* pa[C8::IA];
  const uint8_t* pb[C8::IB];
#pragma unroll
  for (int q = 0; q < C8::IA; ++q) {
    const int chunk = (wave * C8::IA + q) * 64 + lane;  // LDS chunk this lane fills
    const int r = chunk / C::CA, pc = chunk % C::CA;
    pa[q] = a.act + a_src_row(r) * arow + 16 * (pc ^ swz<C::CA>(r));
  }
#pragma unroll
  for (int q = 0; q < C8::IB; ++q) {
    const int chunk = (wave * C8::IB + q) * 64 + lane;
    const int r = chunk / C::CB, pc = chunk % C::CB;
    pb[q] = a.w + ((int64_t)e * a.N + b_row(r)) * wrow + 16 * (pc ^ swz<C::CB>(r));
  }
  // scale copies in 4-byte pieces (a copy writes lane l's piece at 4 l): the [128][8]
  // A-scale slot by the first 32 lanes of each wave (wave w: rows 16 w .. 16 w + 15),
  // the [256][8] B-scale slot by all 64 lanes (wave w: rows 32 w .. 32 w + 31)
  const uint8_t* psa = a.act_scale + a_src_row(16 * wave + ((lane & 31) >> 1)) * srow + 4 * (lane & 1);
  const uint8_t* psb = a.w_scale + ((int64_t)e * a.N + b_row(32 * wave + (lane >> 1))) * srow + 4 * (lane & 1);

  // copy j (0 .. D-1) of stage st into slot sl: A chunks, B chunks, A scales, B scales
  auto issue_one = [&](T3Slot<kActFP4>& sl, int st, int j) {
    if (j < C8::IA) {
      dma16_to_lds(pa[j] + (int64_t)st * C::RA, &sl.A[(wave * C8::IA + j) * 1024]);
    } else if (j < C8::IA + C8::IB) {
      const int q = j - C8::IA;
      dma16_to_lds(pb[q] + (int64_t)st * C::RB, &sl.B[(wave * C8::IB + q) * 1024]);
    } else if (j == C8::IA + C8::IB) {
      if (lane < 32) dma4_to_lds(psa + (int64_t)st * C::SB, &sl.As[wave * 128]);  // one instruction, half the lanes
    } else {
      dma4_to_lds(psb + (int64_t)st * C::SB, &sl.Bs[wave * 256]);
    }
  };
  auto issue = [&](T3Slot<kActFP4>& sl, int st) {
#pragma unroll
    for (int j = 0; j < C8::D; ++j) issue_one(sl, st, j);
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  int arow_l[2], brow_l[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    arow_l[f] = 64 * wm + 32 * f + r32;
    if (kMode == kModeFC1) brow_l[f] = (f == 0 ? 0 : BN / 2) + 32 * wn + r32;
    else brow_l[f] = 64 * wn + 32 * f + r32;
  }

  // compute one stage; ahead of MFMA step s go copies [s DC, (s + 1) DC) of the
  // next stage (when nsl is given), so the copies spread over the stage
  constexpr int DC = (C8::D + C::S - 1) / C::S;
  auto compute = [&](const T3Slot<kActFP4>& sl, T3Slot<kActFP4>* nsl, int nst_) {
    int sa[2], sb[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      sa[f] = *reinterpret_cast<const int*>(&sl.As[arow_l[f] * 8 + 4 * g]);
      sb[f] = *reinterpret_cast<const int*>(&sl.Bs[brow_l[f] * 8 + 4 * g]);
    }
#pragma unroll
    for (int s = 0; s < C::S; ++s) {
      if (nsl) {
#pragma unroll
        for (int j = s * DC; j < (s + 1) * DC && j < C8::D; ++j) issue_one(*nsl, nst_, j);
      }
      __builtin_amdgcn_sched_barrier(0x078F);  // the copies stay in this step; all else may move
      v8i af[2], bf[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int r = arow_l[f];
        const uint8_t* rowp = &sl.A[r * C::RA];
        if (kActFP4) {
          const v4i x4 = *reinterpret_cast<const v4i*>(rowp + 16 * ((C::S * g + s) ^ swz<C::CA>(r)));
          af[f] = v8i{x4[0], x4[1], x4[2], x4[3], 0, 0, 0, 0};
        } else {
          const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * ((2 * s + g) ^ swz<C::CA>(r)));
          const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * ((2 * (C::S + s) + g) ^ swz<C::CA>(r)));
          af[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const int rb = brow_l[f];
        const v4i y4 = *reinterpret_cast<const v4i*>(&sl.B[rb * C::RB + 16 * ((C::S * g + s) ^ swz<C::CB>(rb))]);
        bf[f] = v8i{y4[0], y4[1], y4[2], y4[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          if (s == 0) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 0>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 1) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 1>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 2) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 2>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 3>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
        }
    }
  };

  // ring: at stage st, stages st .. st+NS-2 have been issued; wait for st (leaving
  // the later ones in flight), barrier, refill the slot freed by st-1, compute st
  constexpr int NS = C::NS;
  const int nst = NST > 0 ? NST : (int)(K / C::KS);
  auto slot_of = [&](auto I) -> T3Slot<kActFP4>& {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) {
      return slot0;
    } else if constexpr (i == 1) {
      return slot1;
    } else {
      if constexpr (kActFP4) return slot2;
      else return slot0;  // never reached: FP8 runs a 2-slot ring
    }
  };
  auto step = [&](auto I, int st) {
    constexpr int i = decltype(I)::value;
    constexpr int inext = (i + NS - 1) % NS;
    if (NS == 3 && st + 1 < nst) wait_vmcnt<C8::D>();  // stage st+1 (issued after st) may stay in flight
    else wait_vmcnt<0>();
    lds_barrier();
    compute(slot_of(I), st + NS - 1 < nst ? &slot_of(std::integral_constant<int, inext>{}) : nullptr, st + NS - 1);
  };
  issue(slot0, 0);
  if constexpr (NS == 3) {
    if (nst > 1) issue(slot1, 1);
  }
  auto ring_turn = [&](int st0) {
    step(std::integral_constant<int, 0>{}, st0);
    if (st0 + 1 < nst) step(std::integral_constant<int, 1>{}, st0 + 1);
    if constexpr (NS == 3) {
      if (st0 + 2 < nst) step(std::integral_constant<int, 2>{}, st0 + 2);
    }
  };
  if constexpr (NST > 0) {
#pragma unroll
    for (int st0 = 0; st0 < NST; st0 += NS) ring_turn(st0);
  } else {
    for (int st0 = 0; st0 < nst; st0 += NS) ring_turn(st0);
  }
  lds_barrier();  // every wave is done reading the ring; the slots become staging areas

  // wave w stages in slot0 (w < 4) or slot1 (w >= 4), region (w % 4) x 9216 bytes
  uint8_t* const stage = (wave < 4 ? slot0.A : slot1.A) + (wave & 3) * 9216;
  static_assert(4 * 9216 <= (int)sizeof(T3Slot<kActFP4>), "per-wave staging regions must fit a slot");
  auto lds_wave_fence = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  if (kMode == kModeFC1) {
    // h = silu(gate) * up: 64 rows x 32 I-columns (one quantisation block per row),
    // then lane l requantises row l
    float(*hf)[36] = reinterpret_cast<float(*)[36]>(stage);
    const int64_t icol = (int64_t)n_tile * (BN / 2) + 32 * wn;
    const int64_t hrow = kActFP4 ? a.I / 2 : a.I;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        hf[32 * fm + 8 * (v >> 2) + 4 * g + (v & 3)][r32] = silu_mul(acc[fm][0][v], acc[fm][1][v]);
    lds_wave_fence();
    const int lr = 64 * wm + lane;
    if (lr < m) {
      const int64_t R = row0 + lr;
      quantize_store32<kActFP4>(&hf[lane][0], a.h + R * hrow + icol / (kActFP4 ? 2 : 1),
                                a.h_scale + R * (a.I / 32) + icol / 32);
    }
  } else if (kYBF16) {
    uint16_t(*ob)[72] = reinterpret_cast<uint16_t(*)[72]>(stage);  // 64 x 72 x 2 = 9216 bytes
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int64_t col0 = (int64_t)n_tile * BN + 64 * wn;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          ob[32 * fm + 8 * (v >> 2) + 4 * g + (v & 3)][32 * fn + r32] = (uint16_t)bf16_round(acc[fm][fn][v]);
    lds_wave_fence();
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // 64 rows x 64 columns = 512 pieces of 16 bytes
      const int idx = lane + 64 * j;
      const int rr = idx >> 3, c8 = idx & 7;
      const int lr = 64 * wm + rr;
      if (lr < m)
        *reinterpret_cast<uint4*>(out + (row0 + lr) * a.N + col0 + 8 * c8) = *reinterpret_cast<const uint4*>(&ob[rr][8 * c8]);
    }
  } else {
    float(*of)[68] = reinterpret_cast<float(*)[68]>(stage);  // 32 x 68 x 4 = 8704 bytes
    float* out = static_cast<float*>(a.out);
    const int64_t col0 = (int64_t)n_tile * BN + 64 * wn;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) of[8 * (v >> 2) + 4 * g + (v & 3)][32 * fn + r32] = acc[fm][fn][v];
      lds_wave_fence();
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // 32 rows x 64 columns = 512 pieces of 16 bytes
        const int idx = lane + 64 * j;
        const int rr = idx >> 4, c4 = idx & 15;
        const int lr = 64 * wm + 32 * fm + rr;
        if (lr < m)
          *reinterpret_cast<float4*>(out + (row0 + lr) * a.N + col0 + 4 * c4) = *reinterpret_cast<const float4*>(&of[rr][4 * c4]);
      }
      lds_wave_fence();
    }
  }
}

template <bool kActFP4, int kMode, bool kYBF16>
static void launch_tile8(const GemmArgs& a, int64_t m_units, hipStream_t stream) {
  const int64_t nn = cdiv(a.ntiles, 8);
  const dim3 grid((unsigned)(8 * nn * m_units));
  const int64_t nst = a.K / 256;
  if (nst == 28) gemm_tile8_kernel<kActFP4, kMode, kYBF16, 28><<<grid, 512, 0, stream>>>(a);
  else if (nst == 8) gemm_tile8_kernel<kActFP4, kMode, kYBF16, 8><<<grid, 512, 0, stream>>>(a);
  else gemm_tile8_kernel<kActFP4, kMode, kYBF16, 0><<<grid, 512, 0, stream>>>(a);
}

#ifndef MXF_TILE8
#define MXF_TILE8 1
#endif

template <bool kActFP4, int kMode, bool kYBF16>
static void launch_tile3(const GemmArgs& a, int64_t m_units, hipStream_t stream) {
  const int64_t nn3 = cdiv(a.ntiles, 8);
  const dim3 g3((unsigned)(8 * nn3 * m_units));
  // fully unrolled instances for K = 7168 and K = 2048 (the layer's H and I)
  const int64_t nst = a.K / 256;
  if (nst == 28) gemm_tile3_kernel<kActFP4, kMode, kYBF16, 28><<<g3, 256, 0, stream>>>(a);
  else if (nst == 8) gemm_tile3_kernel<kActFP4, kMode, kYBF16, 8><<<g3, 256, 0, stream>>>(a);
  else gemm_tile3_kernel<kActFP4, kMode, kYBF16, 0><<<g3, 256, 0, stream>>>(a);
}

// the register-streamed kernel addresses every operand with 32-bit byte offsets
static bool fits_tile4(const GemmArgs& a, bool act_fp4) {
  const int64_t lim = (int64_t)1 << 32;
  const int64_t arow = act_fp4 ? a.K / 2 : a.K;
  return a.act_rows * arow < lim && a.N * (a.K / 2) < lim;
}

// Measured on the 2048- and 16384-token layers: with FP8 activations the
// register-streamed kernel is faster (its activation tile is the larger operand
// and stays on the LDS path); with FP4 activations the ring kernel is, because
// per-lane weight loads touch 4x more cache lines per instruction than the
// HBM -> LDS copies of whole 1 KB runs.
template <bool kActFP4>
static void launch_tile_fmt(int mode, bool y_bf16, const GemmArgs& a, int64_t m_units, hipStream_t stream) {
  if (MXF_TILE4 && !kActFP4 && fits_tile4(a, kActFP4)) {
    if (mode == kModeFC1) launch_tile4<kActFP4, kModeFC1, false>(a, m_units, stream);
    else if (mode == kModeDense) launch_tile4<kActFP4, kModeDense, false>(a, m_units, stream);
    else if (y_bf16) launch_tile4<kActFP4, kModeFC2, true>(a, m_units, stream);
    else launch_tile4<kActFP4, kModeFC2, false>(a, m_units, stream);
    return;
  }
  if (MXF_TILE8) {
    if (mode == kModeFC1) launch_tile8<kActFP4, kModeFC1, false>(a, m_units, stream);
    else if (mode == kModeDense) launch_tile8<kActFP4, kModeDense, false>(a, m_units, stream);
    else if (y_bf16) launch_tile8<kActFP4, kModeFC2, true>(a, m_units, stream);
    else launch_tile8<kActFP4, kModeFC2, false>(a, m_units, stream);
    return;
  }
  if (mode == kModeFC1) launch_tile3<kActFP4, kModeFC1, false>(a, m_units, stream);
  else if (mode == kModeDense) launch_tile3<kActFP4, kModeDense, false>(a, m_units, stream);
  else if (y_bf16) launch_tile3<kActFP4, kModeFC2, true>(a, m_units, stream);
  else launch_tile3<kActFP4, kModeFC2, false>(a, m_units, stream);
}

#ifndef MXF_WIDE
#define MXF_WIDE 1
#endif

void launch_tile_gemm(int mode, bool y_bf16, bool act_fp4, const GemmArgs& a, int64_t rows, int64_t groups,
                      hipStream_t stream) {
  // the wide kernel addresses activations and one expert's weights with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 32;
  if (MXF_WIDE && act_fp4 && a.act_rows * (a.K / 2) < lim && a.N * (a.K / 2) < lim) {
    // 256-row units: an upper bound on the units summed over the groups
    launch_wide_gemm(mode, y_bf16, a, cdiv(rows, 256) + groups, stream);
    return;
  }
  const int64_t m_units = cdiv(rows, tile::BM) + groups;
  if (act_fp4) launch_tile_fmt<true>(mode, y_bf16, a, m_units, stream);
  else launch_tile_fmt<false>(mode, y_bf16, a, m_units, stream);
}

}  // namespace mxf
