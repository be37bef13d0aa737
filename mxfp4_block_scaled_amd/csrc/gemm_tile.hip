// LDS-ring MXFP4 GEMM for many rows per expert with E4M3 activations (prefill,
// dense M > 64), on the 32x32x64 scaled MFMA, and the dispatch of the tiled
// GEMMs: E2M1 activations go to the 256 x 256 wide kernel (gemm_wide.hip).
#include "gemm_common.hpp"

namespace mxf {

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

  // wave index through readfirstlane: seen as uniform, LDS-DMA destinations stay scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5,
            r32 = lane & 31;

  // XCD-aware order (block b runs on XCD b % 8). Dense: XCD x owns n-tiles
  // [x*nt/8, (x+1)*nt/8) and walks the row units. Grouped: expert-major items split
  // into one contiguous range per XCD, so an XCD's resident workgroups share
  // activation units and weight tiles in its L2.
  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  int e = 0, n_tile;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
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
  // e is the same in every lane (the work-item lookup broadcasts it); say so, so that the
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
  // Fully unrolled instances for K = 7168 and 2048 where they fit the registers:
  // with fp32 outputs (dense C, FC2 with fp32 y) they would spill about 200 VGPRs,
  // so those take the loop instance (no spills).
  constexpr bool kUnroll = kMode == kModeFC1 || (kMode == kModeFC2 && kYBF16);
  if constexpr (kUnroll) {
    if (nst == 28) {
      gemm_tile4_kernel<kActFP4, kMode, kYBF16, 28><<<grid, 256, 0, stream>>>(a);
      return;
    }
    if (nst == 8) {
      gemm_tile4_kernel<kActFP4, kMode, kYBF16, 8><<<grid, 256, 0, stream>>>(a);
      return;
    }
  }
  gemm_tile4_kernel<kActFP4, kMode, kYBF16, 0><<<grid, 256, 0, stream>>>(a);
}

// Measured on the 2048- and 16384-token layers: with FP8 activations the
// register-streamed kernel is the fastest tiled kernel here (its activation tile is
// the larger operand and stays on the LDS path); with FP4 activations the 256 x 256
// wide kernel is. Both address their operands with 32-bit byte offsets: callers
// check tile_offsets_fit first.
bool tile_offsets_fit(int64_t rows, int64_t K, int64_t N, bool act_fp4) {
  const int64_t lim = (int64_t)1 << 32;
  return rows * (act_fp4 ? K / 2 : K) < lim && N * (K / 2) < lim;
}

int launch_tile_gemm(int mode, bool y_bf16, bool act_fp4, const GemmArgs& a, int64_t rows, int64_t groups,
                     hipStream_t stream) {
  if (!tile_offsets_fit(a.act_rows, a.K, a.N, act_fp4)) return -1;
  if (act_fp4) {
    // 256-row units: an upper bound on the units summed over the groups
    launch_wide_gemm(mode, y_bf16, a, cdiv(rows, 256) + groups, stream);
    return 0;
  }
  const int64_t m_units = cdiv(rows, tile::BM) + groups;
  if (mode == kModeFC1) launch_tile4<false, kModeFC1, false>(a, m_units, stream);
  else if (mode == kModeDense) launch_tile4<false, kModeDense, false>(a, m_units, stream);
  else if (y_bf16) launch_tile4<false, kModeFC2, true>(a, m_units, stream);
  else launch_tile4<false, kModeFC2, false>(a, m_units, stream);
  return 0;
}

}  // namespace mxf
