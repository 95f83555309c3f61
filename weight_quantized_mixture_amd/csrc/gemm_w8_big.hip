// Grouped int8-weight GEMMs for 256-row align blocks (prefill-sized expert
// loads, where the MFMA work dominates), gfx950.
//
// experts_int8 page, ExpertsInt8MoEMethod.create_weights / apply ->
// fused_experts(use_int8_w8a16): h = x dequant(w13[e])^T with the per-row
// scale on the fp32 accumulator, a = silu(h_gate) * h_up, then
// y = a dequant(w2[e])^T.  GEMM1 writes a either as bf16 hi/lo planes
// (hi = rne(a), lo = rne(a - hi)) or, when GEMM2 below runs, directly as
// 16-bit fixed point per (row, 128 columns): a ~= s (256 hi + lo) with
// s = max|a| / 32639 over the group, which is exactly the 128 output columns
// of one GEMM1 workgroup (the two waves sharing a row exchange their row
// maxima through LDS).  GEMM2 then runs the int8 codes of w2 and of a
// through v_mfma_i32_16x16x64_i8 (half the MFMA work of two bf16 planes,
// and 32 instead of 48 KB per stage to copy).
//
// GEMM1 tiling: a workgroup owns one align block (256 rows) and 128 output
// columns, i.e. 128 gate + the matching 128 up rows of w13.  Its 4 waves (one
// per SIMD) form a 2 x 2 grid; a wave owns 128 rows x (64 gate + 64 up)
// columns = 8 x 8 accumulator tiles of v_mfma_f32_16x16x32 (256 accumulator
// registers, which live in the AGPR half of the register file).
// K advances in stages of 64 through a 3-deep LDS ring:
//   * both operands go HBM/L2 -> LDS with global_load_lds_dwordx4 (no
//     staging registers, no LDS store instructions): per stage 32 KB of
//     gathered bf16 activation rows and 16 KB of int8 weight rows;
//   * the operand fragments of stage s+1 are read from LDS while the MFMAs
//     of stage s run, and the int8 weights (-> bf16/fp16, exact) are
//     converted one K half ahead of their MFMAs, so LDS latency and the
//     conversion hide behind 128 MFMAs per wave and stage;
//   * one barrier per stage, after which the copy of stage s+3 goes into the
//     slot stage s was read from;
//   * the 16-byte chunks of every LDS row are XOR-swizzled by row so that the
//     16 rows one MFMA operand read touches fall in distinct bank groups;
// Inside a stage, lane (col, kg) feeds K [16kg, 16kg+8) to the first MFMA and
// [16kg+8, 16kg+16) to the second, for both operands (a dot product does not
// depend on the order of its terms).
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRows = 256;                    // rows per workgroup (= block_m)
constexpr int kOut = 128;                     // output columns per workgroup
constexpr int kBK = 64;                       // K per stage
constexpr int kStages = 3;
constexpr int kARow = kBK * 2;                // bytes per activation row per stage
constexpr int kBRow = kBK;                    // bytes per weight row per stage
constexpr int kAStage = kRows * kARow;        // 32 KB
constexpr int kBStage = 2 * kOut * kBRow;     // 16 KB
constexpr int kStageBytes = kAStage + kBStage;

constexpr int kQMax = 32639;                  // 256 * 127 + 127

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int k1Waves = 4;
constexpr int k1Threads = k1Waves * kWave;
constexpr int k1ADma = kAStage / (k1Threads * 16);  // 16-byte copies per thread per stage
constexpr int k1BDma = kBStage / (k1Threads * 16);
constexpr int k1Dma = k1ADma + k1BDma;

// FP8: w13 holds OCP e4m3fn codes with one scale per expert (fp8 page,
// weight-only path), decoded in pairs by gfx950's conversion instruction.
template <bool F16, bool Q16, bool FP8>
__global__ __launch_bounds__(k1Threads) void gemm1_big_kernel(const Gemm1Args p, int8_t* __restrict__ qhi,
                                                              int8_t* __restrict__ qlo, float* __restrict__ qscale) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar registers
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * kRows;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t Tk = p.Tk, H = p.H, I = p.I;

  // valid rows come first in a block; count them in 16-row tiles
  int nrows = 0;
  for (int r = 0; r < kRows; r += 16)
    if (p.sorted_ids[row0 + r] < Tk) nrows = r + 16;
  int ntw = (nrows - wm * 128) / 16;       // row tiles of this wave
  ntw = ntw < 0 ? 0 : (ntw > 8 ? 8 : ntw);
  const int nst = static_cast<int>(H / kBK);

  // copy sources, as 32-bit byte offsets into buffer resources: x (the
  // launcher checks that its size plus one row stays under 2^32 bytes) and
  // the 128 gate or up rows of w13 this wave copies.  Every lane issues every
  // copy, so the per-thread copy count is fixed; rows that hold no token take
  // the offset one past the end of x, which the buffer's range check turns
  // into a zero fill that reads no memory (those rows' results are dropped).
  const uint32_t xbytes = static_cast<uint32_t>(p.T * H * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, xbytes);
  uint32_t aoffs[k1ADma];
#pragma unroll
  for (int i = 0; i < k1ADma; ++i) {
    const int r = wave * (kRows / k1Waves) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    const int f = r < nrows ? p.sorted_ids[row0 + r] : static_cast<int>(Tk);
    const uint32_t t = f < Tk ? static_cast<uint32_t>(f / static_cast<int>(p.k)) : 0u;
    aoffs[i] = f < Tk ? (t * static_cast<uint32_t>(H) + static_cast<uint32_t>(c * 8)) * 2u : xbytes;
  }
  // a wave copies 64 weight rows of one half (gate for waves 0-1, up for
  // 2-3): row b + 16 i has the swizzle of row b, so one lane offset serves
  // all four copies and the row step goes into the uniform offset
  const int64_t nb = static_cast<int64_t>(blockIdx.x) * kOut;
  const bool up_half = wave >= k1Waves / 2;
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(p.w13 + (static_cast<int64_t>(e) * 2 * I + (up_half ? I : 0) + nb) * p.ldw,
                static_cast<uint32_t>(kOut * p.ldw));
  // LDS row 16 q + r (q < 4, r < 16) of a wave's 64 holds source row 4 r + q,
  // so that MFMA tile q, which takes rows 4 col + q, reads 16 consecutive
  // LDS rows (conflict-free under the swizzle) and lane col ends up with the
  // 4 adjacent output columns 4 col .. 4 col + 3.  Copy i of this lane:
  // LDS row 16 i + lane/4, source row 4 (lane/4) + i.
  uint32_t boffv;
  {
    const int b = wave * (2 * kOut / k1Waves) + (lane >> 2);   // LDS row of copy 0
    const int c = (lane & 3) ^ swz_b(b);                       // the same for every copy i
    boffv = static_cast<uint32_t>(((wave & 1) * 64 + 4 * (lane >> 2)) * p.ldw + c * 16);
  }
  const uint32_t bstep = static_cast<uint32_t>(p.ldw);
  // copy number i (of k1Dma) of stage s into LDS slot `slot`
  auto issue_one = [&](int s, int slot, int i) {
    uint8_t* base = smem + slot * kStageBytes;
    if (i < k1ADma)
      dma16_buf(xr, aoffs[i], static_cast<uint32_t>(s * kBK * 2), base + (wave * (kRows / k1Waves) + i * 8) * kARow);
    else
      dma16_buf(wr, boffv, static_cast<uint32_t>(s * kBK) + (i - k1ADma) * bstep,
                base + kAStage + (wave * (2 * kOut / k1Waves) + (i - k1ADma) * 16) * kBRow);
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this lane's weight rows inside the stage tile: tile j (gate j < 4, up
  // j >= 4) reads LDS rows 16 (j & 3) + col of the wave's 64 (source rows
  // 4 col + (j & 3)), all with the swizzle of LDS row col; the up rows sit
  // kOut rows further
  int boff0;
  {
    const int b = wn * 64 + col;
    boff0 = kAStage + b * kBRow + 16 * (kg ^ swz_b(b));
  }
  // activation fragment offsets: the swizzle of row 16 mt + col depends on mt mod 4
  int aoff[4][2];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    const int r = wm * 128 + m4 * 16 + col;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) aoff[m4][ks] = r * kARow + 16 * ((2 * kg + ks) ^ swz_a(r));
  }

  // main loop over K stages, instantiated for 0, 2, 4, 6 or 8 row tiles per
  // wave so that partly filled blocks skip their empty tiles without branches
  auto run = [&](auto tiles) {
    constexpr int MT = decltype(tiles)::value;
    // Registers: af[mt][h] = activation fragment of row tile mt for K half
    // h; rw[j][h] = the 8 int8 weight codes of column tile j for K half h;
    // cw[h][j] = those codes as a 16-bit MFMA operand.  Half 0 of a stage
    // multiplies with cw[0] while converting the stage's half-1 codes into
    // cw[1] and reading both halves of the next stage's codes (one 16-byte
    // read per tile: conflict-free under the row swizzle, where two 8-byte
    // reads collide in pairs); half 1 multiplies with cw[1] while converting
    // the next stage's half-0 codes into cw[0].  Every register a half has
    // finished with is refilled from the next stage's LDS slot right away.
    u32x4 af[MT > 0 ? MT : 1][2];
    u32x2 rw[8][2];
    u32x4 cw[2][8];
    auto read_a = [&](const uint8_t* st, int mt, int h) {
      af[mt][h] = *reinterpret_cast<const u32x4*>(st + mt / 4 * 64 * kARow + aoff[mt & 3][h]);
    };
    auto read_w = [&](const uint8_t* st, int j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + boff0 + (j & 3) * 16 * kBRow + (j >> 2) * kOut * kBRow);
      rw[j][0] = u32x2{v.x, v.y};
      rw[j][1] = u32x2{v.z, v.w};
    };
    auto conv = [&](int j, int h) {
      u32x2 p0, p1;
      if constexpr (FP8) {
        p0 = u32x2{fp8x2_to_16x2<F16, false>(rw[j][h].x), fp8x2_to_16x2<F16, true>(rw[j][h].x)};
        p1 = u32x2{fp8x2_to_16x2<F16, false>(rw[j][h].y), fp8x2_to_16x2<F16, true>(rw[j][h].y)};
      } else {
        p0 = F16 ? i8x4_to_f16x4(rw[j][h].x) : i8x4_to_bf16x4(rw[j][h].x);
        p1 = F16 ? i8x4_to_f16x4(rw[j][h].y) : i8x4_to_bf16x4(rw[j][h].y);
      }
      cw[h][j] = u32x4{p0.x, p0.y, p1.x, p1.y};
    };
    // column tiles handled in row-tile slot m: [jlo(m), jlo(m + 1))
    constexpr int MT1 = MT > 0 ? MT : 1;
    auto jlo = [](int m) { return m * 8 / MT1; };
    // scheduling of one slot (8 MFMAs, nconv conversions of 12 VALU each, a
    // few LDS reads): MFMA and VALU alternate so that the conversions and
    // address arithmetic issue while the matrix core works (measured: for 8
    // row tiles 2 VALU per MFMA beats 1 or 3; partly filled blocks one less
    // than their conversions need per MFMA)
    auto interleave = []() {
      // VALU per conversion of 8 codes, as the schedule counts them (e4m3
      // takes about 4; counting 8 keeps the fp8 loop free of register spills,
      // whose reloads would wait for every copy in flight each stage: 4 spilt
      // 10 registers, and the fp8 prefill ran 8% slower)
      constexpr int kConv = FP8 ? 8 : 12;
      constexpr int per = (kConv * ((8 + MT1 - 1) / MT1) + 7) / 8 - (MT1 < 8 && !FP8 ? 1 : 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, per, 0);   // VALU
        if (i < 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
        if (i == 4) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // copy to LDS
      }
    };

    // one stage: make stage s+1 visible (every thread's copies of it have
    // landed and every wave has read stage s out of its slot), then multiply
    // stage s while reading stage s+1 and refilling stage s's slot with
    // stage s+3 (the last stage's index past the end: those copies are never
    // read).  The copies are spread over the row-tile slots so that no wave
    // stalls on a burst of them.  The last stage (MORE = false) only
    // multiplies.
    constexpr int kSlots = 2 * MT1;
    auto copies = [&](int s, int m) {
      const int sc = s + 3 < nst ? s + 3 : nst - 1;
#pragma unroll
      for (int i = m * k1Dma / kSlots; i < (m + 1) * k1Dma / kSlots; ++i) issue_one(sc, s % kStages, i);
    };
    auto step = [&](int s, auto more_tag) {
      constexpr bool MORE = decltype(more_tag)::value;
      if constexpr (MORE) {
        wait_vmcnt_lgkm0<k1Dma>();
        stage_barrier();
      }
      if constexpr (MT == 0) {
        if constexpr (MORE) {
#pragma unroll
          for (int m = 0; m < kSlots; ++m) copies(s, m);
        }
      } else {
        const uint8_t* nx = smem + ((s + 1) % kStages) * kStageBytes;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[mt][j] = mfma16<F16>(af[mt][0], cw[0][j], acc[mt][j]);
          if constexpr (MORE) {
            read_a(nx, mt, 0);
            copies(s, mt);
          }
#pragma unroll
          for (int j = jlo(mt); j < jlo(mt + 1); ++j) {
            conv(j, 1);
            if constexpr (MORE) read_w(nx, j);
          }
          interleave();
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[mt][j] = mfma16<F16>(af[mt][1], cw[1][j], acc[mt][j]);
          if constexpr (MORE) {
            read_a(nx, mt, 1);
            copies(s, MT + mt);
#pragma unroll
            for (int j = jlo(mt); j < jlo(mt + 1); ++j) {
              conv(j, 0);
            }
            interleave();
          }
        }
      }
    };

    // stages 0, 1, 2 into slots 0, 1, 2 (indices past the end repeat the
    // last stage), then wait for stage 0
#pragma unroll
    for (int q = 0; q < kStages; ++q)
#pragma unroll
      for (int i = 0; i < k1Dma; ++i) issue_one(q < nst ? q : nst - 1, q, i);
    wait_vmcnt<2 * k1Dma>();
    stage_barrier();
    if constexpr (MT > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        read_a(smem, mt, 0);
        read_a(smem, mt, 1);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        read_w(smem, j);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) conv(j, 0);
    }
    for (int s = 0; s + 1 < nst; ++s) step(s, std::true_type{});
    step(nst - 1, std::false_type{});
  };
  if (ntw > 6) run(std::integral_constant<int, 8>{});
  else if (ntw > 4) run(std::integral_constant<int, 6>{});
  else if (ntw > 2) run(std::integral_constant<int, 4>{});
  else if (ntw > 0) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 0>{});
  wait_vmcnt<0>();   // no copy into LDS outlives the main loop

  // epilogue: scales, SiLU(gate) * up; padding rows get 0.  Lane col holds
  // output columns n0 .. n0 + 3.  The ids of the lane's 32 rows (4
  // consecutive rows per tile) are loaded together up front, so their
  // latency is paid once.
  const int64_t n0 = nb + wn * 64 + 4 * col;
  bool valid[8][4];
  {
    i32x4 ids[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      ids[mt] = *reinterpret_cast<const i32x4*>(p.sorted_ids + row0 + wm * 128 + mt * 16 + kg * 4);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) valid[mt][i] = mt < ntw && ids[mt][i] < Tk;
  }
  float sg[4], su[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sg[j] = FP8 ? p.s13[e] : p.s13[static_cast<int64_t>(e) * 2 * I + n0 + j];
    su[j] = FP8 ? p.s13[e] : p.s13[static_cast<int64_t>(e) * 2 * I + I + n0 + j];
  }
  if constexpr (!Q16) {
    // bf16 hi/lo planes
    uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
    uint16_t* a_lo = a_hi + p.cap * I;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if (mt < ntw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = row0 + wm * 128 + mt * 16 + kg * 4 + i;
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[j] = valid[mt][i] ? silu_mul(acc[mt][j][i] * sg[j], acc[mt][j + 4][i] * su[j]) : 0.0f;
          u32x2 hi, lo;
          split_bf16x4(make_float4(v[0], v[1], v[2], v[3]), hi, lo);
          *reinterpret_cast<u32x2*>(a_hi + r * I + n0) = hi;
          *reinterpret_cast<u32x2*>(a_lo + r * I + n0) = lo;
        }
      }
    }
  } else {
    // 16-bit fixed point per (row, the workgroup's 128 columns).  Row maxima:
    // over this lane's 4 columns, the 16 lanes of the row (xor shuffles
    // inside a 16-lane group), then the other wave of the row through LDS.
    float* rmax = reinterpret_cast<float*>(smem);   // [2][256]; the ring is idle now
    float m[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mm = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = valid[mt][i] ? silu_mul(acc[mt][j][i] * sg[j], acc[mt][j + 4][i] * su[j]) : 0.0f;
          acc[mt][j][i] = v;
          mm = fmaxf(mm, fabsf(v));
        }
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) mm = fmaxf(mm, __shfl_xor(mm, d, kWave));
        m[mt][i] = mm;
      }
    wait_vmcnt_lgkm0<0>();
    stage_barrier();   // every wave is past its last copy and LDS read of the ring
    if (col == 0) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[wn * kRows + wm * 128 + mt * 16 + kg * 4 + i] = m[mt][i];
    }
    wait_lgkm0();
    stage_barrier();
    const int64_t G = I / kOut;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if (mt < ntw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = wm * 128 + mt * 16 + kg * 4 + i;
          const float mm = fmaxf(m[mt][i], rmax[(1 - wn) * kRows + rl]);
          const float inv = mm > 0.0f ? static_cast<float>(kQMax) / mm : 0.0f;
          const int64_t r = row0 + rl;
          uint32_t hw = 0u, lw = 0u;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            int q = static_cast<int>(__builtin_rintf(acc[mt][j][i] * inv));
            q = q < -kQMax ? -kQMax : (q > kQMax ? kQMax : q);
            const int h = (q + 128) >> 8;
            hw |= static_cast<uint32_t>(h & 0xff) << (8 * j);
            lw |= static_cast<uint32_t>((q - 256 * h) & 0xff) << (8 * j);
          }
          *reinterpret_cast<uint32_t*>(qhi + r * I + n0) = hw;
          *reinterpret_cast<uint32_t*>(qlo + r * I + n0) = lw;
          if (wn == 0 && col == 0) qscale[r * G + blockIdx.x] = mm / static_cast<float>(kQMax);
        }
      }
    }
  }
}

// GEMM2 for 256-row blocks on the fixed-point form of a: y = a dequant(w2[e])^T,
// scale on the accumulator.  A workgroup owns 128 rows (half an align block)
// and 256 output columns of one K part (grid z: K cut into `splits` parts of
// whole 128-wide scale groups, partials to y[z]); 8 waves (2 per SIMD) in a
// 2 x 4 grid, each 64 rows x 64 columns (4 x 4 tiles of
// v_mfma_i32_16x16x64_i8, hi and lo codes of a against the same w2
// fragment).  Stages of 64 K through a 4-deep LDS ring filled with
// global_load_lds: 8 KB of hi codes, 8 KB of lo codes, 16 KB of w2 codes and
// each wave's 64 row scales of the stage's group.  The copies of stage s+3
// are requested after the barrier of stage s (past the end of the part the
// last stage's index repeats, into a slot nobody reads), so the copy count
// per stage is fixed.  The two stages of one scale group accumulate in int32
// (|.| < 2^22 per plane), and at the group's end each tile is folded into
// fp32 as s_row * (256 hi + lo) (exact in int32: |.| < 2^30).
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int k2Rows = 128;
constexpr int k2Cols = 256;
constexpr int k2Ring = 4;
constexpr int k2APlane = k2Rows * kBK;                // 8 KB
constexpr int k2BBytes = k2Cols * kBK;                // 16 KB
constexpr int k2SBytes = kWaves * 256;                // 64 scales per wave
constexpr int k2StageBytes = 2 * k2APlane + k2BBytes + k2SBytes;
constexpr int k2ADma = 2 * k2APlane / (kThreads * 16);
static_assert((k2APlane / 16) % (k2ADma * kWave) == 0, "each wave copies codes of one plane");
constexpr int k2BDma = k2BBytes / (kThreads * 16);
constexpr int k2Dma = k2ADma + k2BDma + 1;

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}

__global__ __launch_bounds__(kThreads) void gemm2_big_q16_kernel(const Gemm2Args p, const int8_t* __restrict__ qhi,
                                                                 const int8_t* __restrict__ qlo,
                                                                 const float* __restrict__ qscale) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[k2Ring * k2StageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar registers
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int z = static_cast<int>(blockIdx.z);
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * k2Rows;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[row0 / kRows];
  const int64_t Tk = p.Tk, H = p.H, I = p.I, G = I / 128;

  int nrows = 0;
  for (int r = 0; r < k2Rows; r += 16)
    if (p.sorted_ids[row0 + r] < Tk) nrows = r + 16;
  if (nrows == 0) return;      // the second half of a block may be empty (uniform exit)
  int ntw = (nrows - wm * 64) / 16;
  ntw = ntw < 0 ? 0 : (ntw > 4 ? 4 : ntw);
  // this part's stages: whole scale groups [g0, g1), two 64-K stages each
  const int s0 = static_cast<int>(2 * (z * G / p.splits));
  const int s1 = static_cast<int>(2 * ((z + 1) * G / p.splits));

  // copies: code chunk g = (plane, row, 16-byte position) of the stage's
  // hi/lo codes (LDS position g holds source chunk (g%4) ^ swz_b(row)), w2
  // rows b, and this wave's 64 row scales.  The codes go through buffer
  // resources over this half's rows that hold tokens (nrows * I < 2^31 bytes,
  // as I <= 2^24): the copies of the rows past them fall outside the range,
  // read no memory and fill zeros (those rows' results are dropped), while
  // every lane still issues every copy.  Waves 0-3 copy hi codes, 4-7 lo.
  const __amdgpu_buffer_rsrc_t ar =
      make_rsrc((wave * k2ADma < 8 ? qhi : qlo) + row0 * I, static_cast<uint32_t>(nrows * I));
  uint32_t aoffv[k2ADma];
#pragma unroll
  for (int i = 0; i < k2ADma; ++i) {
    const int g = (wave * k2ADma + i) * kWave + lane;
    const int r = (g % (k2Rows * 4)) / 4;
    const int c = (g & 3) ^ swz_b(r);
    aoffv[i] = static_cast<uint32_t>(r * I + c * 16);
  }
  const int64_t hb = static_cast<int64_t>(blockIdx.x) * k2Cols;
  const int8_t* bsrc[k2BDma];
#pragma unroll
  for (int i = 0; i < k2BDma; ++i) {
    const int b = (wave * k2BDma + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(b);
    bsrc[i] = p.w2 + (static_cast<int64_t>(e) * H + hb + b) * p.ldw + c * 16;
  }
  const float* ssrc = qscale + (row0 + wm * 64 + lane) * G;
  auto issue = [&](int s, int slot) __attribute__((always_inline)) {
    uint8_t* base = smem + slot * k2StageBytes;
#pragma unroll
    for (int i = 0; i < k2ADma; ++i)
      dma16_buf(ar, aoffv[i], static_cast<uint32_t>(s * kBK), base + (wave * k2ADma + i) * 1024);
#pragma unroll
    for (int i = 0; i < k2BDma; ++i)
      dma16(bsrc[i] + static_cast<int64_t>(s) * kBK, base + 2 * k2APlane + (wave * k2BDma + i) * 1024);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)const_cast<float*>(ssrc + s / 2),
                                     (lds_ptr_t)(base + 2 * k2APlane + k2BBytes + wave * 256), 4, 0, 0);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = wn * 64 + 16 * j + col;
    boff[j] = 2 * k2APlane + b * kBK + 16 * (kg ^ swz_b(b));
  }
  int aoff[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int r = wm * 64 + mt * 16 + col;
    aoff[mt] = r * kBK + 16 * (kg ^ swz_b(r));
  }

  auto run = [&](auto tiles) __attribute__((always_inline)) {
    constexpr int MT = decltype(tiles)::value;
    i32x4 ih[MT > 0 ? MT : 1][4], il[MT > 0 ? MT : 1][4];
#pragma unroll
    for (int q = 0; q < k2Ring - 1; ++q) issue(s0 + q < s1 ? s0 + q : s1 - 1, q);
    // one stage: LAST = the second stage of its scale group (accumulate onto
    // the first's int32 results, then fold)
    auto stage = [&](int s, auto last_tag) __attribute__((always_inline)) {
      constexpr bool LAST = decltype(last_tag)::value;
      // this thread's copies of stage s landed (those of s+1, s+2 may still
      // fly) and its LDS reads of stage s-1 done; then the slot of s-1 takes
      // stage s+3
      wait_vmcnt_lgkm0<2 * k2Dma>();
      stage_barrier();
      issue(s + 3 < s1 ? s + 3 : s1 - 1, (s - s0 + 3) % k2Ring);
      const uint8_t* st = smem + ((s - s0) % k2Ring) * k2StageBytes;
      u32x4 bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[j] = *reinterpret_cast<const u32x4*>(st + boff[j]);
      // fold of row tile m: fp32 += s_row * (256 hi + lo)
      auto fold = [&](int m) __attribute__((always_inline)) {
        const f32x4 sr =
            *reinterpret_cast<const f32x4*>(st + 2 * k2APlane + k2BBytes + wave * 256 + 4 * (m * 16 + kg * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][j][i] += sr[i] * static_cast<float>(ih[m][j][i] * 256 + il[m][j][i]);
      };
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 ah = *reinterpret_cast<const u32x4*>(st + aoff[mt]);
        const u32x4 al = *reinterpret_cast<const u32x4*>(st + k2APlane + aoff[mt]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x4 z0 = {0, 0, 0, 0};
          ih[mt][j] = mfma_i8(ah, bq[j], LAST ? ih[mt][j] : z0);
          il[mt][j] = mfma_i8(al, bq[j], LAST ? il[mt][j] : z0);
        }
        if constexpr (LAST) {
          // the previous row tile's fold runs under this tile's MFMAs (its
          // own results are not ready yet); one tile row at a time keeps the
          // scheduler from hoisting every MFMA of the stage first
          if (mt > 0) fold(mt - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (LAST && MT > 0) fold(MT - 1);
    };
    for (int s = s0; s < s1; s += 2) {
      stage(s, std::false_type{});
      stage(s + 1, std::true_type{});
    }
  };
  if (ntw > 3) run(std::integral_constant<int, 4>{});
  else if (ntw > 2) run(std::integral_constant<int, 3>{});
  else if (ntw > 1) run(std::integral_constant<int, 2>{});
  else if (ntw > 0) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});
  wait_vmcnt<0>();   // no copy into LDS outlives the workgroup

  float sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sc[j] = p.s2[static_cast<int64_t>(e) * H + hb + wn * 64 + 16 * j + col];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < ntw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = p.sorted_ids[row0 + wm * 64 + mt * 16 + kg * 4 + i];
        if (f < Tk) {
          float* yr = p.y + (static_cast<int64_t>(z) * Tk + f) * H + hb + wn * 64 + col;
#pragma unroll
          for (int j = 0; j < 4; ++j) yr[16 * j] = acc[mt][j][i] * sc[j];
        }
      }
    }
  }
}

}  // namespace

bool gemm1_w8_big_fits(const Gemm1Args& p) { return (p.T + 1) * p.H * 2 < (int64_t{1} << 32); }

hipError_t launch_gemm2_w8_big_q16(const Gemm2Args& p, const int8_t* qhi, const int8_t* qlo, const float* qscale,
                                   hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.H / k2Cols), static_cast<unsigned>(p.cap / k2Rows),
                  static_cast<unsigned>(p.splits));
  hipLaunchKernelGGL(gemm2_big_q16_kernel, grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
  return hipGetLastError();
}

hipError_t launch_gemm1_w8_big(const Gemm1Args& p, int8_t* qhi, int8_t* qlo, float* qscale, hipStream_t stream) {
  if (!gemm1_w8_big_fits(p)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.I / kOut), static_cast<unsigned>(p.cap / kRows));
  const bool q16 = qhi != nullptr;
#define G1(F, Q) hipLaunchKernelGGL((gemm1_big_kernel<F, Q, false>), grid, dim3(k1Threads), 0, stream, p, qhi, qlo, \
                                    qscale)
#define G1F(F) hipLaunchKernelGGL((gemm1_big_kernel<F, false, true>), grid, dim3(k1Threads), 0, stream, p, qhi, qlo, \
                                  qscale)
  if (p.fp8) {
    // bf16 planes only: the fixed-point form feeds the integer-MFMA GEMM2, which takes int8 w2
    if (q16) return hipErrorInvalidValue;
    if (p.f16) G1F(true);
    else G1F(false);
  } else if (p.f16) {
    if (q16) G1(true, true);
    else G1(true, false);
  } else {
    if (q16) G1(false, true);
    else G1(false, false);
  }
#undef G1
#undef G1F
  return hipGetLastError();
}

}  // namespace moe
