// Grouped int8-weight GEMMs for 256-row align blocks (prefill-sized expert
// loads, where the bf16 MFMA work dominates), gfx950.
//
// experts_int8 page, ExpertsInt8MoEMethod.create_weights / apply ->
// fused_experts(use_int8_w8a16): h = x dequant(w13[e])^T with the per-row
// scale on the fp32 accumulator, a = silu(h_gate) * h_up, written as bf16
// hi/lo planes (hi = rne(a), lo = rne(a - hi)).
//
// Tiling: a workgroup owns one align block (256 rows) and 128 output columns,
// i.e. 128 gate + the matching 128 up rows of w13.  Its 8 waves (two per
// SIMD, so one can issue MFMAs while the other waits for LDS) form a 2 x 4
// grid; a wave owns 128 rows x (32 gate + 32 up) columns = 8 x 4 accumulator
// tiles of v_mfma_f32_16x16x32 (128 accumulator registers).
// K advances in stages of 64 through a 3-deep LDS ring:
//   * both operands go HBM/L2 -> LDS with global_load_lds_dwordx4 (no
//     staging registers, no LDS store instructions): per stage 32 KB of
//     gathered bf16 activation rows and 16 KB of int8 weight rows;
//   * stage s+2 is requested while stage s is multiplied; one barrier per
//     stage, preceded by a wait for this thread's own copies of stage s;
//   * the 16-byte chunks of every LDS row are XOR-swizzled by row so that the
//     16 rows one MFMA operand read touches fall in distinct bank groups;
//   * each wave converts its 4 weight fragments (int8 -> bf16/fp16, exact)
//     once per stage and reuses each for its 8 row tiles; all activation
//     fragments of a stage are read first, then the column tiles are walked
//     one by one so the conversion of one overlaps the MFMAs of the last.
// Inside a stage, lane (col, kg) feeds K [16kg, 16kg+8) to the first MFMA and
// [16kg+8, 16kg+16) to the second, for both operands (a dot product does not
// depend on the order of its terms).
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 256;                    // rows per workgroup (= block_m)
constexpr int kOut = 128;                     // output columns per workgroup
constexpr int kBK = 64;                       // K per stage
constexpr int kStages = 3;
constexpr int kARow = kBK * 2;                // bytes per activation row per stage
constexpr int kBRow = kBK;                    // bytes per weight row per stage
constexpr int kAStage = kRows * kARow;        // 32 KB
constexpr int kBStage = 2 * kOut * kBRow;     // 16 KB
constexpr int kStageBytes = kAStage + kBStage;
constexpr int kADma = kAStage / (kThreads * 16);   // 16-byte copies per thread per stage
constexpr int kBDma = kBStage / (kThreads * 16);

template <bool F16>
__global__ __launch_bounds__(kThreads) void gemm1_big_kernel(const Gemm1Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
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

  // copy sources.  Rows that hold no token read token 0's row (never used):
  // every lane issues every copy, so the per-thread copy count is fixed.
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* asrc[kADma];
#pragma unroll
  for (int i = 0; i < kADma; ++i) {
    const int r = wave * (kRows / kWaves) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    const int f = r < nrows ? p.sorted_ids[row0 + r] : static_cast<int>(Tk);
    const int64_t t = f < Tk ? f / static_cast<int>(p.k) : 0;
    asrc[i] = x + t * H + c * 8;
  }
  const int64_t nb = static_cast<int64_t>(blockIdx.x) * kOut;
  const int8_t* bsrc[kBDma];
#pragma unroll
  for (int i = 0; i < kBDma; ++i) {
    const int b = wave * (2 * kOut / kWaves) + i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(b);
    const int64_t n = b < kOut ? nb + b : I + nb + (b - kOut);
    bsrc[i] = p.w13 + (static_cast<int64_t>(e) * 2 * I + n) * p.ldw + c * 16;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * kStageBytes;
#pragma unroll
    for (int i = 0; i < kADma; ++i)
      dma16(asrc[i] + static_cast<int64_t>(s) * kBK, base + (wave * (kRows / kWaves) + i * 8) * kARow);
#pragma unroll
    for (int i = 0; i < kBDma; ++i)
      dma16(bsrc[i] + static_cast<int64_t>(s) * kBK, base + kAStage + (wave * (2 * kOut / kWaves) + i * 16) * kBRow);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this lane's weight rows inside the stage tile (gate j < 2, up j >= 2)
  int boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = (j < 2 ? wn * 32 + 16 * j : kOut + wn * 32 + 16 * (j - 2)) + col;
    boff[j] = kAStage + b * kBRow + 16 * (kg ^ swz_b(b));
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
    issue(0, 0);
    if (nst > 1) issue(1, 1);
    int slot = 0;
    for (int s = 0; s < nst; ++s) {
      if (s + 1 < nst) wait_vmcnt<kADma + kBDma>();
      else wait_vmcnt<0>();
      stage_barrier();
      if (s + 2 < nst) issue(s + 2, slot == 0 ? 2 : slot - 1);
      const uint8_t* st = smem + slot * kStageBytes;

      // all activation fragments of the stage first, then column tile by
      // column tile: converting tile j+1 overlaps the MFMAs of tile j
      u32x4 q[4], af[MT > 0 ? MT : 1][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = *reinterpret_cast<const u32x4*>(st + boff[j]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint8_t* ar = st + mt / 4 * 64 * kARow;
        af[mt][0] = *reinterpret_cast<const u32x4*>(ar + aoff[mt & 3][0]);
        af[mt][1] = *reinterpret_cast<const u32x4*>(ar + aoff[mt & 3][1]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 b[2];
        i8x16_to_operands<F16>(q[j], b[0], b[1]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma16<F16>(af[mt][ks], b[ks], acc[mt][j]);
      }
      slot = slot == kStages - 1 ? 0 : slot + 1;
    }
  };
  if (ntw > 6) run(std::integral_constant<int, 8>{});
  else if (ntw > 4) run(std::integral_constant<int, 6>{});
  else if (ntw > 2) run(std::integral_constant<int, 4>{});
  else if (ntw > 0) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 0>{});

  // epilogue: scales, SiLU(gate) * up, hi/lo planes; padding rows get 0
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
  uint16_t* a_lo = a_hi + p.cap * I;
  float sg[2], su[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = nb + wn * 32 + 16 * j + col;
    sg[j] = p.s13[static_cast<int64_t>(e) * 2 * I + n];
    su[j] = p.s13[static_cast<int64_t>(e) * 2 * I + I + n];
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt < ntw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + wm * 128 + mt * 16 + kg * 4 + i;
        const bool valid = p.sorted_ids[r] < Tk;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float v = valid ? silu_mul(acc[mt][j][i] * sg[j], acc[mt][j + 2][i] * su[j]) : 0.0f;
          const uint32_t hi = pack_bf16_rne(v, 0.0f) & 0xffffu;
          const uint32_t lo = pack_bf16_rne(v - __uint_as_float(hi << 16), 0.0f) & 0xffffu;
          const int64_t o = r * I + nb + wn * 32 + 16 * j + col;
          a_hi[o] = static_cast<uint16_t>(hi);
          a_lo[o] = static_cast<uint16_t>(lo);
        }
      }
    }
  }
}

// GEMM2 for 256-row blocks: y = (hi + lo) dequant(w2[e])^T, scale on the
// accumulator.  A workgroup owns 128 rows (half an align block) and 256
// output columns; 8 waves in a 2 x 4 grid, each 64 rows x 64 columns (4 x 4
// tiles, both planes of a through the MFMA with the same converted weight
// fragment).  Stages of 64 K in the same 3-deep LDS ring: 2 x 16 KB of the
// hi/lo planes and 16 KB of int8 w2 rows per stage.
constexpr int k2Rows = 128;
constexpr int k2Cols = 256;
constexpr int k2AStage = 2 * k2Rows * kARow;          // 32 KB
constexpr int k2BStage = k2Cols * kBRow;              // 16 KB
constexpr int k2StageBytes = k2AStage + k2BStage;
constexpr int k2ADma = k2AStage / (kThreads * 16);
constexpr int k2BDma = k2BStage / (kThreads * 16);

__global__ __launch_bounds__(kThreads) void gemm2_big_kernel(const Gemm2Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * k2StageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * k2Rows;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[row0 / kRows];
  const int64_t Tk = p.Tk, H = p.H, I = p.I;

  int nrows = 0;
  for (int r = 0; r < k2Rows; r += 16)
    if (p.sorted_ids[row0 + r] < Tk) nrows = r + 16;
  if (nrows == 0) return;      // the second half of a block may be empty (uniform exit)
  int ntw = (nrows - wm * 64) / 16;
  ntw = ntw < 0 ? 0 : (ntw > 4 ? 4 : ntw);
  const int nst = static_cast<int>(I / kBK);

  // A copies: (plane, row) pairs q = 0..255, 8 per copy instruction
  const uint16_t* a16 = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* asrc[k2ADma];
#pragma unroll
  for (int i = 0; i < k2ADma; ++i) {
    const int q = wave * (2 * k2Rows / kWaves) + i * 8 + (lane >> 3);
    const int pl = q / k2Rows, r = q % k2Rows;
    const int c = (lane & 7) ^ swz_a(r);
    asrc[i] = a16 + pl * p.cap * I + (row0 + r) * I + c * 8;
  }
  const int64_t hb = static_cast<int64_t>(blockIdx.x) * k2Cols;
  const int8_t* bsrc[k2BDma];
#pragma unroll
  for (int i = 0; i < k2BDma; ++i) {
    const int b = wave * (k2Cols / kWaves) + i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(b);
    bsrc[i] = p.w2 + (static_cast<int64_t>(e) * H + hb + b) * p.ldw + c * 16;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * k2StageBytes;
#pragma unroll
    for (int i = 0; i < k2ADma; ++i)
      dma16(asrc[i] + static_cast<int64_t>(s) * kBK, base + (wave * (2 * k2Rows / kWaves) + i * 8) * kARow);
#pragma unroll
    for (int i = 0; i < k2BDma; ++i)
      dma16(bsrc[i] + static_cast<int64_t>(s) * kBK, base + k2AStage + (wave * (k2Cols / kWaves) + i * 16) * kBRow);
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
    boff[j] = k2AStage + b * kBRow + 16 * (kg ^ swz_b(b));
  }
  int aoff[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int r = wm * 64 + mt * 16 + col;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) aoff[mt][ks] = r * kARow + 16 * ((2 * kg + ks) ^ swz_a(r));
  }

  auto run = [&](auto tiles) {
    constexpr int MT = decltype(tiles)::value;
    issue(0, 0);
    if (nst > 1) issue(1, 1);
    int slot = 0;
    for (int s = 0; s < nst; ++s) {
      if (s + 1 < nst) wait_vmcnt<k2ADma + k2BDma>();
      else wait_vmcnt<0>();
      stage_barrier();
      if (s + 2 < nst) issue(s + 2, slot == 0 ? 2 : slot - 1);
      const uint8_t* st = smem + slot * k2StageBytes;

      u32x4 q[4], ah[MT > 0 ? MT : 1][2], al[MT > 0 ? MT : 1][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = *reinterpret_cast<const u32x4*>(st + boff[j]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          ah[mt][ks] = *reinterpret_cast<const u32x4*>(st + aoff[mt][ks]);
          al[mt][ks] = *reinterpret_cast<const u32x4*>(st + k2Rows * kARow + aoff[mt][ks]);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 b[2];
        i8x16_to_operands<false>(q[j], b[0], b[1]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma16_bf16(ah[mt][ks], b[ks], acc[mt][j]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma16_bf16(al[mt][ks], b[ks], acc[mt][j]);
        }
      }
      slot = slot == kStages - 1 ? 0 : slot + 1;
    }
  };
  if (ntw > 3) run(std::integral_constant<int, 4>{});
  else if (ntw > 2) run(std::integral_constant<int, 3>{});
  else if (ntw > 1) run(std::integral_constant<int, 2>{});
  else if (ntw > 0) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

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
          float* yr = p.y + static_cast<int64_t>(f) * H + hb + wn * 64 + col;
#pragma unroll
          for (int j = 0; j < 4; ++j) yr[16 * j] = acc[mt][j][i] * sc[j];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm2_w8_big(const Gemm2Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.H / k2Cols), static_cast<unsigned>(p.cap / k2Rows));
  hipLaunchKernelGGL(gemm2_big_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm1_w8_big(const Gemm1Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.I / kOut), static_cast<unsigned>(p.cap / kRows));
  if (p.f16)
    hipLaunchKernelGGL((gemm1_big_kernel<true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm1_big_kernel<false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
