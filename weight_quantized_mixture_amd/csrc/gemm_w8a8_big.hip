// Grouped int8 x int8 GEMMs of the W8A8 layer for 256-row align blocks
// (prefill-sized expert loads, where the MFMA work dominates), gfx950.
//
// fused_moe oracle/int8 page (per-channel int8 weights, per-token dynamic
// int8 activations) on the experts_int8 page's weights:
//   GEMM1: h = s_x[t] s13[e, n] * sum_c qx[t, c] q13[e, n, c], then
//          a = silu(h_gate) * h_up as fp32 rows of the padded block;
//   GEMM2: y = s_a[r] s2[e, h] * sum_i qa[r, i] q2[e, h, i] for the K part of
//          grid z (partials added by the combine).
// Both are the same int8 GEMM: int32 holds the whole K exactly (|sum| <=
// 127^2 K < 2^31 for K < 2^17), so the scales go on the accumulator once at
// the end and no operand needs decoding.
//
// Tiling: a workgroup owns one align block (256 rows) and 256 B rows (GEMM1:
// 128 gate rows and the matching 128 up rows of w13; GEMM2: 256 output
// columns of w2).  Its 4 waves (one per SIMD) form a 2 x 2 grid; a wave owns
// 128 rows x 128 B rows = 8 x 8 tiles of v_mfma_i32_16x16x64_i8 (256 int32
// accumulators in the AGPR half of the register file), one MFMA per tile
// and 64-wide K stage.  K advances through a 4-slot LDS ring filled with
// buffer_load ... lds (16 KB of A rows and 16 KB of B rows per stage):
//   * a stage's fragments are read into registers during the previous stage
//     (A into the row tile's registers once its MFMAs have them; B into the
//     second of two register sets, the stage loop unrolled by two), so the
//     barrier at the start of stage s only has to make stage s+1 visible;
//   * after that barrier the slot of stage s (already in registers) takes
//     stage s+4: three stages are in flight behind the one multiplied;
//   * the 16-byte chunks of the 64-byte LDS rows are XOR-swizzled by row so
//     that the 16 rows one fragment read touches fall in distinct bank groups;
//   * inside each 64-row group of B rows, LDS row 16 q + r holds source row
//     4 r + q, so tile q (16 consecutive LDS rows) gives lane col the source
//     row 4 col + q: the lane ends with 4 adjacent output columns and writes
//     them as one 16-byte store.
// Lane (col, kg) feeds K [16 kg, 16 kg + 16) of the stage for both operands.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 256;                 // A rows per workgroup (= block_m)
constexpr int kBK = 64;                    // K per stage
constexpr int kRing = 4;
constexpr int kPlane = kRows * kBK;        // 16 KB of A rows; the same of B rows
constexpr int kStageBytes = 2 * kPlane;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kCopies = kPlane / (kThreads * 16);   // 16-byte copies per thread and operand per stage
constexpr int kDma = 2 * kCopies;

// c += a b on v_mfma_i32_16x16x64_i8, accumulating in place: with all 256
// AGPRs holding accumulators, the builtin's untied form left the register
// allocator shuffling accumulators through VGPRs every stage (148 moves per
// 64 MFMAs).  Being asm, these MFMAs are invisible to the compiler's hazard
// tracking: the K loop waits out the MFMA latency (mfma_drain) before
// anything else touches the accumulators.
__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  return c;
}

// 24 wait states, more than an MFMA result or operand needs, with nothing
// scheduled across them
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Where this workgroup's operands come from: buffer resources and, per copy
// of this thread, the byte offset of its 16-byte chunk at K = 0 (offsets past
// the resource range fill zeros and read no memory).
struct Sources {
  __amdgpu_buffer_rsrc_t ar, br;
  uint32_t aoff[kCopies], boff[kCopies];
};

// The K loop over stages [s0, s1) for a wave with MT row tiles (0 to 8) and
// the B groups of its 8 column tiles (tile j reads group bgrp[j >> 2]):
// acc[mt][j] += A(row tile mt) B(column tile j) over the stages.
template <int MT>
__device__ __forceinline__ void k_loop(uint8_t* smem, const Sources& src, int s0, int s1, int wm,
                                       const int (&bgrp)[2], i32x4 (&acc)[8][8]) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15;
  const int kg = lane >> 4;
  constexpr int MT1 = MT > 0 ? MT : 1;

  // copy i of this thread: LDS rows wave * 64 + 16 i + lane / 4, chunk lane % 4
  auto issue = [&](int s, int slot) __attribute__((always_inline)) {
    uint8_t* base = smem + slot * kStageBytes;
    const uint32_t so = static_cast<uint32_t>(s * kBK);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) dma16_buf(src.ar, src.aoff[i], so, base + (wave * 64 + i * 16) * kBK);
#pragma unroll
    for (int i = 0; i < kCopies; ++i)
      dma16_buf(src.br, src.boff[i], so, base + kPlane + (wave * 64 + i * 16) * kBK);
  };
  // fragment offsets: rows col (+ 16 mt, + 128 wm) share the swizzle of col
  const int sw = 16 * (kg ^ swz_b(col));
  const int aoffr = (wm * 128 + col) * kBK + sw;
  int boffr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) boffr[j] = kPlane + (bgrp[j >> 2] * 64 + 16 * (j & 3) + col) * kBK + sw;

  u32x4 af[MT1], bf[8];
  auto read_a = [&](const uint8_t* st, int mt) __attribute__((always_inline)) {
    af[mt] = *reinterpret_cast<const u32x4*>(st + aoffr + mt * 16 * kBK);
  };
  auto read_b = [&](const uint8_t* st, int j) __attribute__((always_inline)) {
    bf[j] = *reinterpret_cast<const u32x4*>(st + boffr[j]);
  };

  // stages s0 .. s0+2 into slots 0 .. 2 (indices past the end repeat the last
  // stage, into slots nobody reads), then stage s0's A and B tiles 0-3
#pragma unroll
  for (int q = 0; q < kRing - 1; ++q) issue(s0 + q < s1 ? s0 + q : s1 - 1, q);
  wait_vmcnt<(kRing - 2) * kDma>();
  stage_barrier();
  if constexpr (MT > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) read_a(smem, mt);
#pragma unroll
    for (int j = 0; j < 4; ++j) read_b(smem, j);
  }

  mfma_drain();   // the accumulators' zero fill lands before the first MFMA reads it

  // stage s: half 0 multiplies column tiles 0-3 and reads stage s's B tiles
  // 4-7, half 1 multiplies tiles 4-7 and, with MORE (stage s+1 follows),
  // refills each row tile's A fragment once its last MFMA has it and B tiles
  // 0-3 from stage s+1.  So slot s is read until half 0 of stage s; after the
  // barrier of stage s it is stage s-1's slot that is free, and this
  // thread's copies of stage s+3 go there, spread over the row-tile slots.
  auto step = [&](int s, auto more_tag) __attribute__((always_inline)) {
    constexpr bool MORE = decltype(more_tag)::value;
    if constexpr (MORE) {
      wait_vmcnt_lgkm0<(kRing - 3) * kDma>();   // stage s+1 landed in every thread
      stage_barrier();                          // ... and every wave is done with slot s-1
    }
    const uint8_t* cur = smem + ((s - s0) % kRing) * kStageBytes;
    const uint8_t* nx = smem + ((s - s0 + 1) % kRing) * kStageBytes;
    const int sc = s + kRing - 1 < s1 ? s + kRing - 1 : s1 - 1;
    uint8_t* base = smem + ((s - s0 + kRing - 1) % kRing) * kStageBytes;
    const uint32_t so = static_cast<uint32_t>(sc * kBK);
    auto copy = [&](int i) __attribute__((always_inline)) {
      if (i < kCopies)
        dma16_buf(src.ar, src.aoff[i], so, base + (wave * 64 + i * 16) * kBK);
      else
        dma16_buf(src.br, src.boff[i - kCopies], so, base + kPlane + (wave * 64 + (i - kCopies) * 16) * kBK);
    };
    if constexpr (MT == 0) {
      if constexpr (MORE) {
#pragma unroll
        for (int i = 0; i < kDma; ++i) copy(i);
      }
    } else {
      constexpr int kSlots = 2 * MT;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int j = 4 * h; j < 4 * h + 4; ++j) acc[mt][j] = mfma_i8(af[mt], bf[j], acc[mt][j]);
          if (h == 0) {
#pragma unroll
            for (int j = 4 + mt * 4 / MT; j < 4 + (mt + 1) * 4 / MT; ++j) read_b(cur, j);
          }
          if constexpr (MORE) {
            const int m = h * MT + mt;
#pragma unroll
            for (int i = m * kDma / kSlots; i < (m + 1) * kDma / kSlots; ++i) copy(i);
            if (h == 1) {
              read_a(nx, mt);
#pragma unroll
              for (int j = mt * 4 / MT; j < (mt + 1) * 4 / MT; ++j) read_b(nx, j);
            }
          }
        }
      }
    }
  };
  for (int s = s0; s + 1 < s1; ++s) step(s, std::true_type{});
  step(s1 - 1, std::false_type{});
  wait_vmcnt<0>();   // no copy into LDS outlives the loop
  mfma_drain();
}

// valid rows come first in a block; count them in 16-row tiles
__device__ __forceinline__ int block_rows(const int32_t* sorted_ids, int64_t row0, int64_t Tk) {
  int nrows = 0;
  for (int r = 0; r < kRows; r += 16)
    if (sorted_ids[row0 + r] < Tk) nrows = r + 16;
  return nrows;
}

template <typename F>
__device__ __forceinline__ void dispatch_tiles(int ntw, F&& f) {
  if (ntw > 6) f(std::integral_constant<int, 8>{});
  else if (ntw > 4) f(std::integral_constant<int, 6>{});
  else if (ntw > 2) f(std::integral_constant<int, 4>{});
  else if (ntw > 0) f(std::integral_constant<int, 2>{});
  else f(std::integral_constant<int, 0>{});
}

// copy offsets of B rows: wave w fills B group w (64 LDS rows); copy i lands
// in LDS rows 16 i + lane / 4 of it, source row 4 (lane / 4) + i of the group
// starting at `grow` (rows of `ld` bytes)
__device__ __forceinline__ void b_offsets(uint32_t (&off)[kCopies], int64_t grow, int64_t ld, int lane) {
  const int c = (lane & 3) ^ swz_b(lane >> 2);
#pragma unroll
  for (int i = 0; i < kCopies; ++i)
    off[i] = static_cast<uint32_t>((grow + 4 * (lane >> 2) + i) * ld + c * 16);
}

__global__ __launch_bounds__(kThreads) void gemm1_w8a8_big_kernel(const Gemm1Args p, const int8_t* __restrict__ qx,
                                                                  const float* __restrict__ sx,
                                                                  float* __restrict__ pmax) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * kRows;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t Tk = p.Tk, H = p.H, I = p.I;
  const int nrows = block_rows(p.sorted_ids, row0, Tk);
  int ntw = (nrows - wm * 128) / 16;
  ntw = ntw < 0 ? 0 : (ntw > 8 ? 8 : ntw);

  // A: the token rows of x's codes (rows without a token read past the end);
  // B: gate rows nb + 64 g for groups g = 0, 1 and up rows I + nb + 64 (g - 2)
  Sources src;
  const uint32_t xbytes = static_cast<uint32_t>(p.T * H);
  src.ar = make_rsrc(qx, xbytes);
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = wave * 64 + i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(r);
    const int f = r < nrows ? p.sorted_ids[row0 + r] : static_cast<int>(Tk);
    src.aoff[i] = f < Tk ? static_cast<uint32_t>(f / static_cast<int>(p.k)) * static_cast<uint32_t>(H) +
                               static_cast<uint32_t>(c * 16)
                         : xbytes;
  }
  const int64_t nb = static_cast<int64_t>(blockIdx.x) * 128;
  src.br = make_rsrc(p.w13 + static_cast<int64_t>(e) * 2 * I * p.ldw, static_cast<uint32_t>(2 * I * p.ldw));
  b_offsets(src.boff, (wave < 2 ? nb + 64 * wave : I + nb + 64 * (wave - 2)), p.ldw, lane);

  i32x4 acc[8][8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mt][j] = i32x4{0, 0, 0, 0};
  // column tiles 0-3: gate group wn; 4-7: the matching up group 2 + wn
  const int bgrp[2] = {wn, 2 + wn};
  const int nst = static_cast<int>(H / kBK);
  dispatch_tiles(ntw, [&](auto tiles) __attribute__((always_inline)) {
    k_loop<decltype(tiles)::value>(smem, src, 0, nst, wm, bgrp, acc);
  });

  // epilogue: lane col holds output columns n0 .. n0 + 3 (gate in tiles 0-3,
  // up in 4-7) of rows 4 kg .. 4 kg + 3 of each row tile.  The row's max |a|
  // over these 64 columns (the 16 lanes of the row) goes to its partial
  // maxima pmax[r, 2 blockIdx.x + wn] (I / 64 per row), which the quantizer
  // of a reduces instead of making a first pass over the row.
  const int64_t n0 = nb + wn * 64 + 4 * col;
  float sg[4], su[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    sg[q] = p.s13[static_cast<int64_t>(e) * 2 * I + n0 + q];
    su[q] = p.s13[static_cast<int64_t>(e) * 2 * I + I + n0 + q];
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt < ntw) {
      const i32x4 ids = *reinterpret_cast<const i32x4*>(p.sorted_ids + row0 + wm * 128 + mt * 16 + kg * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + wm * 128 + mt * 16 + kg * 4 + i;
        float m = 0.0f;      // rows without a token: 0, never stored
        if (ids[i] < Tk) {
          const float st = sx[ids[i] / static_cast<int>(p.k)];
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] = silu_mul(static_cast<float>(acc[mt][q][i]) * st * sg[q],
                            static_cast<float>(acc[mt][q + 4][i]) * st * su[q]);
            m = fmaxf(m, fabsf(v[q]));
          }
          *reinterpret_cast<f32x4*>(p.a + r * I + n0) = v;
        }
        // every lane takes part in the shuffles over the row's 16 lanes
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
        if (col == 0 && ids[i] < Tk) pmax[r * (I / 64) + 2 * blockIdx.x + wn] = m;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void gemm2_w8a8_big_kernel(const Gemm2Args p, const int8_t* __restrict__ qa,
                                                                  const float* __restrict__ sa) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int z = static_cast<int>(blockIdx.z);
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * kRows;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t Tk = p.Tk, H = p.H, I = p.I;
  const int nrows = block_rows(p.sorted_ids, row0, Tk);
  int ntw = (nrows - wm * 128) / 16;
  ntw = ntw < 0 ? 0 : (ntw > 8 ? 8 : ntw);
  // this part's stages
  const int nst = static_cast<int>(I / kBK);
  const int s0 = z * nst / p.splits, s1 = (z + 1) * nst / p.splits;

  // A: the block's rows of a's codes that hold tokens (the others fill
  // zeros); B: output columns hb + 64 g of w2 for group g = wave
  Sources src;
  src.ar = make_rsrc(qa + row0 * I, static_cast<uint32_t>(nrows * I));
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = wave * 64 + i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(r);
    src.aoff[i] = static_cast<uint32_t>(r * I + c * 16);
  }
  const int64_t hb = static_cast<int64_t>(blockIdx.x) * 256;
  src.br = make_rsrc(p.w2 + static_cast<int64_t>(e) * H * p.ldw, static_cast<uint32_t>(H * p.ldw));
  b_offsets(src.boff, hb + 64 * wave, p.ldw, lane);

  i32x4 acc[8][8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mt][j] = i32x4{0, 0, 0, 0};
  // column tiles 0-3: group 2 wn; 4-7: group 2 wn + 1
  const int bgrp[2] = {2 * wn, 2 * wn + 1};
  dispatch_tiles(ntw, [&](auto tiles) __attribute__((always_inline)) {
    k_loop<decltype(tiles)::value>(smem, src, s0, s1, wm, bgrp, acc);
  });

  // epilogue: lane col holds output columns hb + 64 g + 4 col .. + 3 of
  // group g = 2 wn + (j >> 2)
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    sc[j] = p.s2[static_cast<int64_t>(e) * H + hb + 64 * (2 * wn + (j >> 2)) + 4 * col + (j & 3)];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt < ntw) {
      const i32x4 ids = *reinterpret_cast<const i32x4*>(p.sorted_ids + row0 + wm * 128 + mt * 16 + kg * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (ids[i] < Tk) {
          const int64_t r = row0 + wm * 128 + mt * 16 + kg * 4 + i;
          const float sr = sa[r];
          float* yr = p.y + (static_cast<int64_t>(z) * Tk + ids[i]) * H + hb + 128 * wn + 4 * col;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = static_cast<float>(acc[mt][4 * g + q][i]) * sr * sc[4 * g + q];
            *reinterpret_cast<f32x4*>(yr + 64 * g) = v;
          }
        }
      }
    }
  }
}

}  // namespace

bool w8a8_big_fits(int64_t T, int64_t H, int64_t I, int64_t bm) {
  return bm == kRows && H % 256 == 0 && I % 128 == 0 && T * H < (int64_t{1} << 32) &&
         2 * I * H < (int64_t{1} << 32) && kRows * I < (int64_t{1} << 31);
}

hipError_t launch_gemm1_w8a8_big(const Gemm1Args& p, const int8_t* qx, const float* sx, float* pmax,
                                 hipStream_t stream) {
  if (!w8a8_big_fits(p.T, p.H, p.I, p.block_m) || p.cap % kRows || p.ldw % 16 || 2 * p.I * p.ldw >= (int64_t{1} << 32))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.I / 128), static_cast<unsigned>(p.cap / kRows));
  hipLaunchKernelGGL(gemm1_w8a8_big_kernel, grid, dim3(kThreads), 0, stream, p, qx, sx, pmax);
  return hipGetLastError();
}

hipError_t launch_gemm2_w8a8_big(const Gemm2Args& p, const int8_t* qa, const float* sa, hipStream_t stream) {
  if (p.H % 256 || p.I % kBK || p.block_m != kRows || p.cap % kRows || p.ldw % 16 || p.splits < 1 ||
      p.splits > p.I / kBK || kRows * p.I >= (int64_t{1} << 31) || p.H * p.ldw >= (int64_t{1} << 32))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.H / 256), static_cast<unsigned>(p.cap / kRows),
                  static_cast<unsigned>(p.splits));
  hipLaunchKernelGGL(gemm2_w8a8_big_kernel, grid, dim3(kThreads), 0, stream, p, qa, sa);
  return hipGetLastError();
}

}  // namespace moe
