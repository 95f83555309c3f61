// Weight-streaming GEMM2 for align blocks of 16 or 32 rows (decode-sized
// batches), fed by direct global -> LDS copies, gfx950: int8 experts
// (gemm2_q16_dma_kernel) and weight-only fp8 experts (gemm2_fp8_dma_kernel).
//
// experts_int8 page, ExpertsInt8MoEMethod.apply -> fused_experts
// (use_int8_w8a16): y = a dequant(w2[e])^T with the per-row scale of w2 on
// the fp32 accumulator.  The intermediate a arrives in the 16-bit fixed-point
// form the 16/32-row GEMM1 writes (a ~= s (256 hi + lo), one scale per row
// and group of 64 columns); the int8 codes of w2 and of both planes go to
// v_mfma_i32_16x16x64_i8 as they are, and each half step folds
// s (256 hi_acc + lo_acc) into the fp32 accumulator: the same products, sums
// and order as gemm2_q16_kernel, so the two give identical results.
//
// A workgroup is one align block (MT 16-row tiles, tiles made of padding
// skipped), 4 waves side by side in N with 32 output columns each, and one
// part of K (grid z).  K advances in steps of 128 through a 3-deep LDS ring
// filled with global_load_lds: per step every wave copies its own 32 rows of
// w2 (4 KB), and the workgroup copies the block's rows of both planes (16-byte
// chunks) and their 2 scales per row (4-byte copies).  Step s+2 is requested
// while step s is multiplied; the waits count copies (every lane issues the
// same number per step), so no load result passes through registers and
// nothing waits for a load issued after the one it needs.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStep = 128;                          // K per step (two scale groups of 64)
constexpr int kNT = 2;                              // 16-column tiles per wave
constexpr int kRing = 3;
constexpr int kWRows = 16 * kNT;                    // w2 rows per wave
constexpr int kWWave = kWRows * kStep;              // 4 KB per wave and step
constexpr int kWStage = 4 * kWWave;                 // 16 KB
constexpr int kWDma = kWWave / (kWave * 16);        // 4 copies per lane and step

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// 4 bytes from global memory to LDS; lane l of the wave lands at lds + 4 l.
__device__ __forceinline__ void dma4(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)const_cast<void*>(src), (lds_ptr_t)lds_wave_base, 4, 0, 0);
}

template <int MT>
struct Q16Ring {
  static constexpr int kAStage = 2 * 16 * MT * kStep;          // both planes of the block's rows
  static constexpr int kADma = kAStage / (kThreads * 16);      // = MT
  static constexpr int kSStage = kThreads * 4;                 // one 4-byte copy per lane (32 MT used)
  static constexpr int kStage = kWStage + kAStage + kSStage;
  static constexpr int kPer = kWDma + kADma + 1;               // copies per lane and step
};

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm2_q16_dma_kernel(const Gemm2Args p, const int8_t* __restrict__ qhi,
                                                                 const int8_t* __restrict__ qlo,
                                                                 const float* __restrict__ qscale) {
  using R = Q16Ring<MT>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * R::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (p.sorted_ids[row0 + mt * 16] < p.Tk) ntiles = mt + 1;

  const int64_t I = p.I, H = p.H, G = I / 64;
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * (4 * kWRows) + wave * kWRows;
  const int total = static_cast<int>(I / kStep);
  const int ib = static_cast<int>(blockIdx.z) * total / p.splits;
  const int iters = (static_cast<int>(blockIdx.z) + 1) * total / p.splits - ib;

  // w2 copies of this lane: row r = 8 i + lane/8 of the wave's 32, LDS slot
  // lane%8 holds chunk (lane%8) ^ swz_a(r)
  const int8_t* wsrc[kWDma];
#pragma unroll
  for (int i = 0; i < kWDma; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    wsrc[i] = p.w2 + (static_cast<int64_t>(e) * H + h0 + r) * p.ldw + static_cast<int64_t>(ib) * kStep + c * 16;
  }
  // plane copies: 8-row group g = wave + 4 q (plane g / (2 MT), rows
  // 8 (g % 2MT) + lane/8), chunks swizzled like the weights
  const int8_t* asrc[R::kADma];
#pragma unroll
  for (int q = 0; q < R::kADma; ++q) {
    const int g = wave + 4 * q;
    const int r = 8 * (g % (2 * MT)) + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    asrc[q] = (g < 2 * MT ? qhi : qlo) + (row0 + r) * I + static_cast<int64_t>(ib) * kStep + c * 16;
  }
  // scale copies: element x = 64 wave + lane is (row x/2, half x%2) for
  // x < 32 MT; the other lanes repeat element 0 into unused LDS
  const int sx = 64 * wave + lane;
  const float* ssrc = qscale + (row0 + (sx < 32 * MT ? sx >> 1 : 0)) * G + static_cast<int64_t>(ib) * 2 +
                      (sx < 32 * MT ? (sx & 1) : 0);
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * R::kStage;
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      dma16(wsrc[i] + static_cast<int64_t>(s) * kStep, base + wave * kWWave + i * 1024);
#pragma unroll
    for (int q = 0; q < R::kADma; ++q)
      dma16(asrc[q] + static_cast<int64_t>(s) * kStep, base + kWStage + (wave + 4 * q) * 1024);
    dma4(ssrc + 2 * s, base + kWStage + R::kAStage + wave * 256);
  };

  // LDS offsets this lane reads: chunks kg and 4 + kg (K 16 kg and
  // 64 + 16 kg) of w2 row 16 j + col, and of plane rows 16 mt + col
  int woff[kNT][2];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int r = 16 * j + col;
    woff[j][0] = wave * kWWave + r * kStep + 16 * (kg ^ swz_a(r));
    woff[j][1] = wave * kWWave + r * kStep + 16 * ((4 + kg) ^ swz_a(r));
  }
  int aoff[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = 16 * mt + col;
    aoff[mt][0] = kWStage + r * kStep + 16 * (kg ^ swz_a(r));
    aoff[mt][1] = kWStage + r * kStep + 16 * ((4 + kg) ^ swz_a(r));
  }
  constexpr int kLoPlane = 16 * MT * kStep;          // lo plane rows follow the hi rows

  // the epilogue's row ids and column scales, loaded now so that no workgroup
  // ends with a round trip to memory after its last step
  int rowf[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rowf[mt][i] = p.sorted_ids[row0 + mt * 16 + kg * 4 + i];
  float csc[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) csc[j] = p.s2[static_cast<int64_t>(e) * H + h0 + 16 * j + col];

  f32x4 acc[MT][kNT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](auto tiles) {
    constexpr int NTL = decltype(tiles)::value;
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j)
      if (j < iters) issue(j, j);
    int slot = 0;
    for (int s = 0; s < iters; ++s) {
      // steps s+1 .. min(s+kRing-2, iters-1) may stay in flight
      if (s + 1 < iters) wait_vmcnt<R::kPer>();
      else wait_vmcnt<0>();
      stage_barrier();
      // the slot of step s-1, which every wave has finished reading
      if (s + kRing - 1 < iters) issue(s + kRing - 1, slot == 0 ? kRing - 1 : slot - 1);
      const uint8_t* st = smem + slot * R::kStage;
      u32x4 b0[kNT], b1[kNT];
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        b0[j] = *reinterpret_cast<const u32x4*>(st + woff[j][0]);
        b1[j] = *reinterpret_cast<const u32x4*>(st + woff[j][1]);
      }
#pragma unroll
      for (int mt = 0; mt < NTL; ++mt) {
        const u32x4 ah0 = *reinterpret_cast<const u32x4*>(st + aoff[mt][0]);
        const u32x4 ah1 = *reinterpret_cast<const u32x4*>(st + aoff[mt][1]);
        const u32x4 al0 = *reinterpret_cast<const u32x4*>(st + kLoPlane + aoff[mt][0]);
        const u32x4 al1 = *reinterpret_cast<const u32x4*>(st + kLoPlane + aoff[mt][1]);
        // scales (row, half) of rows 4 kg + i: [2 i], [2 i + 1]
        const float* sr = reinterpret_cast<const float*>(st + kWStage + R::kAStage) + (16 * mt + 4 * kg) * 2;
        const f32x4 sa = *reinterpret_cast<const f32x4*>(sr);
        const f32x4 sb = *reinterpret_cast<const f32x4*>(sr + 4);
        const float s0[4] = {sa.x, sa.z, sb.x, sb.z}, s1[4] = {sa.y, sa.w, sb.y, sb.w};
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const i32x4 z = {0, 0, 0, 0};
          const i32x4 ih0 = mfma_i8(ah0, b0[j], z), ih1 = mfma_i8(ah1, b1[j], z);
          const i32x4 il0 = mfma_i8(al0, b0[j], z), il1 = mfma_i8(al1, b1[j], z);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[mt][j][i] += s0[i] * static_cast<float>(ih0[i] * 256 + il0[i]) +
                             s1[i] * static_cast<float>(ih1[i] * 256 + il1[i]);
        }
      }
      slot = slot == kRing - 1 ? 0 : slot + 1;
    }
  };
  if constexpr (MT == 2) {
    if (ntiles > 1) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = rowf[mt][i];
        if (f < p.Tk) {
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
#pragma unroll
          for (int j = 0; j < kNT; ++j) yr[16 * j] = acc[mt][j][i] * csc[j];
        }
      }
    }
  }
}

// fp8 page, Fp8MoEMethod (weight-only path): y = a dequant(w2[e])^T with one
// fp32 scale per expert.  The intermediate comes from the 16/32-row GEMM1 as
// two bf16 planes (hi = rne(a), lo = rne(a - hi)); the e4m3fn codes decode
// exactly into bf16 operands (two per conversion instruction) and both planes
// accumulate into one fp32 accumulator, scaled once at the end.
//
// Same workgroup shape as the int8 kernel (one block, 4 waves x 32 columns,
// one K part), with K steps of 64 through a 4-deep ring: per step every wave
// copies its 32 code rows (64 bytes each, 2 KB) and the workgroup both planes
// of the block's rows (128 bytes per row and plane).  Lane (col, kg) takes
// K [16 kg, 16 kg + 16) of the step: one 16-byte chunk of codes (two MFMA
// operands of 8) against chunks 2 kg and 2 kg + 1 of each plane row.
constexpr int kFStep = 64;                          // K per step
constexpr int kFRing = 4;
constexpr int kFWWave = kWRows * kFStep;            // 2 KB of codes per wave and step
constexpr int kFWStage = 4 * kFWWave;               // 8 KB
constexpr int kFWDma = kFWWave / (kWave * 16);      // 2 copies per lane and step

template <int MT>
struct PlaneRing {
  static constexpr int kARow = kFStep * 2;                     // bf16 bytes per row, plane and step
  static constexpr int kAStage = 2 * 16 * MT * kARow;          // both planes of the block's rows
  static constexpr int kADma = kAStage / (kThreads * 16);      // = MT
  static constexpr int kStage = kFWStage + kAStage;
  static constexpr int kPer = kFWDma + kADma;                  // copies per lane and step
};

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm2_fp8_dma_kernel(const Gemm2Args p) {
  using R = PlaneRing<MT>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kFRing * R::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (p.sorted_ids[row0 + mt * 16] < p.Tk) ntiles = mt + 1;

  const int64_t I = p.I, H = p.H;
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * (4 * kWRows) + wave * kWRows;
  const int total = static_cast<int>(I / kFStep);
  const int ib = static_cast<int>(blockIdx.z) * total / p.splits;
  const int iters = (static_cast<int>(blockIdx.z) + 1) * total / p.splits - ib;

  // code copies: row r = 16 i + lane/4 of the wave's 32, LDS slot lane%4
  // holds chunk (lane%4) ^ swz_b(r)
  const int8_t* wsrc[kFWDma];
#pragma unroll
  for (int i = 0; i < kFWDma; ++i) {
    const int r = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(r);
    wsrc[i] = p.w2 + (static_cast<int64_t>(e) * H + h0 + r) * p.ldw + static_cast<int64_t>(ib) * kFStep + c * 16;
  }
  // plane copies: 8-row group g = wave + 4 q (plane g / (2 MT), rows
  // 8 (g % 2MT) + lane/8), chunk (lane%8) ^ swz_a(row)
  const uint16_t* a_hi = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* a_lo = a_hi + p.cap * I;
  const uint16_t* asrc[R::kADma];
#pragma unroll
  for (int q = 0; q < R::kADma; ++q) {
    const int g = wave + 4 * q;
    const int r = 8 * (g % (2 * MT)) + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    asrc[q] = (g < 2 * MT ? a_hi : a_lo) + (row0 + r) * I + static_cast<int64_t>(ib) * kFStep + c * 8;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * R::kStage;
#pragma unroll
    for (int i = 0; i < kFWDma; ++i)
      dma16(wsrc[i] + static_cast<int64_t>(s) * kFStep, base + wave * kFWWave + i * 1024);
#pragma unroll
    for (int q = 0; q < R::kADma; ++q)
      dma16(asrc[q] + static_cast<int64_t>(s) * kFStep, base + kFWStage + (wave + 4 * q) * 1024);
  };

  int woff[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int r = 16 * j + col;
    woff[j] = wave * kFWWave + r * kFStep + 16 * (kg ^ swz_b(r));
  }
  int aoff[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = 16 * mt + col;
    aoff[mt][0] = kFWStage + r * R::kARow + 16 * ((2 * kg) ^ swz_a(r));
    aoff[mt][1] = kFWStage + r * R::kARow + 16 * ((2 * kg + 1) ^ swz_a(r));
  }
  constexpr int kLoPlane = 16 * MT * R::kARow;

  // the epilogue's row ids, loaded now so that no workgroup ends with a round
  // trip to memory after its last step
  int rowf[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rowf[mt][i] = p.sorted_ids[row0 + mt * 16 + kg * 4 + i];
  const float sw = p.s2[e];

  f32x4 acc[MT][kNT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](auto tiles) {
    constexpr int NTL = decltype(tiles)::value;
#pragma unroll
    for (int j = 0; j < kFRing - 1; ++j)
      if (j < iters) issue(j, j);
    int slot = 0;
    for (int s = 0; s < iters; ++s) {
      // steps s+1 .. min(s+kFRing-2, iters-1) may stay in flight
      const int ahead = iters - 1 - s;
      if (ahead >= kFRing - 2) wait_vmcnt<(kFRing - 2) * R::kPer>();
      else if (ahead == 1) wait_vmcnt<R::kPer>();
      else wait_vmcnt<0>();
      stage_barrier();
      if (s + kFRing - 1 < iters) issue(s + kFRing - 1, slot == 0 ? kFRing - 1 : slot - 1);
      const uint8_t* st = smem + slot * R::kStage;
      u32x4 b0[kNT], b1[kNT];
#pragma unroll
      for (int j = 0; j < kNT; ++j)
        fp8x16_to_operands<false>(*reinterpret_cast<const u32x4*>(st + woff[j]), b0[j], b1[j]);
#pragma unroll
      for (int mt = 0; mt < NTL; ++mt) {
        const u32x4 ah0 = *reinterpret_cast<const u32x4*>(st + aoff[mt][0]);
        const u32x4 ah1 = *reinterpret_cast<const u32x4*>(st + aoff[mt][1]);
        const u32x4 al0 = *reinterpret_cast<const u32x4*>(st + kLoPlane + aoff[mt][0]);
        const u32x4 al1 = *reinterpret_cast<const u32x4*>(st + kLoPlane + aoff[mt][1]);
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          acc[mt][j] = mfma16_bf16(ah0, b0[j], acc[mt][j]);
          acc[mt][j] = mfma16_bf16(al0, b0[j], acc[mt][j]);
          acc[mt][j] = mfma16_bf16(ah1, b1[j], acc[mt][j]);
          acc[mt][j] = mfma16_bf16(al1, b1[j], acc[mt][j]);
        }
      }
      slot = slot == kFRing - 1 ? 0 : slot + 1;
    }
  };
  if constexpr (MT == 2) {
    if (ntiles > 1) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = rowf[mt][i];
        if (f < p.Tk) {
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
#pragma unroll
          for (int j = 0; j < kNT; ++j) yr[16 * j] = acc[mt][j][i] * sw;
        }
      }
    }
  }
}

}  // namespace

bool gemm2_fp8_dma_fits(int64_t H, int64_t I, int64_t block_m) {
  return (block_m == 16 || block_m == 32) && H % (4 * kWRows) == 0 && I % kFStep == 0;
}

hipError_t launch_gemm2_fp8_dma(const Gemm2Args& p, hipStream_t stream) {
  if (!gemm2_fp8_dma_fits(p.H, p.I, p.block_m) || p.ldw % 16 != 0 || p.splits < 1 || p.splits > p.I / kFStep)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.H / (4 * kWRows)), static_cast<unsigned>(p.cap / p.block_m),
                  static_cast<unsigned>(p.splits));
  if (p.block_m == 16)
    hipLaunchKernelGGL((gemm2_fp8_dma_kernel<1>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm2_fp8_dma_kernel<2>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

bool gemm2_q16_dma_fits(int64_t H, int64_t I, int64_t block_m, int64_t ldw) {
  return (block_m == 16 || block_m == 32) && H % (4 * kWRows) == 0 && I % kStep == 0 && ldw % 16 == 0;
}

hipError_t launch_gemm2_q16_dma(const Gemm2Args& p, const int8_t* qhi, const int8_t* qlo, const float* qscale,
                                hipStream_t stream) {
  if (!gemm2_q16_dma_fits(p.H, p.I, p.block_m, p.ldw) || p.splits < 1 || p.splits > p.I / kStep)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.H / (4 * kWRows)), static_cast<unsigned>(p.cap / p.block_m),
                  static_cast<unsigned>(p.splits));
  if (p.block_m == 16)
    hipLaunchKernelGGL((gemm2_q16_dma_kernel<1>), grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
  else
    hipLaunchKernelGGL((gemm2_q16_dma_kernel<2>), grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
  return hipGetLastError();
}

}  // namespace moe
