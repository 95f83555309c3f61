// Grouped expert GEMMs with int8 weights (W8A16), gfx950.
//
// experts_int8 page, ExpertsInt8MoEMethod.apply -> fused_experts with
// use_int8_w8a16: the expert weights are int8 with one fp32 scale per output
// channel (create_weights: w13 [E, 2I, H], w2 [E, H, I]).  Here:
//   GEMM1: h = x * dequant(w13[e])^T, with the scale applied to the fp32
//          accumulator, then a = silu(h_gate) * h_up in the epilogue
//          (gate rows 0..I-1 and up rows I..2I-1 of w13, quantizing_weight_loader);
//   GEMM2: y = a * dequant(w2[e])^T, scale on the accumulator.
//
// Tiling for blocks of more than 64 rows (wave64, v_mfma_f32_16x16x32_{bf16,f16}):
//   * a workgroup is 4 waves and one align block of block_m rows, walked in
//     chunks of 16*MT rows; every lane of a wave owns one weight row (MFMA
//     column l%16) and a 32-byte slice of K (l/16), so one wave reads 16 rows x
//     128 contiguous bytes of int8 per K step: whole cache lines, coalesced;
//   * int8 codes (or e4m3fn codes of the weight-only fp8 experts, fp8 page,
//     Fp8MoEMethod: one scale per expert) become bf16/fp16 in registers
//     (exact), the activation rows
//     are gathered through sorted_ids straight into MFMA A operands;
//   * the K order inside a step is permuted identically for A and B, which
//     leaves the dot products unchanged;
//   * GEMM1: each wave owns 16 gate rows and the matching 16 up rows, so the
//     SiLU-and-mul epilogue needs no data exchange;
//   * GEMM1 writes a as two bf16 planes, hi = rne(a) and lo = rne(a - hi)
//     (16 significant bits); GEMM2 feeds both halves through the MFMA with
//     the same dequantized weights;
//     K is cut into `splits` ranges (grid z) whose partial sums the combine
//     kernel adds in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kKStep = 128;

template <int MT, bool F16, bool FP8>
__global__ __launch_bounds__(kGemmThreads) void gemm1_w8_kernel(const Gemm1Args p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * p.block_m;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16;   // first gate row of the wave
  const int64_t I = p.I, H = p.H;

  const int8_t* wg = p.w13 + (static_cast<int64_t>(e) * 2 * I + n0 + col) * p.ldw + kg * 32;
  const int8_t* wu = wg + I * p.ldw;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const float sg = FP8 ? p.s13[e] : p.s13[static_cast<int64_t>(e) * 2 * I + n0 + col];
  const float su = FP8 ? p.s13[e] : p.s13[static_cast<int64_t>(e) * 2 * I + I + n0 + col];

  for (int rc = 0; rc < p.block_m; rc += 16 * MT) {
    const uint16_t* xr[MT];
    bool valid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int f = p.sorted_ids[row0 + rc + mt * 16 + col];
      valid[mt] = f < p.Tk;
      const int64_t t = valid[mt] ? f / p.k : 0;
      xr[mt] = x + t * H + kg * 32;
    }
    f32x4 accg[MT], accu[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t k0 = 0; k0 < H; k0 += kKStep) {
      const u32x4 g0 = *reinterpret_cast<const u32x4*>(wg + k0);
      const u32x4 g1 = *reinterpret_cast<const u32x4*>(wg + k0 + 16);
      const u32x4 u0 = *reinterpret_cast<const u32x4*>(wu + k0);
      const u32x4 u1 = *reinterpret_cast<const u32x4*>(wu + k0 + 16);
      u32x4 bg[4], bu[4];
      w8_operands<F16, FP8>(g0, bg[0], bg[1]);
      w8_operands<F16, FP8>(g1, bg[2], bg[3]);
      w8_operands<F16, FP8>(u0, bu[0], bu[1]);
      w8_operands<F16, FP8>(u1, bu[2], bu[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        u32x4 av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = valid[mt] ? *reinterpret_cast<const u32x4*>(xr[mt] + k0 + 8 * i)
                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[mt] = mfma16<F16>(av[i], bg[i], accg[mt]);
          accu[mt] = mfma16<F16>(av[i], bu[i], accu[mt]);
        }
      }
    }
    uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
    uint16_t* a_lo = a_hi + p.cap * I;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + rc + mt * 16 + kg * 4 + i;
        const float v = silu_mul(accg[mt][i] * sg, accu[mt][i] * su);
        const uint32_t hi = pack_bf16_rne(v, 0.0f) & 0xffffu;
        const uint32_t lo = pack_bf16_rne(v - __uint_as_float(hi << 16), 0.0f) & 0xffffu;
        a_hi[r * I + n0 + col] = static_cast<uint16_t>(hi);
        a_lo[r * I + n0 + col] = static_cast<uint16_t>(lo);
      }
    }
  }
}

template <int MT, bool FP8>
__global__ __launch_bounds__(kGemmThreads) void gemm2_w8_kernel(const Gemm2Args p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * p.block_m;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32;   // first output column of the wave
  const int64_t I = p.I, H = p.H;
  const int64_t kc = I / p.splits;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * kc;

  const int8_t* w0 = p.w2 + (static_cast<int64_t>(e) * H + h0 + col) * p.ldw + kbeg + kg * 32;
  const int8_t* w1 = w0 + 16 * p.ldw;
  const float s0 = FP8 ? p.s2[e] : p.s2[static_cast<int64_t>(e) * H + h0 + col];
  const float s1 = FP8 ? p.s2[e] : p.s2[static_cast<int64_t>(e) * H + h0 + 16 + col];

  const uint16_t* a_hi = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* a_lo = a_hi + p.cap * I;
  for (int rc = 0; rc < p.block_m; rc += 16 * MT) {
    int64_t ar[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ar[mt] = (row0 + rc + mt * 16 + col) * I + kbeg + kg * 32;
    f32x4 acc0[MT], acc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t k0 = 0; k0 < kc; k0 += kKStep) {
      const u32x4 q00 = *reinterpret_cast<const u32x4*>(w0 + k0);
      const u32x4 q01 = *reinterpret_cast<const u32x4*>(w0 + k0 + 16);
      const u32x4 q10 = *reinterpret_cast<const u32x4*>(w1 + k0);
      const u32x4 q11 = *reinterpret_cast<const u32x4*>(w1 + k0 + 16);
      u32x4 b0[4], b1[4];
      w8_operands<false, FP8>(q00, b0[0], b0[1]);
      w8_operands<false, FP8>(q01, b0[2], b0[3]);
      w8_operands<false, FP8>(q10, b1[0], b1[1]);
      w8_operands<false, FP8>(q11, b1[2], b1[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 ahi = *reinterpret_cast<const u32x4*>(a_hi + ar[mt] + k0 + 8 * i);
          const u32x4 alo = *reinterpret_cast<const u32x4*>(a_lo + ar[mt] + k0 + 8 * i);
          acc0[mt] = mfma16_bf16(ahi, b0[i], acc0[mt]);
          acc0[mt] = mfma16_bf16(alo, b0[i], acc0[mt]);
          acc1[mt] = mfma16_bf16(ahi, b1[i], acc1[mt]);
          acc1[mt] = mfma16_bf16(alo, b1[i], acc1[mt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + rc + mt * 16 + kg * 4 + i;
        const int f = p.sorted_ids[r];
        if (f < p.Tk) {
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
          yr[0] = acc0[mt][i] * s0;
          yr[16] = acc1[mt][i] * s1;
        }
      }
    }
  }
}

template <int MT, bool FP8>
hipError_t gemm1_dispatch_dtype(const Gemm1Args& p, dim3 grid, hipStream_t stream) {
  if (p.f16)
    hipLaunchKernelGGL((gemm1_w8_kernel<MT, true, FP8>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm1_w8_kernel<MT, false, FP8>), grid, dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

template <int MT>
hipError_t gemm1_dispatch_fmt(const Gemm1Args& p, dim3 grid, hipStream_t stream) {
  return p.fp8 ? gemm1_dispatch_dtype<MT, true>(p, grid, stream) : gemm1_dispatch_dtype<MT, false>(p, grid, stream);
}

template <int MT>
void gemm2_dispatch_fmt(const Gemm2Args& p, dim3 grid, hipStream_t stream) {
  if (p.fp8)
    hipLaunchKernelGGL((gemm2_w8_kernel<MT, true>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm2_w8_kernel<MT, false>), grid, dim3(kGemmThreads), 0, stream, p);
}

}  // namespace

hipError_t launch_gemm1_w8(const Gemm1Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m));
  if (p.block_m % 64 == 0) return gemm1_dispatch_fmt<4>(p, grid, stream);
  if (p.block_m % 32 == 0) return gemm1_dispatch_fmt<2>(p, grid, stream);
  return gemm1_dispatch_fmt<1>(p, grid, stream);
}

hipError_t launch_gemm2_w8(const Gemm2Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.H / 128), static_cast<unsigned>(p.cap / p.block_m),
                  static_cast<unsigned>(p.splits));
  if (p.block_m % 64 == 0) gemm2_dispatch_fmt<4>(p, grid, stream);
  else if (p.block_m % 32 == 0) gemm2_dispatch_fmt<2>(p, grid, stream);
  else gemm2_dispatch_fmt<1>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
