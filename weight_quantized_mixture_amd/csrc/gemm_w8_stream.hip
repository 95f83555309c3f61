// Weight-streaming grouped GEMM1 for int8 experts when each align block holds
// 16 or 48 rows (decode-sized batches: the weights dominate the bytes).
//
// experts_int8 page, ExpertsInt8MoEMethod.create_weights / apply ->
// fused_experts(use_int8_w8a16): h = x dequant(w13[e])^T with the scale on
// the fp32 accumulator and a = silu(h_gate) * h_up.
//
// Design for HBM-bound streaming on gfx950:
//   * every lane owns one weight row (the MFMA column l%16) and 32 consecutive
//     K per 128-K step, so a wave reads 16 rows x 128 contiguous bytes: whole
//     cache lines, and each byte of the expert's weights is read once per block;
//   * the next step's weights are requested before the current step is
//     converted and multiplied (one step of register prefetch), and the
//     activation operand is requested first so waiting for it never waits
//     for the prefetch;
//   * M-tiles made only of padding rows are skipped (valid rows come first in
//     a block), so a block of 64 rows costs the MFMAs of its real rows;
//   * the 4 waves of a workgroup split K (KW ways) and/or columns (4/KW);
//     K partial sums are added in a fixed order through LDS, so small batches
//     still fill 256 CUs without atomics.
//   * a is written as two bf16 planes, hi = rne(a) and lo = rne(a - hi)
//     (16 significant bits).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 128;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int MT, int KW, bool F16>
__global__ __launch_bounds__(kThreads) void gemm1_stream_kernel(const Gemm1Args p) {
  constexpr int CW = 4 / KW;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int cw = wave % CW;
  const int kw = wave / CW;
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
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * CW) + cw * 16;
  const int total_steps = static_cast<int>(H / kStep);
  const int sbeg = kw * total_steps / KW;
  const int nsteps = (kw + 1) * total_steps / KW - sbeg;
  const int64_t kbeg = static_cast<int64_t>(sbeg) * kStep;
  const int8_t* wg = p.w13 + (static_cast<int64_t>(e) * 2 * I + n0 + col) * p.ldw + kbeg + kg * 32;
  const int8_t* wu = wg + I * p.ldw;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* xr[MT];
  bool valid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int f = p.sorted_ids[row0 + mt * 16 + col];
    valid[mt] = f < p.Tk;
    xr[mt] = x + (valid[mt] ? f / p.k : 0) * H + kbeg + kg * 32;
  }
  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  u32x4 g0 = ld16(wg), g1 = ld16(wg + 16), u0 = ld16(wu), u1 = ld16(wu + 16);
  for (int s = 0; s < nsteps; ++s) {
    const int64_t ko = static_cast<int64_t>(s) * kStep;
    u32x4 av[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[mt][i] = valid[mt] ? ld16(xr[mt] + ko + 8 * i) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    const int64_t kn = (s + 1 < nsteps) ? ko + kStep : ko;     // the last step re-reads itself
    const u32x4 ng0 = ld16(wg + kn), ng1 = ld16(wg + kn + 16);
    const u32x4 nu0 = ld16(wu + kn), nu1 = ld16(wu + kn + 16);
    u32x4 bg[4], bu[4];
    i8x16_to_operands<F16>(g0, bg[0], bg[1]);
    i8x16_to_operands<F16>(g1, bg[2], bg[3]);
    i8x16_to_operands<F16>(u0, bu[0], bu[1]);
    i8x16_to_operands<F16>(u1, bu[2], bu[3]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[mt] = mfma16<F16>(av[mt][i], bg[i], accg[mt]);
          accu[mt] = mfma16<F16>(av[mt][i], bu[i], accu[mt]);
        }
      }
    }
    g0 = ng0; g1 = ng1; u0 = nu0; u1 = nu1;
  }

  if constexpr (KW > 1) {
    __shared__ f32x4 red[KW - 1][CW][MT][2][kWave];
    if (kw > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        red[kw - 1][cw][mt][0][lane] = accg[mt];
        red[kw - 1][cw][mt][1][lane] = accu[mt];
      }
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int j = 0; j < KW - 1; ++j) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        accg[mt] += red[j][cw][mt][0][lane];
        accu[mt] += red[j][cw][mt][1][lane];
      }
    }
  }

  const float sg = p.s13[static_cast<int64_t>(e) * 2 * I + n0 + col];
  const float su = p.s13[static_cast<int64_t>(e) * 2 * I + I + n0 + col];
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
  uint16_t* a_lo = a_hi + p.cap * I;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + mt * 16 + kg * 4 + i;
        const float v = silu_mul(accg[mt][i] * sg, accu[mt][i] * su);
        const uint32_t hi = pack_bf16_rne(v, 0.0f) & 0xffffu;
        const float hf = __uint_as_float(hi << 16);
        const uint32_t lo = pack_bf16_rne(v - hf, 0.0f) & 0xffffu;
        a_hi[r * I + n0 + col] = static_cast<uint16_t>(hi);
        a_lo[r * I + n0 + col] = static_cast<uint16_t>(lo);
      }
    }
  }
}

template <int MT, bool F16>
hipError_t g1_kw(const Gemm1Args& p, int kw, hipStream_t stream) {
  const unsigned by = static_cast<unsigned>(p.cap / p.block_m);
  switch (kw) {
    case 4:
      hipLaunchKernelGGL((gemm1_stream_kernel<MT, 4, F16>), dim3(static_cast<unsigned>(p.I / 16), by),
                         dim3(kThreads), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((gemm1_stream_kernel<MT, 2, F16>), dim3(static_cast<unsigned>(p.I / 32), by),
                         dim3(kThreads), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((gemm1_stream_kernel<MT, 1, F16>), dim3(static_cast<unsigned>(p.I / 64), by),
                         dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_w8_stream(const Gemm1Args& p, int kw, hipStream_t stream) {
  const int mt = p.block_m / 16;
  if (p.f16) {
    if (mt == 4) return g1_kw<4, true>(p, kw, stream);
    if (mt == 3) return g1_kw<3, true>(p, kw, stream);
    if (mt == 2) return g1_kw<2, true>(p, kw, stream);
    return g1_kw<1, true>(p, kw, stream);
  }
  if (mt == 4) return g1_kw<4, false>(p, kw, stream);
  if (mt == 3) return g1_kw<3, false>(p, kw, stream);
  if (mt == 2) return g1_kw<2, false>(p, kw, stream);
  return g1_kw<1, false>(p, kw, stream);
}

}  // namespace moe
