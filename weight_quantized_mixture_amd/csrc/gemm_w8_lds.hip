// Weight-streaming grouped GEMM1 with the activation tile staged in LDS
// (align blocks of 32, 64 or 128 rows: the gathered activations are shared by the
// four waves of a workgroup instead of being fetched once per wave).
//
// experts_int8 page, ExpertsInt8MoEMethod.create_weights / apply ->
// fused_experts(use_int8_w8a16): GEMM1 h = x dequant(w13[e])^T (scale on the
// fp32 accumulator), a = silu(h_gate) * h_up written as bf16 hi/lo planes.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 128;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// GEMM1.  Workgroup: one align block (MT 16-row tiles, padding tiles skipped),
// 4 waves = CW column groups x KW K-ways; wave = NG*16 gate + NG*16 up rows.
// One iteration covers KW*128 of K: wave kw takes sub-step kw.  The gathered
// activation rows of the iteration ([16*MT rows][KW*128] bf16) are staged in
// LDS once and read by every wave; double-buffered, one barrier per iteration.
// Lane (col, kg) reads bytes [16kg, 16kg+16) and [64+16kg, 64+16kg+16) of
// its weight row per 128-K step; the activation operand follows the same K
// order (MFMA i uses K offsets 64*(i/2) + 16kg + 8*(i%2) .. +8).
template <int MT, int KW, int NG, bool F16>
__global__ __launch_bounds__(kThreads) void gemm1_lds_kernel(const Gemm1Args p) {
  constexpr int CW = 4 / KW;
  constexpr int KT = KW * kStep;               // K per iteration
  constexpr int PITCH = KT + 8;                // bf16 elements per LDS row (16-byte pad)
  constexpr int ROWS = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][ROWS * PITCH];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int cw = wave % CW;
  const int kw = wave / CW;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * ROWS;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (p.sorted_ids[row0 + mt * 16] < p.Tk) ntiles = mt + 1;
  const int nrows = ntiles * 16;

  const int64_t I = p.I, H = p.H;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * NG * CW) + cw * 16 * NG;
  const int iters = static_cast<int>(H / KT);
  // weight rows of this lane: gate n0 + 16g + col, up I + n0 + 16g + col
  const int8_t* wbase = p.w13 + (static_cast<int64_t>(e) * 2 * I + n0 + col) * p.ldw + kw * kStep + kg * 16;
  const int64_t gstride = 16 * p.ldw;
  const int64_t ustride = I * p.ldw;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);

  // cooperative A loads: chunk c = (row r, 8-element column group q); chunks = nrows * KT/8
  constexpr int QPR = KT / 8;                  // chunks per row
  constexpr int CPT = (ROWS * QPR + kThreads - 1) / kThreads;
  const uint16_t* srcp[CPT];
  int dsto[CPT];
  bool cvalid[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * kThreads;
    const int r = ci / QPR, q = ci % QPR;
    cvalid[c] = r < nrows;
    int f = p.Tk;
    if (cvalid[c]) f = p.sorted_ids[row0 + r];
    const bool real = cvalid[c] && f < p.Tk;
    srcp[c] = real ? x + static_cast<int64_t>(f / p.k) * H + q * 8 : nullptr;
    dsto[c] = r * PITCH + q * 8;
  }
  auto load_a = [&](int it, u32x4* regs) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      regs[c] = srcp[c] ? ld16(srcp[c] + static_cast<int64_t>(it) * KT) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_a = [&](int buf, const u32x4* regs) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (cvalid[c]) *reinterpret_cast<u32x4*>(&As[buf][dsto[c]]) = regs[c];
  };

  // the epilogue's column scales, loaded now so that no workgroup ends with a
  // round trip to memory after its last step
  float sgv[NG], suv[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    sgv[g] = p.s13[static_cast<int64_t>(e) * 2 * I + n0 + 16 * g + col];
    suv[g] = p.s13[static_cast<int64_t>(e) * 2 * I + I + n0 + 16 * g + col];
  }

  f32x4 accg[MT][NG], accu[MT][NG];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      accg[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  u32x4 areg[CPT];
  load_a(0, areg);
  u32x4 wg0[NG], wg1[NG], wu0[NG], wu1[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    wg0[g] = ld16(wbase + g * gstride);
    wg1[g] = ld16(wbase + g * gstride + 64);
    wu0[g] = ld16(wbase + g * gstride + ustride);
    wu1[g] = ld16(wbase + g * gstride + ustride + 64);
  }
  store_a(0, areg);
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < iters;
    if (more) load_a(it + 1, areg);
    const int64_t kn = static_cast<int64_t>(more ? it + 1 : it) * KT;
    u32x4 ng0[NG], ng1[NG], nu0[NG], nu1[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      ng0[g] = ld16(wbase + g * gstride + kn);
      ng1[g] = ld16(wbase + g * gstride + kn + 64);
      nu0[g] = ld16(wbase + g * gstride + ustride + kn);
      nu1[g] = ld16(wbase + g * gstride + ustride + kn + 64);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      u32x4 bg[4], bu[4];
      i8x16_to_operands<F16>(wg0[g], bg[0], bg[1]);
      i8x16_to_operands<F16>(wg1[g], bg[2], bg[3]);
      i8x16_to_operands<F16>(wu0[g], bu[0], bu[1]);
      i8x16_to_operands<F16>(wu1[g], bu[2], bu[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < ntiles) {
          const uint16_t* ap = &As[buf][(mt * 16 + col) * PITCH + kw * kStep + kg * 16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(ap + (i >> 1) * 64 + (i & 1) * 8);
            accg[mt][g] = mfma16<F16>(av, bg[i], accg[mt][g]);
            accu[mt][g] = mfma16<F16>(av, bu[i], accu[mt][g]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      wg0[g] = ng0[g]; wg1[g] = ng1[g]; wu0[g] = nu0[g]; wu1[g] = nu1[g];
    }
    if (more) store_a(buf ^ 1, areg);
    __syncthreads();
  }

  if constexpr (KW > 1) {
    // reuse the A buffers for the K reduction
    f32x4* red = reinterpret_cast<f32x4*>(&As[0][0]);
    static_assert(sizeof(As) >= (KW - 1) * CW * MT * NG * 2 * kWave * sizeof(f32x4) || KW == 1, "LDS");
    if (kw > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          red[((((kw - 1) * CW + cw) * MT + mt) * NG + g) * 2 * kWave + lane] = accg[mt][g];
          red[((((kw - 1) * CW + cw) * MT + mt) * NG + g) * 2 * kWave + kWave + lane] = accu[mt][g];
        }
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int j = 0; j < KW - 1; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          accg[mt][g] += red[(((j * CW + cw) * MT + mt) * NG + g) * 2 * kWave + lane];
          accu[mt][g] += red[(((j * CW + cw) * MT + mt) * NG + g) * 2 * kWave + kWave + lane];
        }
  }

  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
  uint16_t* a_lo = a_hi + p.cap * I;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t n = n0 + 16 * g + col;
    const float sg = sgv[g], su = suv[g];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = row0 + mt * 16 + kg * 4 + i;
          const float v = silu_mul(accg[mt][g][i] * sg, accu[mt][g][i] * su);
          const uint32_t hi = pack_bf16_rne(v, 0.0f) & 0xffffu;
          const uint32_t lo = pack_bf16_rne(v - __uint_as_float(hi << 16), 0.0f) & 0xffffu;
          a_hi[r * I + n] = static_cast<uint16_t>(hi);
          a_lo[r * I + n] = static_cast<uint16_t>(lo);
        }
      }
    }
  }
}

#define G1L(MT, KW, NG, F16)                                                                        \
  hipLaunchKernelGGL((gemm1_lds_kernel<MT, KW, NG, F16>),                                         \
                     dim3(static_cast<unsigned>(p.I / (16 * NG * (4 / KW))),                      \
                          static_cast<unsigned>(p.cap / p.block_m)),                              \
                     dim3(kThreads), 0, stream, p)

template <bool F16>
hipError_t g1l(const Gemm1Args& p, int mt, int kw, int ng, hipStream_t stream) {
  // LDS per workgroup: 2 x 16*MT x (KW*128 + 8) bf16 -> keep (MT, KW) in {(1,1..4), (2,1..2), (4,1), (8,1)}
  if (mt == 8) {
    G1L(8, 1, 1, F16);
    return hipGetLastError();
  }
  if (mt == 4) kw = 1;
  if (mt == 2 && kw > 2) kw = 2;
  if (ng == 2) {
    if (mt == 4) G1L(4, 1, 2, F16);
    else if (mt == 2) { if (kw == 2) G1L(2, 2, 2, F16); else G1L(2, 1, 2, F16); }
    else { if (kw == 4) G1L(1, 4, 2, F16); else if (kw == 2) G1L(1, 2, 2, F16); else G1L(1, 1, 2, F16); }
  } else {
    if (mt == 4) G1L(4, 1, 1, F16);
    else if (mt == 2) { if (kw == 2) G1L(2, 2, 1, F16); else G1L(2, 1, 1, F16); }
    else { if (kw == 4) G1L(1, 4, 1, F16); else if (kw == 2) G1L(1, 2, 1, F16); else G1L(1, 1, 1, F16); }
  }
  return hipGetLastError();
}
#undef G1L

}  // namespace

hipError_t launch_gemm1_w8_lds(const Gemm1Args& p, int kw, int ng, hipStream_t stream) {
  const int mt = p.block_m / 16;
  return p.f16 ? g1l<true>(p, mt, kw, ng, stream) : g1l<false>(p, mt, kw, ng, stream);
}

}  // namespace moe
