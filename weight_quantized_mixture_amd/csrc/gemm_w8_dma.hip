// Weight-streaming GEMM1 for int8 experts with align blocks of 16 or 32 rows
// (decode-sized batches: the weight bytes dominate), fed by direct
// global -> LDS copies, gfx950.
//
// experts_int8 page, ExpertsInt8MoEMethod.create_weights / apply ->
// fused_experts(use_int8_w8a16): h = x dequant(w13[e])^T with the per-row
// scale on the fp32 accumulator, a = silu(h_gate) * h_up, written either as
// 16-bit fixed point for the integer GEMM2 (the workgroup's 64 columns are
// one scale group: a ~= s (256 hi + lo), s = max |a over the 64| / 32639,
// the waves exchanging their row maxima through LDS), or as bf16 hi/lo planes
// (hi = rne(a), lo = rne(a - hi)) for the 16-bit GEMM2.
//
// A workgroup is one align block (MT 16-row tiles) and 64 output columns;
// each of its 4 waves owns 16 gate rows and the matching 16 up rows of w13.
// K advances in steps of 128 through a 3-deep LDS ring filled with
// global_load_lds_dwordx4: per step every wave copies its own 32 weight rows
// (4 KB) and the workgroup copies the block's activation rows (the gathered
// bf16 rows, 256 bytes each).  Step s+2 is requested while step s is
// converted (int8 or e4m3fn -> bf16/fp16, exact) and multiplied, so the HBM requests
// of a wave never wait for its own arithmetic, and nothing passes through
// registers on the way to LDS.  One barrier per step, after each thread has
// waited for its own copies of that step.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 128;                       // K per step
constexpr int kRing = 3;
constexpr int kWRowsWave = 32;                   // 16 gate + 16 up rows per wave
constexpr int kWWave = kWRowsWave * kStep;       // 4 KB of weights per wave and step
constexpr int kWStage = 4 * kWWave;              // 16 KB
constexpr int kWDma = kWWave / (kWave * 16);     // 4 copies per lane and step

template <int MT>
struct DecodeRing {
  static constexpr int kARow = kStep * 2;                    // bf16 bytes per activation row
  static constexpr int kAStage = 16 * MT * kARow;
  static constexpr int kStage = kWStage + kAStage;
  static constexpr int kADma = kAStage / (kThreads * 16);   // = MT
};

// FP8: w13 holds e4m3fn codes with one scale per expert (fp8 page, weight-only path).
template <int MT, bool F16, bool FP8>
__global__ __launch_bounds__(kThreads) void gemm1_dma_kernel(const Gemm1Args p, int8_t* __restrict__ qhi,
                                                             int8_t* __restrict__ qlo, float* __restrict__ qscale) {
  using R = DecodeRing<MT>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * R::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t Tk = p.Tk, H = p.H, I = p.I;
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (p.sorted_ids[row0 + mt * 16] < Tk) ntiles = mt + 1;
  const int nst = static_cast<int>(H / kStep);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16;

  // weight copies of this lane: row r = 8 i + lane/8 of the wave's 32 rows,
  // LDS slot lane%8 holds chunk (lane%8) ^ swz_a(r)
  const int8_t* wsrc[kWDma];
#pragma unroll
  for (int i = 0; i < kWDma; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    const int64_t n = r < 16 ? n0 + r : I + n0 + (r - 16);
    wsrc[i] = p.w13 + (static_cast<int64_t>(e) * 2 * I + n) * p.ldw + c * 16;
  }
  // activation copies: row r = 4 (wave MT + q) + lane/16, slot lane%16 holds
  // chunk (lane%16) ^ swz_c(r); rows without a token read token 0's row
  // (their results are dropped)
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* asrc[R::kADma];
#pragma unroll
  for (int q = 0; q < R::kADma; ++q) {
    const int r = 4 * (wave * R::kADma + q) + (lane >> 4);
    const int c = (lane & 15) ^ swz_c(r);
    const int f = p.sorted_ids[row0 + r];
    const int64_t t = f < Tk ? f / static_cast<int>(p.k) : 0;
    asrc[q] = x + t * H + c * 8;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * R::kStage;
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      dma16(wsrc[i] + static_cast<int64_t>(s) * kStep, base + wave * kWWave + i * 1024);
#pragma unroll
    for (int q = 0; q < R::kADma; ++q)
      dma16(asrc[q] + static_cast<int64_t>(s) * kStep, base + kWStage + (wave * R::kADma + q) * 1024);
  };

  // LDS offsets this lane reads: weight chunks kg and 4 + kg of its gate row
  // (col) and up row (16 + col); activation chunks 2 kg + 8 (i/2) + i%2 of
  // row 16 mt + col (K offsets 16 kg + 64 (i/2) + 8 (i%2), as the weights)
  int woff[4];
  {
    const int rg = col, ru = 16 + col;
    woff[0] = wave * kWWave + rg * kStep + 16 * (kg ^ swz_a(rg));
    woff[1] = wave * kWWave + rg * kStep + 16 * ((4 + kg) ^ swz_a(rg));
    woff[2] = wave * kWWave + ru * kStep + 16 * (kg ^ swz_a(ru));
    woff[3] = wave * kWWave + ru * kStep + 16 * ((4 + kg) ^ swz_a(ru));
  }
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = kWStage + col * R::kARow + 16 * ((2 * kg + 8 * (i >> 1) + (i & 1)) ^ swz_c(col));

  // what the epilogue reads besides the sums (the column's two scales, which
  // of the lane's rows hold a token) is loaded now, so that no workgroup ends
  // with a round trip to memory after its last step
  const int64_t n = n0 + col;
  const float sg = FP8 ? p.s13[e] : p.s13[static_cast<int64_t>(e) * 2 * I + n];
  const float su = FP8 ? p.s13[e] : p.s13[static_cast<int64_t>(e) * 2 * I + I + n];
  uint32_t rvalid = 0;                               // bit 4 mt + i: row 16 mt + 4 kg + i holds a token
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p.sorted_ids[row0 + mt * 16 + kg * 4 + i] < Tk) rvalid |= 1u << (4 * mt + i);

  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto run = [&](auto tiles) {
    constexpr int NT = decltype(tiles)::value;
    issue(0, 0);
    if (nst > 1) issue(1, 1);
    int slot = 0;
    for (int s = 0; s < nst; ++s) {
      if (s + 1 < nst) wait_vmcnt<kWDma + R::kADma>();
      else wait_vmcnt<0>();
      stage_barrier();
      if (s + 2 < nst) issue(s + 2, slot == 0 ? 2 : slot - 1);
      const uint8_t* st = smem + slot * R::kStage;
      u32x4 bg[4], bu[4];
      w8_operands<F16, FP8>(*reinterpret_cast<const u32x4*>(st + woff[0]), bg[0], bg[1]);
      w8_operands<F16, FP8>(*reinterpret_cast<const u32x4*>(st + woff[1]), bg[2], bg[3]);
      w8_operands<F16, FP8>(*reinterpret_cast<const u32x4*>(st + woff[2]), bu[0], bu[1]);
      w8_operands<F16, FP8>(*reinterpret_cast<const u32x4*>(st + woff[3]), bu[2], bu[3]);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(st + aoff[i] + mt * 16 * R::kARow);
          accg[mt] = mfma16<F16>(av, bg[i], accg[mt]);
          accu[mt] = mfma16<F16>(av, bu[i], accu[mt]);
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

  float v[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[mt][i] = mt < ntiles && ((rvalid >> (4 * mt + i)) & 1u) ? silu_mul(accg[mt][i] * sg, accu[mt][i] * su)
                                                                 : 0.0f;
  if (qhi) {
    // row maxima over the wave's 16 columns (the 16 lanes of one kg), then over the 4 waves
    constexpr int kQMax = 32639;                 // 256 * 127 + 127
    float* red = reinterpret_cast<float*>(smem);  // [4 waves][16 MT rows]
    float m[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = fabsf(v[mt][i]);
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) x = fmaxf(x, __shfl_xor(x, d, kWave));
        m[mt][i] = x;
      }
    __syncthreads();                              // every wave is done with the ring
    if (col == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave * 16 * MT + mt * 16 + kg * 4 + i] = m[mt][i];
    }
    __syncthreads();
    const int64_t G = I / 64;
    // the codes go through an LDS tile [hi, lo][16 MT rows][64 columns] (ring
    // memory past slot 0, free by now) and out in 16-byte pieces, 64
    // contiguous bytes per row and plane: single-byte stores from every lane
    // cost more than the arithmetic of the whole epilogue
    int8_t* qt = reinterpret_cast<int8_t*>(smem + R::kStage);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = mt * 16 + kg * 4 + i;
          const float gm = fmaxf(fmaxf(red[rl], red[16 * MT + rl]), fmaxf(red[32 * MT + rl], red[48 * MT + rl]));
          const float inv = gm > 0.0f ? static_cast<float>(kQMax) / gm : 0.0f;
          int q = static_cast<int>(__builtin_rintf(v[mt][i] * inv));
          q = q < -kQMax ? -kQMax : (q > kQMax ? kQMax : q);
          const int h = (q + 128) >> 8;
          qt[rl * 64 + wave * 16 + col] = static_cast<int8_t>(h);
          qt[(16 * MT + rl) * 64 + wave * 16 + col] = static_cast<int8_t>(q - 256 * h);
          if (wave == 0 && col == 0) qscale[(row0 + rl) * G + blockIdx.x] = gm / static_cast<float>(kQMax);
        }
      }
    }
    __syncthreads();
    {
      constexpr int kChunks = 2 * 16 * MT * 4;     // (plane, row, 16-byte piece)
      const int pl = tid / (16 * MT * 4), rl = (tid / 4) % (16 * MT), c = tid % 4;
      if (tid < kChunks && rl < 16 * ntiles) {
        const u32x4 q16 = *reinterpret_cast<const u32x4*>(qt + (pl * 16 * MT + rl) * 64 + c * 16);
        *reinterpret_cast<u32x4*>((pl ? qlo : qhi) + (row0 + rl) * I + static_cast<int64_t>(blockIdx.x) * 64 + c * 16) =
            q16;
      }
    }
    return;
  }
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
  uint16_t* a_lo = a_hi + p.cap * I;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + mt * 16 + kg * 4 + i;
        const uint32_t hi = pack_bf16_rne(v[mt][i], 0.0f) & 0xffffu;
        const uint32_t lo = pack_bf16_rne(v[mt][i] - __uint_as_float(hi << 16), 0.0f) & 0xffffu;
        a_hi[r * I + n] = static_cast<uint16_t>(hi);
        a_lo[r * I + n] = static_cast<uint16_t>(lo);
      }
    }
  }
}

template <int MT>
hipError_t dma_launch(const Gemm1Args& p, int8_t* qhi, int8_t* qlo, float* qscale, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m));
  if (p.fp8) {
    if (p.f16)
      hipLaunchKernelGGL((gemm1_dma_kernel<MT, true, true>), grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
    else
      hipLaunchKernelGGL((gemm1_dma_kernel<MT, false, true>), grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
  } else {
    if (p.f16)
      hipLaunchKernelGGL((gemm1_dma_kernel<MT, true, false>), grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
    else
      hipLaunchKernelGGL((gemm1_dma_kernel<MT, false, false>), grid, dim3(kThreads), 0, stream, p, qhi, qlo, qscale);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_w8_dma(const Gemm1Args& p, int8_t* qhi, int8_t* qlo, float* qscale, hipStream_t stream) {
  if (p.I % 64 || p.H % kStep || (p.block_m != 16 && p.block_m != 32)) return hipErrorInvalidValue;
  return p.block_m == 16 ? dma_launch<1>(p, qhi, qlo, qscale, stream) : dma_launch<2>(p, qhi, qlo, qscale, stream);
}

}  // namespace moe
