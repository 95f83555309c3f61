// W8A8 GEMMs for align blocks of 16 or 32 rows (decode-sized batches), fed
// by direct global -> LDS copies, gfx950.
//
// fused_moe oracle/int8 page, select_int8_moe_backend: per-channel static
// int8 weights and per-token dynamic int8 activations (the weights are the
// experts_int8 page's).  The products are those of gemm1_w8a8_kernel and
// gemm2_w8a8_kernel, exact in int32 (|sum| <= 127^2 K), so these kernels give
// the same results:
//   GEMM1: h = s_x[t] s13[e, n] sum_c qx[t, c] q13[e, n, c], a = silu(h_gate)
//     h_up as fp32 rows of the padded block, plus the row's max |a| over the
//     workgroup's 64 columns (partial maxima [cap, I/64]), so the quantizer of
//     a makes a single pass;
//   GEMM2: y = s_a[r] s2[e, h] sum_i qa[r, i] q2[e, h, i] over one part of K.
//
// A workgroup is one align block (MT 16-row tiles, padding tiles skipped) and
// 4 waves of 32 weight rows (GEMM1: 16 gate + the matching 16 up rows; GEMM2:
// 32 output columns).  K advances in steps of 128 through a 3-deep LDS ring:
// per step each wave copies its 32 weight rows (4 KB) and 2 MT waves copy 8
// activation rows each (128 bytes per row).  Waits count each wave's own
// copies; one barrier per step.  Lane (col, kg) feeds K [16 kg, 16 kg + 16)
// and [64 + 16 kg, 64 + 16 kg + 16) of the step to the two MFMAs, for the
// weight row col and the activation row col of each tile.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStep = 128;
constexpr int kRing = 3;
constexpr int kWRows = 32;
constexpr int kWWave = kWRows * kStep;              // 4 KB per wave and step
constexpr int kWStage = 4 * kWWave;                 // 16 KB
constexpr int kWDma = kWWave / (kWave * 16);        // 4 copies per lane and step

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

template <int MT>
struct A8Ring {
  static constexpr int kAStage = 16 * MT * kStep;            // the block's activation rows
  static constexpr int kAWaves = kAStage / 1024;             // waves with one activation copy (2 MT)
  static constexpr int kStage = kWStage + kAStage;
};

// Waits until at most `ahead` later steps of this wave's copies are in flight
// (per = copies per step of this wave: kWDma, plus one for an activation wave).
template <int PER>
__device__ __forceinline__ void wait_steps(int ahead) {
  if (ahead >= kRing - 2) wait_vmcnt<(kRing - 2) * PER>();
  else wait_vmcnt<0>();
}

// The ring walk shared by both GEMMs: issue(s, slot) requests step s into a
// slot, body(slot_base) multiplies a step.
template <int MT, typename Issue, typename Body>
__device__ __forceinline__ void ring_walk(uint8_t* smem, int nst, bool a_wave, Issue issue, Body body) {
  using R = A8Ring<MT>;
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j)
    if (j < nst) issue(j, j);
  int slot = 0;
  for (int s = 0; s < nst; ++s) {
    const int ahead = nst - 1 - s;
    if (a_wave) wait_steps<kWDma + 1>(ahead);
    else wait_steps<kWDma>(ahead);
    stage_barrier();
    if (s + kRing - 1 < nst) issue(s + kRing - 1, slot == 0 ? kRing - 1 : slot - 1);
    body(smem + slot * R::kStage);
    slot = slot == kRing - 1 ? 0 : slot + 1;
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm1_w8a8_dma_kernel(const Gemm1Args p, const int8_t* __restrict__ qx,
                                                                  const float* __restrict__ sx, float* __restrict__ pmax) {
  using R = A8Ring<MT>;
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

  // weight copies: row r = 8 i + lane/8 of the wave's 32 (gate rows n0.., then
  // up rows I + n0..), LDS slot lane%8 holds chunk (lane%8) ^ swz_a(r)
  const int8_t* wsrc[kWDma];
#pragma unroll
  for (int i = 0; i < kWDma; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    const int64_t n = r < 16 ? n0 + r : I + n0 + (r - 16);
    wsrc[i] = p.w13 + (static_cast<int64_t>(e) * 2 * I + n) * p.ldw + c * 16;
  }
  // activation copies (waves below 2 MT): rows 8 wave + lane/8 of the block,
  // the codes of their token's x row (rows without a token read token 0's)
  const bool a_wave = wave < R::kAWaves;
  const int8_t* asrc;
  {
    const int r = a_wave ? 8 * wave + (lane >> 3) : 0;
    const int c = (lane & 7) ^ swz_a(r);
    const int f = p.sorted_ids[row0 + r];
    const int64_t t = f < Tk ? f / static_cast<int>(p.k) : 0;
    asrc = qx + t * H + c * 16;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * R::kStage;
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      dma16(wsrc[i] + static_cast<int64_t>(s) * kStep, base + wave * kWWave + i * 1024);
    if (a_wave) dma16(asrc + static_cast<int64_t>(s) * kStep, base + kWStage + wave * 1024);
  };

  int woff[4];
  {
    const int rg = col, ru = 16 + col;
    woff[0] = wave * kWWave + rg * kStep + 16 * (kg ^ swz_a(rg));
    woff[1] = wave * kWWave + rg * kStep + 16 * ((4 + kg) ^ swz_a(rg));
    woff[2] = wave * kWWave + ru * kStep + 16 * (kg ^ swz_a(ru));
    woff[3] = wave * kWWave + ru * kStep + 16 * ((4 + kg) ^ swz_a(ru));
  }
  int aoff[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = 16 * mt + col;
    aoff[mt][0] = kWStage + r * kStep + 16 * (kg ^ swz_a(r));
    aoff[mt][1] = kWStage + r * kStep + 16 * ((4 + kg) ^ swz_a(r));
  }

  // the epilogue's inputs besides the sums (the column's two scales, the
  // rows' token ids and activation scales), loaded now so that no workgroup
  // ends with a chain of memory round trips after its last step
  const int64_t n = n0 + col;
  const float sg = p.s13[static_cast<int64_t>(e) * 2 * I + n];
  const float su = p.s13[static_cast<int64_t>(e) * 2 * I + I + n];
  int rowf[MT][4];
  float rows_sx[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = mt < ntiles ? p.sorted_ids[row0 + mt * 16 + kg * 4 + i] : static_cast<int>(Tk);
      rowf[mt][i] = f;
      rows_sx[mt][i] = f < Tk ? sx[f / p.k] : 0.0f;
    }

  i32x4 accg[MT], accu[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    accg[mt] = i32x4{0, 0, 0, 0};
    accu[mt] = i32x4{0, 0, 0, 0};
  }
  auto run = [&](auto tiles) {
    constexpr int NTL = decltype(tiles)::value;
    ring_walk<MT>(smem, nst, a_wave, issue, [&](const uint8_t* st) {
      const u32x4 g0 = *reinterpret_cast<const u32x4*>(st + woff[0]);
      const u32x4 g1 = *reinterpret_cast<const u32x4*>(st + woff[1]);
      const u32x4 u0 = *reinterpret_cast<const u32x4*>(st + woff[2]);
      const u32x4 u1 = *reinterpret_cast<const u32x4*>(st + woff[3]);
#pragma unroll
      for (int mt = 0; mt < NTL; ++mt) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(st + aoff[mt][0]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(st + aoff[mt][1]);
        accg[mt] = mfma_i8(a0, g0, accg[mt]);
        accg[mt] = mfma_i8(a1, g1, accg[mt]);
        accu[mt] = mfma_i8(a0, u0, accu[mt]);
        accu[mt] = mfma_i8(a1, u1, accu[mt]);
      }
    });
  };
  if constexpr (MT == 2) {
    if (ntiles > 1) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }

  float m[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = row0 + mt * 16 + kg * 4 + i;
      const int f = rowf[mt][i];
      float v = 0.0f;
      if (f < Tk) {
        const float st = rows_sx[mt][i];
        v = silu_mul(static_cast<float>(accg[mt][i]) * st * sg, static_cast<float>(accu[mt][i]) * st * su);
        p.a[r * I + n] = v;
      }
      float x = fabsf(v);
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) x = fmaxf(x, __shfl_xor(x, d, kWave));   // the wave's 16 columns
      m[mt][i] = x;
    }
  // row maxima over the workgroup's 64 columns: the 4 waves through LDS
  float* red = reinterpret_cast<float*>(smem);   // [4 waves][16 MT rows]
  __syncthreads();                               // every wave is done with the ring
  if (col == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * 16 * MT + mt * 16 + kg * 4 + i] = m[mt][i];
  }
  __syncthreads();
  if (wave == 0 && col == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = mt * 16 + kg * 4 + i;
          const float gm = fmaxf(fmaxf(red[rl], red[16 * MT + rl]), fmaxf(red[32 * MT + rl], red[48 * MT + rl]));
          pmax[(row0 + rl) * (I / 64) + blockIdx.x] = gm;
        }
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm2_w8a8_dma_kernel(const Gemm2Args p, const int8_t* __restrict__ qa,
                                                                  const float* __restrict__ sa) {
  using R = A8Ring<MT>;
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

  const int64_t I = p.I, H = p.H;
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * (4 * kWRows) + wave * kWRows;
  const int total = static_cast<int>(I / kStep);
  const int ib = static_cast<int>(blockIdx.z) * total / p.splits;
  const int iters = (static_cast<int>(blockIdx.z) + 1) * total / p.splits - ib;

  const int8_t* wsrc[kWDma];
#pragma unroll
  for (int i = 0; i < kWDma; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    wsrc[i] = p.w2 + (static_cast<int64_t>(e) * H + h0 + r) * p.ldw + static_cast<int64_t>(ib) * kStep + c * 16;
  }
  const bool a_wave = wave < R::kAWaves;
  const int8_t* asrc;
  {
    const int r = a_wave ? 8 * wave + (lane >> 3) : 0;
    const int c = (lane & 7) ^ swz_a(r);
    asrc = qa + (row0 + r) * I + static_cast<int64_t>(ib) * kStep + c * 16;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * R::kStage;
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      dma16(wsrc[i] + static_cast<int64_t>(s) * kStep, base + wave * kWWave + i * 1024);
    if (a_wave) dma16(asrc + static_cast<int64_t>(s) * kStep, base + kWStage + wave * 1024);
  };

  int woff[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
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

  // the epilogue's column scales, row ids and row scales, loaded now so that no
  // workgroup ends with a chain of memory round trips after its last step
  const float s0 = p.s2[static_cast<int64_t>(e) * H + h0 + col];
  const float s1 = p.s2[static_cast<int64_t>(e) * H + h0 + 16 + col];
  int rowf[MT][4];
  float rows_sa[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = row0 + mt * 16 + kg * 4 + i;
      const int f = p.sorted_ids[r];
      rowf[mt][i] = f;
      rows_sa[mt][i] = f < p.Tk ? sa[r] : 0.0f;
    }

  i32x4 acc0[MT], acc1[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc0[mt] = i32x4{0, 0, 0, 0};
    acc1[mt] = i32x4{0, 0, 0, 0};
  }
  auto run = [&](auto tiles) {
    constexpr int NTL = decltype(tiles)::value;
    ring_walk<MT>(smem, iters, a_wave, issue, [&](const uint8_t* st) {
      const u32x4 b00 = *reinterpret_cast<const u32x4*>(st + woff[0][0]);
      const u32x4 b01 = *reinterpret_cast<const u32x4*>(st + woff[0][1]);
      const u32x4 b10 = *reinterpret_cast<const u32x4*>(st + woff[1][0]);
      const u32x4 b11 = *reinterpret_cast<const u32x4*>(st + woff[1][1]);
#pragma unroll
      for (int mt = 0; mt < NTL; ++mt) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(st + aoff[mt][0]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(st + aoff[mt][1]);
        acc0[mt] = mfma_i8(a0, b00, acc0[mt]);
        acc0[mt] = mfma_i8(a1, b01, acc0[mt]);
        acc1[mt] = mfma_i8(a0, b10, acc1[mt]);
        acc1[mt] = mfma_i8(a1, b11, acc1[mt]);
      }
    });
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
          const float sr = rows_sa[mt][i];
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
          yr[0] = static_cast<float>(acc0[mt][i]) * sr * s0;
          yr[16] = static_cast<float>(acc1[mt][i]) * sr * s1;
        }
      }
    }
  }
}

}  // namespace

bool w8a8_dma_fits(int64_t H, int64_t I, int64_t block_m) {
  return (block_m == 16 || block_m == 32) && H % kStep == 0 && I % kStep == 0 && H % (4 * kWRows) == 0;
}

hipError_t launch_gemm1_w8a8_dma(const Gemm1Args& p, const int8_t* qx, const float* sx, float* pmax,
                                 hipStream_t stream) {
  if (!w8a8_dma_fits(p.H, p.I, p.block_m) || p.ldw % 16 != 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m));
  if (p.block_m == 16)
    hipLaunchKernelGGL((gemm1_w8a8_dma_kernel<1>), grid, dim3(kThreads), 0, stream, p, qx, sx, pmax);
  else
    hipLaunchKernelGGL((gemm1_w8a8_dma_kernel<2>), grid, dim3(kThreads), 0, stream, p, qx, sx, pmax);
  return hipGetLastError();
}

hipError_t launch_gemm2_w8a8_dma(const Gemm2Args& p, const int8_t* qa, const float* sa, hipStream_t stream) {
  if (!w8a8_dma_fits(p.H, p.I, p.block_m) || p.ldw % 16 != 0 || p.splits < 1 || p.splits > p.I / kStep)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.H / (4 * kWRows)), static_cast<unsigned>(p.cap / p.block_m),
                  static_cast<unsigned>(p.splits));
  if (p.block_m == 16)
    hipLaunchKernelGGL((gemm2_w8a8_dma_kernel<1>), grid, dim3(kThreads), 0, stream, p, qa, sa);
  else
    hipLaunchKernelGGL((gemm2_w8a8_dma_kernel<2>), grid, dim3(kThreads), 0, stream, p, qa, sa);
  return hipGetLastError();
}

}  // namespace moe
