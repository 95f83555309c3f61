// Grouped int8-weight GEMMs for large align blocks (prefill-sized batches,
// where the bf16 MFMA work dominates), gfx950.
//
// experts_int8 page, ExpertsInt8MoEMethod.create_weights / apply ->
// fused_experts(use_int8_w8a16): GEMM1 h = x dequant(w13[e])^T with the
// scale on the fp32 accumulator and a = silu(h_gate) * h_up (written as bf16
// hi/lo planes); GEMM2 y = (hi + lo) dequant(w2[e])^T.
//
// Tiling: a workgroup owns one align block of 256 rows and 64 output columns
// (GEMM1: 64 gate rows + the matching 64 up rows of w13; GEMM2: 128 rows of
// w2).  Its 4 waves form a 2 x 2 grid; a wave owns 128 rows x 4 16-column
// tiles, i.e. 8 x 4 accumulators of v_mfma_f32_16x16x32.  Per K stage:
//   * the gathered activation rows of the block are copied into LDS once
//     (double-buffered, one barrier per stage) and read by the two waves that
//     share those rows;
//   * each wave loads its own weight bytes from HBM straight into registers
//     (one or two stages ahead) and converts int8 -> bf16/fp16 there; the
//     conversion is paid once per 128 rows of MFMA work;
//   * 16-row groups made only of padding rows are skipped (valid rows come
//     first in a block).
// Per K stage a wave issues 8 x 4 x (BK/32) MFMAs (twice that in GEMM2, for
// the hi and lo halves) against 128 x BK bf16 of LDS reads.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 256;          // rows per workgroup (= block_m)
constexpr int kWaveRows = 128;
constexpr int kMT = kWaveRows / 16; // 16-row tiles per wave
constexpr int kNT = 4;              // 16-column tiles per wave

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// 8 int8 codes -> one 8-wide 16-bit MFMA operand.
template <bool F16>
__device__ __forceinline__ u32x4 i8x8_operand(u32x2 w) {
  u32x2 a, b;
  if constexpr (F16) {
    a = i8x4_to_f16x4(w.x);
    b = i8x4_to_f16x4(w.y);
  } else {
    a = i8x4_to_bf16x4(w.x);
    b = i8x4_to_bf16x4(w.y);
  }
  return u32x4{a.x, a.y, b.x, b.y};
}

// ROLE 1: GEMM1 (A = gathered activations, B = 2 gate + 2 up tiles, SiLU epilogue).
// ROLE 2: GEMM2 (A = hi/lo planes of a, B = 4 consecutive w2 tiles).
template <int ROLE, int BK, int PF, bool F16>
__global__ __launch_bounds__(kThreads, 2) void gemm_prefill_kernel(const Gemm1Args p1, const Gemm2Args p2) {
  constexpr int NPLANE = ROLE == 1 ? 1 : 2;
  constexpr int PITCH = BK + 8;                      // 16-bit elements per LDS row
  constexpr int QPR = BK / 8;                        // 16-byte chunks per row
  constexpr int CPT = kRows * QPR / kThreads;        // chunks per thread per plane
  constexpr int KS = BK / 32;                        // MFMA K steps per stage
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NPLANE][kRows * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15;
  const int kg = lane >> 4;

  const int32_t* sorted_ids = ROLE == 1 ? p1.sorted_ids : p2.sorted_ids;
  const int32_t* npad_ptr = ROLE == 1 ? p1.num_padded : p2.num_padded;
  const int64_t Tk = ROLE == 1 ? p1.Tk : p2.Tk;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * kRows;
  if (row0 >= *npad_ptr) return;
  const int e = (ROLE == 1 ? p1.block_expert : p2.block_expert)[blockIdx.y];

  // valid rows of the block (a multiple of 16 is enough: padding rows are zero)
  int nrows = 0;
  for (int r = 0; r < kRows; r += 16)
    if (sorted_ids[row0 + r] < Tk) nrows = r + 16;
  const int wrows = nrows - wm * kWaveRows;          // rows of this wave's half
  const int ntiles = wrows <= 0 ? 0 : (wrows >= kWaveRows ? kMT : wrows / 16);

  const int64_t H = ROLE == 1 ? p1.H : p2.H;
  const int64_t I = ROLE == 1 ? p1.I : p2.I;
  const int64_t K = ROLE == 1 ? H : I;
  const int64_t ldw = ROLE == 1 ? p1.ldw : p2.ldw;
  const int nstages = static_cast<int>(K / BK);

  // this lane's 4 weight rows
  const int8_t* wrow[kNT];
  if constexpr (ROLE == 1) {
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wn * 32;
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int64_t n = (j < 2 ? 0 : I) + n0 + (j & 1) * 16 + col;
      wrow[j] = p1.w13 + (static_cast<int64_t>(e) * 2 * I + n) * ldw;
    }
  } else {
    const int64_t h0 = static_cast<int64_t>(blockIdx.x) * 128 + wn * 64;
#pragma unroll
    for (int j = 0; j < kNT; ++j) wrow[j] = p2.w2 + (static_cast<int64_t>(e) * H + h0 + 16 * j + col) * ldw;
  }
  // per-lane K offset inside a stage: KS * 8 bytes at kg * KS * 8
  const int kl = kg * KS * 8;

  // cooperative A copy: chunk c of this thread = (row r, 16-byte column q)
  int64_t src[CPT];
  int dst[CPT];
  bool cv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * kThreads;
    const int r = ci / QPR, q = ci % QPR;
    dst[c] = r * PITCH + q * 8;
    cv[c] = r < nrows;
    if constexpr (ROLE == 1) {
      const int f = cv[c] ? sorted_ids[row0 + r] : static_cast<int>(Tk);
      src[c] = f < Tk ? (static_cast<int64_t>(f) / p1.k) * H + q * 8 : -1;
    } else {
      src[c] = (row0 + r) * I + q * 8;
    }
  }
  const uint16_t* xa = ROLE == 1 ? static_cast<const uint16_t*>(p1.x) : reinterpret_cast<const uint16_t*>(p2.a);
  const int64_t plane = ROLE == 1 ? 0 : p2.cap * I;

  auto load_a = [&](int s, u32x4 (&regs)[NPLANE][CPT]) {
    const int64_t ko = static_cast<int64_t>(s) * BK;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int pl = 0; pl < NPLANE; ++pl) {
        if (ROLE == 1)
          regs[pl][c] = (cv[c] && src[c] >= 0) ? ld16(xa + src[c] + ko) : u32x4{0u, 0u, 0u, 0u};
        else
          regs[pl][c] = cv[c] ? ld16(xa + pl * plane + src[c] + ko) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_a = [&](int buf, const u32x4 (&regs)[NPLANE][CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (cv[c]) {
#pragma unroll
        for (int pl = 0; pl < NPLANE; ++pl) *reinterpret_cast<u32x4*>(&As[buf][pl][dst[c]]) = regs[pl][c];
      }
  };
  auto load_b = [&](int s, u32x2 (&w)[kNT][KS / 2 + (KS == 1)], u32x4 (&w4)[kNT]) {
    const int64_t ko = static_cast<int64_t>(s) * BK + kl;
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      if constexpr (KS == 2) w4[j] = ld16(wrow[j] + ko);
      else w[j][0] = ld8(wrow[j] + ko);
    }
  };

  f32x4 acc[kMT][kNT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weights: PF stages in flight ahead of the one being multiplied
  u32x4 areg[NPLANE][CPT];
  u32x2 bw0[kNT][KS / 2 + (KS == 1)], bw1[kNT][KS / 2 + (KS == 1)];
  u32x4 bq0[kNT], bq1[kNT];
  load_a(0, areg);
  load_b(0, bw0, bq0);
  if constexpr (PF == 2) load_b(nstages > 1 ? 1 : 0, bw1, bq1);
  store_a(0, areg);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nstages;
    if (more) load_a(s + 1, areg);
    u32x2 bw2[kNT][KS / 2 + (KS == 1)];
    u32x4 bq2[kNT];
    if constexpr (PF == 2) load_b(s + 2 < nstages ? s + 2 : nstages - 1, bw2, bq2);
    else load_b(more ? s + 1 : s, bw1, bq1);

    // convert the four weight tiles once, then read each activation fragment
    // once and feed it to the four MFMAs that use it
    u32x4 b[kNT][KS];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      if constexpr (KS == 2) {
        if constexpr (ROLE == 1) i8x16_to_operands<F16>(bq0[j], b[j][0], b[j][1]);
        else i8x16_to_operands<false>(bq0[j], b[j][0], b[j][1]);
      } else {
        b[j][0] = i8x8_operand<ROLE == 1 && F16>(bw0[j][0]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt < ntiles) {
        const int o = (wm * kWaveRows + mt * 16 + col) * PITCH + kl;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(&As[buf][0][o + ks * 8]);
          if constexpr (ROLE == 1) {
#pragma unroll
            for (int j = 0; j < kNT; ++j) acc[mt][j] = mfma16<F16>(a0, b[j][ks], acc[mt][j]);
          } else {
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(&As[buf][NPLANE - 1][o + ks * 8]);
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
              acc[mt][j] = mfma16_bf16(a0, b[j][ks], acc[mt][j]);
              acc[mt][j] = mfma16_bf16(a1, b[j][ks], acc[mt][j]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      bq0[j] = bq1[j];
      if constexpr (PF == 2) bq1[j] = bq2[j];
#pragma unroll
      for (int q = 0; q < KS / 2 + (KS == 1); ++q) {
        bw0[j][q] = bw1[j][q];
        if constexpr (PF == 2) bw1[j][q] = bw2[j][q];
      }
    }
    if (more) store_a(buf ^ 1, areg);
    __syncthreads();
  }

  if constexpr (ROLE == 1) {
    uint16_t* a_hi = reinterpret_cast<uint16_t*>(p1.a);
    uint16_t* a_lo = a_hi + p1.cap * I;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wn * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 16 * j + col;
      const float sg = p1.s13[static_cast<int64_t>(e) * 2 * I + n];
      const float su = p1.s13[static_cast<int64_t>(e) * 2 * I + I + n];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt < ntiles) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t r = row0 + wm * kWaveRows + mt * 16 + kg * 4 + i;
            const float v = silu_mul(acc[mt][j][i] * sg, acc[mt][j + 2][i] * su);
            const uint32_t hi = pack_bf16_rne(v, 0.0f) & 0xffffu;
            const uint32_t lo = pack_bf16_rne(v - __uint_as_float(hi << 16), 0.0f) & 0xffffu;
            a_hi[r * I + n] = static_cast<uint16_t>(hi);
            a_lo[r * I + n] = static_cast<uint16_t>(lo);
          }
        }
      }
    }
  } else {
    const int64_t h0 = static_cast<int64_t>(blockIdx.x) * 128 + wn * 64;
    float sc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) sc[j] = p2.s2[static_cast<int64_t>(e) * H + h0 + 16 * j + col];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = sorted_ids[row0 + wm * kWaveRows + mt * 16 + kg * 4 + i];
          if (f < Tk) {
            float* yr = p2.y + static_cast<int64_t>(f) * H + h0 + col;
#pragma unroll
            for (int j = 0; j < kNT; ++j) yr[16 * j] = acc[mt][j][i] * sc[j];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm2_w8_prefill(const Gemm2Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.H / 128), static_cast<unsigned>(p.cap / kRows));
  const Gemm1Args none{};
  hipLaunchKernelGGL((gemm_prefill_kernel<2, 32, 2, false>), grid, dim3(kThreads), 0, stream, none, p);
  return hipGetLastError();
}

}  // namespace moe
