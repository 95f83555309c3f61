// GEMM2 on integer MFMAs for blocks of at most 64 rows (decode-sized
// batches), gfx950.
//
// experts_int8 page, ExpertsInt8MoEMethod.apply -> fused_experts
// (use_int8_w8a16): y = a dequant(w2[e])^T with the per-row scale of w2 on
// the fp32 accumulator.  The int8 codes of w2 are used as they are, by
// v_mfma_i32_16x16x64_i8 (twice the bf16 rate, no decode instructions).
//
// The intermediate a is carried as 16-bit fixed point per (row, group of 128
// columns): a ~= s * (256 * hi + lo) with hi, lo int8 and
// s = max|a over the group| / 32639, so |a - s (256 hi + lo)| <= s / 2
// (relative to the group maximum, 2^-16; the pages' own kernel keeps a in
// bf16, 2^-9 of each element).  Per 128-wide K step a lane runs the MFMAs of
// the hi and lo planes into two int32 accumulators (exact), then folds
// s_row * (256 hi_acc + lo_acc) into its fp32 accumulator.
//
// requant_q16_kernel turns the bf16 hi/lo planes GEMM1 writes into this form
// (16 lanes per (row, group)); rows of 16-row tiles made only of padding are
// skipped, like everywhere else.  Blocks of 16 rows skip that pass: their
// GEMM2 quantizes the (one tile of) planes while staging them in LDS, which
// costs less than a launch when a block holds so few rows.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStep = 128;          // K per iteration = one scale group
constexpr int kQMax = 32639;        // 256 * 127 + 127

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// 16 lanes per (row, group of 128), 8 values per lane: reads the bf16 hi and
// lo planes, writes 128 hi codes, 128 lo codes and one fp32 scale.  Rows of
// tiles made only of padding are left alone (GEMM2 never reads them).
__global__ __launch_bounds__(kThreads) void requant_q16_kernel(const uint16_t* __restrict__ planes, int64_t cap,
                                                               int64_t I, const int32_t* __restrict__ sorted_ids,
                                                               const int32_t* __restrict__ num_padded, int64_t Tk,
                                                               int8_t* __restrict__ qhi, int8_t* __restrict__ qlo,
                                                               float* __restrict__ qscale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane & 15;
  const int64_t G = I / kStep;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + threadIdx.x / 16;
  const int64_t r = w / G, g = w % G;
  const bool live = r < cap;
  const bool valid = live && r < *num_padded && sorted_ids[r & ~int64_t{15}] < Tk;
  const int64_t o = r * I + g * kStep + 8 * sub;
  u32x4 hw = {0u, 0u, 0u, 0u}, lw = {0u, 0u, 0u, 0u};
  if (valid) {
    hw = ld16(planes + o);
    lw = ld16(planes + cap * I + o);
  }
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(hw[i] << 16) + __uint_as_float(lw[i] << 16);
    v[2 * i + 1] = __uint_as_float(hw[i] & 0xffff0000u) + __uint_as_float(lw[i] & 0xffff0000u);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));   // within the 16 lanes
  const float inv = m > 0.0f ? static_cast<float>(kQMax) / m : 0.0f;
  uint32_t hb[2] = {0u, 0u}, lb[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int q = static_cast<int>(__builtin_rintf(v[i] * inv));
    q = q < -kQMax ? -kQMax : (q > kQMax ? kQMax : q);
    const int h = (q + 128) >> 8;
    const int l = q - 256 * h;
    hb[i / 4] |= static_cast<uint32_t>(h & 0xff) << (8 * (i % 4));
    lb[i / 4] |= static_cast<uint32_t>(l & 0xff) << (8 * (i % 4));
  }
  if (valid) {
    *reinterpret_cast<u32x2*>(qhi + o) = u32x2{hb[0], hb[1]};
    *reinterpret_cast<u32x2*>(qlo + o) = u32x2{lb[0], lb[1]};
    if (sub == 0) qscale[r * G + g] = m / static_cast<float>(kQMax);
  }
}

// Workgroup: one align block (MT 16-row tiles, padding tiles skipped), 4
// waves side by side in N, each NT 16-column tiles; K split into p.splits
// parts of whole 128-wide steps (grid z).  The block's hi/lo rows and their
// scales for one step are staged in LDS (double-buffered, one barrier per
// step); lane (col, kg) feeds K [16kg, 16kg+16) and [64+16kg, 64+16kg+16) of
// the step to the two MFMAs of each plane, for both operands.
template <int MT, int NT, bool FQ>
__global__ __launch_bounds__(kThreads) void gemm2_q16_kernel(const Gemm2Args p, const int8_t* __restrict__ qhi,
                                                             const int8_t* __restrict__ qlo,
                                                             const float* __restrict__ qscale) {
  constexpr int ROWS = 16 * MT;
  constexpr int PITCH = kStep + 16;                  // bytes per LDS row (16-byte pad)
  constexpr int CPR = kStep / 16;                    // 16-byte chunks per row and plane
  __shared__ __attribute__((aligned(16))) int8_t As[2][2][ROWS * PITCH];
  __shared__ __attribute__((aligned(16))) float Ss[2][ROWS];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
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

  const int64_t I = p.I, H = p.H, G = I / kStep;
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * (16 * NT * 4) + wave * 16 * NT;
  const int total = static_cast<int>(G);
  const int ib = static_cast<int>(blockIdx.z) * total / p.splits;
  const int iters = (static_cast<int>(blockIdx.z) + 1) * total / p.splits - ib;
  const int8_t* wbase = p.w2 + (static_cast<int64_t>(e) * H + h0 + col) * p.ldw + static_cast<int64_t>(ib) * kStep + kg * 16;
  const int64_t tstride = 16 * p.ldw;

  // cooperative copy of one step of the block's rows into LDS.
  //   FQ = false: chunk c = (plane, row, 16 codes) of the fixed-point form;
  //   FQ = true:  chunk c = (row, 8 values) of the bf16 planes, quantized on
  //   the way (the 16 lanes of a row find its group maximum by shuffles).
  constexpr int NCH = FQ ? ROWS * 16 : 2 * ROWS * CPR;
  constexpr int CPT = (NCH + kThreads - 1) / kThreads;
  int64_t srco[CPT];
  int dsto[CPT];
  bool cv[CPT];
  const int8_t* srcp[CPT];
  const uint16_t* planes = reinterpret_cast<const uint16_t*>(p.a);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * kThreads;
    if constexpr (FQ) {
      const int r = ci / 16, q = ci % 16;
      cv[c] = ci < NCH && r < nrows;
      srcp[c] = nullptr;
      srco[c] = (row0 + r) * I + static_cast<int64_t>(ib) * kStep + q * 8;
      dsto[c] = r * PITCH + q * 8;
    } else {
      const int pl = ci / (ROWS * CPR), rem = ci % (ROWS * CPR);
      const int r = rem / CPR, q = rem % CPR;
      cv[c] = ci < NCH && r < nrows;
      srcp[c] = pl == 0 ? qhi : qlo;
      srco[c] = (row0 + r) * I + static_cast<int64_t>(ib) * kStep + q * 16;
      dsto[c] = (pl * ROWS + r) * PITCH + q * 16;
    }
  }
  constexpr int NREG = FQ ? 2 * CPT : CPT;
  auto load_a = [&](int it, u32x4* regs, float& sreg) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if constexpr (FQ) {
        regs[2 * c] = u32x4{0u, 0u, 0u, 0u};
        regs[2 * c + 1] = u32x4{0u, 0u, 0u, 0u};
        if (cv[c]) {
          regs[2 * c] = ld16(planes + srco[c] + static_cast<int64_t>(it) * kStep);
          regs[2 * c + 1] = ld16(planes + p.cap * I + srco[c] + static_cast<int64_t>(it) * kStep);
        }
      } else {
        if (cv[c]) regs[c] = ld16(srcp[c] + srco[c] + static_cast<int64_t>(it) * kStep);
      }
    }
    if (!FQ && tid < nrows) sreg = qscale[(row0 + tid) * G + ib + it];
  };
  auto store_a = [&](int buf, const u32x4* regs, float sreg) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if constexpr (FQ) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t hw = regs[2 * c][i], lw = regs[2 * c + 1][i];
          v[2 * i] = __uint_as_float(hw << 16) + __uint_as_float(lw << 16);
          v[2 * i + 1] = __uint_as_float(hw & 0xffff0000u) + __uint_as_float(lw & 0xffff0000u);
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
        const float inv = m > 0.0f ? static_cast<float>(kQMax) / m : 0.0f;
        uint32_t hb[2] = {0u, 0u}, lb[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int q = static_cast<int>(__builtin_rintf(v[i] * inv));
          q = q < -kQMax ? -kQMax : (q > kQMax ? kQMax : q);
          const int h = (q + 128) >> 8;
          hb[i / 4] |= static_cast<uint32_t>(h & 0xff) << (8 * (i % 4));
          lb[i / 4] |= static_cast<uint32_t>((q - 256 * h) & 0xff) << (8 * (i % 4));
        }
        if (cv[c]) {
          *reinterpret_cast<u32x2*>(&As[buf][0][dsto[c]]) = u32x2{hb[0], hb[1]};
          *reinterpret_cast<u32x2*>(&As[buf][1][dsto[c]]) = u32x2{lb[0], lb[1]};
          if ((tid & 15) == 0) Ss[buf][(tid + c * kThreads) / 16] = m / static_cast<float>(kQMax);
        }
      } else {
        if (cv[c]) *reinterpret_cast<u32x4*>(&As[buf][0][dsto[c]]) = regs[c];
      }
    }
    if (!FQ && tid < nrows) Ss[buf][tid] = sreg;
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[NREG];
  float sreg = 0.0f;
  if (iters > 0) load_a(0, areg, sreg);
  u32x4 w0[NT], w1[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    w0[j] = iters > 0 ? ld16(wbase + j * tstride) : u32x4{0u, 0u, 0u, 0u};
    w1[j] = iters > 0 ? ld16(wbase + j * tstride + 64) : u32x4{0u, 0u, 0u, 0u};
  }
  if (iters > 0) store_a(0, areg, sreg);
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < iters;
    if (more) load_a(it + 1, areg, sreg);
    const int64_t kn = static_cast<int64_t>(more ? it + 1 : it) * kStep;
    u32x4 n0[NT], n1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      n0[j] = ld16(wbase + j * tstride + kn);
      n1[j] = ld16(wbase + j * tstride + kn + 64);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
        const int o = (mt * 16 + col) * PITCH + kg * 16;
        const u32x4 ah0 = *reinterpret_cast<const u32x4*>(&As[buf][0][o]);
        const u32x4 ah1 = *reinterpret_cast<const u32x4*>(&As[buf][0][o + 64]);
        const u32x4 al0 = *reinterpret_cast<const u32x4*>(&As[buf][1][o]);
        const u32x4 al1 = *reinterpret_cast<const u32x4*>(&As[buf][1][o + 64]);
        const f32x4 sr = *reinterpret_cast<const f32x4*>(&Ss[buf][mt * 16 + kg * 4]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const i32x4 z = {0, 0, 0, 0};
          i32x4 ih = mfma_i8(ah0, w0[j], z);
          ih = mfma_i8(ah1, w1[j], ih);
          i32x4 il = mfma_i8(al0, w0[j], z);
          il = mfma_i8(al1, w1[j], il);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[mt][j][i] += sr[i] * static_cast<float>(ih[i] * 256 + il[i]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      w0[j] = n0[j];
      w1[j] = n1[j];
    }
    if (more) store_a(buf ^ 1, areg, sreg);
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = p.sorted_ids[row0 + mt * 16 + kg * 4 + i];
        if (f < p.Tk) {
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
#pragma unroll
          for (int j = 0; j < NT; ++j)
            yr[16 * j] = acc[mt][j][i] * p.s2[static_cast<int64_t>(e) * H + h0 + 16 * j + col];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_requant_q16(const float* a, int64_t cap, int64_t I, const int32_t* sorted_ids,
                              const int32_t* num_padded, int64_t Tk, int8_t* qhi, int8_t* qlo, float* qscale,
                              hipStream_t stream) {
  const int64_t pairs = cap * (I / kStep);
  const int64_t blocks = (pairs + kThreads / 16 - 1) / (kThreads / 16);
  hipLaunchKernelGGL(requant_q16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(a), cap, I, sorted_ids, num_padded, Tk, qhi, qlo, qscale);
  return hipGetLastError();
}

hipError_t launch_gemm2_q16(const Gemm2Args& p, int nt, const int8_t* qhi, const int8_t* qlo, const float* qscale,
                            hipStream_t stream) {
  const int mt = p.block_m / 16;
  if ((nt != 2 && nt != 4) || p.H % (64 * nt) != 0 || mt < 1 || mt > 4) return hipErrorInvalidValue;
  const unsigned by = static_cast<unsigned>(p.cap / p.block_m), bz = static_cast<unsigned>(p.splits);
#define Q16(MT, NT, FQ)                                                                                   \
  hipLaunchKernelGGL((gemm2_q16_kernel<MT, NT, FQ>), dim3(static_cast<unsigned>(p.H / (64 * NT)), by, bz), \
                     dim3(kThreads), 0, stream, p, qhi, qlo, qscale)
  if (nt == 4) {
    if (mt == 4) Q16(4, 4, false); else if (mt == 3) Q16(3, 4, false); else if (mt == 2) Q16(2, 4, false);
    else Q16(1, 4, true);
  } else {
    if (mt == 4) Q16(4, 2, false); else if (mt == 3) Q16(3, 2, false); else if (mt == 2) Q16(2, 2, false);
    else Q16(1, 2, true);
  }
#undef Q16
  return hipGetLastError();
}

}  // namespace moe
