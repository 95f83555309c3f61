// GEMM2 on integer MFMAs for blocks of at most 64 rows, and 128-row blocks
// as two halves of 64 (decode- and mid-sized batches), gfx950.
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
// requant_q16_kernel turns the bf16 hi/lo planes GEMM1 writes for blocks of
// 48, 64 and 128 rows into this form (16 lanes per (row, group of 128)); rows of
// 16-row tiles made only of padding are skipped, like everywhere else.  For
// blocks of 16 and 32 rows GEMM1 writes the form itself with groups of 64
// columns (its workgroup's width), which GEMM2 reads with one scale per half
// step.
#include "common.hpp"
#include "dma.hpp"
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
// the step to the two MFMAs of each plane, for both operands.  GW is the
// width of a scale group of the intermediate: 128 (one scale per row and
// step, the two MFMAs of a plane chained) or 64 (one per half step: each half
// accumulates and folds on its own).
template <int MT, int NT, int GW>
__global__ __launch_bounds__(kThreads) void gemm2_q16_kernel(const Gemm2Args p, const int8_t* __restrict__ qhi,
                                                             const int8_t* __restrict__ qlo,
                                                             const float* __restrict__ qscale) {
  constexpr int ROWS = 16 * MT;
  constexpr int PITCH = kStep + 16;                  // bytes per LDS row (16-byte pad)
  constexpr int CPR = kStep / 16;                    // 16-byte chunks per row and plane
  constexpr int SPS = kStep / GW;                    // scales per row and step
  __shared__ __attribute__((aligned(16))) int8_t As[2][2][ROWS * PITCH];
  __shared__ __attribute__((aligned(16))) float Ss[2][ROWS * SPS];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  // ROWS rows of an align block (all of it, or one half of a 128-row block)
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * ROWS;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[row0 / p.block_m];
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (p.sorted_ids[row0 + mt * 16] < p.Tk) ntiles = mt + 1;
  if (ntiles == 0) return;                           // the padding half of a 128-row block
  const int nrows = ntiles * 16;

  const int64_t I = p.I, H = p.H, G = I / GW;
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * (16 * NT * 4) + wave * 16 * NT;
  const int total = static_cast<int>(I / kStep);
  const int ib = static_cast<int>(blockIdx.z) * total / p.splits;
  const int iters = (static_cast<int>(blockIdx.z) + 1) * total / p.splits - ib;
  const int8_t* wbase = p.w2 + (static_cast<int64_t>(e) * H + h0 + col) * p.ldw + static_cast<int64_t>(ib) * kStep + kg * 16;
  const int64_t tstride = 16 * p.ldw;

  // cooperative copy of one step of the block's rows into LDS: chunk c =
  // (plane, row, 16 codes) of the fixed-point form.  Chunks of rows past the
  // block's tokens load row 0's chunk again (never stored): every thread
  // issues the same loads each step, so the waits stay exact.
  constexpr int NCH = 2 * ROWS * CPR;
  constexpr int CPT = (NCH + kThreads - 1) / kThreads;
  static_assert(NCH % kThreads == 0, "every thread copies whole chunks");
  int64_t srco[CPT];
  int dsto[CPT];
  bool cv[CPT];
  const int8_t* srcp[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * kThreads;
    const int pl = ci / (ROWS * CPR), rem = ci % (ROWS * CPR);
    const int r = rem / CPR, q = rem % CPR;
    cv[c] = r < nrows;
    srcp[c] = pl == 0 ? qhi : qlo;
    srco[c] = (row0 + (cv[c] ? r : 0)) * I + static_cast<int64_t>(ib) * kStep + q * 16;
    dsto[c] = (pl * ROWS + r) * PITCH + q * 16;
  }
  const int srow = tid < nrows ? tid : 0;

  // Weights, and the block's rows and scales, of step s+2 are requested
  // while step s is multiplied.  They live in rings of three register sets
  // and the loop is unrolled by three, so the rings turn by renaming: copying
  // a register that a load is still filling would wait for that load.  (A
  // fourth set costs more in occupancy than it gains in depth.)
  struct WSet {
    u32x4 w0[NT], w1[NT];
  };
  struct ASet {
    u32x4 r[CPT];
    float s[SPS];
  };
  auto wload = [&](int it, WSet& v) {
    const int64_t kn = static_cast<int64_t>(it) * kStep;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      v.w0[j] = ld16(wbase + j * tstride + kn);
      v.w1[j] = ld16(wbase + j * tstride + kn + 64);
    }
  };
  auto aload = [&](int it, ASet& v) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) v.r[c] = ld16(srcp[c] + srco[c] + static_cast<int64_t>(it) * kStep);
#pragma unroll
    for (int j = 0; j < SPS; ++j) v.s[j] = qscale[(row0 + srow) * G + (ib + it) * SPS + j];
  };
  auto astore = [&](int buf, const ASet& v) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (cv[c]) *reinterpret_cast<u32x4*>(&As[buf][0][dsto[c]]) = v.r[c];
    if (tid < nrows) {
#pragma unroll
      for (int j = 0; j < SPS; ++j) Ss[buf][tid * SPS + j] = v.s[j];
    }
  };

  // the epilogue's row ids (to LDS, read after the loop's barriers) and
  // column scales, loaded now so that no workgroup ends with a round trip to
  // memory after its last step
  __shared__ int rowf[ROWS];
  if (tid < ROWS) rowf[tid] = p.sorted_ids[row0 + tid];
  float csc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) csc[j] = p.s2[static_cast<int64_t>(e) * H + h0 + 16 * j + col];

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int it, const WSet& cur, WSet& ahead, const ASet& anext, ASet& aahead) {
    const int buf = it & 1;
    // step it+2, or the last step again near the end (same addresses, never
    // used): a fixed load count per step
    const int sa = it + 2 < iters ? it + 2 : iters - 1;
    aload(sa, aahead);
    wload(sa, ahead);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
        const int o = (mt * 16 + col) * PITCH + kg * 16;
        const u32x4 ah0 = *reinterpret_cast<const u32x4*>(&As[buf][0][o]);
        const u32x4 ah1 = *reinterpret_cast<const u32x4*>(&As[buf][0][o + 64]);
        const u32x4 al0 = *reinterpret_cast<const u32x4*>(&As[buf][1][o]);
        const u32x4 al1 = *reinterpret_cast<const u32x4*>(&As[buf][1][o + 64]);
        const int so = (mt * 16 + kg * 4) * SPS;
        if constexpr (GW == 128) {
          const f32x4 sr = *reinterpret_cast<const f32x4*>(&Ss[buf][so]);
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const i32x4 z = {0, 0, 0, 0};
            i32x4 ih = mfma_i8(ah0, cur.w0[j], z);
            ih = mfma_i8(ah1, cur.w1[j], ih);
            i32x4 il = mfma_i8(al0, cur.w0[j], z);
            il = mfma_i8(al1, cur.w1[j], il);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][j][i] += sr[i] * static_cast<float>(ih[i] * 256 + il[i]);
          }
        } else {
          // scales (row, half) of rows kg*4 + i: [2 i], [2 i + 1]
          const f32x4 sa4 = *reinterpret_cast<const f32x4*>(&Ss[buf][so]);
          const f32x4 sb4 = *reinterpret_cast<const f32x4*>(&Ss[buf][so + 4]);
          const float s0[4] = {sa4.x, sa4.z, sb4.x, sb4.z}, s1[4] = {sa4.y, sa4.w, sb4.y, sb4.w};
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const i32x4 z = {0, 0, 0, 0};
            const i32x4 ih0 = mfma_i8(ah0, cur.w0[j], z), ih1 = mfma_i8(ah1, cur.w1[j], z);
            const i32x4 il0 = mfma_i8(al0, cur.w0[j], z), il1 = mfma_i8(al1, cur.w1[j], z);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[mt][j][i] += s0[i] * static_cast<float>(ih0[i] * 256 + il0[i]) +
                               s1[i] * static_cast<float>(ih1[i] * 256 + il1[i]);
          }
        }
      }
    }
    if (it + 1 < iters) astore(buf ^ 1, anext);
    // LDS writes done, then the barrier; the loads of later steps stay in
    // flight across it (a full __syncthreads would wait for them too)
    wait_lgkm0();
    stage_barrier();
  };
  WSet q[3];
  ASet ar[3];
  if (iters > 0) {
    aload(0, ar[0]);
    wload(0, q[0]);
    wload(iters > 1 ? 1 : 0, q[1]);
    astore(0, ar[0]);
    aload(iters > 1 ? 1 : 0, ar[1]);
  }
  __syncthreads();
  for (int it = 0; it < iters; it += 3) {
    step(it, q[0], q[2], ar[1], ar[2]);
    if (it + 1 < iters) step(it + 1, q[1], q[0], ar[2], ar[0]);
    if (it + 2 < iters) step(it + 2, q[2], q[1], ar[0], ar[1]);
  }
  wait_vmcnt<0>();   // the last steps' repeat loads land before the registers are reused

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = rowf[mt * 16 + kg * 4 + i];
        if (f < p.Tk) {
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
#pragma unroll
          for (int j = 0; j < NT; ++j) yr[16 * j] = acc[mt][j][i] * csc[j];
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

hipError_t launch_gemm2_q16(const Gemm2Args& p, int nt, int gw, const int8_t* qhi, const int8_t* qlo,
                            const float* qscale, hipStream_t stream) {
  // blocks of up to 64 rows whole, 128-row blocks as two workgroups of 64 rows
  const int rows = p.block_m == 128 ? 64 : p.block_m;
  const int mt = rows / 16;
  if ((nt != 2 && nt != 4) || (gw != 64 && gw != 128) || p.H % (64 * nt) != 0 || p.I % kStep != 0 || mt < 1 ||
      mt > 4 || rows % 16 != 0)
    return hipErrorInvalidValue;
  const unsigned by = static_cast<unsigned>(p.cap / rows), bz = static_cast<unsigned>(p.splits);
#define Q16(MT, NT, GW)                                                                                   \
  hipLaunchKernelGGL((gemm2_q16_kernel<MT, NT, GW>), dim3(static_cast<unsigned>(p.H / (64 * NT)), by, bz), \
                     dim3(kThreads), 0, stream, p, qhi, qlo, qscale)
#define Q16_MT(NT, GW)                                                                                    \
  if (mt == 4) Q16(4, NT, GW); else if (mt == 3) Q16(3, NT, GW); else if (mt == 2) Q16(2, NT, GW); else Q16(1, NT, GW)
  if (gw == 64) {
    if (nt == 4) { Q16_MT(4, 64); } else { Q16_MT(2, 64); }
  } else {
    if (nt == 4) { Q16_MT(4, 128); } else { Q16_MT(2, 128); }
  }
#undef Q16_MT
#undef Q16
  return hipGetLastError();
}

}  // namespace moe
