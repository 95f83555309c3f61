// GEMM2 of the weight-only fp8 layer for 256-row align blocks, gfx950.
//
// fp8 page, Fp8MoEMethod (weight-only path): y = a dequant(w2[e])^T with one
// fp32 scale per expert, where dequant(w2) = e4m3fn value * scale.  The
// intermediate a comes from GEMM1 as two bf16 planes, hi = rne(a) and
// lo = rne(a - hi), so a = hi + lo to 16 significant bits; the e4m3 codes
// decode exactly into bf16 operands (gfx950's conversion instructions, two
// codes per instruction), and both planes accumulate into the same fp32
// accumulator: acc = sum_i (hi_i + lo_i) w_i with no per-group rescaling.
//
// Tiling: a workgroup owns one align block (256 rows) and 256 output columns
// of one K part (grid z: the K stages cut into `splits` parts, partials to
// y[z]).  Its 4 waves (one per SIMD) form a 2 x 2 grid; a wave owns 128 rows
// x 128 columns = 8 x 8 tiles of v_mfma_f32_16x16x32_bf16, two MFMAs (hi, lo)
// per tile and 32-wide K stage, with the 256 accumulators pinned in the AGPR
// half of the register file (in-place asm MFMAs, as the int8 GEMMs of the
// W8A8 layer).  K advances through a 4-slot LDS ring (4 x 40 KB, the whole
// LDS of a CU) filled with buffer_load ... lds: 16 KB of each plane and 8 KB
// of w2 codes per stage.
//   * half 0 of stage s multiplies column tiles 0-3 and reads and decodes the
//     stage's codes of tiles 4-7; half 1 multiplies tiles 4-7, refills each
//     row tile's fragments from stage s+1 once its last MFMA has them, and
//     reads and decodes stage s+1's codes of tiles 0-3;
//   * so slot s is read until half 0 of stage s, and after the barrier of
//     stage s (which makes stage s+1 visible) the slot of stage s-1 takes
//     stage s+3: two stages in flight behind the one multiplied;
//   * A rows (64 bytes) are XOR-swizzled by 16-byte chunk, code rows (32
//     bytes) by flipping their two 16-byte halves every 8 rows, so that the
//     fragment reads of 16 rows do not collide in the banks;
//   * inside each 64-row group of code rows, LDS row 16 q + r holds source
//     row 4 r + q: lane col ends with 4 adjacent output columns.
// Lane (col, kg) feeds K [8 kg, 8 kg + 8) of the stage for both operands.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 256;                    // rows per workgroup (= block_m)
constexpr int kBK = 32;                       // K per stage
constexpr int kRing = 4;
constexpr int kARow = kBK * 2;                // bytes per A row per plane and stage
constexpr int kBRow = kBK;                    // bytes per code row per stage
constexpr int kPlane = kRows * kARow;         // 16 KB
constexpr int kBBytes = 256 * kBRow;          // 8 KB
constexpr int kStageBytes = 2 * kPlane + kBBytes;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kACopies = kPlane / (kThreads * 16);   // 4 per plane and thread
constexpr int kBCopies = kBBytes / (kThreads * 16);  // 2
constexpr int kDma = 2 * kACopies + kBCopies;

static_assert(kRing * kStageBytes <= 160 * 1024, "the ring fits the LDS of a CU");

// acc += a b on v_mfma_f32_16x16x32_bf16, in place (the builtin's untied
// form had the register allocator moving accumulators, as in the int8 GEMMs
// of the W8A8 layer).  The compiler does not see these as MFMAs, so the
// hazards it would cover are covered here: each is preceded by the 2 wait
// states a VALU result (the decoded w2 operand) needs before an MFMA reads
// it, the asm is volatile so that the MFMAs keep their program order, in
// which no accumulator is read by the MFMA right after the one writing it,
// and mfma_drain waits out the last results before anything else reads them.
__device__ __forceinline__ void mfma_acc(f32x4& c, u32x4 a, u32x4 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// swizzle of a 32-byte code row: its two 16-byte halves swap every 8 rows
__device__ __forceinline__ int swz_h(int r) { return (r >> 3) & 1; }

// 8 w2 codes -> one 8-wide bf16 operand, exact
template <bool FP8>
__device__ __forceinline__ u32x4 decode8(u32x2 w) {
  if constexpr (FP8) {
    return u32x4{fp8x2_to_16x2<false, false>(w.x), fp8x2_to_16x2<false, true>(w.x),
                 fp8x2_to_16x2<false, false>(w.y), fp8x2_to_16x2<false, true>(w.y)};
  } else {
    const u32x2 p0 = i8x4_to_bf16x4(w.x), p1 = i8x4_to_bf16x4(w.y);
    return u32x4{p0.x, p0.y, p1.x, p1.y};
  }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void gemm2_planes_kernel(const Gemm2Args p) {
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
  int nrows = 0;
  for (int r = 0; r < kRows; r += 16)
    if (p.sorted_ids[row0 + r] < Tk) nrows = r + 16;
  int ntw = (nrows - wm * 128) / 16;
  ntw = ntw < 0 ? 0 : (ntw > 8 ? 8 : ntw);
  const int nst = static_cast<int>(I / kBK);
  const int s0 = z * nst / p.splits, s1 = (z + 1) * nst / p.splits;

  // A copies: the block's rows of each plane that hold tokens (the others
  // fill zeros); copy i of this thread lands in LDS rows wave * 64 + 16 i +
  // lane / 4, chunk lane % 4 holding source chunk (lane % 4) ^ swz_b(row)
  const uint16_t* hi = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* lo = hi + p.cap * I;
  const uint32_t abytes = static_cast<uint32_t>(nrows * I * 2);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(hi + row0 * I, abytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(lo + row0 * I, abytes);
  uint32_t aoff[kACopies];
#pragma unroll
  for (int i = 0; i < kACopies; ++i) {
    const int r = wave * 64 + i * 16 + (lane >> 2);
    aoff[i] = static_cast<uint32_t>(r * I * 2 + (((lane & 3) ^ swz_b(r)) * 16));
  }
  // code copies: wave w fills code rows 64 w .. 64 w + 63 (output columns
  // hb + 64 w ..); copy i lands in LDS rows 64 w + 32 i + lane / 2, half
  // lane % 2 holding source half (lane % 2) ^ swz_h(row); LDS row 16 q + r of
  // the group holds source row 4 r + q
  const int64_t hb = static_cast<int64_t>(blockIdx.x) * 256;
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(p.w2 + (static_cast<int64_t>(e) * H + hb + 64 * wave) * p.ldw, static_cast<uint32_t>(64 * p.ldw));
  uint32_t boff[kBCopies];
#pragma unroll
  for (int i = 0; i < kBCopies; ++i) {
    const int l = i * 32 + (lane >> 1);          // LDS row inside the group
    const int q = l >> 4, r = l & 15;
    boff[i] = static_cast<uint32_t>((4 * r + q) * p.ldw + (((lane & 1) ^ swz_h(l)) * 16));
  }
  auto copy = [&](int s, int slot, int i) __attribute__((always_inline)) {
    uint8_t* base = smem + slot * kStageBytes;
    if (i < 2 * kACopies) {
      const int pl = i / kACopies, c = i % kACopies;
      dma16_buf(pl ? rl : rh, aoff[c], static_cast<uint32_t>(s * kARow),
                base + pl * kPlane + (wave * 64 + c * 16) * kARow);
    } else {
      const int c = i - 2 * kACopies;
      dma16_buf(rb, boff[c], static_cast<uint32_t>(s * kBRow), base + 2 * kPlane + (wave * 64 + c * 32) * kBRow);
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment offsets (rows col + 16 t share the swizzle of col)
  const int aoffr = (wm * 128 + col) * kARow + 16 * (kg ^ swz_b(col));
  int boffr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int b = (2 * wn + (j >> 2)) * 64 + 16 * (j & 3) + col;
    boffr[j] = 2 * kPlane + b * kBRow + 16 * ((kg >> 1) ^ swz_h(col)) + 8 * (kg & 1);
  }

  auto run = [&](auto tiles) __attribute__((always_inline)) {
    constexpr int MT = decltype(tiles)::value;
    constexpr int MT1 = MT > 0 ? MT : 1;
    u32x4 ah[MT1], al[MT1], bw[8];
    auto read_a = [&](const uint8_t* st, int mt) __attribute__((always_inline)) {
      ah[mt] = *reinterpret_cast<const u32x4*>(st + aoffr + mt * 16 * kARow);
      al[mt] = *reinterpret_cast<const u32x4*>(st + kPlane + aoffr + mt * 16 * kARow);
    };
    auto read_b = [&](const uint8_t* st, int j) __attribute__((always_inline)) {
      bw[j] = decode8<FP8>(*reinterpret_cast<const u32x2*>(st + boffr[j]));
    };
#pragma unroll
    for (int q = 0; q < kRing - 1; ++q)
#pragma unroll
      for (int i = 0; i < kDma; ++i) copy(s0 + q < s1 ? s0 + q : s1 - 1, q, i);
    wait_vmcnt<(kRing - 2) * kDma>();
    stage_barrier();
    if constexpr (MT > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) read_a(smem, mt);
#pragma unroll
      for (int j = 0; j < 4; ++j) read_b(smem, j);
    }
    mfma_drain();

    auto step = [&](int s, auto more_tag) __attribute__((always_inline)) {
      constexpr bool MORE = decltype(more_tag)::value;
      if constexpr (MORE) {
        wait_vmcnt_lgkm0<(kRing - 3) * kDma>();   // stage s+1 landed in every thread
        stage_barrier();                          // ... and every wave is done with slot s-1
      }
      const uint8_t* cur = smem + ((s - s0) % kRing) * kStageBytes;
      const uint8_t* nx = smem + ((s - s0 + 1) % kRing) * kStageBytes;
      const int sc = s + kRing - 1 < s1 ? s + kRing - 1 : s1 - 1;
      const int slot = (s - s0 + kRing - 1) % kRing;
      if constexpr (MT == 0) {
        if constexpr (MORE) {
#pragma unroll
          for (int i = 0; i < kDma; ++i) copy(sc, slot, i);
        }
      } else {
        constexpr int kSlots = 2 * MT;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int j = 4 * h; j < 4 * h + 4; ++j) mfma_acc(acc[mt][j], ah[mt], bw[j]);
#pragma unroll
            for (int j = 4 * h; j < 4 * h + 4; ++j) mfma_acc(acc[mt][j], al[mt], bw[j]);
            if (h == 0) {
#pragma unroll
              for (int j = 4 + mt * 4 / MT; j < 4 + (mt + 1) * 4 / MT; ++j) read_b(cur, j);
            }
            if constexpr (MORE) {
              const int m = h * MT + mt;
#pragma unroll
              for (int i = m * kDma / kSlots; i < (m + 1) * kDma / kSlots; ++i) copy(sc, slot, i);
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
  };
  if (ntw > 6) run(std::integral_constant<int, 8>{});
  else if (ntw > 4) run(std::integral_constant<int, 6>{});
  else if (ntw > 2) run(std::integral_constant<int, 4>{});
  else if (ntw > 0) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 0>{});

  // epilogue: lane col holds output columns hb + 64 g + 4 col .. + 3 of group
  // g = 2 wn + (j >> 2)
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    sc[j] = FP8 ? p.s2[e] : p.s2[static_cast<int64_t>(e) * H + hb + 64 * (2 * wn + (j >> 2)) + 4 * col + (j & 3)];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt < ntw) {
      const i32x4 ids = *reinterpret_cast<const i32x4*>(p.sorted_ids + row0 + wm * 128 + mt * 16 + kg * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (ids[i] < Tk) {
          float* yr = p.y + (static_cast<int64_t>(z) * Tk + ids[i]) * H + hb + 128 * wn + 4 * col;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[mt][4 * g + q][i] * sc[4 * g + q];
            *reinterpret_cast<f32x4*>(yr + 64 * g) = v;
          }
        }
      }
    }
  }
}

}  // namespace

bool gemm2_planes_fits(int64_t H, int64_t I, int64_t bm) {
  return bm == kRows && H % 256 == 0 && I % kBK == 0 && int64_t{kRows} * I * 2 < (int64_t{1} << 32);
}

hipError_t launch_gemm2_w8_planes(const Gemm2Args& p, hipStream_t stream) {
  if (!gemm2_planes_fits(p.H, p.I, p.block_m) || p.cap % kRows || p.ldw % 16 || p.splits < 1 ||
      p.splits > p.I / kBK || 64 * p.ldw >= (int64_t{1} << 32))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.H / 256), static_cast<unsigned>(p.cap / kRows),
                  static_cast<unsigned>(p.splits));
  if (p.fp8)
    hipLaunchKernelGGL(gemm2_planes_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(gemm2_planes_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
