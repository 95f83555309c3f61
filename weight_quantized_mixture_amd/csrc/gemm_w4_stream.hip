// Weight-streaming grouped GEMMs for group-wise uint4 experts (W4A16) when
// each align block holds at most 64 rows.
//
// moe_wna16 page, MoeWNA16Method.create_weights: codes packed along K
// (here 8 per int32, code k at bits 4*(k mod 8)), fp16 scales [E, N, K/g],
// zeros packed along N (8 per int32), W = (q - z) * s with the true zero.
//
// Same structure as the int8 streaming kernels with the activation tile in
// LDS: a workgroup is one align block (16 * MT rows, padding tiles skipped)
// and 4 waves side by side in N; per 128-K step a lane holds one int32x4 of
// its weight row (32 codes), the whole step lies in one group (g is a
// multiple of 128), and the step's MFMA partial sum is multiplied by the
// group scale of the lane's column before it joins the running total, so the
// scale never rounds a weight.  The weights of the next three steps are in
// flight while a step is converted and multiplied (packed rows are short, so a
// wave needs several steps of loads outstanding to cover HBM latency); the
// group scales, zero words and activation rows travel with them, and the
// barrier that ends a step waits for LDS only, so they stay in flight.
//
// fp16 activations: 0x6400 | q is the half 1024 + q and one packed subtraction
// of 1024 + z leaves q - z exactly; decoding nibble pairs (q_i, q_{i+4}) puts
// the MFMA K slots in the order 0,4,1,5,2,6,3,7, so the activation chunks are
// permuted the same way while they are copied into LDS.  GEMM1 writes the
// intermediate as fp16 hi/lo planes in natural order (it must stay inside the
// fp16 range, like the activations), GEMM2 permutes them on the same copy.
// bf16 activations: codes go through fp32 into bf16 (natural order) and the
// planes are bf16.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kStep = 128;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ uint32_t zero_code(const int32_t* qz_e, int64_t G, int64_t g, int64_t n) {
  return (static_cast<uint32_t>(qz_e[(n >> 3) * G + g]) >> (4 * (n & 7))) & 0xFu;
}

// One int32 of 8 codes -> MFMA operand of (q - z).
template <bool F16>
__device__ __forceinline__ u32x4 w4_op(uint32_t w, uint32_t z) {
  u32x4 r;
  if constexpr (F16) {
    const _Float16 zo = static_cast<_Float16>(static_cast<float>(1024u + z));
    const f16x2 off = {zo, zo};
    const uint32_t m = 0x000F000Fu, magic = 0x64006400u;
    r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, (w & m) | magic) - off);
    r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, ((w >> 4) & m) | magic) - off);
    r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, ((w >> 8) & m) | magic) - off);
    r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, ((w >> 12) & m) | magic) - off);
  } else {
    const float zf = static_cast<float>(z);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<float>((w >> (4 * i)) & 0xFu) - zf;
    r.x = pack_hi16(v[0], v[1]);
    r.y = pack_hi16(v[2], v[3]);
    r.z = pack_hi16(v[4], v[5]);
    r.w = pack_hi16(v[6], v[7]);
  }
  return r;
}

// 8 natural-order 16-bit values -> slot order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u32x4 perm0415(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return r;
}

__device__ __forceinline__ void split16(float v, bool f16, uint16_t& hi, uint16_t& lo) {
  if (f16) {
    const _Float16 h = static_cast<_Float16>(v);
    const _Float16 l = static_cast<_Float16>(v - static_cast<float>(h));
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, l);
  } else {
    const uint32_t h = pack_bf16_rne(v, 0.0f) & 0xffffu;
    hi = static_cast<uint16_t>(h);
    lo = static_cast<uint16_t>(pack_bf16_rne(v - __uint_as_float(h << 16), 0.0f) & 0xffffu);
  }
}

// ROLE 1: GEMM1, each wave 16 gate rows + the 16 matching up rows, A = gathered x.
// ROLE 2: GEMM2, each wave NT*16 rows of w2, A = hi/lo planes of the intermediate.
template <int ROLE, int MT, int NT, bool F16>
__global__ __launch_bounds__(kThreads) void gemm_w4_stream_kernel(const Gemm1W4Args p1, const Gemm2W4Args p2) {
  constexpr int NPLANE = ROLE == 1 ? 1 : 2;
  constexpr int ROWS = 16 * MT;
  constexpr int PITCH = kStep + 8;
  constexpr int QPR = kStep / 8;
  constexpr int CPT = (ROWS * QPR + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NPLANE][ROWS * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int32_t* sorted_ids = ROLE == 1 ? p1.sorted_ids : p2.sorted_ids;
  const int64_t Tk = ROLE == 1 ? p1.Tk : p2.Tk;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * ROWS;
  if (row0 >= *(ROLE == 1 ? p1.num_padded : p2.num_padded)) return;
  const int64_t e = (ROLE == 1 ? p1.block_expert : p2.block_expert)[blockIdx.y];
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (sorted_ids[row0 + mt * 16] < Tk) ntiles = mt + 1;
  const int nrows = ntiles * 16;

  const int64_t H = ROLE == 1 ? p1.H : p2.H;
  const int64_t I = ROLE == 1 ? p1.I : p2.I;
  const int64_t K = ROLE == 1 ? H : I;
  const int64_t N = ROLE == 1 ? 2 * I : H;
  const int g = ROLE == 1 ? p1.group : p2.group;
  const int64_t G = K / g;
  const int32_t* qw = ROLE == 1 ? p1.qw : p2.qw;
  const uint16_t* sc = ROLE == 1 ? p1.sc : p2.sc;
  const int32_t* qz_e = (ROLE == 1 ? p1.qz : p2.qz) + e * (N / 8) * G;

  // rows of w owned by this lane (tile j)
  int64_t nrow[NT];
  if constexpr (ROLE == 1) {
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16 + col;
    nrow[0] = n0;
    nrow[1] = I + n0;
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) nrow[j] = static_cast<int64_t>(blockIdx.x) * (64 * NT) + wave * 16 * NT + 16 * j + col;
  }
  const int32_t* wp[NT];
  const uint16_t* sp[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    wp[j] = qw + (e * N + nrow[j]) * (K / 8) + kg * 4;
    sp[j] = sc + (e * N + nrow[j]) * G;
  }

  // K range: GEMM2 cuts K into splits of whole steps
  const int total = static_cast<int>(K / kStep);
  int sbeg = 0, nsteps = total;
  if constexpr (ROLE == 2) {
    sbeg = static_cast<int>(blockIdx.z) * total / p2.splits;
    nsteps = (static_cast<int>(blockIdx.z) + 1) * total / p2.splits - sbeg;
  }

  // cooperative copy of the activation rows of one step into LDS
  int64_t src[CPT];
  int dst[CPT];
  bool cv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ci = tid + c * kThreads;
    const int r = ci / QPR, q = ci % QPR;
    cv[c] = r < nrows;
    dst[c] = r * PITCH + q * 8;
    if constexpr (ROLE == 1) {
      const int f = cv[c] ? sorted_ids[row0 + r] : static_cast<int>(Tk);
      src[c] = f < Tk ? (static_cast<int64_t>(f) / p1.k) * H + q * 8 : -1;
    } else {
      src[c] = (row0 + r) * I + q * 8;
    }
  }
  const uint16_t* xa = ROLE == 1 ? static_cast<const uint16_t*>(p1.x) : reinterpret_cast<const uint16_t*>(p2.a);
  const int64_t plane = ROLE == 1 ? 0 : p2.cap * I;
  // every lane issues every load (rows without a token read offset 0 and
  // are zeroed afterwards), so the number of loads in flight is the same on
  // every path and the compiler's waits stay exact
  int64_t srcs[CPT];
  bool use[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    use[c] = cv[c] && src[c] >= 0;
    srcs[c] = use[c] ? src[c] : 0;
  }
  auto load_a = [&](int s, u32x4 (&regs)[NPLANE][CPT]) {
    const int64_t ko = static_cast<int64_t>(sbeg + s) * kStep;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int pl = 0; pl < NPLANE; ++pl) regs[pl][c] = ld16(xa + pl * plane + srcs[c] + (use[c] ? ko : 0));
  };
  auto store_a = [&](int buf, const u32x4 (&regs)[NPLANE][CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (cv[c]) {
#pragma unroll
        for (int pl = 0; pl < NPLANE; ++pl) {
          const u32x4 v = use[c] ? regs[pl][c] : u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(&As[buf][pl][dst[c]]) = F16 ? perm0415(v) : v;
        }
      }
  };

  // GEMM2's row ids (to LDS, read after the steps' barriers), loaded now so
  // that no workgroup ends with a round trip to memory after its last step
  __shared__ int rowf[ROLE == 2 ? ROWS : 1];
  if constexpr (ROLE == 2) {
    if (tid < ROWS) rowf[tid] = sorted_ids[row0 + tid];
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weights, group scales and zero words of step s+3, and the activation rows
  // of step s+3, are requested while step s is multiplied (a scale or zero
  // fetched in its own step would put a full memory latency on every step).
  // They live in rings of four register sets and the loop is unrolled by
  // four, so the rings turn by renaming: copying a register that a load is
  // still filling would wait for that load.
  struct Pre {
    u32x4 w[NT];
    uint16_t s[NT];    // fp16 group scale
    uint32_t z[NT];    // zero word (8 rows' codes), decoded when used
  };
  auto wload = [&](int s, Pre& v) {
    const int kq = sbeg + s;
    const int grp = kq * kStep / g;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      v.w[j] = ld16(wp[j] + kq * (kStep / 8));
      v.s[j] = sp[j][grp];
      v.z[j] = static_cast<uint32_t>(qz_e[(nrow[j] >> 3) * G + grp]);
    }
  };
  typedef u32x4 ARegs[NPLANE][CPT];
  auto step = [&](int s, const Pre& cur, Pre& ahead, const ARegs& anext, ARegs& aahead) {
    const int buf = s & 1;
    // step s+3, or the last step again near the end (same addresses, never
    // used): an unconditional load count keeps the waits exact
    const int sa = s + 3 < nsteps ? s + 3 : nsteps - 1;
    load_a(sa, aahead);
    wload(sa, ahead);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t z = (cur.z[j] >> (4 * (nrow[j] & 7))) & 0xFu;
      const float scale = f16_to_f32(cur.s[j]);
      u32x4 b[4];
      b[0] = w4_op<F16>(cur.w[j].x, z);
      b[1] = w4_op<F16>(cur.w[j].y, z);
      b[2] = w4_op<F16>(cur.w[j].z, z);
      b[3] = w4_op<F16>(cur.w[j].w, z);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < ntiles) {
          const int o = (mt * 16 + col) * PITCH + kg * 32;
          f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(&As[buf][0][o + 8 * i]);
            part = mfma16<F16>(x0, b[i], part);
            if constexpr (ROLE == 2) {
              const u32x4 x1 = *reinterpret_cast<const u32x4*>(&As[buf][1][o + 8 * i]);
              part = mfma16<F16>(x1, b[i], part);
            }
          }
          acc[mt][j] += part * scale;
        }
      }
    }
    if (s + 1 < nsteps) store_a(buf ^ 1, anext);
    // LDS writes done, then the barrier; the loads of later steps stay in
    // flight across it (a full __syncthreads would wait for them too)
    wait_lgkm0();
    stage_barrier();
  };
  Pre q[4];
  ARegs ar[4];
  if (nsteps > 0) {
    load_a(0, ar[0]);
    wload(0, q[0]);
    wload(nsteps > 1 ? 1 : 0, q[1]);
    wload(nsteps > 2 ? 2 : nsteps - 1, q[2]);
    store_a(0, ar[0]);
    load_a(nsteps > 1 ? 1 : 0, ar[1]);
    load_a(nsteps > 2 ? 2 : nsteps - 1, ar[2]);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; s += 4) {
    step(s, q[0], q[3], ar[1], ar[3]);
    if (s + 1 < nsteps) step(s + 1, q[1], q[0], ar[2], ar[0]);
    if (s + 2 < nsteps) step(s + 2, q[2], q[1], ar[3], ar[1]);
    if (s + 3 < nsteps) step(s + 3, q[3], q[2], ar[0], ar[2]);
  }

  if constexpr (ROLE == 1) {
    uint16_t* a_hi = reinterpret_cast<uint16_t*>(p1.a);
    uint16_t* a_lo = a_hi + p1.cap * I;
    const int64_t n = nrow[0];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = row0 + mt * 16 + kg * 4 + i;
          uint16_t hi, lo;
          split16(silu_mul(acc[mt][0][i], acc[mt][1][i]), F16, hi, lo);
          a_hi[r * I + n] = hi;
          a_lo[r * I + n] = lo;
        }
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = rowf[mt * 16 + kg * 4 + i];
          if (f < Tk) {
            float* yr = p2.y + (static_cast<int64_t>(blockIdx.z) * Tk + f) * H;
#pragma unroll
            for (int j = 0; j < NT; ++j) yr[nrow[j]] = acc[mt][j][i];
          }
        }
      }
    }
  }
}

// GEMM1 for blocks of 16 or 32 rows fed by direct global -> LDS copies (the
// ring of the int8 decode GEMM1, with packed uint4 rows).  A workgroup is one
// align block and 64 output columns; each wave owns 16 gate rows and the
// matching 16 up rows.  Once, before the ring starts, every wave copies as
// dwords its rows' fp16 scales and zero words of every group of the whole K
// (the 16 gate rows' scales are one contiguous span, the up rows' another,
// then 2 rows of zero words each: 20 G dwords per wave, G <= MAXG groups).
// Per 128-K step (one scale group or part of one) every wave copies its 32
// packed rows (64 bytes each, 2 KB) and the workgroup the block's activation
// rows (256 bytes each; rows without a token read token 0's row and their
// results are replaced by 0).  A 4-deep ring keeps steps s+1..s+3 in flight
// while step s is decoded and multiplied; one barrier per step, after each
// thread has waited for its own copies of that step, and the refill of step
// s-1's slot right after it.  Lane (col, kg) takes K [32 kg, 32 kg + 32) of
// its gate and up rows, 8 codes per MFMA, the activation operand read for the
// same K positions (permuted to the fp16 decode's slot order 0,4,1,5,2,6,3,7
// after the LDS read).
//
// The scale area is the tail of the ring's own LDS array: LDS reads from an
// array of its own, while copies into LDS are in flight, make the compiler
// wait for all copies before them (the ring drained every step, measured
// 9-15 us slower at W4A16 T=8..64).  With MAXG = 16 (H = 2048 at groups of
// 128) the 16-row kernel takes 53 KB and three workgroups fit a CU.
constexpr int kW4Ring = 4;
constexpr int kW4WWave = 32 * (kStep / 2);             // 2 KB of packed codes per wave and step
constexpr int kW4WStage = 4 * kW4WWave;
constexpr int kW4WDma = kW4WWave / (kWave * 16);       // 2 copies per lane and step
constexpr int kW4MaxG = 32;                            // most groups per row of any instantiation
template <int MAXG>
constexpr int w4_sz_wave() { return (20 * MAXG + kWave - 1) / kWave * kWave * 4; }   // bytes per wave

template <int MT, bool F16, int MAXG>
__global__ __launch_bounds__(kThreads) void gemm1_w4_dma_kernel(const Gemm1W4Args p) {
  constexpr int kARow = kStep * 2;                     // bytes per activation row and step
  constexpr int kAStage = 16 * MT * kARow;
  constexpr int kADma = kAStage / (kThreads * 16);     // = MT
  constexpr int kStage = kW4WStage + kAStage;
  constexpr int kPer = kW4WDma + kADma;                // copies per thread and step
  constexpr int kSZWave = w4_sz_wave<MAXG>();
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kW4Ring * kStage + 4 * kSZWave];
  uint8_t* const szs = smem + kW4Ring * kStage;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  if (row0 >= *p.num_padded) return;
  const int64_t e = p.block_expert[blockIdx.y];
  const int64_t Tk = p.Tk, H = p.H, I = p.I, N = 2 * I, G = H / p.group;
  int ntiles = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (p.sorted_ids[row0 + mt * 16] < Tk) ntiles = mt + 1;
  const int nst = static_cast<int>(H / kStep);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16;
  auto wrow = [&](int r) -> int64_t { return r < 16 ? n0 + r : I + n0 + (r - 16); };

  // packed-code copies: row r = 16 i + lane/4 of the wave's 32, LDS chunk
  // lane%4 holds source chunk (lane%4) ^ swz_b(r)
  const uint8_t* qwb = reinterpret_cast<const uint8_t*>(p.qw);
  const uint8_t* wsrc[kW4WDma];
#pragma unroll
  for (int i = 0; i < kW4WDma; ++i) {
    const int r = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ swz_b(r);
    wsrc[i] = qwb + (e * N + wrow(r)) * (H / 2) + c * 16;
  }
  // the wave's scale / zero area, dword d: [0, 8G) the gate rows' scales
  // (row-major [16][G] fp16), [8G, 16G) the up rows', [16G, 18G) the gate
  // zero words ([2][G]: rows n0..n0+7, n0+8..n0+15), [18G, 20G) the up ones;
  // dwords past 20 G repeat dword 0 into the area's tail
  uint8_t* sza = szs + wave * kSZWave;

  // activation copies: row r = 4 (wave MT + q) + lane/16, slot lane%16 holds
  // chunk (lane%16) ^ swz_c(r)
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* asrc[kADma];
#pragma unroll
  for (int q = 0; q < kADma; ++q) {
    const int r = 4 * (wave * kADma + q) + (lane >> 4);
    const int c = (lane & 15) ^ swz_c(r);
    const int f = p.sorted_ids[row0 + r];
    const int64_t t = f < Tk ? f / static_cast<int>(p.k) : 0;
    asrc[q] = x + t * H + c * 8;
  }
  auto issue = [&](int s, int slot) {
    uint8_t* base = smem + slot * kStage;
#pragma unroll
    for (int i = 0; i < kW4WDma; ++i)
      dma16(wsrc[i] + static_cast<int64_t>(s) * (kStep / 2), base + wave * kW4WWave + i * 1024);
#pragma unroll
    for (int q = 0; q < kADma; ++q)
      dma16(asrc[q] + static_cast<int64_t>(s) * kStep, base + kW4WStage + (wave * kADma + q) * 1024);
  };

  // LDS offsets this lane reads
  const int wog = wave * kW4WWave + col * (kStep / 2) + 16 * (kg ^ swz_b(col));
  const int wou = wave * kW4WWave + (16 + col) * (kStep / 2) + 16 * (kg ^ swz_b(16 + col));
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = kW4WStage + col * kARow + 16 * ((4 * kg + i) ^ swz_c(col));
  const uint16_t* sgl = reinterpret_cast<const uint16_t*>(sza) + col * G;
  const uint16_t* sul = reinterpret_cast<const uint16_t*>(sza) + (16 + col) * G;
  const uint32_t* zgl = reinterpret_cast<const uint32_t*>(sza) + 16 * G + (col >> 3) * G;
  const uint32_t* zul = reinterpret_cast<const uint32_t*>(sza) + 18 * G + (col >> 3) * G;

  // which of the lane's rows hold a token, read now so that no workgroup ends
  // with a round trip to memory after its last step
  uint32_t rvalid = 0;                               // bit 4 mt + i: row 16 mt + 4 kg + i
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p.sorted_ids[row0 + mt * 16 + kg * 4 + i] < Tk) rvalid |= 1u << (4 * mt + i);
  // the scale area's copies go out after the reads of sorted_ids above are
  // consumed, so their waits do not wait for these copies as well
  {
    const uint32_t* scg = reinterpret_cast<const uint32_t*>(p.sc + (e * N + n0) * G);
    const uint32_t* scu = reinterpret_cast<const uint32_t*>(p.sc + (e * N + I + n0) * G);
    const int32_t* zg = p.qz + (e * (N / 8) + n0 / 8) * G;
    const int32_t* zu = p.qz + (e * (N / 8) + (I + n0) / 8) * G;
    const int64_t g8 = 8 * G;
    for (int j = 0; j * kWave < 20 * G; ++j) {
      const int64_t d = j * kWave + lane;
      const void* src = d < g8             ? static_cast<const void*>(scg + d)
                        : d < 2 * g8       ? static_cast<const void*>(scu + (d - g8))
                        : d < 2 * g8 + 2 * G ? static_cast<const void*>(zg + (d - 2 * g8))
                        : d < 20 * G       ? static_cast<const void*>(zu + (d - 2 * g8 - 2 * G))
                                           : static_cast<const void*>(scg);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)const_cast<void*>(src), (lds_ptr_t)(sza + j * kWave * 4), 4, 0,
                                       0);
    }
  }  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto run = [&](auto tiles) {
    constexpr int NT = decltype(tiles)::value;
#pragma unroll
    for (int q = 0; q < kW4Ring - 1; ++q) issue(q < nst ? q : nst - 1, q);
    for (int s = 0; s < nst; ++s) {
      // this thread's copies of step s (and, at step 0, of the scale area:
      // those were issued first) landed, s+1, s+2 may still fly; then the
      // slot of step s-1 takes step s+3 (past the end the last step again,
      // into a slot nobody reads: a fixed copy count per step)
      wait_vmcnt<(kW4Ring - 2) * kPer>();
      stage_barrier();
      issue(s + 3 < nst ? s + 3 : nst - 1, (s + 3) % kW4Ring);
      const uint8_t* st = smem + (s % kW4Ring) * kStage;
      const u32x4 wg = *reinterpret_cast<const u32x4*>(st + wog);
      const u32x4 wu = *reinterpret_cast<const u32x4*>(st + wou);
      const int grp = static_cast<int>(static_cast<int64_t>(s) * kStep / p.group);
      const float sg = f16_to_f32(sgl[grp]);
      const float su = f16_to_f32(sul[grp]);
      const uint32_t zg = (zgl[grp] >> (4 * (col & 7))) & 0xFu;
      const uint32_t zu = (zul[grp] >> (4 * (col & 7))) & 0xFu;
      u32x4 bg[4], bu[4];
      bg[0] = w4_op<F16>(wg.x, zg);
      bg[1] = w4_op<F16>(wg.y, zg);
      bg[2] = w4_op<F16>(wg.z, zg);
      bg[3] = w4_op<F16>(wg.w, zg);
      bu[0] = w4_op<F16>(wu.x, zu);
      bu[1] = w4_op<F16>(wu.y, zu);
      bu[2] = w4_op<F16>(wu.z, zu);
      bu[3] = w4_op<F16>(wu.w, zu);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        f32x4 pgs = {0.f, 0.f, 0.f, 0.f}, pus = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 av = *reinterpret_cast<const u32x4*>(st + aoff[i] + mt * 16 * kARow);
          if constexpr (F16) av = perm0415(av);
          pgs = mfma16<F16>(av, bg[i], pgs);
          pus = mfma16<F16>(av, bu[i], pus);
        }
        accg[mt] += pgs * sg;
        accu[mt] += pus * su;
      }
    }
  };
  if constexpr (MT == 2) {
    if (ntiles > 1) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 1>{});
  }
  wait_vmcnt<0>();   // no copy into LDS outlives the workgroup

  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.a);
  uint16_t* a_lo = a_hi + p.cap * I;
  const int64_t n = n0 + col;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + mt * 16 + kg * 4 + i;
        uint16_t hi, lo;
        split16(((rvalid >> (4 * mt + i)) & 1u) ? silu_mul(accg[mt][i], accu[mt][i]) : 0.0f, F16, hi, lo);
        a_hi[r * I + n] = hi;
        a_lo[r * I + n] = lo;
      }
    }
  }
}

template <int MT, bool F16>
hipError_t w4d_launch1(const Gemm1W4Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m));
  if (p.H / p.group <= 16)
    hipLaunchKernelGGL((gemm1_w4_dma_kernel<MT, F16, 16>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm1_w4_dma_kernel<MT, F16, kW4MaxG>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int MT, bool F16>
hipError_t w4s_launch1(const Gemm1W4Args& p, hipStream_t stream) {
  const Gemm2W4Args none{};
  hipLaunchKernelGGL((gemm_w4_stream_kernel<1, MT, 2, F16>),
                     dim3(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m)),
                     dim3(kThreads), 0, stream, p, none);
  return hipGetLastError();
}

template <int MT, bool F16>
hipError_t w4s_launch2(const Gemm2W4Args& p, hipStream_t stream) {
  const Gemm1W4Args none{};
  hipLaunchKernelGGL((gemm_w4_stream_kernel<2, MT, 2, F16>),
                     dim3(static_cast<unsigned>(p.H / 128), static_cast<unsigned>(p.cap / p.block_m),
                          static_cast<unsigned>(p.splits)),
                     dim3(kThreads), 0, stream, none, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_w4_stream(const Gemm1W4Args& p, hipStream_t stream) {
  const int mt = p.block_m / 16;
  if (p.f16) {
    if (mt == 4) return w4s_launch1<4, true>(p, stream);
    if (mt == 2) return w4s_launch1<2, true>(p, stream);
    return w4s_launch1<1, true>(p, stream);
  }
  if (mt == 4) return w4s_launch1<4, false>(p, stream);
  if (mt == 2) return w4s_launch1<2, false>(p, stream);
  return w4s_launch1<1, false>(p, stream);
}

hipError_t launch_gemm1_w4_dma(const Gemm1W4Args& p, hipStream_t stream) {
  if (p.H / p.group > kW4MaxG) return hipErrorInvalidValue;
  if (p.block_m == 32) return p.f16 ? w4d_launch1<2, true>(p, stream) : w4d_launch1<2, false>(p, stream);
  return p.f16 ? w4d_launch1<1, true>(p, stream) : w4d_launch1<1, false>(p, stream);
}

hipError_t launch_gemm2_w4_stream(const Gemm2W4Args& p, hipStream_t stream) {
  const int mt = p.block_m / 16;
  if (p.f16) {
    if (mt == 4) return w4s_launch2<4, true>(p, stream);
    if (mt == 2) return w4s_launch2<2, true>(p, stream);
    return w4s_launch2<1, true>(p, stream);
  }
  if (mt == 4) return w4s_launch2<4, false>(p, stream);
  if (mt == 2) return w4s_launch2<2, false>(p, stream);
  return w4s_launch2<1, false>(p, stream);
}

}  // namespace moe
