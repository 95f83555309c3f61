// Grouped expert GEMMs with group-wise uint4 weights and zero points (W4A16), gfx950.
//
// moe_wna16 page, MoeWNA16Method.create_weights: 4-bit codes packed along K
// (8 per int32 here, code k at bits 4*(k mod 8)), scales [E, N, K/g], zeros
// packed along N (8 per int32, row n at bits 4*(n mod 8)); the weight loader
// stores the true zero, so W = (q - z) * s.  Same tiling as the int8 kernels
// (a lane owns one weight row and 32 consecutive K per 128-K step); the group
// size is a multiple of 128, so a whole step lies in one group and its fp32
// partial sum is multiplied by the group scale of the lane's column before it
// is added to the running total (the scale never rounds the weight).
//
// fp16 activations: 0x6400 | nibble is the half 1024 + q, and one packed
// subtraction of 1024 + z gives q - z exactly.  Doing it on the word's
// nibble pairs (q_i, q_{i+4}) puts the MFMA K slots in the order
// 0,4,1,5,2,6,3,7; the activation operand is permuted the same way (v_perm),
// which leaves every dot product unchanged.  GEMM2's fp32 intermediate is
// split into fp16 hi + lo (22 significant bits); like the activations it must
// stay inside the fp16 range.
// bf16 activations: codes go through fp32 (exact) into bf16, natural K order,
// and GEMM2 uses a bf16 hi + lo split.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kKStep = 128;

__device__ __forceinline__ uint32_t zero_of(const int32_t* qz_row8, int64_t G, int64_t g, int64_t n) {
  return (static_cast<uint32_t>(qz_row8[(n >> 3) * G + g]) >> (4 * (n & 7))) & 0xFu;
}

// One int32 of 8 codes -> MFMA operand (8 x 16-bit) of q - z.
template <bool F16>
__device__ __forceinline__ u32x4 w4_operand(uint32_t w, uint32_t z) {
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

// Natural-order 8 x 16-bit activations -> slot order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u32x4 perm_0415(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return r;
}

__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// 8 fp32 values -> hi and lo 16-bit operands, in the slot order the weights use.
template <bool F16>
__device__ __forceinline__ void split_operands(float4 a, float4 b, u32x4& hi, u32x4& lo) {
  if constexpr (F16) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float h[8];
    uint32_t H[4], L[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      H[j] = pack_f16_rne(v[j], v[j + 4]);
      h[j] = static_cast<float>(__builtin_bit_cast(f16x2, H[j]).x);
      h[j + 4] = static_cast<float>(__builtin_bit_cast(f16x2, H[j]).y);
      L[j] = pack_f16_rne(v[j] - h[j], v[j + 4] - h[j + 4]);
    }
    hi = u32x4{H[0], H[1], H[2], H[3]};
    lo = u32x4{L[0], L[1], L[2], L[3]};
  } else {
    u32x2 h0, l0, h1, l1;
    split_bf16x4(a, h0, l0);
    split_bf16x4(b, h1, l1);
    hi = u32x4{h0.x, h0.y, h1.x, h1.y};
    lo = u32x4{l0.x, l0.y, l1.x, l1.y};
  }
}

template <int MT, bool F16>
__global__ __launch_bounds__(kGemmThreads) void gemm1_w4_kernel(const Gemm1W4Args p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * p.block_m;
  if (row0 >= *p.num_padded) return;
  const int64_t e = p.block_expert[blockIdx.y];
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16;
  const int64_t I = p.I, H = p.H, N = 2 * I;
  const int64_t G = H / p.group;
  const int64_t ng = n0 + col, nu = I + n0 + col;

  const int32_t* qg = p.qw + (e * N + ng) * (H / 8) + kg * 4;
  const int32_t* qu = p.qw + (e * N + nu) * (H / 8) + kg * 4;
  const uint16_t* sg = p.sc + (e * N + ng) * G;
  const uint16_t* su = p.sc + (e * N + nu) * G;
  const int32_t* qz = p.qz + e * (N / 8) * G;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);

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
      const int64_t g = k0 / p.group;
      const u32x4 wgv = *reinterpret_cast<const u32x4*>(qg + k0 / 8);
      const u32x4 wuv = *reinterpret_cast<const u32x4*>(qu + k0 / 8);
      const uint32_t zg = zero_of(qz, G, g, ng), zu = zero_of(qz, G, g, nu);
      const float scg = f16_to_f32(sg[g]), scu = f16_to_f32(su[g]);
      u32x4 bg[4], bu[4];
      bg[0] = w4_operand<F16>(wgv.x, zg); bg[1] = w4_operand<F16>(wgv.y, zg);
      bg[2] = w4_operand<F16>(wgv.z, zg); bg[3] = w4_operand<F16>(wgv.w, zg);
      bu[0] = w4_operand<F16>(wuv.x, zu); bu[1] = w4_operand<F16>(wuv.y, zu);
      bu[2] = w4_operand<F16>(wuv.z, zu); bu[3] = w4_operand<F16>(wuv.w, zu);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 sg4 = {0.f, 0.f, 0.f, 0.f}, su4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 av = valid[mt] ? *reinterpret_cast<const u32x4*>(xr[mt] + k0 + 8 * i)
                               : u32x4{0u, 0u, 0u, 0u};
          if constexpr (F16) av = perm_0415(av);
          sg4 = mfma16<F16>(av, bg[i], sg4);
          su4 = mfma16<F16>(av, bu[i], su4);
        }
        accg[mt] += sg4 * scg;
        accu[mt] += su4 * scu;
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + rc + mt * 16 + kg * 4 + i;
        p.a[r * I + n0 + col] = silu_mul(accg[mt][i], accu[mt][i]);
      }
    }
  }
}

template <int MT, bool F16>
__global__ __launch_bounds__(kGemmThreads) void gemm2_w4_kernel(const Gemm2W4Args p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * p.block_m;
  if (row0 >= *p.num_padded) return;
  const int64_t e = p.block_expert[blockIdx.y];
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32;
  const int64_t I = p.I, H = p.H;
  const int64_t G = I / p.group;
  const int64_t kc = I / p.splits;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * kc;
  const int64_t n_0 = h0 + col, n_1 = h0 + 16 + col;

  const int32_t* q0 = p.qw + (e * H + n_0) * (I / 8) + kg * 4;
  const int32_t* q1 = p.qw + (e * H + n_1) * (I / 8) + kg * 4;
  const uint16_t* s0p = p.sc + (e * H + n_0) * G;
  const uint16_t* s1p = p.sc + (e * H + n_1) * G;
  const int32_t* qz = p.qz + e * (H / 8) * G;

  for (int rc = 0; rc < p.block_m; rc += 16 * MT) {
    const float* ar[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ar[mt] = p.a + (row0 + rc + mt * 16 + col) * I + kg * 32;
    f32x4 acc0[MT], acc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t k0 = kbeg; k0 < kbeg + kc; k0 += kKStep) {
      const int64_t g = k0 / p.group;
      const u32x4 w0v = *reinterpret_cast<const u32x4*>(q0 + k0 / 8);
      const u32x4 w1v = *reinterpret_cast<const u32x4*>(q1 + k0 / 8);
      const uint32_t z0 = zero_of(qz, G, g, n_0), z1 = zero_of(qz, G, g, n_1);
      const float sc0 = f16_to_f32(s0p[g]), sc1 = f16_to_f32(s1p[g]);
      u32x4 b0[4], b1[4];
      b0[0] = w4_operand<F16>(w0v.x, z0); b0[1] = w4_operand<F16>(w0v.y, z0);
      b0[2] = w4_operand<F16>(w0v.z, z0); b0[3] = w4_operand<F16>(w0v.w, z0);
      b1[0] = w4_operand<F16>(w1v.x, z1); b1[1] = w4_operand<F16>(w1v.y, z1);
      b1[2] = w4_operand<F16>(w1v.z, z1); b1[3] = w4_operand<F16>(w1v.w, z1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 va = *reinterpret_cast<const float4*>(ar[mt] + k0 + 8 * i);
          const float4 vb = *reinterpret_cast<const float4*>(ar[mt] + k0 + 8 * i + 4);
          u32x4 ahi, alo;
          split_operands<F16>(va, vb, ahi, alo);
          p0 = mfma16<F16>(ahi, b0[i], p0);
          p0 = mfma16<F16>(alo, b0[i], p0);
          p1 = mfma16<F16>(ahi, b1[i], p1);
          p1 = mfma16<F16>(alo, b1[i], p1);
        }
        acc0[mt] += p0 * sc0;
        acc1[mt] += p1 * sc1;
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
          yr[0] = acc0[mt][i];
          yr[16] = acc1[mt][i];
        }
      }
    }
  }
}

template <bool F16>
hipError_t gemm1_w4_mt(const Gemm1W4Args& p, dim3 grid, hipStream_t stream) {
  if (p.block_m % 64 == 0)
    hipLaunchKernelGGL((gemm1_w4_kernel<4, F16>), grid, dim3(kGemmThreads), 0, stream, p);
  else if (p.block_m % 32 == 0)
    hipLaunchKernelGGL((gemm1_w4_kernel<2, F16>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm1_w4_kernel<1, F16>), grid, dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool F16>
hipError_t gemm2_w4_mt(const Gemm2W4Args& p, dim3 grid, hipStream_t stream) {
  if (p.block_m % 64 == 0)
    hipLaunchKernelGGL((gemm2_w4_kernel<4, F16>), grid, dim3(kGemmThreads), 0, stream, p);
  else if (p.block_m % 32 == 0)
    hipLaunchKernelGGL((gemm2_w4_kernel<2, F16>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm2_w4_kernel<1, F16>), grid, dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_w4(const Gemm1W4Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m));
  return p.f16 ? gemm1_w4_mt<true>(p, grid, stream) : gemm1_w4_mt<false>(p, grid, stream);
}

hipError_t launch_gemm2_w4(const Gemm2W4Args& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.H / 128), static_cast<unsigned>(p.cap / p.block_m),
                  static_cast<unsigned>(p.splits));
  return p.f16 ? gemm2_w4_mt<true>(p, grid, stream) : gemm2_w4_mt<false>(p, grid, stream);
}

}  // namespace moe
