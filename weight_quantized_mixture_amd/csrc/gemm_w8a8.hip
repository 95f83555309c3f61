// W8A8: int8 expert weights with int8 activations quantized per token, gfx950
// (fused_moe oracle/int8 page, select_int8_moe_backend: per-channel static
// int8 weights, kInt8StaticChannelSym, and per-token dynamic int8
// activations, kInt8DynamicTokenSym; the weights are the experts_int8 page's).
//
//   act_quant_kernel: one wave per row of a GEMM input (x rows, or rows of the
//     fp32 intermediate a): s = max|row| / 127 and codes rint(v / s) clamped
//     to [-127, 127], fp32 with the IEEE divide (the weights' rule), a zero
//     row gives s = 0 and codes 0;
//   gemm1_w8a8_kernel: h = s_x[t] s13[e, n] * sum_c qx[t, c] q13[e, n, c] on
//     v_mfma_i32_16x16x64_i8 (int32 holds the whole K: |sum| <= 127^2 K),
//     then a = silu(h_gate) * h_up written as fp32 rows of the padded block;
//   gemm2_w8a8_kernel: y = s_a[r] s2[e, h] * sum_i qa[r, i] q2[e, h, i], K cut
//     into equal parts of whole 128-wide steps (grid z) added by the combine.
// Tiling as the 16-bit tiled kernels: 4 waves, one align block per workgroup
// walked in chunks of 16 MT rows; lane (col, kg) feeds K [16 kg, 16 kg + 16)
// and [64 + 16 kg, 64 + 16 kg + 16) of every 128-wide step to the two MFMAs,
// for the weight row col and for the activation row col of each tile.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStep = 128;
constexpr int kQWaves = 4;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

template <int SRC>   // 0 bf16, 1 fp16, 2 fp32
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
  if constexpr (SRC == 0) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else if constexpr (SRC == 1) return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// four consecutive values from element i (a multiple of 4): one 16-byte load
// of fp32, one 8-byte load of 16-bit values
template <int SRC>
__device__ __forceinline__ f32x4 load_act4(const void* p, int64_t i) {
  if constexpr (SRC == 2) {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
    const uint16_t h[4] = {static_cast<uint16_t>(w.x), static_cast<uint16_t>(w.x >> 16), static_cast<uint16_t>(w.y),
                           static_cast<uint16_t>(w.y >> 16)};
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = SRC == 0 ? bf16_to_f32(h[j]) : f16_to_f32(h[j]);
    return v;
  }
}

// One wave per row.  With sorted_ids, row r is quantized only when it holds a
// token (r < *num_padded and sorted_ids[r] < Tk); others are left alone.  With
// pmax, the row's max |v| is the max of its npart partial maxima pmax[r, :]
// (written by the kernel that produced the rows) instead of a first pass over
// the row.  Each lane takes 4 consecutive values per step, 4 steps of the
// wave per loop turn.
template <int SRC>
__global__ __launch_bounds__(kQWaves * kWave) void act_quant_kernel(const void* __restrict__ src, int64_t rows,
                                                                   int64_t K, const int32_t* __restrict__ sorted_ids,
                                                                   const int32_t* __restrict__ num_padded, int64_t Tk,
                                                                   const float* __restrict__ pmax, int64_t npart,
                                                                   int8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kQWaves + threadIdx.x / kWave;
  if (r >= rows) return;                                   // uniform per wave
  if (sorted_ids && (r >= *num_padded || sorted_ids[r] >= Tk)) return;
  const int64_t base = r * K;
  constexpr int64_t kSpan = 4 * kWave;
  float m;
  if (pmax) {
    m = 0.0f;
    for (int64_t i = lane; i < npart; i += kWave) m = fmaxf(m, pmax[r * npart + i]);
    m = wave_max(m);
  } else {
    float m4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t i = lane * 4;
    for (; i + 3 * kSpan < K; i += 4 * kSpan) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 v = load_act4<SRC>(src, base + i + u * kSpan);
        m4[u] = fmaxf(m4[u], fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
      }
    }
    for (; i < K; i += kSpan) {
      const f32x4 v = load_act4<SRC>(src, base + i);
      m4[0] = fmaxf(m4[0], fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
    m = wave_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  }
  const float s = m / 127.0f;
  if (lane == 0) scale[r] = s;
  auto code4 = [&](f32x4 v) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float c = 0.0f;
      if (s != 0.0f) c = fminf(fmaxf(rintf(v[j] / s), -127.0f), 127.0f);
      word |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xffu) << (8 * j);
    }
    return word;
  };
  int64_t i = lane * 4;
  for (; i + 3 * kSpan < K; i += 4 * kSpan) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load_act4<SRC>(src, base + i + u * kSpan);
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint32_t*>(q + base + i + u * kSpan) = code4(v[u]);
  }
  for (; i < K; i += kSpan) *reinterpret_cast<uint32_t*>(q + base + i) = code4(load_act4<SRC>(src, base + i));
}

// One workgroup per (row, chunk of 1024 U values): the same scale and codes
// as act_quant_kernel with every load of the chunk in flight at once (a wave
// walking a whole row pays one memory latency per loop turn).  The row
// maximum comes from pmax or, when one chunk covers the row, from the chunk.
template <int SRC, int U>
__global__ __launch_bounds__(kThreads) void act_quant_rows_kernel(const void* __restrict__ src, int64_t K,
                                                                  const int32_t* __restrict__ sorted_ids,
                                                                  const int32_t* __restrict__ num_padded, int64_t Tk,
                                                                  const float* __restrict__ pmax, int64_t npart,
                                                                  int8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[kThreads / kWave];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  if (sorted_ids && (r >= *num_padded || sorted_ids[r] >= Tk)) return;   // uniform per workgroup
  const int64_t base = r * K;
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * (1024 * U);
  f32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = c0 + (u * kThreads + tid) * 4;
    v[u] = i < K ? load_act4<SRC>(src, base + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m = 0.0f;
  if (pmax) {
    for (int64_t i = tid; i < npart; i += kThreads) m = fmaxf(m, pmax[r * npart + i]);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3]))));
  }
  m = wave_max(m);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m / 127.0f;
  if (blockIdx.y == 0 && tid == 0) scale[r] = s;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = c0 + (u * kThreads + tid) * 4;
    if (i < K) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float c = 0.0f;
        if (s != 0.0f) c = fminf(fmaxf(rintf(v[u][j] / s), -127.0f), 127.0f);
        word |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xffu) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(q + base + i) = word;
    }
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm1_w8a8_kernel(const Gemm1Args p, const int8_t* __restrict__ qx,
                                                              const float* __restrict__ sx) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * p.block_m;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16;
  const int64_t I = p.I, H = p.H;
  const int8_t* wg = p.w13 + (static_cast<int64_t>(e) * 2 * I + n0 + col) * p.ldw + kg * 16;
  const int8_t* wu = wg + I * p.ldw;
  const float sg = p.s13[static_cast<int64_t>(e) * 2 * I + n0 + col];
  const float su = p.s13[static_cast<int64_t>(e) * 2 * I + I + n0 + col];
  float* a = p.a;

  for (int rc = 0; rc < p.block_m; rc += 16 * MT) {
    if (p.sorted_ids[row0 + rc] >= p.Tk) break;             // the rest of the block is padding
    const int8_t* xr[MT];
    bool valid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int f = p.sorted_ids[row0 + rc + mt * 16 + col];
      valid[mt] = f < p.Tk;
      xr[mt] = qx + (valid[mt] ? f / p.k : 0) * H + kg * 16;
    }
    i32x4 accg[MT], accu[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accg[mt] = i32x4{0, 0, 0, 0};
      accu[mt] = i32x4{0, 0, 0, 0};
    }
    for (int64_t k0 = 0; k0 < H; k0 += kStep) {
      const u32x4 g0 = ld16(wg + k0), g1 = ld16(wg + k0 + 64);
      const u32x4 u0 = ld16(wu + k0), u1 = ld16(wu + k0 + 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a0 = valid[mt] ? ld16(xr[mt] + k0) : u32x4{0u, 0u, 0u, 0u};
        const u32x4 a1 = valid[mt] ? ld16(xr[mt] + k0 + 64) : u32x4{0u, 0u, 0u, 0u};
        accg[mt] = mfma_i8(a0, g0, accg[mt]);
        accg[mt] = mfma_i8(a1, g1, accg[mt]);
        accu[mt] = mfma_i8(a0, u0, accu[mt]);
        accu[mt] = mfma_i8(a1, u1, accu[mt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + rc + mt * 16 + kg * 4 + i;
        const int f = p.sorted_ids[r];
        if (f < p.Tk) {
          const float st = sx[f / p.k];
          a[r * I + n0 + col] = silu_mul(static_cast<float>(accg[mt][i]) * st * sg,
                                         static_cast<float>(accu[mt][i]) * st * su);
        }
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gemm2_w8a8_kernel(const Gemm2Args p, const int8_t* __restrict__ qa,
                                                              const float* __restrict__ sa) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * p.block_m;
  if (row0 >= *p.num_padded) return;
  const int e = p.block_expert[blockIdx.y];
  const int64_t h0 = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32;
  const int64_t I = p.I, H = p.H;
  const int64_t kc = I / p.splits;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * kc;
  const int8_t* w0 = p.w2 + (static_cast<int64_t>(e) * H + h0 + col) * p.ldw + kbeg + kg * 16;
  const int8_t* w1 = w0 + 16 * p.ldw;
  const float s0 = p.s2[static_cast<int64_t>(e) * H + h0 + col];
  const float s1 = p.s2[static_cast<int64_t>(e) * H + h0 + 16 + col];

  for (int rc = 0; rc < p.block_m; rc += 16 * MT) {
    if (p.sorted_ids[row0 + rc] >= p.Tk) break;
    const int8_t* ar[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ar[mt] = qa + (row0 + rc + mt * 16 + col) * I + kbeg + kg * 16;
    i32x4 acc0[MT], acc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = i32x4{0, 0, 0, 0};
      acc1[mt] = i32x4{0, 0, 0, 0};
    }
    for (int64_t k0 = 0; k0 < kc; k0 += kStep) {
      const u32x4 b00 = ld16(w0 + k0), b01 = ld16(w0 + k0 + 64);
      const u32x4 b10 = ld16(w1 + k0), b11 = ld16(w1 + k0 + 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 a0 = ld16(ar[mt] + k0), a1 = ld16(ar[mt] + k0 + 64);
        acc0[mt] = mfma_i8(a0, b00, acc0[mt]);
        acc0[mt] = mfma_i8(a1, b01, acc0[mt]);
        acc1[mt] = mfma_i8(a0, b10, acc1[mt]);
        acc1[mt] = mfma_i8(a1, b11, acc1[mt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + rc + mt * 16 + kg * 4 + i;
        const int f = p.sorted_ids[r];
        if (f < p.Tk) {
          const float sr = sa[r];
          float* yr = p.y + (static_cast<int64_t>(blockIdx.z) * p.Tk + f) * H + h0 + col;
          yr[0] = static_cast<float>(acc0[mt][i]) * sr * s0;
          yr[16] = static_cast<float>(acc1[mt][i]) * sr * s1;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_act_quant(const void* src, int src_type, int64_t rows, int64_t K, const int32_t* sorted_ids,
                            const int32_t* num_padded, int64_t Tk, const float* pmax, int64_t npart, int8_t* q,
                            float* scale, hipStream_t stream) {
  if (K % 4 || reinterpret_cast<uintptr_t>(src) % (src_type == 2 ? 16 : 8)) return hipErrorInvalidValue;
  constexpr int kU = 4;
  if (rows <= 0) return hipSuccess;
  if (pmax || K <= 1024 * kU) {
    const dim3 g(static_cast<unsigned>(rows), static_cast<unsigned>((K + 1024 * kU - 1) / (1024 * kU)));
#define AQR(S)                                                                                                   \
  hipLaunchKernelGGL((act_quant_rows_kernel<S, kU>), g, dim3(kThreads), 0, stream, src, K, sorted_ids, num_padded, \
                     Tk, pmax, npart, q, scale)
    if (src_type == 0) AQR(0);
    else if (src_type == 1) AQR(1);
    else AQR(2);
#undef AQR
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((rows + kQWaves - 1) / kQWaves)), block(kQWaves * kWave);
  if (src_type == 0)
    hipLaunchKernelGGL(act_quant_kernel<0>, grid, block, 0, stream, src, rows, K, sorted_ids, num_padded, Tk, pmax, npart,
                       q, scale);
  else if (src_type == 1)
    hipLaunchKernelGGL(act_quant_kernel<1>, grid, block, 0, stream, src, rows, K, sorted_ids, num_padded, Tk, pmax, npart,
                       q, scale);
  else
    hipLaunchKernelGGL(act_quant_kernel<2>, grid, block, 0, stream, src, rows, K, sorted_ids, num_padded, Tk, pmax, npart,
                       q, scale);
  return hipGetLastError();
}

hipError_t launch_gemm1_w8a8(const Gemm1Args& p, const int8_t* qx, const float* sx, hipStream_t stream) {
  if (p.I % 64 || p.H % kStep || p.block_m % 16) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.I / 64), static_cast<unsigned>(p.cap / p.block_m));
  if (p.block_m % 64 == 0)
    hipLaunchKernelGGL((gemm1_w8a8_kernel<4>), grid, dim3(kThreads), 0, stream, p, qx, sx);
  else if (p.block_m % 32 == 0)
    hipLaunchKernelGGL((gemm1_w8a8_kernel<2>), grid, dim3(kThreads), 0, stream, p, qx, sx);
  else
    hipLaunchKernelGGL((gemm1_w8a8_kernel<1>), grid, dim3(kThreads), 0, stream, p, qx, sx);
  return hipGetLastError();
}

hipError_t launch_gemm2_w8a8(const Gemm2Args& p, const int8_t* qa, const float* sa, hipStream_t stream) {
  if (p.H % 128 || p.I % (kStep * p.splits) || p.block_m % 16) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(p.H / 128), static_cast<unsigned>(p.cap / p.block_m),
                  static_cast<unsigned>(p.splits));
  if (p.block_m % 64 == 0)
    hipLaunchKernelGGL((gemm2_w8a8_kernel<4>), grid, dim3(kThreads), 0, stream, p, qa, sa);
  else if (p.block_m % 32 == 0)
    hipLaunchKernelGGL((gemm2_w8a8_kernel<2>), grid, dim3(kThreads), 0, stream, p, qa, sa);
  else
    hipLaunchKernelGGL((gemm2_w8a8_kernel<1>), grid, dim3(kThreads), 0, stream, p, qa, sa);
  return hipGetLastError();
}

}  // namespace moe
