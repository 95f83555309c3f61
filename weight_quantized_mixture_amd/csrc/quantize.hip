// Weight quantizers (offline: run once when the expert weights are loaded).
//
// int8: experts_int8 page, quantize_in_place_and_get_scales -- per output
// channel (row) symmetric: s = max|w| / 127, q = clamp(rint(w / s), -127, 127),
// fp32 IEEE division (HIP's default `/` on float is correctly rounded; no
// fast-math), rint = round half to even (v_rndne_f32).
//
// uint4: moe_wna16 page, MoeWNA16Method.create_weights gives the packed
// layout; the quantizer itself is the min/max reading stated in moe_wq.h.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kQThreads = 256;

// One workgroup per row: a max-abs reduction, then the divide / round / clamp.
__global__ __launch_bounds__(kQThreads) void quantize_int8_rows_kernel(
    const float* __restrict__ w, int64_t K, int8_t* __restrict__ q, float* __restrict__ scale,
    int vec) {
  __shared__ float red[kQThreads / kWave];
  const int64_t row = blockIdx.x;
  const float* wr = w + row * K;
  int8_t* qr = q + row * K;
  const int tid = threadIdx.x;

  float m = 0.0f;
  if (vec) {
    const float4* w4 = reinterpret_cast<const float4*>(wr);
    for (int64_t i = tid; i < K / 4; i += kQThreads) {
      const float4 v = w4[i];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  } else {
    for (int64_t i = tid; i < K; i += kQThreads) m = fmaxf(m, fabsf(wr[i]));
  }
  m = wave_max(m);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < kQThreads / kWave; ++i) m = fmaxf(m, red[i]);

  const float s = m / 127.0f;            // IEEE divide
  if (tid == 0) scale[row] = s;
  const bool zero = (s == 0.0f);

  auto code = [&](float v) -> int {
    if (zero) return 0;
    float r = rintf(v / s);              // IEEE divide, half to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
  };
  if (vec) {
    const float4* w4 = reinterpret_cast<const float4*>(wr);
    uint32_t* q4 = reinterpret_cast<uint32_t*>(qr);
    for (int64_t i = tid; i < K / 4; i += kQThreads) {
      const float4 v = w4[i];
      const uint32_t b0 = static_cast<uint32_t>(code(v.x)) & 0xffu;
      const uint32_t b1 = static_cast<uint32_t>(code(v.y)) & 0xffu;
      const uint32_t b2 = static_cast<uint32_t>(code(v.z)) & 0xffu;
      const uint32_t b3 = static_cast<uint32_t>(code(v.w)) & 0xffu;
      q4[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
  } else {
    for (int64_t i = tid; i < K; i += kQThreads) qr[i] = static_cast<int8_t>(code(wr[i]));
  }
}

// One thread per (expert, octet of rows, group): it quantizes the 8 rows of
// the group one after the other and packs their 8 zero points into one word.
__global__ __launch_bounds__(256) void quantize_w4_kernel(
    const float* __restrict__ w, int64_t E, int64_t N, int64_t K, int group,
    int32_t* __restrict__ qweight, uint16_t* __restrict__ scales, int32_t* __restrict__ qzeros) {
  const int64_t G = K / group;
  const int64_t N8 = N / 8;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= E * N8 * G) return;
  const int64_t g = id % G;
  const int64_t n8 = (id / G) % N8;
  const int64_t e = id / (G * N8);
  uint32_t zword = 0;
  for (int r = 0; r < 8; ++r) {
    const int64_t n = n8 * 8 + r;
    const float* src = w + ((e * N + n) * K + g * group);
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < group; ++i) {
      const float v = src[i];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    const float s32 = (hi - lo) / 15.0f;
    _Float16 s16 = static_cast<_Float16>(s32);     // round to nearest even
    float s = static_cast<float>(s16);
    if (s == 0.0f) {
      s = 1.0f;
      s16 = static_cast<_Float16>(1.0f);
    }
    const float z = fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
    scales[(e * N + n) * G + g] = __builtin_bit_cast(uint16_t, s16);
    zword |= static_cast<uint32_t>(z) << (4 * r);
    int32_t* dst = qweight + ((e * N + n) * (K / 8) + g * (group / 8));
    for (int wi = 0; wi < group / 8; ++wi) {
      uint32_t word = 0;
      for (int j = 0; j < 8; ++j) {
        const float qf = fminf(fmaxf(rintf(src[wi * 8 + j] / s) + z, 0.0f), 15.0f);
        word |= static_cast<uint32_t>(qf) << (4 * j);
      }
      dst[wi] = static_cast<int32_t>(word);
    }
  }
  qzeros[(e * N8 + n8) * G + g] = static_cast<int32_t>(zword);
}

}  // namespace

hipError_t launch_quantize_int8(const float* w, int64_t rows, int64_t K, int8_t* q, float* scale,
                                hipStream_t stream) {
  // rows may exceed the 2^31-1 grid limit only for absurd sizes; chunk anyway
  const int64_t kMaxGrid = 0x7fffffff;
  const int vec = (K % 4 == 0) && (reinterpret_cast<uintptr_t>(w) % 16 == 0) &&
                  (reinterpret_cast<uintptr_t>(q) % 4 == 0);
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGrid) {
    const int64_t n = rows - r0 < kMaxGrid ? rows - r0 : kMaxGrid;
    hipLaunchKernelGGL(quantize_int8_rows_kernel, dim3(static_cast<unsigned>(n)), dim3(kQThreads), 0,
                       stream, w + r0 * K, K, q + r0 * K, scale + r0, vec);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_w4(const float* w, int64_t E, int64_t N, int64_t K, int64_t group,
                              int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                              hipStream_t stream) {
  const int64_t total = E * (N / 8) * (K / group);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(quantize_w4_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, w,
                     E, N, K, static_cast<int>(group), qweight, scales, qzeros);
  return hipGetLastError();
}

}  // namespace moe
