// Weight-only fp8 experts: per-tensor e4m3fn quantization and the merge of
// the two w13 shard scales (fp8 page: Fp8MoEMethod.create_weights and
// process_weights_after_loading; scaled_fp8_quant and per_tensor_dequantize
// are only called there, read here as: scale = max|w| / 448 in fp32, code =
// e4m3fn(clamp(w / scale, -448, 448)) rounded to nearest even, dequantized
// value = fp32(code value * scale)).
//
// The encoder works on the fp32 bit pattern: below 2^-6 the e4m3 grid step is
// 2^-9, so the code is rint(a * 512) (an exact scaling; 8 lands on the code of
// 2^-6); from 2^-6 up the 23-bit mantissa is rounded to 3 bits, half to even,
// a carry moving into the exponent field.  The sign bit is the value's.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), kE4m3Max);
  if (a < 0.015625f) return static_cast<uint8_t>(sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f)));
  const uint32_t u = __float_as_uint(a);
  const uint32_t e = (u >> 23) - 120u;               // e4m3 exponent field: (e_fp32 - 127) + 7
  const uint32_t mant = u & 0x7FFFFFu;
  const uint32_t top = mant >> 20, rest = mant & 0xFFFFFu;
  const uint32_t up = rest > 0x80000u || (rest == 0x80000u && (top & 1u));
  return static_cast<uint8_t>(sign | (((e << 3) | top) + up));
}

// exact value of an e4m3fn code as fp32 (codes 0x7F / 0xFF never come from the encoder)
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t ex = (b >> 3) & 0xFu, m = b & 7u;
  const float mag = ex == 0 ? static_cast<float>(m) * 0.001953125f
                            : __uint_as_float(((ex + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// per-tensor maxima: amax[t] holds the fp32 bits of max |w| of tensor t (non-negative
// floats order like their bit patterns, so an unsigned atomic max is exact and order-free)
__global__ __launch_bounds__(256) void fp8_zero_kernel(uint32_t* __restrict__ amax, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

__global__ __launch_bounds__(256) void fp8_absmax_kernel(const float* __restrict__ w, int64_t per_tensor,
                                                         uint32_t* __restrict__ amax) {
  const int64_t t = blockIdx.y;
  const float* src = w + t * per_tensor;
  float m = 0.0f;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < per_tensor;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    m = fmaxf(m, fabsf(src[i]));
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(amax + t, __float_as_uint(m));
}

// scale[t] = fp32(max / 448) (in place over the maxima)
__global__ __launch_bounds__(256) void fp8_scale_kernel(uint32_t* __restrict__ amax_scale, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) amax_scale[i] = __float_as_uint(__uint_as_float(amax_scale[i]) / kE4m3Max);
}

__global__ __launch_bounds__(256) void fp8_encode_kernel(const float* __restrict__ w, int64_t per_tensor,
                                                         const float* __restrict__ scale, uint8_t* __restrict__ q) {
  const int64_t t = blockIdx.y;
  const float s = scale[t];
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < per_tensor;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float v = w[t * per_tensor + i];
    q[t * per_tensor + i] = s == 0.0f ? static_cast<uint8_t>(0) : f32_to_e4m3_sat(v / s);
  }
}

// w13 of expert e, shard sh (rows [sh I, (sh + 1) I)): dequantize with the shard's scale,
// quantize again with the larger of the two
__global__ __launch_bounds__(256) void fp8_merge_kernel(uint8_t* __restrict__ q13, const float* __restrict__ s_in,
                                                        int64_t IH, float* __restrict__ s_out) {
  const int64_t e = blockIdx.z, sh = blockIdx.y;
  const float s_own = s_in[2 * e + sh];
  const float s_max = fmaxf(s_in[2 * e], s_in[2 * e + 1]);
  uint8_t* base = q13 + (2 * e + sh) * IH;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < IH;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float dq = e4m3_to_f32(base[i]) * s_own;
    base[i] = s_max == 0.0f ? static_cast<uint8_t>(0) : f32_to_e4m3_sat(dq / s_max);
  }
  if (sh == 0 && blockIdx.x == 0 && threadIdx.x == 0) s_out[e] = s_max;
}

unsigned grid_x(int64_t per_tensor) {
  const int64_t b = (per_tensor + 255) / 256;
  return static_cast<unsigned>(b < 1024 ? b : 1024);
}

}  // namespace

hipError_t launch_quantize_fp8(const float* w, int64_t tensors, int64_t per_tensor, uint8_t* q, float* scale,
                               hipStream_t stream) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(scale);
  const unsigned tb = static_cast<unsigned>((tensors + 255) / 256);
  hipLaunchKernelGGL(fp8_zero_kernel, dim3(tb), dim3(256), 0, stream, bits, tensors);
  const dim3 grid(grid_x(per_tensor), static_cast<unsigned>(tensors));
  hipLaunchKernelGGL(fp8_absmax_kernel, grid, dim3(256), 0, stream, w, per_tensor, bits);
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(tb), dim3(256), 0, stream, bits, tensors);
  hipLaunchKernelGGL(fp8_encode_kernel, grid, dim3(256), 0, stream, w, per_tensor, scale, q);
  return hipGetLastError();
}

hipError_t launch_fp8_merge_w13(uint8_t* q13, const float* s_in, int64_t E, int64_t I, int64_t H, float* s_out,
                                hipStream_t stream) {
  const dim3 grid(grid_x(I * H), 2u, static_cast<unsigned>(E));
  hipLaunchKernelGGL(fp8_merge_kernel, grid, dim3(256), 0, stream, q13, s_in, I * H, s_out);
  return hipGetLastError();
}

}  // namespace moe
