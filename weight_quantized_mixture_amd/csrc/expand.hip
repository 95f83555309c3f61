// Routing extensions ahead of the align step.
//
// Shared experts (moe_wna16 page, MoeWNA16Method.apply: shared_experts, whose
// output is added to the routed output): the S shared experts sit after the
// E routed ones in the weight tensors and every token takes all of them with
// weight 1, so the routing of a token grows from k to k + S columns.
//
// apply_router_weight_on_input (experts_int8 page, ExpertsInt8MoEMethod.apply
// -> fused_experts): the routing weight scales the expert's input instead of
// its output.  Every assignment f = t*(k+S) + j then gets its own input row
// rne(w[t, j] * x[t]) (fp32 product rounded to the activation type; weight 1
// for the shared experts), GEMM1 reads row f, and the combine weights are 1.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// One thread per extended assignment (t, j), j < k + S.
__global__ __launch_bounds__(256) void expand_routing_kernel(const float* __restrict__ topk_w,
                                                             const int32_t* __restrict__ topk_ids, int64_t T, int k,
                                                             int S, int E, int weight_on_input,
                                                             float* __restrict__ w_ext,
                                                             int32_t* __restrict__ ids_ext) {
  const int kx = k + S;
  const int64_t f = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (f >= T * kx) return;
  const int64_t t = f / kx;
  const int j = static_cast<int>(f % kx);
  if (j < k) {
    const int32_t id = topk_ids[t * k + j];
    ids_ext[f] = id >= 0 && id < E ? id : -1;      // a routed id never lands on a shared expert
    w_ext[f] = weight_on_input ? 1.0f : topk_w[t * k + j];
  } else {
    ids_ext[f] = E + (j - k);
    w_ext[f] = 1.0f;
  }
}

// One thread per 8 consecutive activations of one extended row.
template <bool F16>
__global__ __launch_bounds__(256) void prescale_input_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ topk_w, int64_t T, int k,
                                                             int S, int64_t H, uint16_t* __restrict__ x_ext) {
  const int kx = k + S;
  const int64_t H8 = H / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= T * kx * H8) return;
  const int64_t f = idx / H8;
  const int64_t h = (idx % H8) * 8;
  const int64_t t = f / kx;
  const int j = static_cast<int>(f % kx);
  const float w = j < k ? topk_w[t * k + j] : 1.0f;
  const u32x4 v = *reinterpret_cast<const u32x4*>(x + t * H + h);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = static_cast<uint16_t>(v[i] & 0xffffu), hi = static_cast<uint16_t>(v[i] >> 16);
    if constexpr (F16) {
      r[i] = static_cast<uint32_t>(f32_to_f16(w * f16_to_f32(lo))) |
             (static_cast<uint32_t>(f32_to_f16(w * f16_to_f32(hi))) << 16);
    } else {
      r[i] = static_cast<uint32_t>(f32_to_bf16(w * bf16_to_f32(lo))) |
             (static_cast<uint32_t>(f32_to_bf16(w * bf16_to_f32(hi))) << 16);
    }
  }
  *reinterpret_cast<u32x4*>(x_ext + f * H + h) = r;
}

}  // namespace

hipError_t launch_expand_routing(const float* topk_w, const int32_t* topk_ids, int64_t T, int k, int S, int E,
                                 int weight_on_input, float* w_ext, int32_t* ids_ext, hipStream_t stream) {
  const int64_t n = T * (k + S);
  hipLaunchKernelGGL(expand_routing_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     topk_w, topk_ids, T, k, S, E, weight_on_input, w_ext, ids_ext);
  return hipGetLastError();
}

hipError_t launch_prescale_input(const void* x, int f16, const float* topk_w, int64_t T, int k, int S, int64_t H,
                                 void* x_ext, hipStream_t stream) {
  if (H % 8) return hipErrorInvalidValue;
  const int64_t n = T * (k + S) * (H / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(prescale_input_kernel<true>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       topk_w, T, k, S, H, static_cast<uint16_t*>(x_ext));
  else
    hipLaunchKernelGGL(prescale_input_kernel<false>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       topk_w, T, k, S, H, static_cast<uint16_t*>(x_ext));
  return hipGetLastError();
}

}  // namespace moe
