// Softmax top-k router, one wave64 per token (the per-token routine is in
// router_dev.hpp; experts_int8 page, ExpertsInt8MoEMethod.apply ->
// select_experts with scoring_func "softmax", top_k, renormalize).
#include "launch.hpp"
#include "router_dev.hpp"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;

__global__ __launch_bounds__(kRouteWaves * kWave) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renormalize,
    float* __restrict__ topk_w, int32_t* __restrict__ topk_ids) {
  __shared__ __attribute__((aligned(16))) uint64_t keys[kRouteWaves][kRankMaxExperts];
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteWaves + (threadIdx.x / kWave);
  if (t >= T) return;
  route_token(logits + t * E, E, k, renormalize, topk_w + t * k, topk_ids + t * k, keys[threadIdx.x / kWave]);
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renormalize,
                        float* topk_w, int32_t* topk_ids, hipStream_t stream) {
  const int64_t blocks = (T + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_topk_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kRouteWaves * kWave),
                     0, stream, logits, T, E, k, renormalize, topk_w, topk_ids);
  return hipGetLastError();
}

}  // namespace moe
