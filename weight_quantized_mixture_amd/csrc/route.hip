// Softmax top-k router (experts_int8 page, ExpertsInt8MoEMethod.apply ->
// select_experts with scoring_func "softmax", top_k, renormalize).
//
// One wave64 per token.  Lane l holds logits l, l+64, ... (E <= 1024, so at
// most 16 per lane).  The softmax denominator is a fixed-order butterfly
// sum; the k winners are found by k rounds of a wave arg-max on the fp32
// logits (equal logits: lower id), so ids are exact comparisons of the
// inputs.  p_j = exp(l_j - max) / sum; with renormalize the chosen p are
// divided by their sum (j ascending), which makes a single winner weigh 1.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;
constexpr int kMaxPerLane = 16;   // 16 * 64 = 1024 experts

__device__ __forceinline__ bool better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

__global__ __launch_bounds__(kRouteWaves * kWave) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renormalize,
    float* __restrict__ topk_w, int32_t* __restrict__ topk_ids) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteWaves + (threadIdx.x / kWave);
  if (t >= T) return;
  const float* lr = logits + t * E;

  float v[kMaxPerLane];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = (e < E) ? lr[e] : -INFINITY;
    if (e < E) m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    if (e < E) z += expf(v[i] - m);
  }
  z = wave_sum(z);

  uint32_t taken = 0;   // bit i: slot i of this lane already chosen
  float psum = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bid)) {
        bv = v[i];
        bid = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oid = __shfl_xor(bid, o, kWave);
      if (better(ov, oid, bv, bid)) {
        bv = ov;
        bid = oid;
      }
    }
    if ((bid & (kWave - 1)) == lane) taken |= 1u << (bid / kWave);
    const float p = expf(bv - m) / z;
    psum += p;
    if (lane == 0) {
      topk_ids[t * k + j] = bid;
      topk_w[t * k + j] = p;
    }
  }
  if (renormalize && lane == 0) {
    for (int j = 0; j < k; ++j) topk_w[t * k + j] = topk_w[t * k + j] / psum;
  }
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
