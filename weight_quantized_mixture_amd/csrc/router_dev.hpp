// Device-side pieces shared by the router and the fused route + align kernel.
//
// Softmax top-k for one token on one wave64 (experts_int8 page,
// ExpertsInt8MoEMethod.apply -> select_experts with scoring_func "softmax",
// top_k, renormalize): lane l holds logits l, l+64, ... (E <= 1024); the
// softmax denominator is a fixed-order butterfly sum; the k winners come from
// k rounds of a wave arg-max on the fp32 logits (equal logits: lower id), so
// ids are exact comparisons of the inputs; p_j = exp(l_j - max) / sum, and
// with renormalize the chosen p are divided by their sum (j ascending).
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kMaxPerLane = 16;   // 16 * 64 = 1024 experts

__device__ __forceinline__ bool route_better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

// Routes token t; lane 0 writes topk_w[t*k + j] and topk_ids[t*k + j].
__device__ __forceinline__ void route_token(const float* __restrict__ lr, int E, int k, int renormalize,
                                            float* __restrict__ tw, int32_t* __restrict__ ti) {
  const int lane = threadIdx.x & (kWave - 1);
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
  float my_p = 0.0f;    // lane j keeps the j-th winner (k <= 64)
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((taken >> i) & 1u) && route_better(v[i], e, bv, bid)) {
        bv = v[i];
        bid = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oid = __shfl_xor(bid, o, kWave);
      if (route_better(ov, oid, bv, bid)) {
        bv = ov;
        bid = oid;
      }
    }
    if ((bid & (kWave - 1)) == lane) taken |= 1u << (bid / kWave);
    const float p = expf(bv - m) / z;
    psum += p;
    if (j < kWave) {
      if (lane == j) {
        my_p = p;
        my_id = bid;
      }
    } else if (lane == 0) {
      ti[j] = bid;
      tw[j] = p;
    }
  }
  // the first 64 winners are written by the lanes that hold them (no store is
  // read back); renormalisation divides by the sum taken in j order
  if (lane < k) {
    ti[lane] = my_id;
    tw[lane] = renormalize ? my_p / psum : my_p;
  }
  if (renormalize && lane == 0) {
    for (int j = kWave; j < k; ++j) tw[j] = tw[j] / psum;
  }
}

}  // namespace moe
