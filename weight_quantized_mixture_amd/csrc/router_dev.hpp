// Device-side pieces shared by the router and the fused route + align kernel.
//
// Softmax top-k for one token on one wave64 (experts_int8 page,
// ExpertsInt8MoEMethod.apply -> select_experts with scoring_func "softmax",
// top_k, renormalize): lane l holds logits l, l+64, ... (E <= 1024); the
// softmax denominator is a fixed-order butterfly sum; the winners are ordered
// by fp32 logit, descending, equal logits by lower id, so ids are exact
// comparisons of the inputs; p_j = exp(l_j - max) / sum, and with
// renormalize the chosen p are divided by their sum.
//   * E <= 256 (route_token_rank): every logit's rank (the number of logits
//     that beat it) is counted against all E keys in LDS; the logits of rank
//     j < k are winner j.  Two comparisons per pair, no shuffle chains.
//   * larger E (route_token_argmax): k rounds of a wave arg-max.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kMaxPerLane = 16;   // 16 * 64 = 1024 experts
constexpr int kRankMaxExperts = 256;   // rank path: per-wave LDS of 256 keys

// 64-bit key ordering logits as the router does: larger logit first, equal
// logits by lower id (-0 is taken as +0, as the float comparison does).
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~e);
}

// E <= 64 NPL; `keys` is this wave's LDS area of kRankMaxExperts keys.
template <int NPL>
__device__ __forceinline__ void route_token_rank(const float* __restrict__ lr, int E, int k, int renormalize,
                                                 float* __restrict__ tw, int32_t* __restrict__ ti,
                                                 uint64_t* __restrict__ keys) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[NPL];
  uint64_t key[NPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    v[i] = (e < E) ? lr[e] : -INFINITY;
    key[i] = route_key(v[i], e);
    if (e < E) m = fmaxf(m, v[i]);
    keys[e] = e < E ? key[i] : 0ull;   // slots past E never win
  }
  m = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    if (lane + i * kWave < E) z += expf(v[i] - m);
  z = wave_sum(z);
  // the wave's own LDS writes are visible to its reads after they complete
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_wave_barrier();
  int rank[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) rank[i] = 0;
  // 8 pairs of keys per turn, all read before the first comparison (read one
  // at a time, each pair costs a full LDS latency: 64 turns at E = 128).
  // Turns past E read the zero keys the lanes wrote after the last expert
  // (they write all 64 NPL slots, a multiple of the 16 keys a turn reads),
  // which no key exceeds.
  const int epairs = (E + 1) / 2;
  for (int q = 0; q < epairs; q += 8) {
    u32x4 kk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kk[j] = *reinterpret_cast<const u32x4*>(keys + 2 * (q + j));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t k0 = (static_cast<uint64_t>(kk[j].y) << 32) | kk[j].x;
      const uint64_t k1 = (static_cast<uint64_t>(kk[j].w) << 32) | kk[j].z;
#pragma unroll
      for (int i = 0; i < NPL; ++i) rank[i] += (k0 > key[i] ? 1 : 0) + (k1 > key[i] ? 1 : 0);
    }
  }
  float pc[NPL];
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    pc[i] = 0.0f;
    if (e < E && rank[i] < k) {
      pc[i] = expf(v[i] - m) / z;
      psum += pc[i];
    }
  }
  if (renormalize) psum = wave_sum(psum);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E && rank[i] < k) {
      ti[rank[i]] = e;
      tw[rank[i]] = renormalize ? pc[i] / psum : pc[i];
    }
  }
}

__device__ __forceinline__ bool route_better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

// k rounds of a wave arg-max (any E <= 1024).
__device__ __forceinline__ void route_token_argmax(const float* __restrict__ lr, int E, int k, int renormalize,
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

// Routes one token: writes topk_w[0..k) and topk_ids[0..k) of it.  `keys`
// is this wave's LDS area of kRankMaxExperts keys (used when E <= 256).
__device__ __forceinline__ void route_token(const float* __restrict__ lr, int E, int k, int renormalize,
                                            float* __restrict__ tw, int32_t* __restrict__ ti,
                                            uint64_t* __restrict__ keys) {
  if (E <= kWave) route_token_rank<1>(lr, E, k, renormalize, tw, ti, keys);
  else if (E <= 2 * kWave) route_token_rank<2>(lr, E, k, renormalize, tw, ti, keys);
  else if (E <= kRankMaxExperts) route_token_rank<4>(lr, E, k, renormalize, tw, ti, keys);
  else route_token_argmax(lr, E, k, renormalize, tw, ti);
}

}  // namespace moe
