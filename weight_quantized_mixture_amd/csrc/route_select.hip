// Routing with the options select_experts takes on the pages: scoring
// function (softmax or sigmoid), grouped top-k (num_expert_group groups of
// consecutive experts, topk_group of them kept), a score-correction bias that
// only steers the choice, and a routed scaling factor on the weights
// (experts_int8 page, ExpertsInt8MoEMethod.apply -> select_experts;
// moe_wna16 page, MoeWNA16Method.apply_monolithic).
//
// One wave64 per token, lane l holding experts l, l+64, ... (E <= 1024):
//   * scores s_e in fp64 (softmax with a fixed-order butterfly sum, or
//     sigmoid), so that their fp32 rounding is the correctly rounded value
//     (up to fp64's own error) on every side that takes decisions on it;
//   * choice key: the fp32 logit without a bias (the order of the scores),
//     else fp32(s_e) + bias_e added in fp32; keys become 64-bit integers that
//     order larger keys first and equal keys by lower id;
//   * groups: lane g < G takes the largest key of group g; a group stays when
//     fewer than topk_group groups beat it; the keys of the other experts are
//     set to 0, which never wins;
//   * every expert counts the keys in LDS that beat it; rank j < k is winner j;
//   * weights: the chosen s, renormalised in fp64 when asked, times the
//     scaling factor, rounded to fp32.
#include "launch.hpp"
#include "router_dev.hpp"

namespace moe {

namespace {

constexpr int kSelWaves = 4;
constexpr int kSelMaxGroups = 64;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The wave's own LDS writes are visible to its reads after they complete.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_wave_barrier();
}

template <int NPL>
__global__ __launch_bounds__(kSelWaves * kWave) void route_select_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renormalize, int sigmoid, int G, int topk_group,
    const float* __restrict__ bias, float scale, float* __restrict__ topk_w, int32_t* __restrict__ topk_ids) {
  __shared__ __attribute__((aligned(16))) uint64_t keys_all[kSelWaves][NPL * kWave];
  __shared__ uint64_t gkeys_all[kSelWaves][kSelMaxGroups];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kSelWaves + w;
  if (t >= T) return;                      // uniform per wave
  uint64_t* keys = keys_all[w];
  uint64_t* gkeys = gkeys_all[w];
  const float* lr = logits + t * E;

  float lf[NPL];
  double s[NPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    lf[i] = e < E ? lr[e] : -INFINITY;
    if (e < E) m = fmaxf(m, lf[i]);
  }
  if (!sigmoid) {
    m = wave_max(m);
    double z = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      s[i] = e < E ? exp(static_cast<double>(lf[i]) - static_cast<double>(m)) : 0.0;
      z += s[i];
    }
    z = wave_sum_f64(z);
#pragma unroll
    for (int i = 0; i < NPL; ++i) s[i] /= z;
  } else {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      s[i] = e < E ? 1.0 / (1.0 + exp(-static_cast<double>(lf[i]))) : 0.0;
    }
  }

  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    const float c = bias ? static_cast<float>(s[i]) + bias[e < E ? e : 0] : lf[i];
    key[i] = e < E ? route_key(c, e) : 0ull;
  }

  if (G > 1) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      if (e < E) keys[e] = key[i];
    }
    wave_lds_sync();
    const int gs = E / G;
    uint64_t gk = 0;
    if (lane < G)
      for (int j = 0; j < gs; ++j) {
        const uint64_t v = keys[lane * gs + j];
        gk = v > gk ? v : gk;
      }
    gkeys[lane] = gk;
    wave_lds_sync();
    int grank = 0;
    if (lane < G)
      for (int g = 0; g < G; ++g) grank += gkeys[g] > gk ? 1 : 0;
    const uint64_t keep = __ballot(lane < G && grank < topk_group);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((keep >> (e / gs)) & 1ull)) key[i] = 0ull;
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E) keys[e] = key[i];
  }
  wave_lds_sync();

  int rank[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) rank[i] = 0;
  for (int q = 0; q < E; ++q) {
    const uint64_t kq = keys[q];
#pragma unroll
    for (int i = 0; i < NPL; ++i) rank[i] += kq > key[i] ? 1 : 0;
  }
  double psum = 0.0;
  bool win[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    win[i] = e < E && key[i] != 0ull && rank[i] < k;
    if (win[i]) psum += s[i];
  }
  psum = wave_sum_f64(psum);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    if (win[i]) {
      const double wv = (renormalize ? s[i] / psum : s[i]) * static_cast<double>(scale);
      topk_ids[t * k + rank[i]] = lane + i * kWave;
      topk_w[t * k + rank[i]] = static_cast<float>(wv);
    }
  }
}

}  // namespace

hipError_t launch_route_select(const float* logits, int64_t T, int E, int k, int renormalize, int sigmoid, int G,
                               int topk_group, const float* bias, float scale, float* topk_w, int32_t* topk_ids,
                               hipStream_t stream) {
  if (E < 1 || E > 16 * kWave || (G > 1 && (G > kSelMaxGroups || E % G != 0))) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((T + kSelWaves - 1) / kSelWaves)), block(kSelWaves * kWave);
#define SEL(NPL)                                                                                         \
  hipLaunchKernelGGL(route_select_kernel<NPL>, grid, block, 0, stream, logits, T, E, k, renormalize, sigmoid, \
                     G, topk_group, bias, scale, topk_w, topk_ids)
  if (E <= kWave) SEL(1);
  else if (E <= 2 * kWave) SEL(2);
  else if (E <= 4 * kWave) SEL(4);
  else if (E <= 8 * kWave) SEL(8);
  else SEL(16);
#undef SEL
  return hipGetLastError();
}

}  // namespace moe
