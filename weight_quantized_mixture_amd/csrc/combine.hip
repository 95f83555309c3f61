// Routing-weighted top-k combine (experts_int8 page, ExpertsInt8MoEMethod.apply:
// fused_experts with apply_router_weight_on_input=False, so the routing weight
// multiplies each expert's output; inplace=True lets `out` be the input buffer).
//
// out[t, h] = sum_j topk_w[t, j] * sum_s y[s, t*k + j, h], fp32, j and s
// ascending, one writer per output element (no atomics: bitwise deterministic),
// then rounded to the activation type.  Each thread owns 4 consecutive h.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// BATCH: the split partials of a row are loaded 8 at a time so that their
// loads are in flight together (the sums still run in ascending s); only for
// many splits, which come with few tokens: the batch needs 96 registers where
// the plain loop needs 26, which would cut the occupancy of the large-T
// launches.
template <bool F16, bool BATCH>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int splits,
                                                      int64_t T, int k, int64_t H, int E,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ topk_ids,
                                                      void* __restrict__ out) {
  const int64_t H4 = H / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= T * H4) return;
  const int64_t t = idx / H4;
  const int64_t h = (idx % H4) * 4;
  const int64_t Tk = T * k;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int64_t f = t * k + j;
    const int e = topk_ids[f];
    if (e < 0 || e >= E) continue;
    const float wj = topk_w[f];
    float4 ys = *reinterpret_cast<const float4*>(y + f * H + h);
    int s = 1;
    for (; BATCH && s + 7 < splits; s += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(y + ((s + u) * Tk + f) * H + h);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ys.x += v[u].x; ys.y += v[u].y; ys.z += v[u].z; ys.w += v[u].w;
      }
    }
    for (; s < splits; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(y + (s * Tk + f) * H + h);
      ys.x += v.x; ys.y += v.y; ys.z += v.z; ys.w += v.w;
    }
    acc.x += wj * ys.x; acc.y += wj * ys.y; acc.z += wj * ys.z; acc.w += wj * ys.w;
  }
  uint2 packed;
  if constexpr (F16) {
    packed.x = static_cast<uint32_t>(f32_to_f16(acc.x)) | (static_cast<uint32_t>(f32_to_f16(acc.y)) << 16);
    packed.y = static_cast<uint32_t>(f32_to_f16(acc.z)) | (static_cast<uint32_t>(f32_to_f16(acc.w)) << 16);
  } else {
    packed.x = pack_bf16_rne(acc.x, acc.y);
    packed.y = pack_bf16_rne(acc.z, acc.w);
  }
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * H + h) = packed;
}

// Few tokens (decode): the latency of one dependent load is most of the
// kernel, so every partial of the thread's 4 outputs and every slot's id and
// weight are requested before the first is used.  KMAX x SMAX <= 32 register
// slots cover k <= KMAX slots of splits <= SMAX partials; slots past (k,
// splits) re-read a valid partial and are not added, so the loads need no
// branches.  Same sums, in the same order, as combine_kernel.
template <bool F16, int KMAX, int SMAX>
__global__ __launch_bounds__(256) void combine_few_kernel(const float* __restrict__ y, int splits,
                                                          int64_t T, int k, int64_t H, int E,
                                                          const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ topk_ids,
                                                          void* __restrict__ out) {
  const int64_t H4 = H / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= T * H4) return;
  const int64_t t = idx / H4;
  const int64_t h = (idx % H4) * 4;
  const int64_t Tk = T * k;
  float4 v[KMAX][SMAX];
  int eid[KMAX];
  float wk[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int64_t f = t * k + (j < k ? j : 0);
    eid[j] = topk_ids[f];
    wk[j] = topk_w[f];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int64_t sl = s < splits ? s : 0;
      v[j][s] = *reinterpret_cast<const float4*>(y + (sl * Tk + f) * H + h);
    }
  }
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float4 ys = v[j][0];
#pragma unroll
    for (int s = 1; s < SMAX; ++s) {
      if (s < splits) {
        ys.x += v[j][s].x; ys.y += v[j][s].y; ys.z += v[j][s].z; ys.w += v[j][s].w;
      }
    }
    if (j < k && eid[j] >= 0 && eid[j] < E) {
      const float wj = wk[j];
      acc.x += wj * ys.x; acc.y += wj * ys.y; acc.z += wj * ys.z; acc.w += wj * ys.w;
    }
  }
  uint2 packed;
  if constexpr (F16) {
    packed.x = static_cast<uint32_t>(f32_to_f16(acc.x)) | (static_cast<uint32_t>(f32_to_f16(acc.y)) << 16);
    packed.y = static_cast<uint32_t>(f32_to_f16(acc.z)) | (static_cast<uint32_t>(f32_to_f16(acc.w)) << 16);
  } else {
    packed.x = pack_bf16_rne(acc.x, acc.y);
    packed.y = pack_bf16_rne(acc.z, acc.w);
  }
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * H + h) = packed;
}

// Few tokens with more (slot, split) partials than combine_few_kernel holds
// in registers (k <= 16 slots, splits <= SMAX): a workgroup covers 64
// consecutive 4-element groups, wave w sums the split partials of slots w,
// w+4, ... (all loads of a slot in flight together, added in ascending s)
// into LDS, and wave 0 adds the weighted slots in ascending j.  Same sums, in
// the same order, as combine_kernel; each slot's partials cost one memory
// round trip instead of one per split.
constexpr int kWideMaxK = 16;

template <bool F16, int SMAX>
__global__ __launch_bounds__(256) void combine_wide_kernel(const float* __restrict__ y, int splits,
                                                           int64_t T, int k, int64_t H, int E,
                                                           const float* __restrict__ topk_w,
                                                           const int32_t* __restrict__ topk_ids,
                                                           void* __restrict__ out) {
  __shared__ float4 part[kWideMaxK][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t H4 = H / 4;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool live = g < T * H4;
  const int64_t t = live ? g / H4 : 0;
  const int64_t h = live ? (g % H4) * 4 : 0;
  const int64_t Tk = T * k;
  // ids and weights of every slot requested before the partials (wave 0
  // uses them after the barrier); slots past k re-read slot 0
  int eid[kWideMaxK];
  float wk[kWideMaxK];
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < kWideMaxK; ++j) {
      const int64_t f = t * k + (j < k ? j : 0);
      eid[j] = topk_ids[f];
      wk[j] = topk_w[f];
    }
  }
  // a workgroup's 64 groups may straddle two tokens: slot data per lane
  for (int j = wave; j < k; j += 4) {
    const int64_t f = t * k + j;
    float4 v[SMAX];
#pragma unroll
    for (int sp = 0; sp < SMAX; ++sp) {
      const int64_t sl = sp < splits ? sp : 0;
      v[sp] = *reinterpret_cast<const float4*>(y + (sl * Tk + f) * H + h);
    }
    float4 ys = v[0];
#pragma unroll
    for (int sp = 1; sp < SMAX; ++sp) {
      if (sp < splits) {
        ys.x += v[sp].x; ys.y += v[sp].y; ys.z += v[sp].z; ys.w += v[sp].w;
      }
    }
    part[j][lane] = ys;
  }
  __syncthreads();
  if (wave != 0 || !live) return;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kWideMaxK; ++j) {
    if (j < k && eid[j] >= 0 && eid[j] < E) {
      const float wj = wk[j];
      const float4 ys = part[j][lane];
      acc.x += wj * ys.x; acc.y += wj * ys.y; acc.z += wj * ys.z; acc.w += wj * ys.w;
    }
  }
  uint2 packed;
  if constexpr (F16) {
    packed.x = static_cast<uint32_t>(f32_to_f16(acc.x)) | (static_cast<uint32_t>(f32_to_f16(acc.y)) << 16);
    packed.y = static_cast<uint32_t>(f32_to_f16(acc.z)) | (static_cast<uint32_t>(f32_to_f16(acc.w)) << 16);
  } else {
    packed.x = pack_bf16_rne(acc.x, acc.y);
    packed.y = pack_bf16_rne(acc.z, acc.w);
  }
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * H + h) = packed;
}

}  // namespace

hipError_t launch_combine(const float* y, int splits, int64_t T, int k, int64_t H, int E,
                          const float* topk_w, const int32_t* topk_ids, int f16, void* out,
                          hipStream_t stream) {
  const int64_t n = T * (H / 4);
  const int64_t blocks = (n + 255) / 256;
  if (blocks <= 256) {
    // few tokens: the first (KMAX, SMAX) shape that holds (k, splits)
#define FEW(KM, SM)                                                                                         \
  if (k <= KM && splits <= SM) {                                                                           \
    if (f16)                                                                                                \
      hipLaunchKernelGGL((combine_few_kernel<true, KM, SM>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, \
                         stream, y, splits, T, k, H, E, topk_w, topk_ids, out);                             \
    else                                                                                                    \
      hipLaunchKernelGGL((combine_few_kernel<false, KM, SM>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, \
                         stream, y, splits, T, k, H, E, topk_w, topk_ids, out);                             \
    return hipGetLastError();                                                                               \
  }
    FEW(2, 1)
    FEW(2, 2)
    FEW(2, 4)
    FEW(2, 16)
    FEW(8, 1)
    FEW(8, 2)
    FEW(8, 4)
#undef FEW
    // more partials per slot: the slots spread over the waves
    if (k <= kWideMaxK && splits <= 16) {
      const unsigned wblocks = static_cast<unsigned>((n + kWave - 1) / kWave);
#define WIDE(SM)                                                                                            \
  if (splits <= SM) {                                                                                      \
    if (f16)                                                                                                \
      hipLaunchKernelGGL((combine_wide_kernel<true, SM>), dim3(wblocks), dim3(256), 0, stream, y, splits, T, k, \
                         H, E, topk_w, topk_ids, out);                                                      \
    else                                                                                                    \
      hipLaunchKernelGGL((combine_wide_kernel<false, SM>), dim3(wblocks), dim3(256), 0, stream, y, splits, T, \
                         k, H, E, topk_w, topk_ids, out);                                                   \
    return hipGetLastError();                                                                               \
  }
      WIDE(8)
      WIDE(16)
#undef WIDE
    }
  }
#define COMBINE(F, B)                                                                                    \
  hipLaunchKernelGGL((combine_kernel<F, B>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, y, splits, \
                     T, k, H, E, topk_w, topk_ids, out)
  const bool batch = splits > 8;
  if (f16) {
    if (batch) COMBINE(true, true);
    else COMBINE(true, false);
  } else {
    if (batch) COMBINE(false, true);
    else COMBINE(false, false);
  }
#undef COMBINE
  return hipGetLastError();
}

}  // namespace moe
