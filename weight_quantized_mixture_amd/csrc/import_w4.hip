// Import of 4-bit GPTQ / AWQ checkpoint tensors into this library's layout
// (moe_wna16 page, MoeWNA16Method.get_weight_loader: convert_awq_tensor,
// convert_gptq_int4_qzeros, moe_wna16_weight_loader; MoeWNA16Method.create_weights:
// the group size is halved until it divides H and I and the loaded scales
// and zeros are repeated to match).
//
// Inputs of one [N, K] matrix (N output rows, K reduction):
//   AWQ:  qweight int32 [K, N/8] packed along N in AWQ's order (nibble p holds
//         column (0,2,4,6,1,3,5,7)[p]: column c sits in nibble (0,4,1,5,2,6,3,7)[c],
//         the page's reverse order), qzeros int32 [Gin, N/8] the same way;
//   GPTQ: qweight int32 [K/8, N] packed along K (code k at bits 4(k mod 8)),
//         qzeros int32 [Gin, N/8] of zero - 1 packed along N; the loader adds 1
//         to each nibble and re-packs the pair in uint8 arithmetic (so a stored
//         15 carries into the next nibble, as the page's byte sum does);
//   both: scales fp16 [Gin, N].
// Outputs: qweight int32 [N, K/8] (code k at bits 4(k mod 8)), scales fp16
// [N, K/g'], qzeros int32 [N/8, K/g'] (row n at bits 4(n mod 8)); output
// group j' takes input group j' / repeat.  Integer work only: bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// nibble of AWQ's packing that holds column c of a group of eight
__device__ __forceinline__ int awq_nibble(int c) { return (c & 1) ? 4 + (c >> 1) : (c >> 1); }

// One thread per output code word [n, k8].
__global__ __launch_bounds__(256) void import_codes_kernel(int gptq, const int32_t* __restrict__ qw, int64_t N,
                                                           int64_t K, int32_t* __restrict__ out) {
  const int64_t K8 = K / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= N * K8) return;
  const int64_t n = idx / K8, k8 = idx % K8;
  if (gptq) {
    out[idx] = qw[k8 * N + n];
    return;
  }
  const int sh = 4 * awq_nibble(static_cast<int>(n & 7));
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t src = static_cast<uint32_t>(qw[(k8 * 8 + i) * (N / 8) + n / 8]);
    w |= ((src >> sh) & 0xFu) << (4 * i);
  }
  out[idx] = static_cast<int32_t>(w);
}

// true zero of row n in input group j
__device__ __forceinline__ uint32_t import_zero(int gptq, const int32_t* __restrict__ qz, int64_t N, int64_t j,
                                                int64_t n) {
  const uint32_t word = static_cast<uint32_t>(qz[j * (N / 8) + n / 8]);
  if (!gptq) return (word >> (4 * awq_nibble(static_cast<int>(n & 7)))) & 0xFu;
  const uint32_t b = (word >> (8 * ((n & 7) >> 1))) & 0xFFu;         // the byte of rows 2m, 2m+1
  const uint32_t page = ((b & 0xFu) + 1u + 16u * ((b >> 4) + 1u)) & 0xFFu;
  return (n & 1) ? page >> 4 : page & 0xFu;
}

// One thread per output zero word [n8, j'].
__global__ __launch_bounds__(256) void import_zeros_kernel(int gptq, const int32_t* __restrict__ qz, int64_t N,
                                                           int64_t Gout, int64_t repeat, int32_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= (N / 8) * Gout) return;
  const int64_t n8 = idx / Gout, jo = idx % Gout, j = jo / repeat;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= import_zero(gptq, qz, N, j, n8 * 8 + i) << (4 * i);
  out[idx] = static_cast<int32_t>(w);
}

// One thread per output scale [n, j'].
__global__ __launch_bounds__(256) void import_scales_kernel(const uint16_t* __restrict__ sc, int64_t N, int64_t Gout,
                                                            int64_t repeat, uint16_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= N * Gout) return;
  const int64_t n = idx / Gout, jo = idx % Gout;
  out[idx] = sc[(jo / repeat) * N + n];
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

}  // namespace

hipError_t launch_import_w4(int gptq, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                            int64_t N, int64_t K, int64_t group_out, int64_t repeat, int32_t* out_qweight,
                            uint16_t* out_scales, int32_t* out_qzeros, hipStream_t stream) {
  if (N % 8 || K % 8 || group_out < 1 || K % group_out || repeat < 1) return hipErrorInvalidValue;
  const int64_t Gout = K / group_out;
  hipLaunchKernelGGL(import_codes_kernel, dim3(blocks_for(N * (K / 8))), dim3(256), 0, stream, gptq, qweight, N, K,
                     out_qweight);
  hipLaunchKernelGGL(import_zeros_kernel, dim3(blocks_for((N / 8) * Gout)), dim3(256), 0, stream, gptq, qzeros, N,
                     Gout, repeat, out_qzeros);
  hipLaunchKernelGGL(import_scales_kernel, dim3(blocks_for(N * Gout)), dim3(256), 0, stream, scales, N, Gout, repeat,
                     out_scales);
  return hipGetLastError();
}

}  // namespace moe
