// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C-ABI layer before these are called; the launchers only shape the grids.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Per-row symmetric int8 quantizer over `rows` rows of K fp32 values.
hipError_t launch_quantize_int8(const float* w, int64_t rows, int64_t K, int8_t* q, float* scale,
                                hipStream_t stream);

// Group-wise uint4 quantizer over E experts of [N, K].
hipError_t launch_quantize_w4(const float* w, int64_t E, int64_t N, int64_t K, int64_t group,
                              int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                              hipStream_t stream);

// Softmax top-k router, one wave per token.
hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renormalize,
                        float* topk_w, int32_t* topk_ids, hipStream_t stream);

// Routing with scoring function, grouped top-k, correction bias and scaling factor, one wave per token
// (E <= 1024; G <= 64 groups dividing E when G > 1).
hipError_t launch_route_select(const float* logits, int64_t T, int E, int k, int renormalize, int sigmoid, int G,
                               int topk_group, const float* bias, float scale, float* topk_w, int32_t* topk_ids,
                               hipStream_t stream);

// Routing followed by the padded-block align in one workgroup (small batches).
hipError_t launch_route_align(const float* logits, int64_t T, int E, int k, int renormalize, float* topk_w,
                              int32_t* topk_ids, int block_m, int64_t cap, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* num_padded, hipStream_t stream);

// Padded-block align, one workgroup.
hipError_t launch_align(const int32_t* topk_ids, int64_t Tk, int E, int block_m, int64_t cap,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t stream);

struct Gemm1Args {
  const void* x;          // [T, H] bf16 / fp16
  int f16;                // activation type is fp16
  int64_t T, H, I, k, Tk;
  const int8_t* w13;      // [E, 2I, ldw]
  const float* s13;       // [E, 2I]
  int64_t ldw;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int block_m;
  int64_t cap;
  float* a;               // int8 path: two bf16 planes [2, cap, I] (hi, lo); uint4 path: fp32 [cap, I]
  int fp8;                // w13 holds e4m3fn codes and s13 one scale per expert [E]
};
hipError_t launch_gemm1_w8(const Gemm1Args& p, hipStream_t stream);
// Weight-streaming variant for block_m <= 64; kw = K-ways inside a workgroup (1, 2, 4).
hipError_t launch_gemm1_w8_stream(const Gemm1Args& p, int kw, hipStream_t stream);

struct Gemm2Args {
  const float* a;         // two bf16 planes [2, cap, I] written by GEMM1
  int64_t H, I, Tk;
  const int8_t* w2;       // [E, H, ldw]
  const float* s2;        // [E, H]
  int64_t ldw;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int block_m;
  int64_t cap;
  int splits;
  float* y;               // [splits, Tk, H]
  int fp8;                // w2 holds e4m3fn codes and s2 one scale per expert [E]
};
hipError_t launch_gemm2_w8(const Gemm2Args& p, hipStream_t stream);
// LDS-staged GEMM1 for blocks of 32 or 64 rows (kw <= 2 at 32, 1 at 64; ng = 16-column groups per wave).
hipError_t launch_gemm1_w8_lds(const Gemm1Args& p, int kw, int ng, hipStream_t stream);
// GEMM1 for blocks of 16 or 32 rows on a 3-step LDS ring of direct global -> LDS copies; with qhi the
// intermediate goes out as 16-bit fixed point in groups of 64 columns (hi, lo codes [cap, I], scales
// [cap, I/64]), else as bf16 hi/lo planes into p.a.
hipError_t launch_gemm1_w8_dma(const Gemm1Args& p, int8_t* qhi, int8_t* qlo, float* qscale, hipStream_t stream);
// Intermediate as 16-bit fixed point per (row, 128 columns) for the integer-MFMA GEMM2 (blocks of
// at most 64 rows): requant turns GEMM1's bf16 hi/lo planes into hi/lo int8 codes and scales;
// nt = 16-column tiles per wave (2 or 4).
hipError_t launch_requant_q16(const float* a, int64_t cap, int64_t I, const int32_t* sorted_ids,
                              const int32_t* num_padded, int64_t Tk, int8_t* qhi, int8_t* qlo, float* qscale,
                              hipStream_t stream);
// gw = columns per scale group of the fixed-point intermediate (64 or 128).
hipError_t launch_gemm2_q16(const Gemm2Args& p, int nt, int gw, const int8_t* qhi, const int8_t* qlo,
                            const float* qscale, hipStream_t stream);
// Blocks of 16 or 32 rows, intermediate in the 16-bit fixed-point form with
// 64-column scale groups (written by the 16/32-row GEMM1): w2 and the planes
// streamed through an LDS ring by global -> LDS copies, 128 columns per
// workgroup.  Same sums, in the same order, as launch_gemm2_q16 with gw 64.
bool gemm2_q16_dma_fits(int64_t H, int64_t I, int64_t block_m, int64_t ldw);
hipError_t launch_gemm2_q16_dma(const Gemm2Args& p, const int8_t* qhi, const int8_t* qlo, const float* qscale,
                                hipStream_t stream);
// Weight-only fp8, blocks of 16 or 32 rows: the bf16 planes GEMM1 writes and
// the e4m3fn codes of w2 streamed the same way (any split count up to I/64).
bool gemm2_fp8_dma_fits(int64_t H, int64_t I, int64_t block_m);
hipError_t launch_gemm2_fp8_dma(const Gemm2Args& p, hipStream_t stream);
// block_m == 256 GEMMs with both operands copied straight into a 3-stage LDS ring
// (GEMM2 needs H to be a multiple of 256).
// the 256-row GEMM1 addresses x with 32-bit byte offsets ((T + 1) * H * 2 < 2^32)
bool gemm1_w8_big_fits(const Gemm1Args& p);
// qhi == nullptr: bf16 planes into p.a; else the 16-bit fixed-point form
// (hi, lo codes [cap, I], scales [cap, I/128]) that launch_gemm2_w8_big_q16 reads.
hipError_t launch_gemm1_w8_big(const Gemm1Args& p, int8_t* qhi, int8_t* qlo, float* qscale, hipStream_t stream);
// 256-row blocks, H a multiple of 256.
hipError_t launch_gemm2_w8_big_q16(const Gemm2Args& p, const int8_t* qhi, const int8_t* qlo, const float* qscale,
                                   hipStream_t stream);

struct Gemm1W4Args {
  const void* x;
  int f16;
  int64_t T, H, I, k, Tk;
  const int32_t* qw;      // [E, 2I, H/8]
  const uint16_t* sc;     // [E, 2I, H/g]
  const int32_t* qz;      // [E, 2I/8, H/g]
  int group;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int block_m;
  int64_t cap;
  float* a;
};
hipError_t launch_gemm1_w4(const Gemm1W4Args& p, hipStream_t stream);

struct Gemm2W4Args {
  const float* a;
  int f16;                // use the fp16 MFMA path (activations are fp16)
  int64_t H, I, Tk;
  const int32_t* qw;      // [E, H, I/8]
  const uint16_t* sc;     // [E, H, I/g]
  const int32_t* qz;      // [E, H/8, I/g]
  int group;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int block_m;
  int64_t cap;
  int splits;
  float* y;
};
hipError_t launch_gemm2_w4(const Gemm2W4Args& p, hipStream_t stream);
// Weight-streaming uint4 variants for blocks of 16, 32 or 64 rows (intermediate as 16-bit hi/lo planes).
hipError_t launch_gemm1_w4_stream(const Gemm1W4Args& p, hipStream_t stream);
// uint4 GEMM1 for blocks of 16 or 32 rows on a 4-step ring of direct global -> LDS copies
// (needs the fp16 scales 4-byte aligned).
hipError_t launch_gemm1_w4_dma(const Gemm1W4Args& p, hipStream_t stream);
hipError_t launch_gemm2_w4_stream(const Gemm2W4Args& p, hipStream_t stream);

// Shared experts / routing weight on the input: routing extended to k + S columns (shared experts
// E .. E+S-1 with weight 1; weights 1 everywhere when the weight goes on the input), and the input rows
// rne(w * x[t]) of every extended assignment.
hipError_t launch_expand_routing(const float* topk_w, const int32_t* topk_ids, int64_t T, int k, int S, int E,
                                 int weight_on_input, float* w_ext, int32_t* ids_ext, hipStream_t stream);
hipError_t launch_prescale_input(const void* x, int f16, const float* topk_w, int64_t T, int k, int S, int64_t H,
                                 void* x_ext, hipStream_t stream);

// 4-bit GPTQ (gptq = 1) or AWQ (gptq = 0) checkpoint tensors of one [N, K] matrix -> this library's
// layout; output groups of group_out columns, group j' from input group j' / repeat.
hipError_t launch_import_w4(int gptq, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                            int64_t N, int64_t K, int64_t group_out, int64_t repeat, int32_t* out_qweight,
                            uint16_t* out_scales, int32_t* out_qzeros, hipStream_t stream);

// Per-tensor e4m3fn quantization of `tensors` fp32 tensors of per_tensor values (scale[t] = max|w| / 448).
hipError_t launch_quantize_fp8(const float* w, int64_t tensors, int64_t per_tensor, uint8_t* q, float* scale,
                               hipStream_t stream);
// w13 codes [E, 2I, H] with shard scales [E, 2] -> codes under the larger scale, scales [E].
hipError_t launch_fp8_merge_w13(uint8_t* q13, const float* s_in, int64_t E, int64_t I, int64_t H, float* s_out,
                                hipStream_t stream);

// W8A8: per-row int8 quantization of a GEMM input (src_type 0 bf16, 1 fp16, 2 fp32, src 8- / 16-byte
// aligned, K a multiple of 4; with sorted_ids only the rows that hold a token; with pmax each row's
// max |v| is the max of its npart partial maxima [rows, npart], written by the producer of the rows),
// and the two int8 x int8 GEMMs.
hipError_t launch_act_quant(const void* src, int src_type, int64_t rows, int64_t K, const int32_t* sorted_ids,
                            const int32_t* num_padded, int64_t Tk, const float* pmax, int64_t npart, int8_t* q,
                            float* scale, hipStream_t stream);
hipError_t launch_gemm1_w8a8(const Gemm1Args& p, const int8_t* qx, const float* sx, hipStream_t stream);
hipError_t launch_gemm2_w8a8(const Gemm2Args& p, const int8_t* qa, const float* sa, hipStream_t stream);
// W8A8 with blocks of 16 or 32 rows: weights and activation codes streamed
// through an LDS ring (same results as the two launchers above); GEMM1 also
// leaves the rows' partial maxima of |a| over 64 columns in pmax [cap, I/64].
bool w8a8_dma_fits(int64_t H, int64_t I, int64_t block_m);
hipError_t launch_gemm1_w8a8_dma(const Gemm1Args& p, const int8_t* qx, const float* sx, float* pmax,
                                 hipStream_t stream);
hipError_t launch_gemm2_w8a8_dma(const Gemm2Args& p, const int8_t* qa, const float* sa, hipStream_t stream);
// The W8A8 GEMMs for 256-row blocks (H a multiple of 256, I of 128): one align block x 256 weight rows
// per workgroup on a 4-slot LDS ring of direct global -> LDS copies; GEMM2 over p.splits K parts of
// whole 64-wide steps.  w8a8_big_fits: the shapes they take (T = rows of x's codes).
bool w8a8_big_fits(int64_t T, int64_t H, int64_t I, int64_t bm);
// GEMM2 for 256-row blocks on GEMM1's bf16 hi/lo planes with e4m3fn (p.fp8) or int8 w2 codes: one align
// block x 256 output columns per workgroup, p.splits K parts of whole 32-wide steps.
bool gemm2_planes_fits(int64_t H, int64_t I, int64_t bm);
hipError_t launch_gemm2_w8_planes(const Gemm2Args& p, hipStream_t stream);
// pmax [cap, I/64]: max |a| of each row over each wave's 64 columns.
hipError_t launch_gemm1_w8a8_big(const Gemm1Args& p, const int8_t* qx, const float* sx, float* pmax,
                                 hipStream_t stream);
hipError_t launch_gemm2_w8a8_big(const Gemm2Args& p, const int8_t* qa, const float* sa, hipStream_t stream);

// Weighted top-k combine of the split partials.
hipError_t launch_combine(const float* y, int splits, int64_t T, int k, int64_t H, int E,
                          const float* topk_w, const int32_t* topk_ids, int f16, void* out,
                          hipStream_t stream);

}  // namespace moe
