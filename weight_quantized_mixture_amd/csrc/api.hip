// C ABI of the MoE library: argument checks, workspace layout and the launch
// sequence.  Every check runs on the host before anything is enqueued, so an
// error leaves the stream untouched (the pages raise ValueError for a bad
// shard or bit width and NotImplementedError for unsupported features:
// experts_int8 page, quantizing_weight_loader and apply; moe_wna16 page,
// MoeWNA16Method.__init__).
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/moe_wq.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxExperts = 1024;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

int64_t capacity(int64_t T, int64_t k, int64_t E, int64_t bm) {
  const int64_t tk = T * k;
  if (tk <= 0 || bm <= 0) return 0;
  const int64_t ne = E < tk ? E : tk;
  return (tk + ne * (bm - 1)) / bm * bm;
}

// Rows per align block.  Batches whose experts hold at most about 64 rows
// take the weight-streaming kernels: the block (16, 32 or 64 rows) is sized
// to cover the expected largest expert (mean + 3 sigma of a binomial count),
// so each expert's weights are read once; large int8 experts (w13 of 32 MiB
// or more) expected past 80 rows take 128-row blocks, still streamed.
// Experts with 128 rows or more on average take 256-row blocks of the
// MFMA-tiled kernels.
int64_t auto_block_m(int64_t T, int64_t E, int64_t k, bool w8 = false, int64_t H = 0, int64_t I = 0) {
  const double avg = static_cast<double>(T) * k / E;
  if (avg >= 128.0) return 256;                 // MFMA-bound: large tiles
  const double need = avg + 3.0 * std::sqrt(avg) + 1.0;
  if (need <= 16.0) return 16;
  if (need <= 32.0) return 32;
  // Well past 64 rows a 128-row block reads each weight row once for two
  // 64-row blocks' worth of tokens: measured 8-14% faster for Mixtral T=256
  // and 384 (117 MB of w13 per expert), 23% slower at T=192 (most experts
  // still fit 64 rows), 3-10% slower for the fine-grained shape (5.8 MB per
  // expert, whose second reads mostly hit the 256 MB Infinity Cache)
  return w8 && need > 80.0 && 2 * H * I >= (int64_t{1} << 25) ? 128 : 64;
}

bool use_prefill(int64_t bm) { return bm == 256; }

// Blocks of 16 and 32 rows: GEMM1 (the DMA-fed kernel) writes the 16-bit
// fixed-point form itself, in groups of 64 columns.  48, 64 and 128 rows:
// GEMM1 writes bf16 planes and a requant pass turns them into groups of 128.
bool q16_from_gemm1(int64_t bm) { return bm == 16 || bm == 32; }
bool needs_requant(int64_t bm) { return (bm > 32 && bm <= 64) || bm == 128; }

// The intermediate of the int8 path:
//   blocks of 16 / 32 rows: int8 hi codes [cap, I], lo codes [cap, I], fp32
//     scales [cap, I/64] at offset 0;
//   48 / 64 / 128 rows: bf16 hi/lo planes [2, cap, I] followed by hi codes, lo
//     codes and scales [cap, I/128];
//   256-row blocks with prefill_q16: hi, lo codes and scales [cap, I/128] at
//     offset 0, in the planes' space;
//   otherwise (and for the other weight formats) the bf16 planes.
struct Q16 {
  int8_t* hi;
  int8_t* lo;
  float* scale;
};

size_t planes_bytes(int64_t cap, int64_t I) { return align_up(static_cast<size_t>(cap) * static_cast<size_t>(I) * 4); }

size_t intermediate_bytes(int64_t cap, int64_t I, int64_t bm, bool w8) {
  if (w8 && q16_from_gemm1(bm))
    return 2 * align_up(static_cast<size_t>(cap) * static_cast<size_t>(I)) +
           align_up(static_cast<size_t>(cap) * static_cast<size_t>(I / 64) * 4);
  size_t b = planes_bytes(cap, I);
  if (w8 && needs_requant(bm)) {
    b += 2 * align_up(static_cast<size_t>(cap) * static_cast<size_t>(I));
    b += align_up(static_cast<size_t>(cap) * static_cast<size_t>(I / 128) * 4);
  }
  return b;
}

Q16 q16_at(const float* a, int64_t cap, int64_t I, size_t offset) {
  char* base = const_cast<char*>(reinterpret_cast<const char*>(a)) + offset;
  const size_t codes = align_up(static_cast<size_t>(cap) * static_cast<size_t>(I));
  return Q16{reinterpret_cast<int8_t*>(base), reinterpret_cast<int8_t*>(base + codes),
             reinterpret_cast<float*>(base + 2 * codes)};
}

// 256-row blocks keep the intermediate as 16-bit fixed point (written by
// GEMM1's epilogue, read by the integer-MFMA GEMM2) when both 256-row
// kernels apply; otherwise as bf16 planes.  Decided from (T, H, block_m),
// which every stage call knows, so GEMM1 and GEMM2 always agree.
bool prefill_q16(int64_t T, int64_t H, int64_t bm) {
  return use_prefill(bm) && H % 256 == 0 && (T + 1) * H * 2 < (int64_t{1} << 32);
}

// Weight-streaming kernels: blocks of up to 64 rows, and 128 (GEMM1 with eight
// row tiles, GEMM2 on each 64-row half).
bool use_stream(int64_t bm) { return bm <= 64 || bm == 128; }

// Rough count of align blocks that hold rows (the exact count stays on the
// device): the blocks the assignments fill, plus half a block of padding for
// each expert expected to be hit when T tokens pick k of E at random.
int64_t blocks_estimate(int64_t T, int64_t E, int64_t k, int64_t bm) {
  const int64_t tk = T * k;
  const double miss = std::pow(1.0 - static_cast<double>(k) / static_cast<double>(E), static_cast<double>(T));
  const int64_t hit = static_cast<int64_t>(std::ceil(static_cast<double>(E) * (1.0 - miss)));
  const int64_t ne = hit < tk ? hit : tk;
  return (tk + bm - 1) / bm + ne / 2;
}

// ---- GEMM1 ----
// Register-streaming kernel (blocks of 16 or 48 rows): K-ways inside the
// workgroup until about 4096 waves keep every CU streaming.
constexpr int64_t kTargetWaves = 4096;

int gemm1_kways(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm) {
  const int64_t waves1 = (I / 16) * blocks_estimate(T, E, k, bm);
  int kw = 1;
  while (kw < 4 && waves1 * kw < kTargetWaves && H / 128 >= 2 * kw) kw *= 2;
  return kw;
}

hipError_t run_gemm1(const moe::Gemm1Args& p, int64_t T, int64_t E, hipStream_t stream) {
  if (use_prefill(p.block_m) && moe::gemm1_w8_big_fits(p)) {
    if (prefill_q16(T, p.H, p.block_m)) {
      const Q16 q = q16_at(p.a, p.cap, p.I, 0);
      return moe::launch_gemm1_w8_big(p, q.hi, q.lo, q.scale, stream);
    }
    return moe::launch_gemm1_w8_big(p, nullptr, nullptr, nullptr, stream);
  }
  if (!use_stream(p.block_m)) return moe::launch_gemm1_w8(p, stream);
  if (q16_from_gemm1(p.block_m)) {
    const Q16 q = q16_at(p.a, p.cap, p.I, 0);
    return moe::launch_gemm1_w8_dma(p, q.hi, q.lo, q.scale, stream);
  }
  if (p.block_m == 64 || p.block_m == 128) return moe::launch_gemm1_w8_lds(p, 1, 1, stream);
  return moe::launch_gemm1_w8_stream(p, gemm1_kways(T, p.H, p.I, E, p.k, p.block_m), stream);
}

// ---- GEMM2 ----
// Blocks of at most 64 rows: integer-MFMA kernel on the 16-bit fixed-point
// form of a (requantized after GEMM1), 4 or 2 column tiles per wave and K cut
// into `splits` parts so that about 512 workgroups are in flight.  256-row
// blocks: the LDS-ring kernel on the bf16 planes.  Other block sizes: the
// generic tiled kernel (equal splits of whole 128-wide steps).
bool gemm2_int8(int64_t bm) { return bm <= 64 || bm == 128; }


// Expected rows per active expert above 2.5: narrower waves (more
// workgroups) stream better; with fewer rows, 4 column tiles per wave.
// Measured on the Mixtral decode shape (E 8, H 4096): 2 tiles faster by 8%
// at 3 to 6 rows per expert, 4 tiles by 1-8% at 1.5 to 2.2 rows.  Blocks of
// 48 rows and more: 2 tiles (with three register sets of loads in flight, 4
// tiles take 384 registers and leave one wave per SIMD).
// Four tiles cover 256 columns per workgroup, so they need H a multiple of
// 256; otherwise two tiles (128 columns, which every H the layer accepts fills).
int gemm2_nt(int64_t T, int64_t H, int64_t E, int64_t k, int64_t bm) {
  if (H % 256 != 0) return 2;
  if (moe::gemm2_q16_dma_fits(H, 128, bm, 16)) return 2;   // the LDS-ring kernel: 2 tiles per wave
  if (bm >= 48) return 2;   // 48/64-row blocks: four tiles would leave one wave per SIMD
  const double miss = std::pow(1.0 - static_cast<double>(k) / static_cast<double>(E), static_cast<double>(T));
  const double hit = static_cast<double>(E) * (1.0 - miss);
  return static_cast<double>(T * k) / (hit > 1.0 ? hit : 1.0) > 2.5 ? 2 : 4;
}

int64_t gemm2_splits(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm, bool tiled = false) {
  const int64_t steps = I / 128;
  const int64_t blocks = blocks_estimate(T, E, k, bm);
  if (!tiled && use_prefill(bm)) {
    if (!prefill_q16(T, H, bm)) return 1;
    // 128-row halves x 256 columns per workgroup, one workgroup per CU.  When
    // they fill at most two rounds of 256 CUs, the split count (1, 2 or 4
    // parts of whole 128-wide groups) with the shortest run in rounds, each
    // extra part charged 5% for its partials' round trip through the combine
    const int64_t wgs = 2 * blocks * (H / 256);
    if (wgs > 512) return 1;
    int64_t best = 1;
    double best_t = 1e30;
    for (int64_t sp = 1; sp <= 4 && sp <= steps; sp *= 2) {
      const double t = std::ceil(static_cast<double>(wgs * sp) / 256.0) / static_cast<double>(sp) *
                       (1.0 + 0.05 * static_cast<double>(sp - 1));
      if (t < best_t) {
        best_t = t;
        best = sp;
      }
    }
    return best;
  }
  if (tiled || !gemm2_int8(bm)) {
    // tiled kernel: 128 columns x one split per workgroup, equal splits
    const int64_t ntiles = H / 128;
    int64_t want = 1;
    while (ntiles * blocks * want < 1024 && want < 64) want *= 2;
    int64_t best = 1;
    for (int64_t sp = 1; sp <= want && sp <= steps; ++sp)
      if (steps % sp == 0) best = sp;
    return best;
  }
  // GEMM2 runs 128-row blocks as two 64-row halves
  const int64_t groups = (H / (64 * gemm2_nt(T, H, E, k, bm))) * blocks * (bm > 64 ? bm / 64 : 1);
  int64_t sp = 1;
  while (sp * 2 <= 16 && sp * 2 <= steps && groups * sp * 2 <= 512) sp *= 2;
  return sp;
}

int64_t splits_for(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm) {
  return gemm2_splits(T, H, I, E, k, bm);
}

// uint4 GEMM2 splits: the streaming kernel (blocks of 16/32/64 rows) takes any
// count up to I/128 (about 512 workgroups in flight); the tiled kernel needs
// equal parts of whole 128-wide steps.
bool w4_stream(int64_t bm) { return bm == 16 || bm == 32 || bm == 64; }

int64_t w4_splits(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm) {
  if (!w4_stream(bm)) return gemm2_splits(T, H, I, E, k, bm, true);
  const int64_t groups = (H / 128) * blocks_estimate(T, E, k, bm);
  int64_t sp = 1;
  while (sp * 2 <= 16 && sp * 2 <= I / 128 && groups * sp * 2 <= 512) sp *= 2;
  return sp;
}

hipError_t run_gemm1_and_requant(const moe::Gemm1Args& p, int64_t T, int64_t E, hipStream_t stream) {
  hipError_t e = run_gemm1(p, T, E, stream);
  if (e != hipSuccess || !needs_requant(p.block_m)) return e;
  const Q16 q = q16_at(p.a, p.cap, p.I, planes_bytes(p.cap, p.I));
  return moe::launch_requant_q16(p.a, p.cap, p.I, p.sorted_ids, p.num_padded, p.Tk, q.hi, q.lo, q.scale, stream);
}

hipError_t run_gemm2(const moe::Gemm2Args& p, int64_t T, int64_t E, int64_t k, hipStream_t stream) {
  if (prefill_q16(T, p.H, p.block_m)) {
    const Q16 q = q16_at(p.a, p.cap, p.I, 0);
    return moe::launch_gemm2_w8_big_q16(p, q.hi, q.lo, q.scale, stream);
  }
  if (!gemm2_int8(p.block_m)) return moe::launch_gemm2_w8(p, stream);
  const int nt = gemm2_nt(T, p.H, E, k, p.block_m);
  if (q16_from_gemm1(p.block_m)) {
    const Q16 q = q16_at(p.a, p.cap, p.I, 0);
    if (moe::gemm2_q16_dma_fits(p.H, p.I, p.block_m, p.ldw))
      return moe::launch_gemm2_q16_dma(p, q.hi, q.lo, q.scale, stream);
    return moe::launch_gemm2_q16(p, nt, 64, q.hi, q.lo, q.scale, stream);
  }
  const Q16 q = q16_at(p.a, p.cap, p.I, planes_bytes(p.cap, p.I));
  return moe::launch_gemm2_q16(p, nt, 128, q.hi, q.lo, q.scale, stream);
}

enum class Fmt { W8, W4, FP8, W8A8 };

// W8A8 intermediate: the GEMM1 input's int8 codes [xrows, H] and scales
// [xrows], the fp32 intermediate a [cap, I], its codes [cap, I] and scales
// [cap], and the rows' partial maxima of |a| [cap, I/64] (the 256-row GEMM1
// writes them).
struct A8 {
  int8_t* qx;
  float* sx;
  float* a;
  int8_t* qa;
  float* sa;
  float* pmax;
};

size_t w8a8_bytes(int64_t cap, int64_t I, int64_t xrows, int64_t H) {
  const size_t c = static_cast<size_t>(cap), r = static_cast<size_t>(xrows);
  return align_up(r * static_cast<size_t>(H)) + align_up(r * 4) + align_up(c * static_cast<size_t>(I) * 4) +
         align_up(c * static_cast<size_t>(I)) + align_up(c * 4) + align_up(c * static_cast<size_t>(I / 64) * 4);
}

A8 w8a8_at(float* base, int64_t cap, int64_t I, int64_t xrows, int64_t H) {
  char* b = reinterpret_cast<char*>(base);
  const size_t c = static_cast<size_t>(cap), r = static_cast<size_t>(xrows);
  A8 v{};
  v.qx = reinterpret_cast<int8_t*>(b);  b += align_up(r * static_cast<size_t>(H));
  v.sx = reinterpret_cast<float*>(b);   b += align_up(r * 4);
  v.a = reinterpret_cast<float*>(b);    b += align_up(c * static_cast<size_t>(I) * 4);
  v.qa = reinterpret_cast<int8_t*>(b);  b += align_up(c * static_cast<size_t>(I));
  v.sa = reinterpret_cast<float*>(b);   b += align_up(c * 4);
  v.pmax = reinterpret_cast<float*>(b);
  return v;
}

struct Layout {
  int64_t cap, nblocks, splits;
  size_t off_sorted, off_block, off_npad, off_a, off_y, off_ids_ext, off_w_ext, off_x_ext, total;
};

// Workspace regions, 256-byte aligned: align outputs, the intermediate, the
// split partials y; with `expand` (shared experts or weight on input) the
// extended routing [T, k]; with `woi` the scaled input rows [T*k, H].
// E and k here count the shared experts too.
Layout layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm, int64_t splits, Fmt fmt,
              bool expand = false, bool woi = false) {
  Layout L{};
  L.cap = capacity(T, k, E, bm);
  L.nblocks = bm > 0 ? L.cap / bm : 0;
  L.splits = splits;
  const size_t Tk = static_cast<size_t>(T * k);
  size_t o = 0;
  L.off_sorted = o; o += align_up(static_cast<size_t>(L.cap) * 4);
  L.off_block = o;  o += align_up(static_cast<size_t>(L.nblocks) * 4);
  L.off_npad = o;   o += align_up(4);
  L.off_a = o;
  o += fmt == Fmt::W8A8 ? w8a8_bytes(L.cap, I, woi ? T * k : T, H) : intermediate_bytes(L.cap, I, bm, fmt == Fmt::W8);
  L.off_y = o;      o += align_up(static_cast<size_t>(splits) * Tk * static_cast<size_t>(H) * 4);
  if (expand) {
    L.off_ids_ext = o; o += align_up(Tk * 4);
    L.off_w_ext = o;   o += align_up(Tk * 4);
  }
  if (woi) {
    L.off_x_ext = o;   o += align_up(Tk * static_cast<size_t>(H) * 2);
  }
  L.total = o;
  return L;
}

int check_block_m(int64_t bm) {
  if (bm < 16 || bm > 256 || bm % 16 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "block_m must be a multiple of 16 in [16, 256], got %lld",
                static_cast<long long>(bm));
  return MOE_OK;
}

int check_layer_dims(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0");
  if (H < 1 || I < 1 || E < 1 || k < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "H, I, E and k must be >= 1");
  if (k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "k (%lld) > E (%lld)", (long long)k, (long long)E);
  if (E > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "E > %lld", (long long)kMaxExperts);
  if (H > (int64_t{1} << 24) || I > (int64_t{1} << 24))
    return fail(MOE_ERR_UNSUPPORTED, "H and I above 2^24 are not supported");
  if (H % 128 != 0 || I % 128 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "H (%lld) and I (%lld) must be multiples of 128",
                (long long)H, (long long)I);
  return MOE_OK;
}

int check_act(int act) {
  if (act != MOE_BF16 && act != MOE_FP16)
    return fail(MOE_ERR_UNSUPPORTED, "act_dtype %d is neither MOE_BF16 nor MOE_FP16", act);
  return MOE_OK;
}


// Checks of the routing options (moe_route_select); a NULL pointer is the default routing.
int check_routing(int64_t T, int64_t E, int64_t k, const moe_routing* r) {
  if (T < 0 || E < 1 || k < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0, E >= 1, k >= 1");
  if (k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "k (%lld) > E (%lld)", (long long)k, (long long)E);
  if (E > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "E > %lld", (long long)kMaxExperts);
  if (!r) return MOE_OK;
  if (r->scoring != MOE_SCORING_SOFTMAX && r->scoring != MOE_SCORING_SIGMOID)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown scoring %d", r->scoring);
  if (!std::isfinite(r->routed_scaling_factor))
    return fail(MOE_ERR_INVALID_ARGUMENT, "routed_scaling_factor must be finite");
  const int64_t G = r->num_expert_group;
  if (G < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_expert_group must be >= 0");
  if (G > 1) {
    if (G > 64) return fail(MOE_ERR_UNSUPPORTED, "num_expert_group above 64");
    if (E % G) return fail(MOE_ERR_INVALID_ARGUMENT, "num_expert_group %lld does not divide E %lld", (long long)G,
                           (long long)E);
    if (r->topk_group < 1 || r->topk_group > G)
      return fail(MOE_ERR_INVALID_ARGUMENT, "topk_group must be in [1, num_expert_group]");
    if (k > r->topk_group * (E / G))
      return fail(MOE_ERR_INVALID_ARGUMENT, "k exceeds the experts of the kept groups");
  }
  return MOE_OK;
}

bool default_routing(const moe_routing* r) {
  return !r || (r->scoring == MOE_SCORING_SOFTMAX && r->num_expert_group <= 1 && !r->e_score_correction_bias &&
                r->routed_scaling_factor == 1.0f);
}

hipError_t launch_routing(const float* logits, int64_t T, int64_t E, int64_t k, const moe_routing* r, float* tw,
                          int32_t* ti, hipStream_t stream) {
  if (default_routing(r))
    return moe::launch_route(logits, T, static_cast<int>(E), static_cast<int>(k), r ? r->renormalize : 1, tw, ti,
                             stream);
  const int G = r->num_expert_group > 1 ? static_cast<int>(r->num_expert_group) : 0;
  return moe::launch_route_select(logits, T, static_cast<int>(E), static_cast<int>(k), r->renormalize,
                                  r->scoring == MOE_SCORING_SIGMOID, G, G ? static_cast<int>(r->topk_group) : 0,
                                  r->e_score_correction_bias, r->routed_scaling_factor, tw, ti, stream);
}

constexpr int64_t kFusedRouteTokens = 8;

struct Opts {
  int64_t S;     // shared experts after the routed ones
  bool woi;      // routing weight applied to the input
};

Opts opts_of(const moe_fused_opts* fo) {
  return fo ? Opts{fo->num_shared_experts, fo->apply_router_weight_on_input != 0} : Opts{0, false};
}

// W8A8 with 256-row blocks: the big int8 GEMMs (the x codes may have T k rows
// when the routing weight scales the input)
bool w8a8_big(int64_t T, int64_t H, int64_t I, int64_t k, int64_t bm) {
  return moe::w8a8_big_fits(T * k, H, I, bm);
}

// GEMM2 kernels with one 256-row block x 256 columns per workgroup and CU
// (W8A8 and fp8 prefill): when they fill at most two rounds of 256 CUs, the K
// split (1, 2 or 4 parts) with the shortest run in rounds, each extra part
// charged 5% for its partials' round trip through the combine
int64_t big_tile_splits(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm) {
  const int64_t wgs = blocks_estimate(T, E, k, bm) * (H / 256);
  if (wgs > 512) return 1;
  int64_t best = 1;
  double best_t = 1e30;
  for (int64_t sp = 1; sp <= 4 && sp <= I / 64; sp *= 2) {
    const double t = std::ceil(static_cast<double>(wgs * sp) / 256.0) / static_cast<double>(sp) *
                     (1.0 + 0.05 * static_cast<double>(sp - 1));
    if (t < best_t) {
      best_t = t;
      best = sp;
    }
  }
  return best;
}

int64_t splits_fmt(Fmt fmt, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm) {
  if (fmt == Fmt::W8) return splits_for(T, H, I, E, k, bm);
  if (fmt == Fmt::W4) return w4_splits(T, H, I, E, k, bm);
  if (fmt == Fmt::W8A8 && w8a8_big(T, H, I, k, bm)) return big_tile_splits(T, H, I, E, k, bm);
  if (fmt == Fmt::W8A8 && moe::w8a8_dma_fits(H, I, bm)) return gemm2_splits(T, H, I, E, k, bm);
  if (fmt == Fmt::FP8 && moe::gemm2_planes_fits(H, I, bm)) return big_tile_splits(T, H, I, E, k, bm);
  if (fmt == Fmt::FP8 && moe::gemm2_fp8_dma_fits(H, I, bm)) return gemm2_splits(T, H, I, E, k, bm);
  return gemm2_splits(T, H, I, E, k, bm, true);     // fp8, W8A8: the tiled GEMM2, equal parts
}

// Workspace of a layer call; 0 for bad sizes.
size_t workspace_for(Fmt fmt, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t bm,
                     const moe_fused_opts* fo) {
  const Opts o = opts_of(fo);
  if (T <= 0 || H < 1 || I < 1 || E < 1 || k < 1 || o.S < 0) return 0;
  const int64_t Ex = E + o.S, kx = k + o.S;
  if (bm == 0) bm = auto_block_m(T, Ex, kx, fmt == Fmt::W8, H, I);
  if (bm < 16 || bm > 256 || bm % 16) return 0;
  return layout(T, H, I, Ex, kx, bm, splits_fmt(fmt, T, H, I, Ex, kx, bm), fmt, o.S > 0 || o.woi, o.woi).total;
}

// What the GEMMs of a format need, set up by layer_front.
struct Front {
  const void* x;               // GEMM1's activation rows
  int64_t Tg, kg;              // rows of x; assignment f reads row f / kg
  int64_t T, Tk, Ex, kx, bm, splits, cap;
  int32_t* sorted;
  int32_t* blocks;
  int32_t* npad;
  float* a;
  float* y;
  const float* cw;             // combine weights and ids [T, kx]
  const int32_t* cids;
};

// Checks, workspace layout, routing (from logits, with the routing options),
// the shared-expert / weight-on-input extension and the align.  Returns MOE_OK
// and fills F; T = 0 returns MOE_OK with F->T = 0 and nothing enqueued.
int layer_front(Fmt fmt, const void* x, int act, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                const moe_fused_opts* fo, const float* logits, const moe_routing* r, float* tw_out,
                int32_t* ti_out, const float* tw, const int32_t* ti, int64_t block_m, void* workspace,
                size_t workspace_bytes, hipStream_t stream, Front* F) {
  int st;
  const Opts o = opts_of(fo);
  if (o.S < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_shared_experts must be >= 0");
  if ((st = check_layer_dims(T, H, I, E, k)) != MOE_OK) return st;
  const int64_t Ex = E + o.S, kx = k + o.S;
  if (Ex > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "routed plus shared experts above %lld", (long long)kMaxExperts);
  if ((st = check_act(act)) != MOE_OK) return st;
  if (logits && (st = check_routing(T, E, k, r)) != MOE_OK) return st;
  const int64_t bm = block_m == 0 ? auto_block_m(T, Ex, kx, fmt == Fmt::W8, H, I) : block_m;
  if ((st = check_block_m(bm)) != MOE_OK) return st;
  F->T = 0;
  if (T == 0) return ok();
  if (T * kx > 0x7fffffffLL) return fail(MOE_ERR_UNSUPPORTED, "T*k above 2^31-1");
  if (!x || !workspace) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (logits ? (!tw_out || !ti_out) : (!tw || !ti)) return fail(MOE_ERR_INVALID_ARGUMENT, "null routing pointer");
  if (!aligned(x, 16) || !aligned(workspace, kAlign))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x must be 16-byte and the workspace 256-byte aligned");
  const bool expand = o.S > 0 || o.woi;
  const int64_t splits = splits_fmt(fmt, T, H, I, Ex, kx, bm);
  const Layout L = layout(T, H, I, Ex, kx, bm, splits, fmt, expand, o.woi);
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", L.total, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  F->sorted = reinterpret_cast<int32_t*>(ws + L.off_sorted);
  F->blocks = reinterpret_cast<int32_t*>(ws + L.off_block);
  F->npad = reinterpret_cast<int32_t*>(ws + L.off_npad);
  F->a = reinterpret_cast<float*>(ws + L.off_a);
  F->y = reinterpret_cast<float*>(ws + L.off_y);
  F->T = T; F->Tk = T * kx; F->Ex = Ex; F->kx = kx; F->bm = bm; F->splits = splits; F->cap = L.cap;
  const int bmi = static_cast<int>(bm);
  hipError_t e = hipSuccess;
  bool aligned_done = false;
  if (logits) {
    if (!expand && default_routing(r) && T <= kFusedRouteTokens) {
      // up to 8 tokens one workgroup routes (one wave per token) and aligns: one launch less
      e = moe::launch_route_align(logits, T, static_cast<int>(E), static_cast<int>(k), r ? r->renormalize : 1,
                                  tw_out, ti_out, bmi, L.cap, F->sorted, F->blocks, F->npad, stream);
      aligned_done = true;
    } else {
      e = launch_routing(logits, T, E, k, r, tw_out, ti_out, stream);
    }
    if (e != hipSuccess) return hip_status(e, "route");
    tw = tw_out;
    ti = ti_out;
  }
  F->x = x; F->Tg = T; F->kg = kx; F->cw = tw; F->cids = ti;
  if (expand) {
    float* w_ext = reinterpret_cast<float*>(ws + L.off_w_ext);
    int32_t* ids_ext = reinterpret_cast<int32_t*>(ws + L.off_ids_ext);
    e = moe::launch_expand_routing(tw, ti, T, static_cast<int>(k), static_cast<int>(o.S), static_cast<int>(E),
                                   o.woi ? 1 : 0, w_ext, ids_ext, stream);
    if (e != hipSuccess) return hip_status(e, "expand routing");
    F->cw = w_ext;
    F->cids = ids_ext;
    if (o.woi) {
      void* x_ext = ws + L.off_x_ext;
      e = moe::launch_prescale_input(x, act == MOE_FP16, tw, T, static_cast<int>(k), static_cast<int>(o.S), H,
                                     x_ext, stream);
      if (e != hipSuccess) return hip_status(e, "scale input");
      F->x = x_ext; F->Tg = T * kx; F->kg = 1;
    }
  }
  if (!aligned_done) {
    e = moe::launch_align(F->cids, F->Tk, static_cast<int>(Ex), bmi, L.cap, F->sorted, F->blocks, F->npad, stream);
    if (e != hipSuccess) return hip_status(e, "align");
  }
  return MOE_OK;
}

// The weighted combine of the split partials into `out`.
int layer_back(const Front& F, int64_t H, int act, void* out, hipStream_t stream) {
  return hip_status(moe::launch_combine(F.y, static_cast<int>(F.splits), F.T, static_cast<int>(F.kx), H,
                                        static_cast<int>(F.Ex), F.cw, F.cids, act == MOE_FP16, out, stream),
                    "combine");
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_UNKNOWN_STATUS";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_quantize_weights_int8(const float* w, int64_t E, int64_t N, int64_t K, int8_t* q,
                              float* scale, hipStream_t stream) {
  if (E < 1 || N < 1 || K < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "E, N and K must be >= 1");
  if (!w || !q || !scale) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(moe::launch_quantize_int8(w, E * N, K, q, scale, stream), "quantize_int8");
}

int moe_route_topk(const float* logits, int64_t T, int64_t E, int64_t k, int renormalize,
                   float* topk_w, int32_t* topk_ids, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0, E >= 1, k >= 1");
  if (k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "k (%lld) > E (%lld)", (long long)k, (long long)E);
  if (E > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "E > %lld", (long long)kMaxExperts);
  if (T == 0) return ok();
  if (!logits || !topk_w || !topk_ids) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(moe::launch_route(logits, T, static_cast<int>(E), static_cast<int>(k),
                                      renormalize, topk_w, topk_ids, stream),
                    "route_topk");
}

int moe_route_select(const float* logits, int64_t T, int64_t E, int64_t k, const moe_routing* routing,
                     float* topk_w, int32_t* topk_ids, hipStream_t stream) {
  int st;
  if ((st = check_routing(T, E, k, routing)) != MOE_OK) return st;
  if (T == 0) return ok();
  if (!logits || !topk_w || !topk_ids) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(launch_routing(logits, T, E, k, routing, topk_w, topk_ids, stream), "route_select");
}

int64_t moe_align_capacity(int64_t T, int64_t k, int64_t E, int64_t block_m) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1) return 0;
  return capacity(T, k, E, block_m);
}

int moe_align_block(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                    int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                    hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0, k >= 1, E >= 1, block_m >= 1");
  if (E > kMaxExperts || block_m > 1024)
    return fail(MOE_ERR_UNSUPPORTED, "E or block_m above 1024");
  if (!num_padded) return fail(MOE_ERR_INVALID_ARGUMENT, "null num_padded");
  const int64_t tk = T * k;
  if (tk > 0x7fffffffLL) return fail(MOE_ERR_UNSUPPORTED, "T*k above 2^31-1");
  if (tk == 0)   // the kernel with no assignments only writes *num_padded = 0
    return hip_status(moe::launch_align(topk_ids, 0, static_cast<int>(E), static_cast<int>(block_m), 0,
                                        sorted_ids, block_expert, num_padded, stream),
                      "align");
  if (!topk_ids || !sorted_ids || !block_expert) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  const int64_t cap = capacity(T, k, E, block_m);
  return hip_status(moe::launch_align(topk_ids, tk, static_cast<int>(E), static_cast<int>(block_m), cap,
                                      sorted_ids, block_expert, num_padded, stream),
                    "align");
}

int64_t moe_w8a16_block_m(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  if (T < 0 || E < 1 || k < 1) return 16;
  return auto_block_m(T, E, k, true, H, I);
}

int64_t moe_w8a16_splits(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m) {
  if (T <= 0 || H < 128 || I < 128 || E < 1 || k < 1) return 1;
  if (block_m == 0) block_m = auto_block_m(T, E, k, true, H, I);
  return splits_for(T, H, I, E, k, block_m);
}

size_t moe_w8a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                                 int64_t block_m) {
  return workspace_for(Fmt::W8, T, H, I, E, k, block_m, nullptr);
}

size_t moe_w8a16_workspace_bytes_ex(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                    const moe_fused_opts* opts) {
  return workspace_for(Fmt::W8, T, H, I, E, k, block_m, opts);
}

size_t moe_w8a16_intermediate_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m) {
  if (T <= 0 || I < 1 || E < 1 || k < 1) return 0;
  if (block_m == 0) block_m = auto_block_m(T, E, k, true, H, I);
  if (block_m < 16 || block_m > 256 || block_m % 16) return 0;
  return intermediate_bytes(capacity(T, k, E, block_m), I, block_m, true);
}

int moe_w8a16_gemm1(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E,
                    int64_t k, const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                    const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, int64_t block_m, float* a, hipStream_t stream) {
  int st;
  if ((st = check_layer_dims(T, H, I, E, k)) != MOE_OK) return st;
  if ((st = check_act(act_dtype)) != MOE_OK) return st;
  if ((st = check_block_m(block_m)) != MOE_OK) return st;
  const int64_t ldw = w13_row_stride ? w13_row_stride : H;
  if (ldw < H || ldw % 16) return fail(MOE_ERR_INVALID_ARGUMENT, "w13_row_stride must be >= H and a multiple of 16");
  if (T == 0) return ok();
  if (!x || !w13 || !w13_scale || !sorted_ids || !block_expert || !num_padded || !a)
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(a, 16))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x, w13 and a must be 16-byte aligned");
  moe::Gemm1Args p{};
  p.x = x; p.f16 = act_dtype == MOE_FP16; p.T = T; p.H = H; p.I = I; p.k = k; p.Tk = T * k;
  p.w13 = w13; p.s13 = w13_scale; p.ldw = ldw;
  p.sorted_ids = sorted_ids; p.block_expert = block_expert; p.num_padded = num_padded;
  p.block_m = static_cast<int>(block_m); p.cap = capacity(T, k, E, block_m); p.a = a;
  return hip_status(run_gemm1(p, T, E, stream), "gemm1_w8");
}

int moe_w8a16_requant(float* a, int64_t T, int64_t I, int64_t E, int64_t k, const int32_t* sorted_ids,
                      const int32_t* num_padded, int64_t block_m, hipStream_t stream) {
  int st;
  if (T < 0 || E < 1 || k < 1 || k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0, 1 <= k <= E");
  if (I < 128 || I % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "I must be a positive multiple of 128");
  if ((st = check_block_m(block_m)) != MOE_OK) return st;
  if (T == 0 || !needs_requant(block_m)) return ok();
  if (!a || !sorted_ids || !num_padded) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(a, 16)) return fail(MOE_ERR_INVALID_ARGUMENT, "a must be 16-byte aligned");
  const int64_t cap = capacity(T, k, E, block_m);
  const Q16 q = q16_at(a, cap, I, planes_bytes(cap, I));
  return hip_status(moe::launch_requant_q16(a, cap, I, sorted_ids, num_padded, T * k, q.hi, q.lo, q.scale, stream),
                    "requant");
}

int moe_w8a16_gemm2(const float* a, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                    const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                    const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, int64_t block_m, int64_t splits, float* y,
                    hipStream_t stream) {
  int st;
  if ((st = check_layer_dims(T, H, I, E, k)) != MOE_OK) return st;
  if ((st = check_block_m(block_m)) != MOE_OK) return st;
  const int64_t ldw = w2_row_stride ? w2_row_stride : I;
  if (ldw < I || ldw % 16) return fail(MOE_ERR_INVALID_ARGUMENT, "w2_row_stride must be >= I and a multiple of 16");
  if (splits < 1 || splits > I / 128 ||
      (!gemm2_int8(block_m) && !prefill_q16(T, H, block_m) && (I / 128) % splits != 0))
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "splits must be in [1, I/128] and divide I/128 when block_m > 64 (except for 256-row blocks "
                "with H a multiple of 256)");
  if (T == 0) return ok();
  if (!a || !w2 || !w2_scale || !sorted_ids || !block_expert || !num_padded || !y)
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(a, 16) || !aligned(w2, 16)) return fail(MOE_ERR_INVALID_ARGUMENT, "a and w2 must be 16-byte aligned");
  moe::Gemm2Args p{};
  p.a = a; p.H = H; p.I = I; p.Tk = T * k; p.w2 = w2; p.s2 = w2_scale; p.ldw = ldw;
  p.sorted_ids = sorted_ids; p.block_expert = block_expert; p.num_padded = num_padded;
  p.block_m = static_cast<int>(block_m); p.cap = capacity(T, k, E, block_m);
  p.splits = static_cast<int>(splits); p.y = y;
  return hip_status(run_gemm2(p, T, E, k, stream), "gemm2_w8");
}

int moe_combine_topk(const float* y, int64_t splits, int64_t T, int64_t k, int64_t H, int64_t E,
                     const float* topk_w, const int32_t* topk_ids, int act_dtype, void* out,
                     hipStream_t stream) {
  int st;
  if ((st = check_act(act_dtype)) != MOE_OK) return st;
  if (T < 0 || k < 1 || H < 1 || E < 1 || splits < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0 and k, H, E, splits >= 1");
  if (H % 4) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a multiple of 4");
  if (T == 0) return ok();
  if (!y || !topk_w || !topk_ids || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(y, 16) || !aligned(out, 8)) return fail(MOE_ERR_INVALID_ARGUMENT, "y / out misaligned");
  return hip_status(moe::launch_combine(y, static_cast<int>(splits), T, static_cast<int>(k), H,
                                        static_cast<int>(E), topk_w, topk_ids,
                                        act_dtype == MOE_FP16, out, stream),
                    "combine");
}

}  // extern "C"

namespace {

// Route (when logits are given) + align + GEMM1 + GEMM2 + combine.
int forward_w8(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
               const int8_t* w13, const float* w13_scale, int64_t w13_row_stride, const int8_t* w2,
               const float* w2_scale, int64_t w2_row_stride, const float* logits, const moe_routing* routing,
               float* topk_w_out, int32_t* topk_ids_out, const float* topk_w, const int32_t* topk_ids,
               const moe_fused_opts* fo, int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  const int64_t ld13 = w13_row_stride ? w13_row_stride : H;
  const int64_t ld2 = w2_row_stride ? w2_row_stride : I;
  if (ld13 < H || ld13 % 16 || ld2 < I || ld2 % 16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "row strides must cover the row and be multiples of 16");
  if (T > 0 && (!w13 || !w13_scale || !w2 || !w2_scale || !out)) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (T > 0 && (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(out, 8)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "w13, w2 16-byte and out 8-byte alignment required");
  Front F{};
  int st = layer_front(Fmt::W8, x, act_dtype, T, H, I, E, k, fo, logits, routing, topk_w_out, topk_ids_out, topk_w,
                       topk_ids, block_m, workspace, workspace_bytes, stream, &F);
  if (st != MOE_OK || F.T == 0) return st;
  moe::Gemm1Args p1{};
  p1.x = F.x; p1.f16 = act_dtype == MOE_FP16; p1.T = F.Tg; p1.H = H; p1.I = I; p1.k = F.kg; p1.Tk = F.Tk;
  p1.w13 = w13; p1.s13 = w13_scale; p1.ldw = ld13; p1.sorted_ids = F.sorted; p1.block_expert = F.blocks;
  p1.num_padded = F.npad; p1.block_m = static_cast<int>(F.bm); p1.cap = F.cap; p1.a = F.a;
  hipError_t e;
  if ((e = run_gemm1_and_requant(p1, F.Tg, F.Ex, stream)) != hipSuccess) return hip_status(e, "gemm1_w8");
  moe::Gemm2Args p2{};
  p2.a = F.a; p2.H = H; p2.I = I; p2.Tk = F.Tk; p2.w2 = w2; p2.s2 = w2_scale; p2.ldw = ld2;
  p2.sorted_ids = F.sorted; p2.block_expert = F.blocks; p2.num_padded = F.npad;
  p2.block_m = static_cast<int>(F.bm); p2.cap = F.cap; p2.splits = static_cast<int>(F.splits); p2.y = F.y;
  if ((e = run_gemm2(p2, F.Tg, F.Ex, F.kg, stream)) != hipSuccess) return hip_status(e, "gemm2_w8");
  return layer_back(F, H, act_dtype, out, stream);
}

}  // namespace

extern "C" {

int moe_w8a16_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E,
                      int64_t k, const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                      const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                      const float* topk_w, const int32_t* topk_ids, int64_t block_m, void* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_w8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                    nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, nullptr, block_m, out, workspace,
                    workspace_bytes, stream);
}

int moe_w8a16_forward_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                         const int8_t* w13, const float* w13_scale, int64_t w13_row_stride, const int8_t* w2,
                         const float* w2_scale, int64_t w2_row_stride, const float* topk_w, const int32_t* topk_ids,
                         const moe_fused_opts* opts, int64_t block_m, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return forward_w8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                    nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, opts, block_m, out, workspace,
                    workspace_bytes, stream);
}

int moe_w8a16_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                    const float* router_logits, int renormalize,
                    const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                    const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                    float* topk_w, int32_t* topk_ids, int64_t block_m, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !router_logits) return fail(MOE_ERR_INVALID_ARGUMENT, "null router_logits");
  const moe_routing r{MOE_SCORING_SOFTMAX, renormalize, 0, 0, nullptr, 1.0f};
  return forward_w8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                    router_logits, &r, topk_w, topk_ids, nullptr, nullptr, nullptr, block_m, out, workspace,
                    workspace_bytes, stream);
}

int moe_w8a16_apply_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                       const float* router_logits, const moe_routing* routing, const int8_t* w13,
                       const float* w13_scale, int64_t w13_row_stride, const int8_t* w2, const float* w2_scale,
                       int64_t w2_row_stride, const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids,
                       int64_t block_m, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !router_logits) return fail(MOE_ERR_INVALID_ARGUMENT, "null router_logits");
  return forward_w8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                    router_logits, routing, topk_w, topk_ids, nullptr, nullptr, opts, block_m, out, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Forward without allocation: the workspace is a static device array
// ---------------------------------------------------------------------------

namespace {

// Device-resident workspace of moe_w8a16_forward_noalloc.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never a device address: its device
// address is looked up once per device with hipGetSymbolAddress and only that
// pointer is handed to kernels.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_w8a16_forward_noalloc(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E,
                              int64_t k, const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                              const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                              const float* topk_w, const int32_t* topk_ids, int64_t block_m, void* out,
                              hipStream_t stream) {
  int st;
  if ((st = check_layer_dims(T, H, I, E, k)) != MOE_OK) return st;
  const int64_t bm = block_m == 0 ? auto_block_m(T, E, k, true, H, I) : block_m;
  if ((st = check_block_m(bm)) != MOE_OK) return st;
  if (T == 0) return ok();
  const size_t need = workspace_for(Fmt::W8, T, H, I, E, k, bm, nullptr);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "this batch needs %zu bytes of workspace; the static scratch of the no-alloc forward holds %zu "
                "(use moe_w8a16_forward with a caller workspace)",
                need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
  return forward_w8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                    nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, nullptr, bm, out, ws,
                    MOE_NOALLOC_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------------------
// W4A16
// ---------------------------------------------------------------------------

int moe_quantize_weights_w4(const float* w, int64_t E, int64_t N, int64_t K, int64_t group_size,
                            int32_t* qweight, uint16_t* scales, int32_t* qzeros, hipStream_t stream) {
  if (E < 1 || N < 1 || K < 1 || group_size < 8)
    return fail(MOE_ERR_INVALID_ARGUMENT, "E, N, K >= 1 and group_size >= 8 required");
  if (N % 8 || group_size % 8 || K % group_size)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need N %% 8 == 0, group_size %% 8 == 0, K %% group_size == 0");
  if (!w || !qweight || !scales || !qzeros) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(moe::launch_quantize_w4(w, E, N, K, group_size, qweight, scales, qzeros, stream),
                    "quantize_w4");
}

size_t moe_w4a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                                 int64_t block_m) {
  return workspace_for(Fmt::W4, T, H, I, E, k, block_m, nullptr);
}

size_t moe_w4a16_workspace_bytes_ex(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                    const moe_fused_opts* opts) {
  return workspace_for(Fmt::W4, T, H, I, E, k, block_m, opts);
}

}  // extern "C"

namespace {

int forward_w4(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
               const int32_t* w13_qweight, const uint16_t* w13_scales, const int32_t* w13_qzeros,
               const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros, int64_t group_size,
               const float* logits, const moe_routing* routing, float* topk_w_out, int32_t* topk_ids_out,
               const float* topk_w, const int32_t* topk_ids, const moe_fused_opts* fo, int64_t block_m, void* out,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (group_size < 128 || group_size % 128 || H % group_size || I % group_size)
    return fail(MOE_ERR_UNSUPPORTED, "group_size must be a multiple of 128 dividing H and I (got %lld)",
                (long long)group_size);
  if (T > 0 && (!w13_qweight || !w13_scales || !w13_qzeros || !w2_qweight || !w2_scales || !w2_qzeros || !out))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (T > 0 && (!aligned(w13_qweight, 16) || !aligned(w2_qweight, 16) || !aligned(out, 8)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "alignment: qweights 16 bytes, out 8");
  Front F{};
  int st = layer_front(Fmt::W4, x, act_dtype, T, H, I, E, k, fo, logits, routing, topk_w_out, topk_ids_out, topk_w,
                       topk_ids, block_m, workspace, workspace_bytes, stream, &F);
  if (st != MOE_OK || F.T == 0) return st;
  moe::Gemm1W4Args p1{};
  p1.x = F.x; p1.f16 = act_dtype == MOE_FP16; p1.T = F.Tg; p1.H = H; p1.I = I; p1.k = F.kg; p1.Tk = F.Tk;
  p1.qw = w13_qweight; p1.sc = w13_scales; p1.qz = w13_qzeros; p1.group = static_cast<int>(group_size);
  p1.sorted_ids = F.sorted; p1.block_expert = F.blocks; p1.num_padded = F.npad;
  p1.block_m = static_cast<int>(F.bm); p1.cap = F.cap; p1.a = F.a;
  // blocks of 16 or 32 rows: the DMA-fed ring (it copies the fp16 scales as
  // dwords, at most 32 scale groups per row)
  const bool w4_dma = (F.bm == 16 || F.bm == 32) && aligned(w13_scales, 4) && H / group_size <= 32;
  hipError_t e = w4_dma ? moe::launch_gemm1_w4_dma(p1, stream)
                        : (w4_stream(F.bm) ? moe::launch_gemm1_w4_stream(p1, stream) : moe::launch_gemm1_w4(p1, stream));
  if (e != hipSuccess) return hip_status(e, "gemm1_w4");
  moe::Gemm2W4Args p2{};
  p2.a = F.a; p2.f16 = act_dtype == MOE_FP16; p2.H = H; p2.I = I; p2.Tk = F.Tk;
  p2.qw = w2_qweight; p2.sc = w2_scales; p2.qz = w2_qzeros; p2.group = static_cast<int>(group_size);
  p2.sorted_ids = F.sorted; p2.block_expert = F.blocks; p2.num_padded = F.npad;
  p2.block_m = static_cast<int>(F.bm); p2.cap = F.cap; p2.splits = static_cast<int>(F.splits); p2.y = F.y;
  if ((e = w4_stream(F.bm) ? moe::launch_gemm2_w4_stream(p2, stream) : moe::launch_gemm2_w4(p2, stream)) !=
      hipSuccess)
    return hip_status(e, "gemm2_w4");
  return layer_back(F, H, act_dtype, out, stream);
}

}  // namespace

extern "C" {

int moe_w4a16_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E,
                      int64_t k, const int32_t* w13_qweight, const uint16_t* w13_scales,
                      const int32_t* w13_qzeros, const int32_t* w2_qweight,
                      const uint16_t* w2_scales, const int32_t* w2_qzeros, int64_t group_size,
                      const float* topk_w, const int32_t* topk_ids, int64_t block_m, void* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_w4(x, act_dtype, T, H, I, E, k, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales,
                    w2_qzeros, group_size, nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, nullptr, block_m, out,
                    workspace, workspace_bytes, stream);
}

int moe_w4a16_forward_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                         const int32_t* w13_qweight, const uint16_t* w13_scales, const int32_t* w13_qzeros,
                         const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros,
                         int64_t group_size, const float* topk_w, const int32_t* topk_ids,
                         const moe_fused_opts* opts, int64_t block_m, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return forward_w4(x, act_dtype, T, H, I, E, k, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales,
                    w2_qzeros, group_size, nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, opts, block_m, out,
                    workspace, workspace_bytes, stream);
}

int moe_w4a16_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                    const float* router_logits, int renormalize,
                    const int32_t* w13_qweight, const uint16_t* w13_scales, const int32_t* w13_qzeros,
                    const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros,
                    int64_t group_size, float* topk_w, int32_t* topk_ids, int64_t block_m, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !router_logits) return fail(MOE_ERR_INVALID_ARGUMENT, "null router_logits");
  const moe_routing r{MOE_SCORING_SOFTMAX, renormalize, 0, 0, nullptr, 1.0f};
  return forward_w4(x, act_dtype, T, H, I, E, k, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales,
                    w2_qzeros, group_size, router_logits, &r, topk_w, topk_ids, nullptr, nullptr, nullptr, block_m,
                    out, workspace, workspace_bytes, stream);
}

int moe_w4a16_apply_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                       const float* router_logits, const moe_routing* routing, const int32_t* w13_qweight,
                       const uint16_t* w13_scales, const int32_t* w13_qzeros, const int32_t* w2_qweight,
                       const uint16_t* w2_scales, const int32_t* w2_qzeros, int64_t group_size,
                       const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids, int64_t block_m, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !router_logits) return fail(MOE_ERR_INVALID_ARGUMENT, "null router_logits");
  return forward_w4(x, act_dtype, T, H, I, E, k, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales,
                    w2_qzeros, group_size, router_logits, routing, topk_w, topk_ids, nullptr, nullptr, opts, block_m,
                    out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// GPTQ / AWQ import
// ---------------------------------------------------------------------------

extern "C" {

int moe_wna16_group_size(int64_t H, int64_t I, int64_t group_size, int64_t* group, int64_t* repeat) {
  if (H < 1 || I < 1 || group_size < 1 || !group || !repeat)
    return fail(MOE_ERR_INVALID_ARGUMENT, "need H, I, group_size >= 1 and output pointers");
  int64_t g = group_size, r = 1;
  while (I % g || H % g) {
    g /= 2;
    r *= 2;
    if (g < 32) return fail(MOE_ERR_INVALID_ARGUMENT, "the group size would fall below 32");
  }
  *group = g;
  *repeat = r;
  return ok();
}

int moe_w4_import(int format, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales, int64_t N,
                  int64_t K, int64_t group_size, int64_t repeat, int32_t* out_qweight, uint16_t* out_scales,
                  int32_t* out_qzeros, hipStream_t stream) {
  if (format != MOE_W4_AWQ && format != MOE_W4_GPTQ) return fail(MOE_ERR_INVALID_ARGUMENT, "unknown format %d", format);
  if (N < 8 || K < 8 || N % 8 || K % 8) return fail(MOE_ERR_INVALID_ARGUMENT, "N and K must be positive multiples of 8");
  if (repeat < 1 || group_size < 1 || group_size % repeat)
    return fail(MOE_ERR_INVALID_ARGUMENT, "repeat must be >= 1 and divide group_size");
  const int64_t gout = group_size / repeat;
  if (K % gout) return fail(MOE_ERR_INVALID_ARGUMENT, "the output group %lld does not divide K %lld", (long long)gout,
                            (long long)K);
  if (!qweight || !qzeros || !scales || !out_qweight || !out_scales || !out_qzeros)
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(moe::launch_import_w4(format == MOE_W4_GPTQ, qweight, qzeros, scales, N, K, gout, repeat,
                                          out_qweight, out_scales, out_qzeros, stream),
                    "import_w4");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Weight-only fp8 (e4m3fn) experts
// ---------------------------------------------------------------------------

namespace {

int forward_fp8(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                const uint8_t* w13, const float* w13_scale, int64_t w13_row_stride, const uint8_t* w2,
                const float* w2_scale, int64_t w2_row_stride, const float* logits, const moe_routing* routing,
                float* topk_w_out, int32_t* topk_ids_out, const float* topk_w, const int32_t* topk_ids,
                const moe_fused_opts* fo, int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  const int64_t ld13 = w13_row_stride ? w13_row_stride : H;
  const int64_t ld2 = w2_row_stride ? w2_row_stride : I;
  if (ld13 < H || ld13 % 16 || ld2 < I || ld2 % 16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "row strides must cover the row and be multiples of 16");
  if (T > 0 && (!w13 || !w13_scale || !w2 || !w2_scale || !out)) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (T > 0 && (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(out, 8)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "w13, w2 16-byte and out 8-byte alignment required");
  Front F{};
  int st = layer_front(Fmt::FP8, x, act_dtype, T, H, I, E, k, fo, logits, routing, topk_w_out, topk_ids_out, topk_w,
                       topk_ids, block_m, workspace, workspace_bytes, stream, &F);
  if (st != MOE_OK || F.T == 0) return st;
  moe::Gemm1Args p1{};
  p1.x = F.x; p1.f16 = act_dtype == MOE_FP16; p1.T = F.Tg; p1.H = H; p1.I = I; p1.k = F.kg; p1.Tk = F.Tk;
  p1.w13 = reinterpret_cast<const int8_t*>(w13); p1.s13 = w13_scale; p1.ldw = ld13; p1.sorted_ids = F.sorted;
  p1.block_expert = F.blocks; p1.num_padded = F.npad; p1.block_m = static_cast<int>(F.bm); p1.cap = F.cap;
  p1.a = F.a; p1.fp8 = 1;
  hipError_t e;
  if (F.bm == 16 || F.bm == 32) e = moe::launch_gemm1_w8_dma(p1, nullptr, nullptr, nullptr, stream);
  else if (use_prefill(F.bm) && moe::gemm1_w8_big_fits(p1)) e = moe::launch_gemm1_w8_big(p1, nullptr, nullptr, nullptr, stream);
  else e = moe::launch_gemm1_w8(p1, stream);
  if (e != hipSuccess) return hip_status(e, "gemm1_fp8");
  moe::Gemm2Args p2{};
  p2.a = F.a; p2.H = H; p2.I = I; p2.Tk = F.Tk; p2.w2 = reinterpret_cast<const int8_t*>(w2); p2.s2 = w2_scale;
  p2.ldw = ld2; p2.sorted_ids = F.sorted; p2.block_expert = F.blocks; p2.num_padded = F.npad;
  p2.block_m = static_cast<int>(F.bm); p2.cap = F.cap; p2.splits = static_cast<int>(F.splits); p2.y = F.y; p2.fp8 = 1;
  e = moe::gemm2_planes_fits(H, I, F.bm)       ? moe::launch_gemm2_w8_planes(p2, stream)
      : moe::gemm2_fp8_dma_fits(H, I, F.bm) ? moe::launch_gemm2_fp8_dma(p2, stream)
                                             : moe::launch_gemm2_w8(p2, stream);
  if (e != hipSuccess) return hip_status(e, "gemm2_fp8");
  return layer_back(F, H, act_dtype, out, stream);
}

}  // namespace

extern "C" {

int moe_quantize_weights_fp8(const float* w, int64_t E, int64_t N, int64_t K, uint8_t* q, float* scale,
                             hipStream_t stream) {
  if (E < 1 || N < 1 || K < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "E, N and K must be >= 1");
  if (E > 65535) return fail(MOE_ERR_UNSUPPORTED, "more than 65535 tensors");
  if (!w || !q || !scale) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(moe::launch_quantize_fp8(w, E, N * K, q, scale, stream), "quantize_fp8");
}

int moe_fp8_merge_w13_scales(uint8_t* w13, const float* w13_shard_scales, int64_t E, int64_t I, int64_t H,
                             float* w13_scale, hipStream_t stream) {
  if (E < 1 || I < 1 || H < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "E, I and H must be >= 1");
  if (E > 65535) return fail(MOE_ERR_UNSUPPORTED, "more than 65535 experts");
  if (!w13 || !w13_shard_scales || !w13_scale) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  return hip_status(moe::launch_fp8_merge_w13(w13, w13_shard_scales, E, I, H, w13_scale, stream), "fp8_merge");
}

size_t moe_wfp8a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                   const moe_fused_opts* opts) {
  return workspace_for(Fmt::FP8, T, H, I, E, k, block_m, opts);
}

int moe_wfp8a16_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                        const uint8_t* w13, const float* w13_scale, int64_t w13_row_stride, const uint8_t* w2,
                        const float* w2_scale, int64_t w2_row_stride, const float* topk_w, const int32_t* topk_ids,
                        const moe_fused_opts* opts, int64_t block_m, void* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return forward_fp8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                     nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, opts, block_m, out, workspace,
                     workspace_bytes, stream);
}

int moe_wfp8a16_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                      const float* router_logits, const moe_routing* routing, const uint8_t* w13,
                      const float* w13_scale, int64_t w13_row_stride, const uint8_t* w2, const float* w2_scale,
                      int64_t w2_row_stride, const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids,
                      int64_t block_m, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !router_logits) return fail(MOE_ERR_INVALID_ARGUMENT, "null router_logits");
  return forward_fp8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                     router_logits, routing, topk_w, topk_ids, nullptr, nullptr, opts, block_m, out, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// W8A8: int8 weights, int8 activations quantized per token
// ---------------------------------------------------------------------------

namespace {

int forward_w8a8(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                 const int8_t* w13, const float* w13_scale, int64_t w13_row_stride, const int8_t* w2,
                 const float* w2_scale, int64_t w2_row_stride, const float* logits, const moe_routing* routing,
                 float* topk_w_out, int32_t* topk_ids_out, const float* topk_w, const int32_t* topk_ids,
                 const moe_fused_opts* fo, int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  const int64_t ld13 = w13_row_stride ? w13_row_stride : H;
  const int64_t ld2 = w2_row_stride ? w2_row_stride : I;
  if (ld13 < H || ld13 % 16 || ld2 < I || ld2 % 16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "row strides must cover the row and be multiples of 16");
  if (T > 0 && (!w13 || !w13_scale || !w2 || !w2_scale || !out)) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (T > 0 && (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(out, 8)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "w13, w2 16-byte and out 8-byte alignment required");
  Front F{};
  int st = layer_front(Fmt::W8A8, x, act_dtype, T, H, I, E, k, fo, logits, routing, topk_w_out, topk_ids_out, topk_w,
                       topk_ids, block_m, workspace, workspace_bytes, stream, &F);
  if (st != MOE_OK || F.T == 0) return st;
  const A8 v = w8a8_at(F.a, F.cap, I, F.Tg, H);
  hipError_t e = moe::launch_act_quant(F.x, act_dtype == MOE_FP16 ? 1 : 0, F.Tg, H, nullptr, nullptr, 0, nullptr, 0,
                                       v.qx, v.sx, stream);
  if (e != hipSuccess) return hip_status(e, "quantize x");
  moe::Gemm1Args p1{};
  p1.x = F.x; p1.f16 = act_dtype == MOE_FP16; p1.T = F.Tg; p1.H = H; p1.I = I; p1.k = F.kg; p1.Tk = F.Tk;
  p1.w13 = w13; p1.s13 = w13_scale; p1.ldw = ld13; p1.sorted_ids = F.sorted; p1.block_expert = F.blocks;
  p1.num_padded = F.npad; p1.block_m = static_cast<int>(F.bm); p1.cap = F.cap; p1.a = v.a;
  // the same choice as the split count of the workspace layout (row strides past 2^32 bytes per
  // expert make the big launchers fail the call)
  const bool big = w8a8_big(T, H, I, F.kx, F.bm);
  const bool dma = !big && moe::w8a8_dma_fits(H, I, F.bm);
  // the 256-row and the 16/32-row GEMM1 also leave the rows' partial maxima of |a|, so the
  // quantizer of a makes one pass over it
  e = big   ? moe::launch_gemm1_w8a8_big(p1, v.qx, v.sx, v.pmax, stream)
      : dma ? moe::launch_gemm1_w8a8_dma(p1, v.qx, v.sx, v.pmax, stream)
            : moe::launch_gemm1_w8a8(p1, v.qx, v.sx, stream);
  if (e != hipSuccess) return hip_status(e, "gemm1_w8a8");
  e = moe::launch_act_quant(v.a, 2, F.cap, I, F.sorted, F.npad, F.Tk, big || dma ? v.pmax : nullptr, I / 64, v.qa,
                            v.sa, stream);
  if (e != hipSuccess) return hip_status(e, "quantize a");
  moe::Gemm2Args p2{};
  p2.a = v.a; p2.H = H; p2.I = I; p2.Tk = F.Tk; p2.w2 = w2; p2.s2 = w2_scale; p2.ldw = ld2;
  p2.sorted_ids = F.sorted; p2.block_expert = F.blocks; p2.num_padded = F.npad;
  p2.block_m = static_cast<int>(F.bm); p2.cap = F.cap; p2.splits = static_cast<int>(F.splits); p2.y = F.y;
  e = big   ? moe::launch_gemm2_w8a8_big(p2, v.qa, v.sa, stream)
      : dma ? moe::launch_gemm2_w8a8_dma(p2, v.qa, v.sa, stream)
            : moe::launch_gemm2_w8a8(p2, v.qa, v.sa, stream);
  if (e != hipSuccess) return hip_status(e, "gemm2_w8a8");
  return layer_back(F, H, act_dtype, out, stream);
}

}  // namespace

extern "C" {

int moe_quantize_act_int8(const void* x, int act_dtype, int64_t T, int64_t H, int8_t* q, float* scale,
                          hipStream_t stream) {
  int st;
  if ((st = check_act(act_dtype)) != MOE_OK) return st;
  if (T < 0 || H < 1 || H % 4) return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0 and H a positive multiple of 4");
  if (T == 0) return ok();
  if (!x || !q || !scale) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "q must be 4-byte aligned");
  if (!aligned(x, 8)) return fail(MOE_ERR_INVALID_ARGUMENT, "x must be 8-byte aligned");
  return hip_status(moe::launch_act_quant(x, act_dtype == MOE_FP16 ? 1 : 0, T, H, nullptr, nullptr, 0, nullptr, 0,
                                          q, scale, stream),
                    "quantize_act_int8");
}

size_t moe_w8a8_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                const moe_fused_opts* opts) {
  return workspace_for(Fmt::W8A8, T, H, I, E, k, block_m, opts);
}

int moe_w8a8_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                     const int8_t* w13, const float* w13_scale, int64_t w13_row_stride, const int8_t* w2,
                     const float* w2_scale, int64_t w2_row_stride, const float* topk_w, const int32_t* topk_ids,
                     const moe_fused_opts* opts, int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return forward_w8a8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                      nullptr, nullptr, nullptr, nullptr, topk_w, topk_ids, opts, block_m, out, workspace,
                      workspace_bytes, stream);
}

int moe_w8a8_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                   const float* router_logits, const moe_routing* routing, const int8_t* w13, const float* w13_scale,
                   int64_t w13_row_stride, const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                   const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids, int64_t block_m, void* out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T > 0 && !router_logits) return fail(MOE_ERR_INVALID_ARGUMENT, "null router_logits");
  return forward_w8a8(x, act_dtype, T, H, I, E, k, w13, w13_scale, w13_row_stride, w2, w2_scale, w2_row_stride,
                      router_logits, routing, topk_w, topk_ids, nullptr, nullptr, opts, block_m, out, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"
