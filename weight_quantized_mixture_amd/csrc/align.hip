// Token -> expert align: histogram, prefix scan, padded-block permutation.
//
// The pages only call the fused expert kernel that consumes this grouping
// (experts_int8 page, ExpertsInt8MoEMethod.apply); the definition is in
// moe_wq.h.  One workgroup of 8 waves does all of it, with no atomics on
// positions, so the result is the unique stable order.  Up to 512
// assignments align_small below takes them one per thread; up to 16 chunks
// of 512 with chunks * E <= 1536, align_seg (a kernel of its own) ranks every
// chunk at once (see there); otherwise:
//   1. histogram of valid ids (LDS integer atomics: counts are order free);
//   2. wave 0 scans the padded counts into block offsets and writes the
//      block -> expert table; all threads write the padding sentinels;
//   3. the flat indices are walked in chunks of 512; inside a wave, lanes
//      with the same expert find each other with ballots over the id bits
//      (their rank is a popcount of the lower lanes), per-wave counts go to
//      LDS, and each element's slot is off[e] + done[e] + (counts of earlier
//      waves of the chunk) + rank.
#include "common.hpp"
#include "launch.hpp"
#include "router_dev.hpp"

namespace moe {

namespace {

constexpr int kAlignWaves = 8;
constexpr int kAlignThreads = kAlignWaves * kWave;
constexpr int kMaxExperts = 1024;

// The ids of the flat indices a thread handles are loaded once, all before
// the first use, when T*k <= kIdsInRegs * 512 (a loop that loads, waits and
// uses would pay one memory latency per 512 ids, twice).
constexpr int kIdsInRegs = 16;

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4 and 8 lanes inside each row of 16 (lanes shifted in from outside the row
// read 0), then lane 15 of rows 0 and 2 added to rows 1 and 3 and lane 31 to
// rows 2 and 3 (row broadcasts).  Six dependent adds instead of six
// LDS-path shuffles.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// 2. exclusive scan of the padded counts into block offsets (wave 0, 64
// experts per step); then the block -> expert table, the sentinels inside
// each expert's last block and those of the unused blocks and rows.
__device__ __forceinline__ void pad_and_tables(const int* cnt, int* off, int* total_padded, int E, int bm,
                                               int64_t cap, int sentinel, int32_t* __restrict__ sorted_ids,
                                               int32_t* __restrict__ block_expert,
                                               int32_t* __restrict__ num_padded) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int c = (e < E) ? cnt[e] : 0;
      const int p = (c + bm - 1) / bm * bm;
      const int incl = wave_incl_scan(p);
      if (e < E) off[e] = carry + incl - p;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      *total_padded = carry;
      *num_padded = carry;
    }
  }
  __syncthreads();

  const int used = *total_padded;
  for (int e = tid; e < E; e += kAlignThreads) {
    const int c = cnt[e];
    const int p = (c + bm - 1) / bm * bm;
    for (int b = off[e] / bm; b < (off[e] + p) / bm; ++b) block_expert[b] = e;
    for (int r = off[e] + c; r < off[e] + p; ++r) sorted_ids[r] = sentinel;
  }
  for (int64_t b = used / bm + tid; b < cap / bm; b += kAlignThreads) block_expert[b] = -1;
  for (int64_t r = used + tid; r < cap; r += kAlignThreads) sorted_ids[r] = sentinel;
}

// The rank of each lane's id among the lanes of its wave holding the same
// expert (lanes with e < 0 take part in nothing), and the size of its group:
// ballots over the id bits narrow the mask to the lanes with the same id.
__device__ __forceinline__ int wave_match_rank(int e, int nbits, int* group) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool active = e >= 0;
  uint64_t mask = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = active && ((e >> b) & 1);
    const uint64_t bal = __ballot(bit);
    mask &= bit ? bal : ~bal;
  }
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  *group = __popcll(mask);
  return __popcll(mask & lower);
}

template <bool REGS>
__device__ __forceinline__ void align_body(
    const int32_t* __restrict__ ids, int64_t Tk, int E, int bm, int64_t cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts];
  __shared__ int done[kMaxExperts];
  __shared__ int wc[kAlignWaves][kMaxExperts];
  __shared__ int total_padded;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int sentinel = static_cast<int>(Tk);

  int reg_ids[REGS ? kIdsInRegs : 1];
  auto id_of = [&](int u, int64_t f) -> int {
    int e;
    if constexpr (REGS) e = reg_ids[u];
    else e = f < Tk ? ids[f] : -1;
    return (e >= 0 && e < E) ? e : -1;
  };
  if constexpr (REGS) {
#pragma unroll
    for (int u = 0; u < kIdsInRegs; ++u) {
      const int64_t f = static_cast<int64_t>(u) * kAlignThreads + tid;
      reg_ids[u] = f < Tk ? ids[f] : -1;
    }
  }
  const int nchunks = static_cast<int>((Tk + kAlignThreads - 1) / kAlignThreads);

  for (int e = tid; e < E; e += kAlignThreads) {
    cnt[e] = 0;
    done[e] = 0;
  }
  __syncthreads();

  // 1. histogram
  if constexpr (REGS) {
#pragma unroll
    for (int u = 0; u < kIdsInRegs; ++u) {
      const int e = id_of(u, 0);
      if (e >= 0) atomicAdd(&cnt[e], 1);
    }
  } else {
    for (int64_t f = tid; f < Tk; f += kAlignThreads) {
      const int e = id_of(0, f);
      if (e >= 0) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();

  pad_and_tables(cnt, off, &total_padded, E, bm, cap, sentinel, sorted_ids, block_expert, num_padded);

  // 3. stable scatter
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  auto chunk = [&](int u) {
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) wc[i / E][i % E] = 0;
    __syncthreads();
    const int64_t f = static_cast<int64_t>(u) * kAlignThreads + tid;
    const int e = id_of(u, f);
    const bool active = (e >= 0);
    int group;
    const int rank = wave_match_rank(e, nbits, &group);
    if (active && rank == 0) wc[wave][e] = group;
    __syncthreads();
    if (active) {
      int pos = off[e] + done[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wc[w][e];
      sorted_ids[pos] = static_cast<int32_t>(f);
    }
    __syncthreads();
    for (int x = tid; x < E; x += kAlignThreads) {
      int s = 0;
      for (int w = 0; w < kAlignWaves; ++w) s += wc[w][x];
      done[x] += s;
    }
    __syncthreads();
  };
  if constexpr (REGS) {
#pragma unroll
    for (int u = 0; u < kIdsInRegs; ++u)
      if (u < nchunks) chunk(u);
  } else {
    for (int u = 0; u < nchunks; ++u) chunk(u);
  }
}

// Up to 16 chunks of 512 assignments with chunks * E <= 1536 (for example
// 6144 assignments of 64 experts, 8192 of 8): each thread keeps its 16 ids
// and their in-wave ranks in registers; the leaders of each (chunk, wave,
// expert) group store the group's size in LDS, all chunks at once; then, per
// (chunk, expert), the sizes become exclusive prefixes over the waves of the
// chunk and the chunk totals, per expert, exclusive prefixes over the chunks
// (their sum is the expert's count).  Flat index f = 512 chunk + 64 wave +
// lane, so the slot off[e] + (chunks before) + (waves before) + rank is the
// stable position.  Three barriers before the offsets scan, none per chunk,
// no atomics.
constexpr int kSegChunks = 16;
constexpr int kSegCells = 1536;                  // chunks * E at most

__device__ __forceinline__ void align_seg(const int32_t* __restrict__ ids, int64_t Tk, int E, int bm, int64_t cap,
                                          int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                                          int32_t* __restrict__ num_padded) {
  __shared__ int seg[kSegCells * kAlignWaves];  // [chunk][wave][E]
  __shared__ int cpre[kSegCells];               // [chunk][E]
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts];
  __shared__ int total_padded;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int nchunks = static_cast<int>((Tk + kAlignThreads - 1) / kAlignThreads);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  int ev[kSegChunks];
#pragma unroll
  for (int u = 0; u < kSegChunks; ++u) {
    const int64_t f = static_cast<int64_t>(u) * kAlignThreads + tid;
    const int e = f < Tk ? ids[f] : -1;
    ev[u] = (e >= 0 && e < E) ? e : -1;
  }
  for (int i = tid; i < nchunks * kAlignWaves * E; i += kAlignThreads) seg[i] = 0;
  __syncthreads();
  int rank[kSegChunks];
#pragma unroll
  for (int u = 0; u < kSegChunks; ++u) {
    rank[u] = 0;
    if (u < nchunks) {
      int group;
      rank[u] = wave_match_rank(ev[u], nbits, &group);
      if (ev[u] >= 0 && rank[u] == 0) seg[(u * kAlignWaves + wave) * E + ev[u]] = group;
    }
  }
  __syncthreads();
  for (int task = tid; task < nchunks * E; task += kAlignThreads) {
    const int u = task / E, e = task - u * E;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = seg[(u * kAlignWaves + w) * E + e];
      seg[(u * kAlignWaves + w) * E + e] = sum;
      sum += c;
    }
    cpre[task] = sum;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    int sum = 0;
    for (int u = 0; u < nchunks; ++u) {
      const int c = cpre[u * E + e];
      cpre[u * E + e] = sum;
      sum += c;
    }
    cnt[e] = sum;
  }
  __syncthreads();
  pad_and_tables(cnt, off, &total_padded, E, bm, cap, static_cast<int>(Tk), sorted_ids, block_expert, num_padded);
#pragma unroll
  for (int u = 0; u < kSegChunks; ++u) {
    const int e = ev[u];
    if (u < nchunks && e >= 0) {
      const int pos = off[e] + cpre[u * E + e] + seg[(u * kAlignWaves + wave) * E + e] + rank[u];
      sorted_ids[pos] = static_cast<int32_t>(static_cast<int64_t>(u) * kAlignThreads + tid);
    }
  }
}

// At most one id per thread (T*k <= 512), the decode case: the same result
// as align_body with fewer dependent steps.  Lanes with the same expert find
// each other with ballots over the id bits once; the leader of each group
// writes the wave's count, and one pass per expert turns the waves' counts
// into the expert's total and exclusive per-wave offsets (no LDS atomics);
// after the scan every thread writes its own assignment's row, and the
// sentinels and the block table are written per row and per block from an
// LDS table of each used block's expert (no loops over an expert's rows).
__device__ __forceinline__ void align_small(const int32_t* __restrict__ ids, int Tk, int E, int bm, int64_t cap,
                                            int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                                            int32_t* __restrict__ num_padded) {
  __shared__ int s_wc[kAlignWaves][kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_blk[kAlignThreads];   // used blocks <= sum of ceil(count / bm) <= T*k
  __shared__ int s_used;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int raw = tid < Tk ? ids[tid] : -1;
  const int e = (raw >= 0 && raw < E) ? raw : -1;
#pragma unroll
  for (int w = 0; w < kAlignWaves; ++w)
    for (int x = tid; x < E; x += kAlignThreads) s_wc[w][x] = 0;
  __syncthreads();

  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const bool active = e >= 0;
  uint64_t mask = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = active && ((e >> b) & 1);
    const uint64_t bal = __ballot(bit);
    mask &= bit ? bal : ~bal;
  }
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int rank = __popcll(mask & lower);
  if (active && rank == 0) s_wc[wave][e] = __popcll(mask);
  __syncthreads();

  for (int x = tid; x < E; x += kAlignThreads) {
    int pre = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = s_wc[w][x];
      s_wc[w][x] = pre;
      pre += c;
    }
    s_cnt[x] = pre;
  }
  __syncthreads();

  // exclusive scan of the padded counts (wave 0, 64 experts per step)
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int x = base + lane;
      const int c = (x < E) ? s_cnt[x] : 0;
      const int pc = (c + bm - 1) / bm * bm;
      const int incl = wave_incl_scan(pc);
      if (x < E) s_off[x] = carry + incl - pc;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      s_used = carry;
      *num_padded = carry;
    }
  }
  __syncthreads();

  for (int x = tid; x < E; x += kAlignThreads) {
    const int nb = (s_cnt[x] + bm - 1) / bm;
    for (int b = 0; b < nb; ++b) s_blk[s_off[x] / bm + b] = x;
  }
  if (active) sorted_ids[s_off[e] + s_wc[wave][e] + rank] = tid;
  __syncthreads();
  const int64_t ublocks = s_used / bm;
  const int sentinel = Tk;
  for (int64_t b = tid; b < cap / bm; b += kAlignThreads) block_expert[b] = b < ublocks ? s_blk[b] : -1;
  for (int64_t r = tid; r < cap; r += kAlignThreads) {
    const int64_t b = r / bm;
    if (b >= ublocks) {
      sorted_ids[r] = sentinel;
    } else {
      const int x = s_blk[b];
      if (r - s_off[x] >= s_cnt[x]) sorted_ids[r] = sentinel;   // padding row of expert x's last block
    }
  }
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t Tk, int E, int bm, int64_t cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  if (Tk <= kAlignThreads)
    align_small(ids, static_cast<int>(Tk), E, bm, cap, sorted_ids, block_expert, num_padded);
  else if (Tk <= static_cast<int64_t>(kIdsInRegs) * kAlignThreads)
    align_body<true>(ids, Tk, E, bm, cap, sorted_ids, block_expert, num_padded);
  else
    align_body<false>(ids, Tk, E, bm, cap, sorted_ids, block_expert, num_padded);
}

// align_seg in a launch of its own (its LDS would not fit beside the other
// paths' in one kernel).
__global__ __launch_bounds__(kAlignThreads) void align_seg_kernel(
    const int32_t* __restrict__ ids, int64_t Tk, int E, int bm, int64_t cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  align_seg(ids, Tk, E, bm, cap, sorted_ids, block_expert, num_padded);
}

bool seg_fits(int64_t Tk, int E) {
  const int64_t nchunks = (Tk + kAlignThreads - 1) / kAlignThreads;
  return Tk > kAlignThreads && nchunks <= kSegChunks && nchunks * E <= kSegCells;
}

// Routing and align in one launch (small batches): the 8 waves route the
// tokens round-robin, then the same workgroup groups the ids it just wrote.
__global__ __launch_bounds__(kAlignThreads) void route_align_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renormalize,
    float* __restrict__ topk_w, int32_t* __restrict__ topk_ids, int bm, int64_t cap,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ __attribute__((aligned(16))) uint64_t keys[kAlignWaves][kRankMaxExperts];
  const int wave = threadIdx.x / kWave;
  for (int64_t t = wave; t < T; t += kAlignWaves)
    route_token(logits + t * E, E, k, renormalize, topk_w + t * k, topk_ids + t * k, keys[wave]);
  __syncthreads();
  if (T * k <= kAlignThreads)
    align_small(topk_ids, static_cast<int>(T * k), E, bm, cap, sorted_ids, block_expert, num_padded);
  else
    align_body<true>(topk_ids, T * k, E, bm, cap, sorted_ids, block_expert, num_padded);
}

}  // namespace

hipError_t launch_route_align(const float* logits, int64_t T, int E, int k, int renormalize, float* topk_w,
                              int32_t* topk_ids, int block_m, int64_t cap, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* num_padded, hipStream_t stream) {
  hipLaunchKernelGGL(route_align_kernel, dim3(1), dim3(kAlignThreads), 0, stream, logits, T, E, k, renormalize,
                     topk_w, topk_ids, block_m, cap, sorted_ids, block_expert, num_padded);
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* topk_ids, int64_t Tk, int E, int block_m, int64_t cap,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t stream) {
  if (seg_fits(Tk, E))
    hipLaunchKernelGGL(align_seg_kernel, dim3(1), dim3(kAlignThreads), 0, stream, topk_ids, Tk, E,
                       block_m, cap, sorted_ids, block_expert, num_padded);
  else
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, stream, topk_ids, Tk, E,
                       block_m, cap, sorted_ids, block_expert, num_padded);
  return hipGetLastError();
}

}  // namespace moe
