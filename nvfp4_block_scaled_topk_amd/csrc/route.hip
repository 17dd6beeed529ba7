// route.hip -- top-k routing of a whole token batch and the per-expert row lists.
//
// A whole batch is routed in one run so every selected expert is read once for all
// of its rows [FP4-Local checkpoints on DGX Spark, §4 Round 1, #740 and #808]. The
// weights are the renormalized softmax over the selected logits (the router
// normalization policy the pages name, [bloomery 0.3.9 release notes, Fixed, #772],
// read as softmax -> top-k -> renormalize).
//
// Kernel 1 (16 tokens per block, 256 threads): for E <= 256 and k <= 16 each token
// owns one 16-lane row of a wave (four tokens a wave at a time) and finds its k best
// (logit desc, index asc) by k rounds of a row argmax built from DPP lane exchanges;
// larger E or k fall back to a wave per token and wave-wide shuffles. The choice is on
// the logits, or on the float32 sums logit + bias[e] when a correction bias is given;
// the weights follow from the unbiased logits under the router's normalization policy,
// a named value on the pages [bloomery 0.3.9 release notes, From our contributors,
// #772]: softmax renormalized over the selected (the default), softmax over all
// experts, sigmoid renormalized over the selected, or sigmoid. Wave 0 then ranks every assignment among the block's
// earlier assignments to the same expert, 64 at a time: ten ballots over the expert
// index bits give each lane the mask of lanes with its expert, and a per-expert running
// count in LDS carries across chunks. Then p = offset[e] + (earlier blocks' count of e)
// + rank for every assignment: up to 64 token blocks, one more kernel whose blocks each
// sum the per-expert counts of the blocks before them and of all blocks, scan over
// experts and scatter; beyond that two kernels, so that the work stays linear in the
// batch: a scan over token blocks per expert, then the scan over experts and the scatter.
// No atomics: the row lists are the same bits on every run. A batch of at most 16 tokens
// runs as one launch (scan and scatter in the same block).
#include "device.hpp"
#include "internal.hpp"
#include "route_device.hpp"

namespace moe {

constexpr int kRouteTokensPerBlock = 16;  // measured against 8, 32 and 64 (8: no faster at 512 tokens)
constexpr int kRouteThreads = 256;
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;
constexpr int kRouteDirectScanMax = 64;  // token blocks up to which each scatter block sums the counts itself

// PLAIN: the default policy without a bias, compiled with both as constants (the other
// policies' code drops out)
template <int EPL, bool PLAIN>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias_arg, int policy_arg, int T, int E, int k,
    int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ ws_rank, int32_t* __restrict__ ws_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_rows,
    int32_t* __restrict__ row_of) {
  constexpr int kWaves = kRouteThreads / 64;
  __shared__ int s_ids[kRouteTokensPerBlock * kMaxTopK];
  __shared__ int s_rank[kRouteTokensPerBlock * kMaxTopK];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];

  const float* const bias = PLAIN ? nullptr : bias_arg;
  const int policy = PLAIN ? 0 : policy_arg;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t_begin = blockIdx.x * kRouteTokensPerBlock;
  const int t_end = min(T, t_begin + kRouteTokensPerBlock);
  const int ntok = t_end - t_begin;

  for (int e = threadIdx.x; e < E; e += kRouteThreads) s_cnt[e] = 0;
  constexpr int kRowEpl = EPL <= 4 ? EPL * 4 : 1;  // experts a lane holds in the row path
  if (EPL <= 4 && k <= 16) {
    // top-k: one 16-lane row per token, 4 tokens per wave at once
    const int gl = lane & 15;
    for (int tl = wave * 4 + (lane >> 4); tl < ntok; tl += kWaves * 4) {
      const int t = t_begin + tl;
      float my_w;
      int my_i;
      row_topk<kRowEpl>(logits + (size_t)t * E, bias, E, k, gl, policy, my_i, my_w);
      if (gl < k) {
        topk_ids[(size_t)t * k + gl] = my_i;
        topk_w[(size_t)t * k + gl] = my_w;
        s_ids[tl * k + gl] = my_i;
      }
    }
  } else
  // top-k: one wave per token, tokens interleaved over the waves
  for (int tl = wave; tl < ntok; tl += kWaves) {
    const int t = t_begin + tl;
    const float* row = logits + (size_t)t * E;
    float v[EPL];
    int ix[EPL];
    // selection values: the logits, or the float32 sums logit + bias[e] (-0.0 ties +0.0)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? (bias ? row[e] + bias[e] : row[e]) : -__builtin_inff();
      ix[j] = e < E ? e : 0x7FFFFFFF;
    }
    float my_v = 0.0f;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
      float bv = v[0];
      int bi = ix[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j)
        if (route_better(v[j], ix[j], bv, bi)) { bv = v[j]; bi = ix[j]; }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (route_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (ix[j] == bi) { v[j] = -__builtin_inff(); ix[j] = 0x7FFFFFFF; }
      if (lane == r) { my_v = bv; my_i = bi; }
    }
    // weights under the policy (as in the row path), from the unbiased logits
    const bool sel = lane < k;
    const float my_l = sel ? (bias ? row[sel ? my_i : 0] : my_v) : -__builtin_inff();
    auto wmax = [](float m) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      return m;
    };
    auto wsum = [](float s) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      return s;
    };
    float wt;
    if (policy <= 1) {
      float m, denom, ex = 0.0f;
      if (policy == 0) {
        m = bias ? wmax(my_l) : __shfl(my_v, 0);  // without a bias, the first choice
        if (sel) ex = exp_diff(my_l, m);
        denom = wsum(ex);
      } else {
        float lm = -__builtin_inff(), ls = 0.0f;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + 64 * j < E) lm = fmaxf(lm, row[lane + 64 * j]);
        m = wmax(lm);
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + 64 * j < E) ls += exp_diff(row[lane + 64 * j], m);
        denom = wsum(ls);
        if (sel) ex = exp_diff(my_l, m);
      }
      wt = ex / denom;
    } else {
      const float sg = sel ? sigmoid_f32(my_l) : 0.0f;
      wt = policy == 2 ? sg / wsum(sg) : sg;
    }
    if (sel) {
      topk_ids[(size_t)t * k + lane] = my_i;
      topk_w[(size_t)t * k + lane] = wt;
      s_ids[tl * k + lane] = my_i;
    }
  }
  __syncthreads();

  const int nas = ntok * k;
  if (wave == 0) wave_rank_assignments(s_ids, nas, s_rank, s_cnt, lane);
  __syncthreads();

  if (gridDim.x == 1) {
    // whole batch in this block: scan and scatter here
    block_exclusive_scan(s_cnt, s_off, E);
    for (int e = threadIdx.x; e <= E; e += kRouteThreads) expert_offsets[e] = s_off[e];
    for (int a = threadIdx.x; a < nas; a += kRouteThreads) {
      const int p = s_off[s_ids[a]] + s_rank[a];
      sorted_rows[p] = a;
      row_of[a] = p;
    }
    return;
  }
  const size_t a0 = (size_t)t_begin * k;
  for (int a = threadIdx.x; a < nas; a += kRouteThreads) ws_rank[a0 + a] = s_rank[a];
  // counts expert-major ([E][blocks]): the per-expert scan over blocks reads a contiguous row
  for (int e = threadIdx.x; e < E; e += kRouteThreads) ws_counts[(size_t)e * gridDim.x + blockIdx.x] = s_cnt[e];
}

// Few token blocks (nblocks <= kRouteDirectScanMax): one block per token block finds its
// base per expert (the counts of the blocks before it) and every expert's total by
// summing the counts itself, scans over experts, and scatters its own assignments. Each
// block reads all nblocks * E counts, so this is only used while that is small; larger
// batches take the two-level form below (route_block_scan_kernel, route_scatter_kernel),
// whose work grows linearly with the batch.
__global__ __launch_bounds__(kRouteThreads) void route_scan_scatter_kernel(
    const int32_t* __restrict__ topk_ids, int T, int E, int k, int nblocks,
    const int32_t* __restrict__ ws_rank, const int32_t* __restrict__ ws_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_rows,
    int32_t* __restrict__ row_of) {
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int before = 0, total = 0;
    int j = 0;
    // 32 loads in flight a thread (integer sums: the grouping does not matter)
    for (; j + 32 <= nblocks; j += 32) {
      int c[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) c[u] = ws_counts[(size_t)e * nblocks + j + u];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        before += (j + u < b) ? c[u] : 0;
        total += c[u];
      }
    }
    for (; j < nblocks; ++j) {
      const int c = ws_counts[(size_t)e * nblocks + j];
      before += (j < b) ? c : 0;
      total += c;
    }
    s_base[e] = before;
    s_tot[e] = total;
  }
  __syncthreads();
  block_exclusive_scan(s_tot, s_off, E);
  if (b == 0)
    for (int e = threadIdx.x; e <= E; e += kRouteThreads) expert_offsets[e] = s_off[e];
  const int a_begin = b * kRouteTokensPerBlock * k;
  const int a_end = min(T * k, a_begin + kRouteTokensPerBlock * k);
  for (int a = a_begin + threadIdx.x; a < a_end; a += kRouteThreads) {
    const int e = topk_ids[a];
    const int p = s_off[e] + s_base[e] + ws_rank[a];
    sorted_rows[p] = a;
    row_of[a] = p;
  }
}

// Many token blocks, first level: one block per expert turns the expert's row of counts
// (one count a token block) into exclusive prefix sums in place (each token block's base
// for the expert) and writes the expert's total. Integer sums: any grouping gives the same
// values, so the row lists are those of the one-level form.
__global__ __launch_bounds__(kRouteThreads) void route_block_scan_kernel(int nblocks, int32_t* __restrict__ ws_counts,
                                                                         int32_t* __restrict__ ws_total) {
  constexpr int kChunk = 1024;
  __shared__ int s_in[kChunk];
  __shared__ int s_out[kChunk + 1];
  int32_t* const row = ws_counts + (size_t)blockIdx.x * nblocks;
  int carry = 0;
  for (int c0 = 0; c0 < nblocks; c0 += kChunk) {
    const int n = min(kChunk, nblocks - c0);
    for (int i = threadIdx.x; i < n; i += kRouteThreads) s_in[i] = row[c0 + i];
    __syncthreads();
    block_exclusive_scan(s_in, s_out, n);  // ends with a barrier
    for (int i = threadIdx.x; i < n; i += kRouteThreads) row[c0 + i] = carry + s_out[i];
    carry += s_out[n];
    __syncthreads();  // before the next chunk overwrites s_in / s_out
  }
  if (threadIdx.x == 0) ws_total[blockIdx.x] = carry;
}

// Second level: one block per token block scans the E totals (the expert offsets; block 0
// writes them) and scatters its own assignments to offset + its base + its rank.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t* __restrict__ topk_ids, int T, int E, int k, int nblocks, const int32_t* __restrict__ ws_rank,
    const int32_t* __restrict__ ws_base, const int32_t* __restrict__ ws_total, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ row_of) {
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) s_tot[e] = ws_total[e];
  __syncthreads();
  block_exclusive_scan(s_tot, s_off, E);
  if (b == 0)
    for (int e = threadIdx.x; e <= E; e += kRouteThreads) expert_offsets[e] = s_off[e];
  const int a_begin = b * kRouteTokensPerBlock * k;
  const int a_end = min(T * k, a_begin + kRouteTokensPerBlock * k);
  for (int a = a_begin + threadIdx.x; a < a_end; a += kRouteThreads) {
    const int e = topk_ids[a];
    const int p = s_off[e] + ws_base[(size_t)e * nblocks + b] + ws_rank[a];
    sorted_rows[p] = a;
    row_of[a] = p;
  }
}

size_t route_workspace_bytes(int T, int E, int k) {
  const size_t nb = ((size_t)T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
  if (nb <= 1) return 0;
  // ranks [T * k], counts [E][nb], totals [E]
  return ((size_t)T * k + nb * (size_t)E + (size_t)E) * sizeof(int32_t);
}

hipError_t launch_route(const float* logits, const float* bias, int policy, int T, int E, int k, int32_t* ids,
                        float* w,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* row_of, void* ws,
                        hipStream_t stream) {
  const int nb = (T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
  int32_t* ws_rank = nullptr;
  int32_t* ws_counts = nullptr;
  if (nb > 1) {
    ws_rank = static_cast<int32_t*>(ws);
    ws_counts = ws_rank + (size_t)T * k;
  }
  const int epl = (E + 63) / 64;
  dim3 grid(nb), block(kRouteThreads);
  const bool plain = policy == 0 && bias == nullptr;
#define MOE_ROUTE_LAUNCH(N)                                                                                    \
  do {                                                                                                         \
    if (plain)                                                                                                 \
      hipLaunchKernelGGL((route_topk_kernel<N, true>), grid, block, 0, stream, logits, bias, policy, T, E, k,  \
                         ids, w, ws_rank, ws_counts, offsets, sorted_rows, row_of);                            \
    else                                                                                                       \
      hipLaunchKernelGGL((route_topk_kernel<N, false>), grid, block, 0, stream, logits, bias, policy, T, E, k, \
                         ids, w, ws_rank, ws_counts, offsets, sorted_rows, row_of);                            \
  } while (0)
  if (epl <= 1) MOE_ROUTE_LAUNCH(1);
  else if (epl <= 2) MOE_ROUTE_LAUNCH(2);
  else if (epl <= 4) MOE_ROUTE_LAUNCH(4);
  else if (epl <= 8) MOE_ROUTE_LAUNCH(8);
  else MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nb <= 1) return err;
  if (nb <= kRouteDirectScanMax) {
    hipLaunchKernelGGL(route_scan_scatter_kernel, dim3(nb), dim3(kRouteThreads), 0, stream, ids, T, E, k, nb,
                       ws_rank, ws_counts, offsets, sorted_rows, row_of);
    return hipGetLastError();
  }
  int32_t* const ws_total = ws_counts + (size_t)nb * E;
  hipLaunchKernelGGL(route_block_scan_kernel, dim3(E), dim3(kRouteThreads), 0, stream, nb, ws_counts, ws_total);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(kRouteThreads), 0, stream, ids, T, E, k, nb, ws_rank,
                     ws_counts, ws_total, offsets, sorted_rows, row_of);
  return hipGetLastError();
}

}  // namespace moe
