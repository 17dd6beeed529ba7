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
// count in LDS carries across chunks. Kernel 2 (one block per token block): each block
// sums the per-expert counts of the blocks before it and of all blocks, scans over
// experts, and scatters p = offset[e] + (earlier blocks' count of e) + rank. No
// atomics: the row lists are the same bits on every run. A batch of at most 16 tokens
// runs as one launch (scan and scatter in the same block).
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kRouteTokensPerBlock = 16;  // measured against 32 and 64: more blocks, shorter chains
constexpr int kRouteThreads = 256;
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ bool route_better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Lane exchange inside rows of 16 lanes (DPP, no LDS round trip): CTRL is a gfx9 DPP
// control -- 0xB1 / 0x4E swap lanes at distance 1 / 2 inside each quad, 0x141 mirrors
// each half row (8 lanes), 0x140 mirrors the row.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ void row_sum_step(float& s) {
  s += dpp_f<CTRL>(s);
}

// Routing key of (logit v, expert e): one unsigned 64-bit integer whose order is the
// selection order -- v descending (its bits made order-preserving, -0.0 taken as +0.0),
// then e ascending -- so a comparison is one 64-bit compare. Key 0 (below every real
// key) marks a padding or already-selected slot.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);  // -0.0 + 0.0 = +0.0
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float route_key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int route_key_expert(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
template <int CTRL>
__device__ __forceinline__ void row_keymax_step(uint64_t& k) {
  const uint64_t o = ((uint64_t)(uint32_t)dpp_i<CTRL>((int)(k >> 32)) << 32) | (uint32_t)dpp_i<CTRL>((int)(uint32_t)k);
  k = o > k ? o : k;
}

template <int CTRL>
__device__ __forceinline__ void row_max_step(float& m) {
  m = fmaxf(m, dpp_f<CTRL>(m));
}
__device__ __forceinline__ float row_sum16(float s) {
  row_sum_step<0xB1>(s);
  row_sum_step<0x4E>(s);
  row_sum_step<0x141>(s);
  row_sum_step<0x140>(s);
  return s;
}
__device__ __forceinline__ float row_max16(float m) {
  row_max_step<0xB1>(m);
  row_max_step<0x4E>(m);
  row_max_step<0x141>(m);
  row_max_step<0x140>(m);
  return m;
}
// e^(l - m), with the rounding error of l - m carried into the exponential to first order
__device__ __forceinline__ float exp_diff(float l, float m) {
  const float s = l - m;
  const float bb = s - l;
  const float err = (l - (s - bb)) + (-m - bb);
  const float e0 = expf(s);
  return fmaf(e0, err, e0);
}
__device__ __forceinline__ float sigmoid_f32(float l) { return 1.0f / (1.0f + expf(-l)); }

// Top-k of one token held by a 16-lane row (lane gl of the row holds experts gl + 16j,
// j < EPL), k <= 16: k rounds of a row maximum over routing keys -- of the logits, or of
// the float32 sums logit + bias[e] when a correction bias is given (it moves the choice
// only). Lane gl < k gets the gl-th choice in my_i and its weight under `policy` in
// my_w: 0 softmax over the selected logits, 1 softmax over all E logits, 2 sigmoid
// renormalized over the selected, 3 sigmoid.
template <int EPL>
__device__ __forceinline__ void row_topk(const float* __restrict__ row, const float* __restrict__ bias, int E, int k,
                                         int gl, int policy, int& my_i, float& my_w) {
  uint64_t key[EPL];
  float lg[EPL];  // the unbiased logits (-inf past E)
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = gl + 16 * j;
    lg[j] = e < E ? row[e] : -__builtin_inff();
    key[j] = e < E ? route_key(bias ? lg[j] + bias[e] : lg[j], e) : 0ull;
  }
  uint64_t mine = 0ull, top = 0ull;
  for (int r = 0; r < k; ++r) {
    // the lane's best key, by a pairwise tree (short dependency chains)
    uint64_t t[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) t[j] = key[j];
#pragma unroll
    for (int w = 1; w < EPL; w *= 2)
#pragma unroll
      for (int j = 0; j + w < EPL; j += 2 * w) t[j] = t[j + w] > t[j] ? t[j + w] : t[j];
    uint64_t best = t[0];
    row_keymax_step<0xB1>(best);
    row_keymax_step<0x4E>(best);
    row_keymax_step<0x141>(best);
    row_keymax_step<0x140>(best);
    // the selected slot (keys are distinct: the low word names the expert)
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if ((uint32_t)key[j] == (uint32_t)best) key[j] = 0ull;
    if (gl == r) mine = best;
    if (r == 0) top = best;  // the first choice, in every lane of the row
  }
  const bool sel = gl < k;
  my_i = route_key_expert(mine);
  // the unbiased logit of this lane's choice (without a bias, the key's own value)
  const float my_l = sel ? (bias ? row[sel ? my_i : 0] : route_key_value(mine)) : -__builtin_inff();
  if (policy <= 1) {
    float m, denom;
    float ex = 0.0f;
    if (policy == 0) {
      // without a bias the first choice holds the largest selected logit
      m = bias ? row_max16(my_l) : route_key_value(top);
      if (sel) ex = exp_diff(my_l, m);
      denom = row_sum16(ex);
    } else {
      float lm = lg[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j) lm = fmaxf(lm, lg[j]);
      m = row_max16(lm);
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (gl + 16 * j < E) ls += exp_diff(lg[j], m);
      denom = row_sum16(ls);
      if (sel) ex = exp_diff(my_l, m);
    }
    my_w = ex / denom;
  } else {
    const float sg = sel ? sigmoid_f32(my_l) : 0.0f;
    my_w = policy == 2 ? sg / row_sum16(sg) : sg;
  }
}

// Exclusive scan of s_in[0..n) in LDS (n <= 1024) by the block's first wave, 64
// entries a step: an inclusive scan inside each 16-lane row by four DPP row shifts
// (lanes shifted in from outside the row add 0), then the row totals read into scalar
// registers and added to the rows above; writes s_out[0..n], s_out[n] = total.
__device__ void block_exclusive_scan(const int* s_in, int* s_out, int n) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    for (int base = 0; base < n; base += 64) {
      const int e = base + lane;
      const int v = e < n ? s_in[e] : 0;
      int incl = v;
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);  // row_shr:1
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);  // row_shr:2
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);  // row_shr:4
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);  // row_shr:8
      const int r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31);
      const int r2 = __builtin_amdgcn_readlane(incl, 47), r3 = __builtin_amdgcn_readlane(incl, 63);
      const int row = lane >> 4;
      const int above = (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
      if (e < n) s_out[e] = run + above + incl - v;
      run += r0 + r1 + r2 + r3;
    }
    if (lane == 0) s_out[n] = run;
  }
  __syncthreads();
}

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

  // ranks, by wave 0, 64 assignments at a time in assignment order: lanes holding the
  // same expert are found with one ballot per bit of the expert index; the rank is the
  // number of such lanes below plus the expert's running count (s_cnt), which the
  // expert's last lane in the chunk then advances.
  const int nas = ntok * k;
  if (wave == 0) {
    for (int base = 0; base < nas; base += 64) {
      const int a = base + lane;
      const int e = a < nas ? s_ids[a] : -1;
      uint64_t same = __ballot(e >= 0);
#pragma unroll
      for (int bit = 0; bit < 10; ++bit) {
        const uint64_t b1 = __ballot(e >= 0 && ((e >> bit) & 1));
        same &= ((e >> bit) & 1) ? b1 : ~b1;
      }
      const uint64_t below = (1ull << lane) - 1ull;
      const int before = __popcll(same & below);
      const bool last = (same & ~below & ~(1ull << lane)) == 0;
      int r = 0;
      if (e >= 0) r = s_cnt[e] + before;
      __builtin_amdgcn_wave_barrier();
      if (e >= 0) {
        s_rank[a] = r;
        if (last) s_cnt[e] = r + 1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
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
  for (int e = threadIdx.x; e < E; e += kRouteThreads) ws_counts[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// One block per token block: this block's base per expert (counts of the blocks before
// it), every expert's total, the scan over experts, and the scatter of its own
// assignments.
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
    for (; j + 8 <= nblocks; j += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = ws_counts[(size_t)(j + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        before += (j + u < b) ? c[u] : 0;
        total += c[u];
      }
    }
    for (; j < nblocks; ++j) {
      const int c = ws_counts[(size_t)j * E + e];
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

size_t route_workspace_bytes(int T, int E, int k) {
  const size_t nb = ((size_t)T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
  if (nb <= 1) return 0;
  return ((size_t)T * k + nb * (size_t)E) * sizeof(int32_t);
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
  hipLaunchKernelGGL(route_scan_scatter_kernel, dim3(nb), dim3(kRouteThreads), 0, stream, ids, T, E, k, nb,
                     ws_rank, ws_counts, offsets, sorted_rows, row_of);
  return hipGetLastError();
}

}  // namespace moe
