// route_device.hpp -- the per-token top-k and routing weights (device code), shared by
// the routing kernel and the few-token FFN launch that routes its own tokens.
//
// Selection order: logit (or logit + correction bias, in fp32) descending, expert index
// ascending, -0.0 equal to +0.0. Weights under the router's normalization policy, a
// named value on the pages [bloomery 0.3.9 release notes, From our contributors, #772].
#pragma once
#include "device.hpp"

namespace moe {

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
__device__ inline void block_exclusive_scan(const int* s_in, int* s_out, int n) {
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

// Stable ranks, by one wave, 64 assignments at a time in assignment order (experts <
// 1024): lanes holding the same expert are found with one ballot per bit of the expert
// index; the rank is the number of such lanes below plus the expert's running count
// (s_cnt, zero on entry), which the expert's last lane in the chunk then advances. On
// return s_cnt holds every expert's count. The caller synchronizes before reading.
__device__ inline void wave_rank_assignments(const int* s_ids, int nas, int* s_rank, int* s_cnt, int lane) {
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

}  // namespace moe
