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

// Routing key of (value v, expert e): a double whose order is the selection order -- v
// descending, then e ascending, -0.0 taken as +0.0 -- so one v_max_f64 compares two keys.
// v becomes the double of the same value (exact), whose 29 low significand bits are then
// zero; the low 10 of them take the tie-break, 1023 - e above zero and e below (a larger
// magnitude is the smaller key there), which cannot reach the next representable value
// of v. Zero, whose double has no exponent, is given 2^-500 (below every nonzero fp32
// magnitude, and a normal number, so no denormal meets the compare); infinities are given
// +-2^200 and NaN +-2^201 by its sign bit (outside the contract, but kept finite, ordered
// and distinct). Every key is finite and keys of distinct experts differ; -inf marks an
// empty slot (expert index E <= 1024).
__device__ __forceinline__ double route_keyd(float v, int e) {
  const float w = v + 0.0f;  // -0.0 + 0.0 = +0.0
  const uint32_t wb = __builtin_bit_cast(uint32_t, w);
  double d;
  if (w != w) d = (wb & 0x80000000u) ? -0x1p201 : 0x1p201;
  else if (__builtin_isinf(w)) d = w > 0.0f ? 0x1p200 : -0x1p200;
  else if (w == 0.0f) d = 0x1p-500;
  else d = (double)w;
  const uint64_t b = __builtin_bit_cast(uint64_t, d);
  return __builtin_bit_cast(double, b | (d > 0.0 ? (uint64_t)(1023 - e) : (uint64_t)e));
}
__device__ __forceinline__ int route_keyd_expert(double key) {
  const uint64_t b = __builtin_bit_cast(uint64_t, key);
  return key > 0.0 ? 1023 - (int)(b & 1023u) : (int)(b & 1023u);
}
// the key's value as the fp32 it came from (the mapped zero, infinities and NaN back)
__device__ __forceinline__ float route_keyd_value(double key) {
  const double d = __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, key) & ~(uint64_t)1023u);
  const double a = __builtin_fabs(d);
  if (a >= 0x1p201) return __builtin_nanf("");
  if (a >= 0x1p200) return d > 0.0 ? __builtin_inff() : -__builtin_inff();
  if (a <= 0x1p-400) return 0.0f;
  return (float)d;
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)b), hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// the largest key of a 16-lane row, in every lane of the row
__device__ __forceinline__ double row_keymax16(double k) {
  k = __builtin_fmax(k, dpp_d<0xB1>(k));
  k = __builtin_fmax(k, dpp_d<0x4E>(k));
  k = __builtin_fmax(k, dpp_d<0x141>(k));
  k = __builtin_fmax(k, dpp_d<0x140>(k));
  return k;
}
// the largest key of the wave, in every lane: the row maxima, then gfx950's swaps of
// lane rows (v_permlane16_swap: rows 0 <-> 1 and 2 <-> 3; v_permlane32_swap: the two
// halves of the wave), called with both operands the same value so that its two results
// are a lane's value and its partner's
__device__ __forceinline__ double swap_keymax(double k, bool rows32) {
  const uint64_t b = __builtin_bit_cast(uint64_t, k);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  uint32_t l0, l1, h0, h1;
  if (rows32) {
    const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = pl[0]; l1 = pl[1]; h0 = ph[0]; h1 = ph[1];
  } else {
    const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = pl[0]; l1 = pl[1]; h0 = ph[0]; h1 = ph[1];
  }
  const double x = __builtin_bit_cast(double, ((uint64_t)h0 << 32) | l0);
  const double y = __builtin_bit_cast(double, ((uint64_t)h1 << 32) | l1);
  return __builtin_fmax(x, y);
}
__device__ __forceinline__ double wave_keymax(double k) {
  k = row_keymax16(k);
  k = swap_keymax(k, false);
  return swap_keymax(k, true);
}
// Sort N keys in descending order: Batcher's odd-even merge sort (N a power of two),
// each comparator one fmax and one fmin.
template <int N>
__device__ __forceinline__ void sort_keys_desc(double (&a)[N]) {
  static_assert((N & (N - 1)) == 0, "power of two");
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int q = p; q >= 1; q >>= 1)
#pragma unroll
      for (int j = q % p; j + q < N; j += 2 * q)
#pragma unroll
        for (int i = 0; i < q; ++i)
          if (i + j + q < N && (i + j) / (2 * p) == (i + j + q) / (2 * p)) {
            const double x = a[i + j], y = a[i + j + q];
            a[i + j] = __builtin_fmax(x, y);
            a[i + j + q] = __builtin_fmin(x, y);
          }
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
// j < EPL), k <= 16, by routing keys -- of the logits, or of the float32 sums logit +
// bias[e] when a correction bias is given (it moves the choice only). Each lane sorts its
// own keys once; then each of k rounds takes the row maximum of the lanes' first keys and
// the lane that held it moves on to its next one. Lane gl < k gets the gl-th choice in
// my_i and its weight under `policy` in my_w: 0 softmax over the selected logits, 1
// softmax over all E logits, 2 sigmoid renormalized over the selected, 3 sigmoid.
template <int EPL>
__device__ __forceinline__ void row_topk(const float* __restrict__ row, const float* __restrict__ bias, int E, int k,
                                         int gl, int policy, int& my_i, float& my_w) {
  constexpr int N = EPL <= 4 ? 4 : EPL <= 8 ? 8 : 16;  // slots, a power of two (empty ones -inf)
  double key[N];
  float lg[EPL];  // the unbiased logits (-inf past E)
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = gl + 16 * j;
    lg[j] = e < E ? row[e] : -__builtin_inff();
    key[j] = e < E ? route_keyd(bias ? lg[j] + bias[e] : lg[j], e) : -__builtin_inf();
  }
#pragma unroll
  for (int j = EPL; j < N; ++j) key[j] = -__builtin_inf();
  sort_keys_desc(key);
  double mine = -__builtin_inf(), top = -__builtin_inf();
  for (int r = 0; r < k; ++r) {
    const double best = row_keymax16(key[0]);
    if (gl == r) mine = best;
    if (r == 0) top = best;  // the first choice, in every lane of the row
    // the lane that held it (keys are distinct) moves on; slots past k are never reached
    if (key[0] == best) {
#pragma unroll
      for (int j = 0; j + 1 < N; ++j)
        if (j + 1 < k) key[j] = key[j + 1];
      key[N - 1] = -__builtin_inf();
    }
  }
  const bool sel = gl < k;
  my_i = route_keyd_expert(mine);
  // the unbiased logit of this lane's choice (without a bias, the key's own value)
  const float my_l = sel ? (bias ? row[sel ? my_i : 0] : route_keyd_value(mine)) : -__builtin_inff();
  if (policy <= 1) {
    float m, denom;
    float ex = 0.0f;
    if (policy == 0) {
      // without a bias the first choice holds the largest selected logit
      m = bias ? row_max16(my_l) : route_keyd_value(top);
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


// Top-k of one token held by a whole wave (lane l holds experts l + 64j, j < EPW), k <=
// 16, the default policy without a bias: the selection of row_topk with the rows' work
// spread over 64 lanes (shorter per-lane lists, one wave a token). Lane l < k gets the l-th
// choice and its weight; the weights are formed exactly as in row_topk (the choices in
// lanes 0..15, the same row sum), so both give the same bits.
template <int EPW>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int lane, int& my_i,
                                          float& my_w) {
  constexpr int N = EPW <= 1 ? 1 : EPW <= 2 ? 2 : 4;
  double key[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int e = lane + 64 * j;
    key[j] = j < EPW && e < E ? route_keyd(row[e], e) : -__builtin_inf();
  }
  sort_keys_desc(key);
  double mine = -__builtin_inf(), top = -__builtin_inf();
  for (int r = 0; r < k; ++r) {
    const double best = wave_keymax(key[0]);
    if (lane == r) mine = best;
    if (r == 0) top = best;
    if (key[0] == best) {
#pragma unroll
      for (int j = 0; j + 1 < N; ++j)
        if (j + 1 < k) key[j] = key[j + 1];
      key[N - 1] = -__builtin_inf();
    }
  }
  const bool sel = lane < k;
  my_i = route_keyd_expert(mine);
  const float my_l = sel ? route_keyd_value(mine) : -__builtin_inff();
  const float m = route_keyd_value(top);
  const float ex = sel ? exp_diff(my_l, m) : 0.0f;
  my_w = ex / row_sum16(ex);
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
