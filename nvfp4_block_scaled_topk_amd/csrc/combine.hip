// combine.hip -- the router-weighted sum of each token's expert rows.
//
// The pages fold the card sum of the expert outputs into the combine [FP4-Local
// checkpoints on DGX Spark, §4 Round 1, #701] and keep the rows wide until that sum
// ([same page, §4 remaining items, #914]: rows rounded to nearest even, the block's
// sum widening them). Here the expert rows stay fp32 and are summed in fp32 in the
// token's top-k order, then rounded once to bf16: out[t] = bf16_rne(sum_j w_tj * y[row_of[t*k+j]]).
// Pure streaming: each thread owns 4 consecutive columns of one token (128-bit loads).
//
// With a shared expert beside the routed ones [same page, §4 Round 1, #686], its add
// folds into this producer (the pages fold the shared-expert add into the kernels
// that produce it [same page, §4 remaining items]): out[t] = bf16_rne(sum_j w_tj *
// y[...] + g_t * S[t]), g_t = sigmoid(gate logit of t) (1 without a gate), the shared
// row S kept fp32 and added after the routed sum, before the single rounding. The
// block's residual row x[t] (bf16) folds in the same way, added last.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kCombineThreads = 256;

// The rows are read once: non-temporal loads.
__device__ __forceinline__ float4 ldnt_f4(const float* p) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Tokens TT*blockIdx.x .. + TT - 1, columns (blockIdx.y * kCombineThreads + thread) * 4 ..
// + 3 of each. With k <= 8 every row load of the block's tokens is issued before the
// first sum (a row slot past k repeats row k - 1 and adds nothing); larger k sums eight
// rows at a time.
template <bool SHARED, bool RESID, int TT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ y_rows, const int32_t* __restrict__ row_of,
    const float* __restrict__ w, int T, int k, int d, const float* __restrict__ s_rows,
    const float* __restrict__ s_gate, const uint16_t* __restrict__ resid, uint16_t* __restrict__ out) {
  const int c = (blockIdx.y * kCombineThreads + threadIdx.x) * 4;
  if (c >= d) return;
  float4 acc[TT];
  float4 v[TT][8];
#pragma unroll
  for (int q = 0; q < TT; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
#pragma unroll
    for (int q = 0; q < TT; ++q) {
      const int t = min((int)blockIdx.x * TT + q, T - 1);
      // the token's row positions are the same for the whole block: scalar loads
      const int32_t* const ro = row_of + (size_t)t * k;
#pragma unroll
      for (int u = 0; u < 8; ++u) v[q][u] = ldnt_f4(y_rows + (size_t)ro[min(j0 + u, k - 1)] * d + c);
    }
#pragma unroll
    for (int q = 0; q < TT; ++q) {
      const int t = min((int)blockIdx.x * TT + q, T - 1);
      const float* const wt = w + (size_t)t * k;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < k) {
          const float wj = wt[j0 + u];
          acc[q].x = fmaf(wj, v[q][u].x, acc[q].x);
          acc[q].y = fmaf(wj, v[q][u].y, acc[q].y);
          acc[q].z = fmaf(wj, v[q][u].z, acc[q].z);
          acc[q].w = fmaf(wj, v[q][u].w, acc[q].w);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int t = (int)blockIdx.x * TT + q;
    if (t >= T) break;
    float4 a4 = acc[q];
    if constexpr (SHARED) {
      const float4 sv = *reinterpret_cast<const float4*>(s_rows + (size_t)t * d + c);
      const float g = s_gate ? 1.0f / (1.0f + expf(-s_gate[t])) : 1.0f;
      a4.x = fmaf(g, sv.x, a4.x);
      a4.y = fmaf(g, sv.y, a4.y);
      a4.z = fmaf(g, sv.z, a4.z);
      a4.w = fmaf(g, sv.w, a4.w);
    }
    if constexpr (RESID) {
      const uint2 xr = *reinterpret_cast<const uint2*>(resid + (size_t)t * d + c);
      a4.x += bf16_to_f32((uint16_t)(xr.x & 0xFFFFu));
      a4.y += bf16_to_f32((uint16_t)(xr.x >> 16));
      a4.z += bf16_to_f32((uint16_t)(xr.y & 0xFFFFu));
      a4.w += bf16_to_f32((uint16_t)(xr.y >> 16));
    }
    uint2 o;
    o.x = (uint32_t)bf16_rne(a4.x) | ((uint32_t)bf16_rne(a4.y) << 16);
    o.y = (uint32_t)bf16_rne(a4.z) | ((uint32_t)bf16_rne(a4.w) << 16);
    *reinterpret_cast<uint2*>(out + (size_t)t * d + c) = o;
  }
}

constexpr int kCombineTokens = 1;  // tokens a block (2 and 4 measured no faster)

hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* w, int T, int k,
                          int d, const float* s_rows, const float* s_gate, const uint16_t* resid, uint16_t* out,
                          hipStream_t stream) {
  constexpr int TT = kCombineTokens;
  dim3 grid((T + TT - 1) / TT, (d / 4 + kCombineThreads - 1) / kCombineThreads);
  if (s_rows && resid)
    hipLaunchKernelGGL((combine_kernel<true, true, TT>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w,
                       T, k, d, s_rows, s_gate, resid, out);
  else if (s_rows)
    hipLaunchKernelGGL((combine_kernel<true, false, TT>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w,
                       T, k, d, s_rows, s_gate, nullptr, out);
  else if (resid)
    hipLaunchKernelGGL((combine_kernel<false, true, TT>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w,
                       T, k, d, nullptr, nullptr, resid, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, false, TT>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w,
                       T, k, d, nullptr, nullptr, nullptr, out);
  return hipGetLastError();
}

}  // namespace moe
