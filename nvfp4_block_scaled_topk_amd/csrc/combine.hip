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

template <bool SHARED, bool RESID>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ y_rows, const int32_t* __restrict__ row_of,
    const float* __restrict__ w, int T, int k, int d, const float* __restrict__ s_rows,
    const float* __restrict__ s_gate, const uint16_t* __restrict__ resid, uint16_t* __restrict__ out) {
  // the token's row positions and weights are the same for the whole block: scalar loads
  const int t = blockIdx.x;
  const int32_t* const ro = row_of + (size_t)t * k;
  const float* const wt = w + (size_t)t * k;
  const int c = (blockIdx.y * kCombineThreads + threadIdx.x) * 4;
  if (c >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 sv;
  if constexpr (SHARED) sv = *reinterpret_cast<const float4*>(s_rows + (size_t)t * d + c);
  uint2 xr;
  if constexpr (RESID) xr = *reinterpret_cast<const uint2*>(resid + (size_t)t * d + c);
  // eight rows' loads in flight at once (a group past k repeats row k-1 and adds
  // nothing), then the sums in top-k order
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const float4*>(y_rows + (size_t)ro[min(j0 + u, k - 1)] * d + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        const float wj = wt[j0 + u];
        acc.x = fmaf(wj, v[u].x, acc.x);
        acc.y = fmaf(wj, v[u].y, acc.y);
        acc.z = fmaf(wj, v[u].z, acc.z);
        acc.w = fmaf(wj, v[u].w, acc.w);
      }
    }
  }
  if constexpr (SHARED) {
    const float g = s_gate ? 1.0f / (1.0f + expf(-s_gate[t])) : 1.0f;
    acc.x = fmaf(g, sv.x, acc.x);
    acc.y = fmaf(g, sv.y, acc.y);
    acc.z = fmaf(g, sv.z, acc.z);
    acc.w = fmaf(g, sv.w, acc.w);
  }
  if constexpr (RESID) {
    acc.x += bf16_to_f32((uint16_t)(xr.x & 0xFFFFu));
    acc.y += bf16_to_f32((uint16_t)(xr.x >> 16));
    acc.z += bf16_to_f32((uint16_t)(xr.y & 0xFFFFu));
    acc.w += bf16_to_f32((uint16_t)(xr.y >> 16));
  }
  uint2 o;
  o.x = (uint32_t)bf16_rne(acc.x) | ((uint32_t)bf16_rne(acc.y) << 16);
  o.y = (uint32_t)bf16_rne(acc.z) | ((uint32_t)bf16_rne(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * d + c) = o;
}

hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* w, int T, int k,
                          int d, const float* s_rows, const float* s_gate, const uint16_t* resid, uint16_t* out,
                          hipStream_t stream) {
  dim3 grid(T, (d / 4 + kCombineThreads - 1) / kCombineThreads);
  if (s_rows && resid)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w, T, k,
                       d, s_rows, s_gate, resid, out);
  else if (s_rows)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w, T, k,
                       d, s_rows, s_gate, nullptr, out);
  else if (resid)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w, T, k,
                       d, nullptr, nullptr, resid, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, dim3(kCombineThreads), 0, stream, y_rows, row_of, w, T,
                       k, d, nullptr, nullptr, nullptr, out);
  return hipGetLastError();
}

}  // namespace moe
