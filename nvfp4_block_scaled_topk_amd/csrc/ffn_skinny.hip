// ffn_skinny.hip -- the weight-streaming kernels as launches of their own, for calls
// whose experts all have at most 16 rows (few tokens, too wide for the one-launch
// decode kernel): the grouped GEMM would have no tiles. Each launch runs the streaming
// phase of skinny_device.hpp on as many blocks as the device holds at once, taking
// items blockIdx.x, blockIdx.x + gridDim.x, ...
#include "skinny_device.hpp"

namespace moe {

template <int MODE>  // 0: gate/up/SwiGLU -> H (bf16); 1: down -> y_rows (fp32)
__global__ __launch_bounds__(kSkThreads, 2) void ffn_skinny_kernel(FFNArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kSkLdsBytes];
  skinny_phase<MODE>(a, lds, nullptr);
}

template <int MODE>
static hipError_t launch_skinny(const FFNArgs& a, hipStream_t stream) {
  int blocks = 0;
  hipError_t err = resident_blocks(reinterpret_cast<const void*>(&ffn_skinny_kernel<MODE>), kSkThreads, 0, blocks);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_skinny_kernel<MODE>, dim3(blocks), dim3(kSkThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ffn_skinny_gateup(const FFNArgs& a, hipStream_t stream) { return launch_skinny<0>(a, stream); }
hipError_t launch_ffn_skinny_down(const FFNArgs& a, hipStream_t stream) { return launch_skinny<1>(a, stream); }

}  // namespace moe
