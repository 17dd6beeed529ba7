// router.hip -- the router projection: logits[t][e] = sum_i x[t][i] * W_r[e][i].
//
// The router matrix stays in its stored BF16 words [FP4-Local checkpoints on DGX
// Spark, §4 Round 1, #732] and the logits are summed on a float32 tile [same page,
// §4 Round 1, #763]: here bf16 x bf16 products on the 16x16x32 bf16 MFMA with fp32
// accumulation. A block of 8 waves owns 32 tokens x 32 experts (two 16-row tiles of
// each: four MFMAs a 32-element chunk of K); the waves split K in eight contiguous
// ranges and their partial tiles are added in LDS in wave order, so the result does
// not depend on timing. Operands come straight from memory (no LDS staging): a lane
// reads 16 bytes of one row a chunk -- the activation rows of its tokens and the
// router rows of its experts -- through buffer descriptors, so rows past T or E read
// zeros. The contraction index inside a chunk is permuted identically on both sides
// (lane group g holds elements 8g .. 8g + 7), which leaves the sums unchanged.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kRtWaves = 8;
constexpr int kRtThreads = 64 * kRtWaves;
constexpr int kRtTile = 32;   // tokens and experts a block owns
constexpr int kRtUnroll = 4;  // chunks a wave loads before their MFMAs
constexpr uint32_t kRtOOB = 0x80000000u;  // a buffer offset past every record: reads zeros

typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rt_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(kRtThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ wr, int T, int d,
                                                                   int E, float* __restrict__ logits) {
  __shared__ floatx4 red[kRtWaves][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * kRtTile, e0 = blockIdx.y * kRtTile;
  const __amdgpu_buffer_rsrc_t xrs = rt_rsrc(x, (uint32_t)((size_t)T * d * 2));
  const __amdgpu_buffer_rsrc_t wrs = rt_rsrc(wr, (uint32_t)((size_t)E * d * 2));
  // byte offset of this lane's 16 bytes in chunk 0 of each of its rows (past the end: OOB)
  uint32_t xo[2], wo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 16 * i + col, e = e0 + 16 * i + col;
    xo[i] = t < T ? (uint32_t)t * (uint32_t)(d * 2) + 16u * grp : kRtOOB;
    wo[i] = e < E ? (uint32_t)e * (uint32_t)(d * 2) + 16u * grp : kRtOOB;
  }
  const bool two_tok = t0 + 16 < T, two_exp = e0 + 16 < E;  // block-uniform
  const int nch = d / 32;
  const int c0 = nch * wave / kRtWaves, c1 = nch * (wave + 1) / kRtWaves;
  floatx4 acc[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
  for (int c = c0; c < c1; c += kRtUnroll) {
    u32x4r a[kRtUnroll][2], b[kRtUnroll][2];
#pragma unroll
    for (int u = 0; u < kRtUnroll; ++u) {
      // a chunk past the wave's range reads zeros (offset past every record) and adds
      // nothing; row offsets plus chunk offsets stay below 2^32 (T * d * 2 < 2^31)
      const bool in = c + u < c1;
      const uint32_t ko = (uint32_t)(c + u) * 64u;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[u][i] = (i == 0 || two_tok) ? __builtin_amdgcn_raw_buffer_load_b128(xrs, in ? xo[i] + ko : kRtOOB, 0, 0)
                                      : u32x4r{0u, 0u, 0u, 0u};
        b[u][i] = (i == 0 || two_exp) ? __builtin_amdgcn_raw_buffer_load_b128(wrs, in ? wo[i] + ko : kRtOOB, 0, 0)
                                      : u32x4r{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kRtUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if ((i == 0 || two_tok) && (j == 0 || two_exp))
            acc[i][j] = mfma16(__builtin_bit_cast(bf16x8, b[u][j]), __builtin_bit_cast(bf16x8, a[u][i]), acc[i][j]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) red[wave][2 * i + j][lane] = acc[i][j];
  __syncthreads();
  // waves 0-3 each finish one 16 x 16 tile: the eight partial tiles in wave order
  if (wave < 4) {
    const int i = wave >> 1, j = wave & 1;
    floatx4 s = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kRtWaves; ++w) s += red[w][wave][lane];
    // lane (col, grp) holds experts 4 grp .. 4 grp + 3 of the tile's token col
    const int t = t0 + 16 * i + col, e = e0 + 16 * j + 4 * grp;
    if (t < T) {
      float* const dst = logits + (size_t)t * E + e;
      if ((E & 3) == 0 && e + 3 < E) {
        *reinterpret_cast<float4*>(dst) = make_float4(s[0], s[1], s[2], s[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < E) dst[r] = s[r];
      }
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_r, int T, int d, int E, float* logits,
                                hipStream_t stream) {
  dim3 grid((T + kRtTile - 1) / kRtTile, (E + kRtTile - 1) / kRtTile);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(kRtThreads), 0, stream, x, w_r, T, d, E, logits);
  return hipGetLastError();
}

}  // namespace moe
