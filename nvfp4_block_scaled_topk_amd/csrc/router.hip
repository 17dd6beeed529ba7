// router.hip -- the router projection: logits[t][e] = sum_i x[t][i] * W_r[e][i].
//
// The router matrix stays in its stored BF16 words [FP4-Local checkpoints on DGX
// Spark, §4 Round 1, #732] and the logits are summed on a float32 tile [same page,
// §4 Round 1, #763]: here bf16 x bf16 products on the 16x16x32 bf16 MFMA with fp32
// accumulation. A block of 8 waves owns 16 NT tokens x 16 NE experts (NT x NE MFMA
// tiles a 32-element chunk of K): 64 x 64 for batches, 32 x 32 when E <= 32 (operand
// bytes fetched per FLOP halve with each doubling of the tile, and they bound this
// kernel), 16 x 16
// for a few tokens (more blocks, and every load of a wave's K range in flight at
// once); the waves split K in eight contiguous ranges and their partial tiles are
// added in LDS in a fixed order, so the result does not depend on timing. Operands come straight from memory (no LDS staging): a lane
// reads 16 bytes of one row a chunk -- the activation rows of its tokens and the
// router rows of its experts -- through buffer descriptors, so rows past T or E read
// zeros. The contraction index inside a chunk is permuted identically on both sides
// (lane group g holds elements 8g .. 8g + 7), which leaves the sums unchanged.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kRtWaves = 8;
constexpr int kRtThreads = 64 * kRtWaves;
constexpr int kRtLoads = 16;  // 16-byte loads a lane issues before their MFMAs
constexpr uint32_t kRtOOB = 0x80000000u;  // a buffer offset past every record: reads zeros

typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rt_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

template <int NT, int NE>
__global__ __launch_bounds__(kRtThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ wr, int T, int d,
                                                                   int E, float* __restrict__ logits) {
  constexpr int kUnroll = kRtLoads / (NT + NE);  // chunks loaded before their MFMAs
  // partial tiles of up to eight waves at once (64 KB): one step for up to 8 tiles a
  // wave, a pairwise tree for 16
  constexpr int kRedWaves = NT * NE <= 8 ? kRtWaves : kRtWaves / 2;
  __shared__ floatx4 red[kRedWaves][NT * NE][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * 16 * NT, e0 = blockIdx.y * 16 * NE;
  const __amdgpu_buffer_rsrc_t xrs = rt_rsrc(x, (uint32_t)((size_t)T * d * 2));
  const __amdgpu_buffer_rsrc_t wrs = rt_rsrc(wr, (uint32_t)((size_t)E * d * 2));
  // byte offset of this lane's 16 bytes in chunk 0 of each of its rows (past the end: OOB)
  uint32_t xo[NT], wo[NE];
  bool tin[NT], ein[NE];  // 16-row tiles with at least one row in range (block-uniform)
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = t0 + 16 * i + col;
    xo[i] = t < T ? (uint32_t)t * (uint32_t)(d * 2) + 16u * grp : kRtOOB;
    tin[i] = t0 + 16 * i < T;
  }
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int e = e0 + 16 * j + col;
    wo[j] = e < E ? (uint32_t)e * (uint32_t)(d * 2) + 16u * grp : kRtOOB;
    ein[j] = e0 + 16 * j < E;
  }
  const int nch = d / 32;
  const int c0 = nch * wave / kRtWaves, c1 = nch * (wave + 1) / kRtWaves;
  floatx4 acc[NT][NE];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NE; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int c = c0; c < c1; c += kUnroll) {
    u32x4r a[kUnroll][NT], b[kUnroll][NE];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // a chunk past the wave's range reads zeros (offset past every record) and adds
      // nothing; row offsets plus chunk offsets stay below 2^32 (T * d * 2 < 2^31)
      const bool in = c + u < c1;
      const uint32_t ko = (uint32_t)(c + u) * 64u;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        a[u][i] = tin[i] ? __builtin_amdgcn_raw_buffer_load_b128(xrs, in ? xo[i] + ko : kRtOOB, 0, 0)
                         : u32x4r{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < NE; ++j)
        b[u][j] = ein[j] ? __builtin_amdgcn_raw_buffer_load_b128(wrs, in ? wo[j] + ko : kRtOOB, 0, 0)
                         : u32x4r{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < NE; ++j) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (tin[i] && ein[j])
            acc[i][j] = mfma16(__builtin_bit_cast(bf16x8, b[u][j]), __builtin_bit_cast(bf16x8, a[u][i]), acc[i][j]);
        }
      }
    }
  }
  // lane (col, grp) of tile (i, j) holds experts 4 grp .. 4 grp + 3 of the tile's token col
  auto store = [&](int i, int j, const floatx4& s) {
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
  };
  if constexpr (NT * NE <= 8) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < NE; ++j) red[wave][NE * i + j][lane] = acc[i][j];
    __syncthreads();
    // waves 0 .. NT NE - 1 each finish one 16 x 16 tile: the eight partial tiles in wave order
    if (wave < NT * NE) {
      const int i = wave / NE, j = wave - i * NE;
      floatx4 s = red[0][wave][lane];
#pragma unroll
      for (int w = 1; w < kRtWaves; ++w) s += red[w][wave][lane];
      store(i, j, s);
    }
  } else {
    // pairwise: wave w < h adds wave w + h's tiles, for h = 4, 2, 1; wave 0 stores
#pragma unroll
    for (int h = kRtWaves / 2; h >= 1; h /= 2) {
      if (wave >= h && wave < 2 * h) {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int j = 0; j < NE; ++j) red[wave - h][NE * i + j][lane] = acc[i][j];
      }
      __syncthreads();
      if (wave < h) {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int j = 0; j < NE; ++j) acc[i][j] += red[wave][NE * i + j][lane];
      }
      __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < NE; ++j) store(i, j, acc[i][j]);
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_r, int T, int d, int E, float* logits,
                                hipStream_t stream) {
  if (T <= 16) {
    dim3 grid(1, (E + 15) / 16);
    hipLaunchKernelGGL((router_logits_kernel<1, 1>), grid, dim3(kRtThreads), 0, stream, x, w_r, T, d, E, logits);
  } else {
    if (E > 32) {
      dim3 grid((T + 63) / 64, (E + 63) / 64);
      hipLaunchKernelGGL((router_logits_kernel<4, 4>), grid, dim3(kRtThreads), 0, stream, x, w_r, T, d, E, logits);
    } else {
      dim3 grid((T + 31) / 32, (E + 31) / 32);
      hipLaunchKernelGGL((router_logits_kernel<2, 2>), grid, dim3(kRtThreads), 0, stream, x, w_r, T, d, E, logits);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
