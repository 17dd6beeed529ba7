// ffn_decode.hip -- the expert FFN for a few tokens (decode): weight streaming.
//
// With a few tokens every selected expert has at most a handful of rows, and the
// layer's time is the time to read the selected experts' weight bytes once. The pages
// read each selected expert once for all of its rows [FP4-Local checkpoints on DGX
// Spark, §4 Round 1, #808]; here one 16x16x32 bf16 MFMA tile covers all of an
// expert's rows (<= 16), so each weight byte is read once whatever the row count.
//
// Mapping (per wave): 16 weight rows (output features) x up to 16 routed rows. Each
// lane streams one weight row's packed codes with 128-bit loads (32 E2M1 codes = two
// scale blocks) and decodes them in registers into four MFMA operands. Within a 128-
// element chunk, lane group g (lane / 16) holds elements [32g, 32g + 32) and MFMA
// step s takes elements 32g + 8s .. 32g + 8s + 7 of every group -- a permutation of
// the contraction index, applied identically to the activation operand, so the sums
// are unchanged. A block of KSPLIT waves splits K and reduces in LDS in wave order.
//
// Gate, up and SwiGLU run in one launch [same page, §4 Round 1, #766]: the gate and up
// tiles of the same 16 features share the activation operand, and the epilogue forms
// H = bf16_rne(silu(ts_g * G) * (ts_u * U)). The down launch then reads H.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kDecodeKsplitGU = 4;
constexpr int kDecodeKsplitDown = 2;

// The u-th expert (in index order) whose row list is non-empty; wave-wide, every lane
// gets the answer. Returns false when fewer than u + 1 experts have rows.
__device__ bool find_touched_expert(const int32_t* __restrict__ offsets, int E, int u, int& e_out,
                                    int& r0, int& r1) {
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int o0 = 0, c = 0;
    if (e < E) {
      o0 = offsets[e];
      c = offsets[e + 1] - o0;
    }
    const uint64_t nz = __ballot(c > 0);
    const int n = __popcll(nz);
    if (u < seen + n) {
      const int rank = __popcll(nz & ((1ull << lane) - 1ull));
      const uint64_t hit = __ballot(c > 0 && rank == u - seen);
      const int src = __ffsll((unsigned long long)hit) - 1;
      e_out = base + src;
      r0 = __shfl(o0, src);
      r1 = r0 + __shfl(c, src);
      return true;
    }
    seen += n;
  }
  return false;
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word_of(const u32x4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Accumulates NW weight matrices (rows wrow[i], K = K elements) against one activation
// row per lane column, over 128-element chunks [c_begin, c_end) and, when `tail`, the
// 32-element chunks past the last full 128 chunk.
template <int NW>
__device__ __forceinline__ void decode_accumulate(const uint8_t* const (&wq)[NW],
                                                  const uint8_t* const (&wsc)[NW],
                                                  const uint16_t* __restrict__ act, bool valid,
                                                  int K, int c_begin, int c_end, bool tail,
                                                  floatx4 (&acc)[NW]) {
  const int grp = (threadIdx.x & 63) >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  int c = c_begin;
  // two chunks in flight per iteration
  for (; c + 1 < c_end; c += 2) {
    u32x4 q[2][NW];
    uint32_t sc[2][NW];
    u32x4 xv[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int K0 = (c + h) * 128;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        q[h][i] = ldg_u32x4(wq[i] + K0 / 2 + 16 * grp);
        sc[h][i] = *reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * grp);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[h][s] = valid ? ldg_u32x4(act + K0 + 32 * grp + 8 * s) : zero;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const E4M3Split s0 = e4m3_split(sc[h][i] & 0xFFu);
        const E4M3Split s1 = e4m3_split(sc[h][i] >> 8);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 wv = nvfp4x8_to_bf16(word_of(q[h][i], s), s < 2 ? s0 : s1);
          acc[i] = mfma16(wv, u32x4_as_bf16x8(xv[h][s]), acc[i]);
        }
      }
    }
  }
  for (; c < c_end; ++c) {
    const int K0 = c * 128;
    u32x4 q[NW];
    uint32_t sc[NW];
    u32x4 xv[4];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      q[i] = ldg_u32x4(wq[i] + K0 / 2 + 16 * grp);
      sc[i] = *reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * grp);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) xv[s] = valid ? ldg_u32x4(act + K0 + 32 * grp + 8 * s) : zero;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const E4M3Split s0 = e4m3_split(sc[i] & 0xFFu);
      const E4M3Split s1 = e4m3_split(sc[i] >> 8);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 wv = nvfp4x8_to_bf16(word_of(q[i], s), s < 2 ? s0 : s1);
        acc[i] = mfma16(wv, u32x4_as_bf16x8(xv[s]), acc[i]);
      }
    }
  }
  if (tail) {
    // 32-element chunks: lane group g holds elements K0 + 8g .. K0 + 8g + 7
    for (int K0 = (K / 128) * 128; K0 < K; K0 += 32) {
      const u32x4 xv = valid ? ldg_u32x4(act + K0 + 8 * grp) : zero;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq[i] + K0 / 2 + 4 * grp);
        const E4M3Split s = e4m3_split(wsc[i][K0 / 16 + (grp >> 1)]);
        acc[i] = mfma16(nvfp4x8_to_bf16(q, s), u32x4_as_bf16x8(xv), acc[i]);
      }
    }
  }
}

template <int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void ffn_decode_gateup_kernel(FFNArgs a) {
  __shared__ floatx4 red[KSPLIT][2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ft = blockIdx.x;  // 16-feature tile of f
  int e, r0, r1;
  if (!find_touched_expert(a.offsets, a.E, blockIdx.y, e, r0, r1)) return;
  const int ne = r1 - r0;  // <= kDecodeMaxRows (host-checked through T)
  const int col = lane & 15, grp = lane >> 4;
  const size_t wrow = (size_t)e * a.f + ft * 16 + col;
  const uint8_t* const wq[2] = {a.gate_q + wrow * (a.d / 2), a.up_q + wrow * (a.d / 2)};
  const uint8_t* const wsc[2] = {a.gate_s + wrow * (a.d / 16), a.up_s + wrow * (a.d / 16)};
  const bool valid = col < ne;
  const uint16_t* act = a.x + (size_t)(valid ? a.sorted_rows[r0 + col] / a.k : 0) * a.d;
  floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int nch = a.d / 128;
  decode_accumulate<2>(wq, wsc, act, valid, a.d, nch * wave / KSPLIT, nch * (wave + 1) / KSPLIT,
                       wave == KSPLIT - 1, acc);
  red[wave][0][lane] = acc[0];
  red[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave != 0 || !valid) return;
  floatx4 G = red[0][0][lane], U = red[0][1][lane];
#pragma unroll
  for (int w = 1; w < KSPLIT; ++w) {
    G += red[w][0][lane];
    U += red[w][1][lane];
  }
  const float tg = a.gate_ts[e], tu = a.up_ts[e];
  uint32_t hb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(silu_f32(tg * G[r]) * (tu * U[r]));
  // lane holds token column `col`, features 4*grp .. 4*grp + 3 of the tile
  uint2 v;
  v.x = hb[0] | (hb[1] << 16);
  v.y = hb[2] | (hb[3] << 16);
  *reinterpret_cast<uint2*>(a.h + (size_t)(r0 + col) * a.f + ft * 16 + 4 * grp) = v;
}

template <int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void ffn_decode_down_kernel(FFNArgs a) {
  __shared__ floatx4 red[KSPLIT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dt = blockIdx.x;  // 16-column tile of d
  int e, r0, r1;
  if (!find_touched_expert(a.offsets, a.E, blockIdx.y, e, r0, r1)) return;
  const int ne = r1 - r0;
  const int col = lane & 15, grp = lane >> 4;
  const size_t wrow = (size_t)e * a.d + dt * 16 + col;
  const uint8_t* const wq[1] = {a.down_q + wrow * (a.f / 2)};
  const uint8_t* const wsc[1] = {a.down_s + wrow * (a.f / 16)};
  const bool valid = col < ne;
  const uint16_t* act = a.h + (size_t)(valid ? r0 + col : 0) * a.f;
  floatx4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  const int nch = a.f / 128;
  decode_accumulate<1>(wq, wsc, act, valid, a.f, nch * wave / KSPLIT, nch * (wave + 1) / KSPLIT,
                       wave == KSPLIT - 1, acc);
  red[wave][lane] = acc[0];
  __syncthreads();
  if (wave != 0 || !valid) return;
  floatx4 O = red[0][lane];
#pragma unroll
  for (int w = 1; w < KSPLIT; ++w) O += red[w][lane];
  const float td = a.down_ts[e];
  float4 v;
  v.x = td * O[0];
  v.y = td * O[1];
  v.z = td * O[2];
  v.w = td * O[3];
  *reinterpret_cast<float4*>(a.y_rows + (size_t)(r0 + col) * a.d + dt * 16 + 4 * grp) = v;
}

hipError_t launch_ffn_decode(const FFNArgs& a, hipStream_t stream) {
  const int max_touched = (int)std::min<long long>(a.E, (long long)a.T * a.k);
  hipLaunchKernelGGL(ffn_decode_gateup_kernel<kDecodeKsplitGU>, dim3(a.f / 16, max_touched),
                     dim3(64 * kDecodeKsplitGU), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_decode_down_kernel<kDecodeKsplitDown>, dim3(a.d / 16, max_touched),
                     dim3(64 * kDecodeKsplitDown), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
