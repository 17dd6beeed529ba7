// ffn_skinny.hip -- the expert FFN of the experts that receive few rows of a prompt
// batch.
//
// Routing skew leaves most selected experts of a prompt batch with a handful of rows
// (at 4096 tokens over 256 experts, top-8, the median selected expert has 9 rows), and
// a grouped-GEMM tile of 256 rows would spend a full tile's weight decode on them. The
// pages read each selected expert's weights once for all of its rows
// [FP4-Local checkpoints on DGX Spark, §4 Round 1, #808]; so these experts (at most
// kSkinnyRows rows each) take the weight-streaming form of the decode path instead:
// one 16x16x32 bf16 MFMA tile covers all rows of an expert, each lane streams one
// weight row's packed codes with 128-bit loads, decodes them in registers, and four
// waves split K and add their sums in LDS in wave order. The grouped GEMM skips these
// experts. Two launches, gate/up/SwiGLU (-> H, bf16) then down (-> fp32 rows), each a
// grid-stride loop over (expert, 16 features or columns) items built on the device
// from expert_offsets.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kSkThreads = 256;  // 4 waves split K
constexpr int kSkWaves = 4;
constexpr int kSkMaxE = 1024;
constexpr int kSkScr = 2048;  // LDS a wave uses to rearrange a chunk pair of one tile

// Accumulates NW weight tiles of 16 rows (wq: row 0 of each tile, row stride wstride
// bytes; wsc: the scale row of this lane's column) against one activation row per lane
// column (act), over 128-element chunks [c_begin, c_end) and, when `tail`, the
// 32-element chunks past the last full 128. A pair of chunks is loaded at a time, along
// the rows: load i of a tile gives lane group lane / 8 the 128 bytes (one cache line) of
// row 8i + lane / 8, so a load touches 8 lines instead of 64 bytes of 16 rows; the wave
// then rearranges the pair through its 2 KB LDS scratch `scr` into the MFMA operand
// layout (lane group g: elements 32g .. 32g + 31 of each chunk). Lanes of missing rows
// (!valid) load no activations: with a few rows an expert, that keeps the activation
// traffic far below the weight traffic.
template <int NW>
__device__ __forceinline__ void decode_accumulate(const uint8_t* const (&wq)[NW], size_t wstride,
                                                  const uint8_t* const (&wsc)[NW],
                                                  const uint16_t* __restrict__ act, bool valid,
                                                  int K, int c_begin, int c_end, bool tail,
                                                  floatx4 (&acc)[NW], unsigned char* scr) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int grp8 = lane >> 3, seg8 = lane & 7;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  __amdgpu_buffer_rsrc_t rs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    rs[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wq[i]), 0, (int)(16 * wstride), 0x00020000);
  // pairs start at even chunks, so a pair is one aligned 128-byte line of each row; a
  // chunk of a pair outside [c_begin, c_end) reads nothing (an offset past the buffer)
  for (int c = c_begin & ~1; c < c_end; c += 2) {
    const int mc = c + (seg8 >> 2);  // this lane's chunk
    const uint32_t lo = mc >= c_begin && mc < c_end ? (uint32_t)(grp8 * wstride) + (uint32_t)(c * 64 + 16 * seg8)
                                                    : 0x80000000u;
    u32x4 lq[NW][2];
    uint32_t sc[NW][2];
    u32x4 xv[2][4];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs[i], (int)lo, (int)(8 * h * wstride), kWeightAux);
        lq[i][h] = u32x4{v.x, v.y, v.z, v.w};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = c + j >= c_begin && c + j < c_end ? c + j : c_begin;
        sc[i][j] = *reinterpret_cast<const uint16_t*>(wsc[i] + cc * 8 + 2 * grp);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cc = c + j >= c_begin && c + j < c_end ? c + j : c_begin;
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[j][s] = valid ? ldg_u32x4(act + cc * 128 + 32 * grp + 8 * s) : zero;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      // piece (row r, 16-byte segment s) at r * 128 + ((s + r / 2) mod 8) * 16: both the
      // stores and the loads hit 16 distinct 16-byte bank groups per 16 lanes
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + grp8;
        *reinterpret_cast<u32x4v*>(scr + r * 128 + ((seg8 + (r >> 1)) & 7) * 16) =
            u32x4v{lq[i][h].x, lq[i][h].y, lq[i][h].z, lq[i][h].w};
      }
      __builtin_amdgcn_wave_barrier();
      u32x4 q[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4v v = *reinterpret_cast<const u32x4v*>(scr + col * 128 + ((4 * j + grp + (col >> 1)) & 7) * 16);
        q[j] = u32x4{v.x, v.y, v.z, v.w};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (c + j >= c_begin && c + j < c_end) {
          const E4M3Split s0 = e4m3_split_b<0>(sc[i][j]);
          const E4M3Split s1 = e4m3_split_b<1>(sc[i][j]);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 wv = nvfp4x8_to_bf16(word_of(q[j], s), s < 2 ? s0 : s1);
            acc[i] = mfma16(wv, u32x4_as_bf16x8(xv[j][s]), acc[i]);
          }
        }
      }
    }
  }
  if (tail) {
    // 32-element chunks: lane group g holds elements K0 + 8g .. K0 + 8g + 7 of row col
    for (int K0 = (K / 128) * 128; K0 < K; K0 += 32) {
      const u32x4 xv = valid ? ldg_u32x4(act + K0 + 8 * grp) : zero;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq[i] + (size_t)col * wstride + K0 / 2 + 4 * grp);
        const E4M3Split s = e4m3_split(wsc[i][K0 / 16 + (grp >> 1)]);
        acc[i] = mfma16(nvfp4x8_to_bf16(q, s), u32x4_as_bf16x8(xv), acc[i]);
      }
    }
  }
}

// Short K ranges (fewer than four chunks a wave): the same products with the codes
// loaded straight in the operand layout (one weight row per lane column: wq / wsc) against one
// activation row per lane column (act), over 128-element chunks [c_begin, c_end) and,
// when `tail`, the 32-element chunks past the last full 128. Two chunks' loads are in
// flight at a time. Lanes of missing rows (!valid) load no activations: with a few
// rows an expert, that keeps the activation traffic far below the weight traffic.
template <int NW>
__device__ __forceinline__ void decode_accumulate_lanes(const uint8_t* const (&wq)[NW],
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
        q[h][i] = ldg_nt_u32x4(wq[i] + K0 / 2 + 16 * grp);
        sc[h][i] = *reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * grp);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[h][s] = valid ? ldg_u32x4(act + K0 + 32 * grp + 8 * s) : zero;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const E4M3Split s0 = e4m3_split_b<0>(sc[h][i]);
        const E4M3Split s1 = e4m3_split_b<1>(sc[h][i]);
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
      q[i] = ldg_nt_u32x4(wq[i] + K0 / 2 + 16 * grp);
      sc[i] = *reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * grp);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) xv[s] = valid ? ldg_u32x4(act + K0 + 32 * grp + 8 * s) : zero;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const E4M3Split s0 = e4m3_split_b<0>(sc[i]);
      const E4M3Split s1 = e4m3_split_b<1>(sc[i]);
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

// Experts with 1 .. kSkinnyRows rows, in index order, into LDS; returns their number.
__device__ int skinny_list(const int32_t* __restrict__ offsets, int E, int* s_off, int* s_e, int* s_r0,
                           int* s_n, int* s_cnt) {
  for (int i = threadIdx.x; i <= E; i += kSkThreads) s_off[i] = offsets[i];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int seen = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int o0 = 0, c = 0;
      if (e < E) {
        o0 = s_off[e];
        c = s_off[e + 1] - o0;
      }
      const bool pick = c >= 1 && c <= kSkinnyRows;
      const uint64_t m = __ballot(pick);
      if (pick) {
        const int r = seen + __popcll(m & ((1ull << lane) - 1ull));
        s_e[r] = e;
        s_r0[r] = o0;
        s_n[r] = c;
      }
      seen += __popcll(m);
    }
    if (lane == 0) *s_cnt = seen;
  }
  __syncthreads();
  return *s_cnt;
}

__global__ __launch_bounds__(kSkThreads) void ffn_skinny_gateup_kernel(FFNArgs a) {
  __shared__ int s_off[kSkMaxE + 1];
  __shared__ int s_e[kSkMaxE], s_r0[kSkMaxE], s_n[kSkMaxE];
  __shared__ int s_cnt;
  __shared__ floatx4 red[kSkWaves][2][64];
  __shared__ __attribute__((aligned(16))) unsigned char s_scr[kSkWaves][kSkScr];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int U = skinny_list(a.offsets, a.E, s_off, s_e, s_r0, s_n, &s_cnt);
  const int nft = a.f / 16;
  const int nch = a.d / 128;
  for (int i = blockIdx.x; i < U * nft; i += gridDim.x) {
    const int u = i / nft, ft = i - u * nft;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    const size_t wrow0 = (size_t)e * a.f + ft * 16, wrow = wrow0 + col;
    const uint8_t* const wq[2] = {a.gate_q + wrow0 * (a.d / 2), a.up_q + wrow0 * (a.d / 2)};
    const uint8_t* const wsc[2] = {a.gate_s + wrow * (a.d / 16), a.up_s + wrow * (a.d / 16)};
    const bool valid = col < ne;
    const uint16_t* act = a.x + (size_t)(a.sorted_rows[r0 + (valid ? col : 0)] / a.k) * a.d;
    floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (nch >= 4 * kSkWaves) {
      decode_accumulate<2>(wq, a.d / 2, wsc, act, valid, a.d, nch * wave / kSkWaves, nch * (wave + 1) / kSkWaves,
                           wave == kSkWaves - 1, acc, s_scr[wave]);
    } else {
      const uint8_t* const wql[2] = {wq[0] + (size_t)col * (a.d / 2), wq[1] + (size_t)col * (a.d / 2)};
      decode_accumulate_lanes<2>(wql, wsc, act, valid, a.d, nch * wave / kSkWaves, nch * (wave + 1) / kSkWaves,
                                 wave == kSkWaves - 1, acc);
    }
    red[wave][0][lane] = acc[0];
    red[wave][1][lane] = acc[1];
    __syncthreads();
    if (wave == 0 && valid) {
      floatx4 G = red[0][0][lane], Uv = red[0][1][lane];
#pragma unroll
      for (int w = 1; w < kSkWaves; ++w) {
        G += red[w][0][lane];
        Uv += red[w][1][lane];
      }
      const float tg = a.gate_ts[e], tu = a.up_ts[e];
      uint32_t hb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(silu_f32(tg * G[r]) * (tu * Uv[r]));
      // lane holds routed row `col`, features 4*grp .. 4*grp + 3 of the tile
      uint2 v;
      v.x = hb[0] | (hb[1] << 16);
      v.y = hb[2] | (hb[3] << 16);
      *reinterpret_cast<uint2*>(a.h + (size_t)(r0 + col) * a.f + ft * 16 + 4 * grp) = v;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSkThreads) void ffn_skinny_down_kernel(FFNArgs a) {
  __shared__ int s_off[kSkMaxE + 1];
  __shared__ int s_e[kSkMaxE], s_r0[kSkMaxE], s_n[kSkMaxE];
  __shared__ int s_cnt;
  __shared__ floatx4 red[kSkWaves][64];
  __shared__ __attribute__((aligned(16))) unsigned char s_scr[kSkWaves][kSkScr];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int U = skinny_list(a.offsets, a.E, s_off, s_e, s_r0, s_n, &s_cnt);
  const int ndt = a.d / 16;
  const int nch = a.f / 128;
  for (int i = blockIdx.x; i < U * ndt; i += gridDim.x) {
    const int u = i / ndt, dt = i - u * ndt;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    const size_t wrow0 = (size_t)e * a.d + dt * 16, wrow = wrow0 + col;
    const uint8_t* const wq[1] = {a.down_q + wrow0 * (a.f / 2)};
    const uint8_t* const wsc[1] = {a.down_s + wrow * (a.f / 16)};
    const bool valid = col < ne;
    const uint16_t* act = a.h + (size_t)(r0 + (valid ? col : 0)) * a.f;
    floatx4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    if (nch >= 4 * kSkWaves) {
      decode_accumulate<1>(wq, a.f / 2, wsc, act, valid, a.f, nch * wave / kSkWaves, nch * (wave + 1) / kSkWaves,
                           wave == kSkWaves - 1, acc, s_scr[wave]);
    } else {
      const uint8_t* const wql[1] = {wq[0] + (size_t)col * (a.f / 2)};
      decode_accumulate_lanes<1>(wql, wsc, act, valid, a.f, nch * wave / kSkWaves, nch * (wave + 1) / kSkWaves,
                                 wave == kSkWaves - 1, acc);
    }
    red[wave][lane] = acc[0];
    __syncthreads();
    if (wave == 0 && valid) {
      floatx4 O = red[0][lane];
#pragma unroll
      for (int w = 1; w < kSkWaves; ++w) O += red[w][lane];
      const float td = a.down_ts[e];
      float4 v;
      v.x = td * O[0];
      v.y = td * O[1];
      v.z = td * O[2];
      v.w = td * O[3];
      *reinterpret_cast<float4*>(a.y_rows + (size_t)(r0 + col) * a.d + dt * 16 + 4 * grp) = v;
    }
    __syncthreads();
  }
}

// The grid-stride loops run on as many blocks as the device holds at once (one round of
// blocks: each reads the expert offsets once).
hipError_t launch_ffn_skinny_gateup(const FFNArgs& a, hipStream_t stream) {
  int blocks = 0;
  hipError_t err = resident_blocks(reinterpret_cast<const void*>(&ffn_skinny_gateup_kernel), kSkThreads, 0, blocks);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_skinny_gateup_kernel, dim3(blocks), dim3(kSkThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ffn_skinny_down(const FFNArgs& a, hipStream_t stream) {
  int blocks = 0;
  hipError_t err = resident_blocks(reinterpret_cast<const void*>(&ffn_skinny_down_kernel), kSkThreads, 0, blocks);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_skinny_down_kernel, dim3(blocks), dim3(kSkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
