// ffn_skinny.hip -- the expert FFN of the experts that receive few rows of a prompt
// batch.
//
// Routing skew leaves most selected experts of a prompt batch with a handful of rows
// (at 4096 tokens over 256 experts, top-8, the median selected expert has 9 rows), and
// a grouped-GEMM tile of 256 rows would spend a full tile's weight decode on them. The
// pages read each selected expert's weights once for all of its rows
// [FP4-Local checkpoints on DGX Spark, §4 Round 1, #808]; so these experts (at most
// kSkinnyRows rows each) take the weight-streaming form of the decode path instead:
// one 16x16x32 bf16 MFMA tile covers all rows of an expert, the codes stream in with
// 128-bit loads and are decoded in registers, and four waves split K and add their
// sums in LDS in wave order. The grouped GEMM skips these experts. Two launches,
// gate/up/SwiGLU (-> H, bf16) then down (-> fp32 rows), each a grid-stride loop over
// items built on the device from expert_offsets: (expert, 32 features) of gate and up,
// (expert, 64 columns) of down, four 16-row weight tiles an item that share each
// activation load (the activation operands, mostly lanes of missing rows, are what the
// load data path carries most of).
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kSkThreads = 256;  // 4 waves split K
constexpr int kSkWaves = 4;
constexpr int kSkMaxE = 1024;
constexpr int kSkScr = 2048;  // LDS a wave uses to rearrange a chunk pair of one tile
constexpr int kSkGuTiles = 2;  // 16-feature tiles of a gate/up item (each of gate and up)
constexpr int kSkDnTiles = 4;  // 16-column tiles of a down item (one per wave in the sums)

constexpr uint32_t kSkOOB = 0x80000000u;  // a buffer offset past every record: reads zeros

// 8 activation elements (bf16) at element `k` of a lane's row: the row starts at byte
// offset aoff of the activation buffer; lanes of missing rows carry kSkOOB and read
// zeros without a memory access.
__device__ __forceinline__ u32x4 act_load(__amdgpu_buffer_rsrc_t ars, uint32_t aoff, int k) {
  typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));
  const u32x4a v = __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff + (uint32_t)k * 2u), 0, 0);
  return u32x4{v.x, v.y, v.z, v.w};
}

// Accumulates NW weight tiles of 16 rows (wq: row 0 of each tile, row stride wstride
// bytes; tiles nvalid.. are absent and read zeros; wsc: the scale row of this lane's
// column) against one activation row per lane column (at byte offset aoff of the
// activation buffer), over 128-element chunks [c_begin, c_end) and, when `tail`, the
// 32-element chunks past the last full 128. The NW tiles share each activation load.
// A pair of chunks is loaded at a time, along the rows: load i of a tile gives lane
// group lane / 8 the 128 bytes (one cache line) of row 8i + lane / 8, so a load touches
// 8 lines instead of 64 bytes of 16 rows; the wave then rearranges the pair through its
// 2 KB LDS scratch `scr` into the MFMA operand layout (lane group g: elements
// 32g .. 32g + 31 of each chunk). Lanes of missing rows (aoff past the buffer) load no
// activations.
template <int NW>
__device__ __forceinline__ void decode_accumulate(const uint8_t* const (&wq)[NW], int nvalid, size_t wstride,
                                                  const uint8_t* const (&wsc)[NW],
                                                  __amdgpu_buffer_rsrc_t ars, uint32_t aoff,
                                                  int K, int c_begin, int c_end, bool tail,
                                                  floatx4 (&acc)[NW], unsigned char* scr) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int grp8 = lane >> 3, seg8 = lane & 7;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  __amdgpu_buffer_rsrc_t rs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    rs[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wq[i]), 0, i < nvalid ? (int)(16 * wstride) : 0,
                                              0x00020000);
  // pairs start at even chunks, so a pair is one aligned 128-byte line of each row; a
  // chunk of a pair outside [c_begin, c_end) reads nothing (an offset past the buffer)
  struct Pair {
    u32x4 lq[NW][2];   // [tile][rows 0-7 / 8-15], as loaded
    uint32_t sc[NW][2];
    u32x4 xv[2][4];
  };
  auto load_pair = [&](int c, Pair& P) {
    const int mc = c + (seg8 >> 2);  // this lane's chunk
    const uint32_t lo = mc >= c_begin && mc < c_end ? (uint32_t)(grp8 * wstride) + (uint32_t)(c * 64 + 16 * seg8)
                                                    : 0x80000000u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs[i], (int)lo, (int)(8 * h * wstride), kWeightAux);
        P.lq[i][h] = u32x4{v.x, v.y, v.z, v.w};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = c + j >= c_begin && c + j < c_end ? c + j : c_begin;
        P.sc[i][j] = *reinterpret_cast<const uint16_t*>(wsc[i] + cc * 8 + 2 * grp);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cc = c + j >= c_begin && c + j < c_end ? c + j : c_begin;
#pragma unroll
      for (int s = 0; s < 4; ++s) P.xv[j][s] = act_load(ars, aoff, cc * 128 + 32 * grp + 8 * s);
    }
  };
  auto compute_pair = [&](int c, const Pair& P) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      // piece (row r, 16-byte segment s) at r * 128 + ((s + r / 2) mod 8) * 16: both the
      // stores and the loads hit 16 distinct 16-byte bank groups per 16 lanes
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + grp8;
        *reinterpret_cast<u32x4v*>(scr + r * 128 + ((seg8 + (r >> 1)) & 7) * 16) =
            u32x4v{P.lq[i][h].x, P.lq[i][h].y, P.lq[i][h].z, P.lq[i][h].w};
      }
      __builtin_amdgcn_wave_barrier();
      u32x4 q[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4v v = *reinterpret_cast<const u32x4v*>(scr + col * 128 + ((4 * j + grp + (col >> 1)) & 7) * 16);
        q[j] = u32x4{v.x, v.y, v.z, v.w};
      }
      __builtin_amdgcn_wave_barrier();
      // a chunk outside [c_begin, c_end) has zero codes (read past the buffer): its
      // products are +-0 and leave the sums' bits unchanged
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const E4M3Split s0 = e4m3_split_b<0>(P.sc[i][j]);
        const E4M3Split s1 = e4m3_split_b<1>(P.sc[i][j]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 wv = nvfp4x8_to_bf16(word_of(q[j], s), s < 2 ? s0 : s1);
          acc[i] = mfma16(wv, u32x4_as_bf16x8(P.xv[j][s]), acc[i]);
        }
      }
    }
  };
  // Two pairs in flight: the next pair's loads are issued before the current pair is
  // computed. Every path consumes each load it issues (no load past the last pair),
  // so the loads outstanding at each wait are a fixed count.
  const int c0 = c_begin & ~1;
  const int np = c_end > c0 ? (c_end - c0 + 1) / 2 : 0;
  if (np > 0) {
    Pair P0, P1;
    load_pair(c0, P0);
    int p = 0;
    for (; p + 2 < np; p += 2) {
      load_pair(c0 + 2 * (p + 1), P1);
      compute_pair(c0 + 2 * p, P0);
      load_pair(c0 + 2 * (p + 2), P0);
      compute_pair(c0 + 2 * (p + 1), P1);
    }
    if (p + 1 < np) {
      load_pair(c0 + 2 * (p + 1), P1);
      compute_pair(c0 + 2 * p, P0);
      compute_pair(c0 + 2 * (p + 1), P1);
    } else {
      compute_pair(c0 + 2 * p, P0);
    }
  }
  if (tail) {
    // 32-element chunks: lane group g holds elements K0 + 8g .. K0 + 8g + 7 of row col
    for (int K0 = (K / 128) * 128; K0 < K; K0 += 32) {
      const u32x4 xv = act_load(ars, aoff, K0 + 8 * grp);
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq[i] + (size_t)col * wstride + K0 / 2 + 4 * grp);
        const E4M3Split s = e4m3_split(wsc[i][K0 / 16 + (grp >> 1)]);
        acc[i] = mfma16(nvfp4x8_to_bf16(q, s), u32x4_as_bf16x8(xv), acc[i]);
      }
    }
  }
}

// Short K ranges (at most four chunks a wave): the same products with the codes loaded
// straight in the operand layout (lane (grp, col): 16 bytes of weight row col; wq: row 0
// of each tile, row stride wstride bytes, tiles nvalid.. absent; wsc: the scale row of
// this lane's column) against one activation row per lane column (at byte offset aoff
// of the activation buffer), over 128-element chunks [c_begin, c_end) and, when `tail`,
// the 32-element chunks past the last full 128. The loads of up to four chunks are
// issued together (slots past c_end load and compute nothing). Lanes of missing rows
// (aoff past the buffer) load no activations.
template <int NW>
__device__ __forceinline__ void decode_accumulate_lanes(const uint8_t* const (&wq)[NW], int nvalid, size_t wstride,
                                                  const uint8_t* const (&wsc)[NW],
                                                  __amdgpu_buffer_rsrc_t ars, uint32_t aoff,
                                                  int K, int c_begin, int c_end, bool tail,
                                                  floatx4 (&acc)[NW]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  __amdgpu_buffer_rsrc_t rs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    rs[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wq[i]), 0, i < nvalid ? (int)(16 * wstride) : 0,
                                              0x00020000);
  const uint32_t wrow = (uint32_t)(col * wstride) + (uint32_t)(16 * grp);
  // N chunks from cb: every load first, then the products (straight-line code for each
  // count, so no load waits behind another chunk's products)
  auto run = [&](int cb, auto n_const) {
    constexpr int N = decltype(n_const)::value;
    u32x4 q[N][NW];
    uint32_t sc[N][NW];
    u32x4 xv[N][4];
#pragma unroll
    for (int h = 0; h < N; ++h) {
      const int K0 = (cb + h) * 128;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs[i], (int)(wrow + (uint32_t)(K0 / 2)), 0, kWeightAux);
        q[h][i] = u32x4{v.x, v.y, v.z, v.w};
        sc[h][i] = *reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * grp);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[h][s] = act_load(ars, aoff, K0 + 32 * grp + 8 * s);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first product
#pragma unroll
    for (int h = 0; h < N; ++h) {
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
  };
  int cb = c_begin;
  for (; cb + 4 <= c_end; cb += 4) run(cb, std::integral_constant<int, 4>{});
  switch (c_end - cb) {
    case 3: run(cb, std::integral_constant<int, 3>{}); break;
    case 2: run(cb, std::integral_constant<int, 2>{}); break;
    case 1: run(cb, std::integral_constant<int, 1>{}); break;
    default: break;
  }
  if (tail) {
    // 32-element chunks: lane group g holds elements K0 + 8g .. K0 + 8g + 7
    for (int K0 = (K / 128) * 128; K0 < K; K0 += 32) {
      const u32x4 xv = act_load(ars, aoff, K0 + 8 * grp);
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq[i] + (size_t)col * wstride + K0 / 2 + 4 * grp);
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

__global__ __launch_bounds__(kSkThreads, 2) void ffn_skinny_gateup_kernel(FFNArgs a) {
  __shared__ int s_off[kSkMaxE + 1];
  __shared__ int s_e[kSkMaxE], s_r0[kSkMaxE], s_n[kSkMaxE];
  __shared__ int s_cnt;
  __shared__ floatx4 red[2][kSkWaves][2 * kSkGuTiles][64];  // two items' partial sums, alternating
  __shared__ __attribute__((aligned(16))) unsigned char s_scr[kSkWaves][kSkScr];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int U = skinny_list(a.offsets, a.E, s_off, s_e, s_r0, s_n, &s_cnt);
  // x as one buffer (T d 2 < 2^31 bytes, checked by the entry points)
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, (int)((uint32_t)a.T * (uint32_t)a.d * 2u), 0x00020000);
  const int nfg = a.f / (16 * kSkGuTiles);  // f is a multiple of 32
  const int nch = a.d / 128;
  const int items = U * nfg;
  // the sorted_rows entry of routed row `col` of item `it` (rows past the expert's last
  // repeat it), loaded one item ahead so that the activation loads need not wait for it
  auto srow_of = [&](int it) {
    const int uu = it / nfg;
    return a.sorted_rows[s_r0[uu] + min(col, s_n[uu] - 1)];
  };
  int srow = (int)blockIdx.x < items ? srow_of(blockIdx.x) : 0;
  int buf = 0;
  for (int i = blockIdx.x; i < items; i += gridDim.x, buf ^= 1) {
    const int u = i / nfg, fg = i - u * nfg;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    // tiles: gate features 16t.., t < kSkGuTiles, then up
    const size_t wrow0 = (size_t)e * a.f + (size_t)fg * (16 * kSkGuTiles);
    const uint8_t* wq[2 * kSkGuTiles];
    const uint8_t* wsc[2 * kSkGuTiles];
#pragma unroll
    for (int t = 0; t < kSkGuTiles; ++t) {
      wq[t] = a.gate_q + (wrow0 + 16 * t) * (a.d / 2);
      wq[kSkGuTiles + t] = a.up_q + (wrow0 + 16 * t) * (a.d / 2);
      wsc[t] = a.gate_s + (wrow0 + 16 * t + col) * (a.d / 16);
      wsc[kSkGuTiles + t] = a.up_s + (wrow0 + 16 * t + col) * (a.d / 16);
    }
    const bool valid = col < ne;
    // the activation row of routed row `col` (x row sorted_rows[r0 + col] / k)
    const uint32_t aoff = valid ? (uint32_t)(srow / a.k) * (uint32_t)(a.d * 2) : kSkOOB;
    if (i + (int)gridDim.x < items) srow = srow_of(i + gridDim.x);
    // the tensor scales, loaded with the weights (the epilogue needs them)
    const float tg = a.gate_ts[e], tu = a.up_ts[e];
    floatx4 acc[2 * kSkGuTiles];
#pragma unroll
    for (int t = 0; t < 2 * kSkGuTiles; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (nch >= 4 * kSkWaves) {
      decode_accumulate<2 * kSkGuTiles>(wq, 2 * kSkGuTiles, a.d / 2, wsc, xrs, aoff, a.d, nch * wave / kSkWaves,
                                        nch * (wave + 1) / kSkWaves, wave == kSkWaves - 1, acc, s_scr[wave]);
    } else {
      decode_accumulate_lanes<2 * kSkGuTiles>(wq, 2 * kSkGuTiles, a.d / 2, wsc, xrs, aoff, a.d, nch * wave / kSkWaves,
                                              nch * (wave + 1) / kSkWaves, wave == kSkWaves - 1, acc);
    }
#pragma unroll
    for (int t = 0; t < 2 * kSkGuTiles; ++t) red[buf][wave][t][lane] = acc[t];
    // one barrier an item: the next item writes the other half of red, and the one
    // after it is written only after this barrier's successor, which the summing
    // waves reach once their sums below are done
    __syncthreads();
    if (wave < kSkGuTiles && valid) {
      // wave t sums feature tile t: gate partials [t], up partials [kSkGuTiles + t]
      const int t = wave;
      floatx4 G = red[buf][0][t][lane], Uv = red[buf][0][kSkGuTiles + t][lane];
#pragma unroll
      for (int w = 1; w < kSkWaves; ++w) {
        G += red[buf][w][t][lane];
        Uv += red[buf][w][kSkGuTiles + t][lane];
      }
      uint32_t hb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(silu_f32(tg * G[r]) * (tu * Uv[r]));
      // lane holds routed row `col`, features 4*grp .. 4*grp + 3 of tile t
      uint2 v;
      v.x = hb[0] | (hb[1] << 16);
      v.y = hb[2] | (hb[3] << 16);
      *reinterpret_cast<uint2*>(a.h + (size_t)(r0 + col) * a.f + (size_t)fg * (16 * kSkGuTiles) + 16 * t + 4 * grp) = v;
    }
  }
}

__global__ __launch_bounds__(kSkThreads, 2) void ffn_skinny_down_kernel(FFNArgs a) {
  __shared__ int s_off[kSkMaxE + 1];
  __shared__ int s_e[kSkMaxE], s_r0[kSkMaxE], s_n[kSkMaxE];
  __shared__ int s_cnt;
  __shared__ floatx4 red[2][kSkWaves][kSkDnTiles][64];  // two items' partial sums, alternating
  __shared__ __attribute__((aligned(16))) unsigned char s_scr[kSkWaves][kSkScr];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int U = skinny_list(a.offsets, a.E, s_off, s_e, s_r0, s_n, &s_cnt);
  // H as one buffer (T k f 2 < 2^31 bytes, checked by the entry points)
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
      a.h, 0, (int)((uint32_t)a.T * (uint32_t)a.k * (uint32_t)a.f * 2u), 0x00020000);
  const int ndt = a.d / 16;
  const int ndg = (ndt + kSkDnTiles - 1) / kSkDnTiles;  // column groups (the last may be short)
  const int nch = a.f / 128;
  int buf = 0;
  for (int i = blockIdx.x; i < U * ndg; i += gridDim.x, buf ^= 1) {
    const int u = i / ndg, dg = i - u * ndg;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    const int nt = min(kSkDnTiles, ndt - dg * kSkDnTiles);  // tiles of this group
    const uint8_t* wq[kSkDnTiles];
    const uint8_t* wsc[kSkDnTiles];
#pragma unroll
    for (int t = 0; t < kSkDnTiles; ++t) {
      // absent tiles (t >= nt) point at tile 0 and read zeros
      const size_t wrow0 = (size_t)e * a.d + (size_t)(dg * kSkDnTiles + (t < nt ? t : 0)) * 16;
      wq[t] = a.down_q + wrow0 * (a.f / 2);
      wsc[t] = a.down_s + (wrow0 + col) * (a.f / 16);
    }
    const bool valid = col < ne;
    // H row r0 + col
    const uint32_t aoff = valid ? (uint32_t)(r0 + col) * (uint32_t)(a.f * 2) : kSkOOB;
    const float td = a.down_ts[e];  // loaded with the weights (the epilogue needs it)
    floatx4 acc[kSkDnTiles];
#pragma unroll
    for (int t = 0; t < kSkDnTiles; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (nch >= 4 * kSkWaves) {
      decode_accumulate<kSkDnTiles>(wq, nt, a.f / 2, wsc, hrs, aoff, a.f, nch * wave / kSkWaves,
                                    nch * (wave + 1) / kSkWaves, wave == kSkWaves - 1, acc, s_scr[wave]);
    } else {
      decode_accumulate_lanes<kSkDnTiles>(wq, nt, a.f / 2, wsc, hrs, aoff, a.f, nch * wave / kSkWaves,
                                          nch * (wave + 1) / kSkWaves, wave == kSkWaves - 1, acc);
    }
#pragma unroll
    for (int t = 0; t < kSkDnTiles; ++t) red[buf][wave][t][lane] = acc[t];
    __syncthreads();  // one barrier an item (red alternates, as in the gate/up kernel)
    if (wave < nt && valid) {
      // wave t sums column tile t
      const int t = wave;
      floatx4 O = red[buf][0][t][lane];
#pragma unroll
      for (int w = 1; w < kSkWaves; ++w) O += red[buf][w][t][lane];
      float4 v;
      v.x = td * O[0];
      v.y = td * O[1];
      v.z = td * O[2];
      v.w = td * O[3];
      *reinterpret_cast<float4*>(a.y_rows + (size_t)(r0 + col) * a.d + (size_t)(dg * kSkDnTiles + t) * 16 + 4 * grp) = v;
    }
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
