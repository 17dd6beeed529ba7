// skinny_device.hpp -- the weight-streaming form of the expert FFN (device code), for
// the experts that receive few rows of a prompt batch.
//
// Routing skew leaves most selected experts of a prompt batch with a handful of rows
// (at 4096 tokens over 256 experts, top-8, the median selected expert has 9 rows), and
// a grouped-GEMM tile of 128 rows would spend a full tile's weight decode on them. The
// pages read each selected expert's weights once for all of its rows
// [FP4-Local checkpoints on DGX Spark, §4 Round 1, #808]; so these experts (at most
// kSkinnyRows rows each) take the weight-streaming form of the decode path instead:
// one or two 16x16x32 bf16 MFMA column tiles cover all rows of an expert (one 16-row
// set, or two for 17..32 rows), the codes stream in with 128-bit loads and are decoded
// in registers once for every row set, and four waves split K and add their sums in
// LDS in wave order. Items are built on the device from expert_offsets: (expert, 32
// features) of gate and up for one row set, (expert, 16 features) for two, (expert, 64
// or 32 columns) of down; an item's four tile-by-set accumulators share each activation
// load (the activation operands, mostly lanes of missing rows, are what the load data
// path carries most of).
//
// The grouped GEMM kernels run these items after their own tiles, taking them from a
// counter (ffn_prompt.hip); the standalone kernels (ffn_skinny.hip) run them for calls
// that have no GEMM tiles.
#pragma once
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kSkThreads = 256;  // 4 waves split K
constexpr int kSkWaves = 4;
constexpr int kSkMaxE = 1024;
constexpr int kSkScrScale = 2048;          // the part of it that regroups two pairs' block scales
constexpr int kSkScr = 2048 + kSkScrScale;  // LDS a wave uses to rearrange a chunk pair of one tile

constexpr uint32_t kSkOOB = 0x80000000u;  // a buffer offset past every record: reads zeros

// 8 activation elements (bf16) at element `k` of a lane's row: the row starts at byte
// offset aoff of the activation buffer; lanes of missing rows carry kSkOOB and read
// zeros without a memory access.
__device__ __forceinline__ u32x4 act_load(__amdgpu_buffer_rsrc_t ars, uint32_t aoff, int k) {
  typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));
  const u32x4a v = __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff + (uint32_t)k * 2u), 0, 0);
  return u32x4{v.x, v.y, v.z, v.w};
}

// Lane col of each 16-lane row takes the 16 bytes of lane col + SH (a DPP row shift;
// lanes whose source lies past their row take zeros).
template <int SH>
__device__ __forceinline__ u32x4 rows_shl(const u32x4& v) {
  if constexpr (SH == 0) {
    return v;
  } else {
    return u32x4{(uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0x100 + SH, 0xF, 0xF, true),
                 (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0x100 + SH, 0xF, 0xF, true),
                 (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, 0x100 + SH, 0xF, 0xF, true),
                 (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, 0x100 + SH, 0xF, 0xF, true)};
  }
}

// Activation rows packed PK to a lane row (PK = 1, 2, 4), for one row set of at most
// 16 / PK rows: lane col holds row col mod (16 / PK), and its 16-byte load q brings the
// 8-element group act_group(q, col) of the four (s = 0..3) its lane group needs from a
// 128-element chunk, so a chunk takes 4 / PK loads instead of four. The operand of group
// s is then load s / PK shifted down by (s mod PK) (16 / PK) lanes; lanes past the rows
// hold other groups' elements, which feed only the products of missing rows.
template <int PK>
__device__ __forceinline__ int act_group(int q, int col) {
  return q * PK + col / (16 / PK);
}
template <int PK>
__device__ __forceinline__ u32x4 act_operand(const u32x4 (&v)[4 / PK], int s) {
  if constexpr (PK == 1) {
    return v[s];
  } else if constexpr (PK == 2) {
    return (s & 1) ? rows_shl<8>(v[s >> 1]) : v[s >> 1];
  } else {
    return s == 0 ? v[0] : s == 1 ? rows_shl<4>(v[0]) : s == 2 ? rows_shl<8>(v[0]) : rows_shl<12>(v[0]);
  }
}

// Accumulates NW weight tiles of 16 rows (wq: row 0 of each tile, row stride wstride
// bytes; tiles nvalid.. are absent and read zeros; wsc: the scale row of this lane's
// column) against RS sets of 16 activation rows, one row per lane column in each (at
// byte offset aoff[r] of the activation buffer), into acc[tile][set], over 128-element
// chunks [c_begin, c_end) and, when `tail`, the 32-element chunks past the last full
// 128. The NW tiles share each activation load and the RS sets each decoded weight.
// A pair of chunks is loaded at a time, along the rows: load i of a tile gives lane
// group lane / 8 the 128 bytes (one cache line) of row 8i + lane / 8, so a load touches
// 8 lines instead of 64 bytes of 16 rows; the wave then rearranges the pair through its
// 2 KB LDS scratch `scr` into the MFMA operand layout (lane group g: elements
// 32g .. 32g + 31 of each chunk). Lanes of missing rows (aoff past the buffer) load no
// activations. Block scales: K is a multiple of 256, so a scale row holds whole 16-byte
// pairs; the loads of every other pair bring the scales of that pair and the next one
// for all NW tiles' rows, 16 bytes a lane, two lanes a row (lane l: row 32h + l / 2 of
// the NW * 16, through the per-lane pointer wsl2[h], pair l mod 2), so a load touches 32
// rows' lines instead of 64; the wave regroups both pairs through the last kSkScrScale
// bytes of its scratch (1 KB a pair).
// PK > 1 (one row set): activation rows packed PK to a lane row (act_operand).
template <int NW, int RS, int PK = 1>
__device__ __forceinline__ void decode_accumulate(const uint8_t* const (&wq)[NW], int nvalid, size_t wstride,
                                                  const uint8_t* const (&wsl2)[NW / 2],
                                                  __amdgpu_buffer_rsrc_t ars, const uint32_t (&aoff)[RS],
                                                  int c_begin, int c_end, floatx4 (&acc)[NW][RS],
                                                  unsigned char* scr) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, col = lane & 15;
  const int grp8 = lane >> 3, seg8 = lane & 7;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  __amdgpu_buffer_rsrc_t rs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    rs[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wq[i]), 0, i < nvalid ? (int)(16 * wstride) : 0,
                                              0x00020000);
  // pairs start at even chunks (c0, c0 + 2, ...), so a pair is one aligned 128-byte line
  // of each row; a chunk of a pair outside [c_begin, c_end) reads nothing (an offset past
  // the buffer). The scale loads of an even pair p also bring pair p + 1's scales (the
  // last pair's again where p is the last).
  const int c0 = c_begin & ~1;
  const int np = c_end > c0 ? (c_end - c0 + 1) / 2 : 0;
  const int c_last = c0 + 2 * (np - 1);
  struct Pair {
    u32x4 lq[NW][2];   // [tile][rows 0-7 / 8-15], as loaded
    u32x4 scq[NW / 2];  // even pairs: this lane's 16 scale bytes of its row and pair
    u32x4 xv[RS][2][4 / PK];
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
    }
    // a chunk of a pair outside [c_begin, c_end) gets its own scales (its codes are
    // zero, so they scale nothing)
    if (((c - c0) & 2) == 0) {
      const int cq = min(c + 2 * (lane & 1), c_last);
#pragma unroll
      for (int h = 0; h < NW / 2; ++h) P.scq[h] = *reinterpret_cast<const u32x4*>(wsl2[h] + cq * 8);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cc = c + j >= c_begin && c + j < c_end ? c + j : c_begin;
#pragma unroll
      for (int r = 0; r < RS; ++r)
#pragma unroll
        for (int q = 0; q < 4 / PK; ++q)
          P.xv[r][j][q] = act_load(ars, aoff[r], cc * 128 + 32 * grp + 8 * act_group<PK>(q, col));
    }
  };
  auto compute_pair = [&](int c, const Pair& P) {
    // lane l's bytes (chunk c: x, y; chunk c + 1: z, w) regrouped as four dwords, dword g
    // holding what lane group g of the lane's row needs, then read back per tile:
    // scw[i] = [chunk c: bytes 2 grp, 2 grp + 1 | chunk c + 1: the same] of tile i, row col
    // (even pairs first write both pairs' regrouped scales: pair p + j at j KB, row
    // 32h + l / 2 at 16 (32h + l / 2))
    uint32_t scw[NW];
    {
      unsigned char* const ss = scr + kSkScr - kSkScrScale;
      const bool even = ((c - c0) & 2) == 0;
      if (even) {
#pragma unroll
        for (int h = 0; h < NW / 2; ++h)
          *reinterpret_cast<u32x4v*>(ss + (lane & 1) * 1024 + (32 * h + (lane >> 1)) * 16) =
              u32x4v{__builtin_amdgcn_perm(P.scq[h].z, P.scq[h].x, 0x05040100u),
                     __builtin_amdgcn_perm(P.scq[h].z, P.scq[h].x, 0x07060302u),
                     __builtin_amdgcn_perm(P.scq[h].w, P.scq[h].y, 0x05040100u),
                     __builtin_amdgcn_perm(P.scq[h].w, P.scq[h].y, 0x07060302u)};
        __builtin_amdgcn_wave_barrier();
      }
#pragma unroll
      for (int i = 0; i < NW; ++i)
        scw[i] = *reinterpret_cast<const uint32_t*>(ss + (even ? 0 : 1024) + (i * 16 + col) * 16 + grp * 4);
      __builtin_amdgcn_wave_barrier();
    }
    u32x4 xo[RS][2][4];  // the activation operands, shared by the NW tiles
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) xo[r][j][s] = act_operand<PK>(P.xv[r][j], s);
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
        const E4M3Split s0 = j == 0 ? e4m3_split_b<0>(scw[i]) : e4m3_split_b<2>(scw[i]);
        const E4M3Split s1 = j == 0 ? e4m3_split_b<1>(scw[i]) : e4m3_split_b<3>(scw[i]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 wv = nvfp4x8_to_bf16(word_of(q[j], s), s < 2 ? s0 : s1);
#pragma unroll
          for (int r = 0; r < RS; ++r) acc[i][r] = mfma16(wv, u32x4_as_bf16x8(xo[r][j][s]), acc[i][r]);
        }
      }
    }
  };
  // One row set: two pairs in flight (the next pair's loads are issued before the
  // current pair is computed). Every path consumes each load it issues (no load past
  // the last pair), so the loads outstanding at each wait are a fixed count.
  if constexpr (RS > 1) {
    // two row sets: one pair at a time (a second pair's activation operands would not
    // fit in the registers)
    for (int p = 0; p < np; ++p) {
      Pair P;
      load_pair(c0 + 2 * p, P);
      compute_pair(c0 + 2 * p, P);
    }
  } else if (np > 0) {
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
}

// Short K ranges (at most four chunks a wave), and any K range when K is not a multiple
// of 256 (in rounds of four chunks): the same products with the codes loaded
// straight in the operand layout (lane (grp, col): 16 bytes of weight row col; wq: row 0
// of each tile, row stride wstride bytes, tiles nvalid.. absent; wsc: the scale row of
// this lane's column) against RS sets of 16 activation rows (row col of set r at byte
// offset aoff[r] of the activation buffer), over 128-element chunks [c_begin, c_end)
// and, when `tail`, the 32-element chunks past the last full 128. The loads of up to
// four chunks (two with two row sets) are issued together. Lanes of missing rows (aoff
// past the buffer) load no activations. With SCQ (K a multiple of 256) the block scales
// come as in decode_accumulate, a 16-byte load a lane for each chunk pair (through
// wsl), regrouped through the wave's scratch `scr`.
template <int NW, int RS, bool SCQ, int PK = 1>
__device__ __forceinline__ void decode_accumulate_lanes(const uint8_t* const (&wq)[NW], int nvalid, size_t wstride,
                                                  const uint8_t* const (&wsc)[NW], const uint8_t* wsl,
                                                  __amdgpu_buffer_rsrc_t ars, const uint32_t (&aoff)[RS],
                                                  int K, int c_begin, int c_end, bool tail,
                                                  floatx4 (&acc)[NW][RS], unsigned char* scr) {
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
    constexpr int NPM = N / 2 + 1;  // chunk pairs that can hold N chunks
    u32x4 q[N][NW];
    uint32_t sc[N][NW];
    u32x4 scq[SCQ ? NPM : 1];
    u32x4 xv[N][RS][4 / PK];
    const int pf = cb >> 1, pl = (cb + N - 1) >> 1;  // SCQ: first and last pair of the chunks
    if constexpr (SCQ) {
#pragma unroll
      for (int p = 0; p < NPM; ++p) scq[p] = *reinterpret_cast<const u32x4*>(wsl + min(pf + p, pl) * 16);
    }
#pragma unroll
    for (int h = 0; h < N; ++h) {
      const int K0 = (cb + h) * 128;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs[i], (int)(wrow + (uint32_t)(K0 / 2)), 0, kWeightAux);
        q[h][i] = u32x4{v.x, v.y, v.z, v.w};
        if constexpr (!SCQ) sc[h][i] = *reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * grp);
      }
#pragma unroll
      for (int r = 0; r < RS; ++r)
#pragma unroll
        for (int q = 0; q < 4 / PK; ++q) xv[h][r][q] = act_load(ars, aoff[r], K0 + 32 * grp + 8 * act_group<PK>(q, col));
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first product
    if constexpr (SCQ) {
      // pair p's bytes regrouped as in decode_accumulate (1 KB a pair), then chunk h's two
      // bytes of tile i, row col, lane group grp read back
#pragma unroll
      for (int p = 0; p < NPM; ++p)
        *reinterpret_cast<u32x4v*>(scr + p * 1024 + lane * 16) =
            u32x4v{__builtin_amdgcn_perm(scq[p].z, scq[p].x, 0x05040100u), __builtin_amdgcn_perm(scq[p].z, scq[p].x, 0x07060302u),
                   __builtin_amdgcn_perm(scq[p].w, scq[p].y, 0x05040100u), __builtin_amdgcn_perm(scq[p].w, scq[p].y, 0x07060302u)};
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < N; ++h)
#pragma unroll
        for (int i = 0; i < NW; ++i)
          sc[h][i] = *reinterpret_cast<const uint16_t*>(scr + (((cb + h) >> 1) - pf) * 1024 + (i * 16 + col) * 16 +
                                                        grp * 4 + ((cb + h) & 1) * 2);
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int h = 0; h < N; ++h) {
      u32x4 xo[RS][4];  // chunk h's activation operands, shared by the NW tiles
#pragma unroll
      for (int r = 0; r < RS; ++r)
#pragma unroll
        for (int s = 0; s < 4; ++s) xo[r][s] = act_operand<PK>(xv[h][r], s);
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const E4M3Split s0 = e4m3_split_b<0>(sc[h][i]);
        const E4M3Split s1 = e4m3_split_b<1>(sc[h][i]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 wv = nvfp4x8_to_bf16(word_of(q[h][i], s), s < 2 ? s0 : s1);
#pragma unroll
          for (int r = 0; r < RS; ++r) acc[i][r] = mfma16(wv, u32x4_as_bf16x8(xo[r][s]), acc[i][r]);
        }
      }
    }
  };
  int cb = c_begin;
  if constexpr (RS == 1) {
    for (; cb + 4 <= c_end; cb += 4) run(cb, std::integral_constant<int, 4>{});
    switch (c_end - cb) {
      case 3: run(cb, std::integral_constant<int, 3>{}); break;
      case 2: run(cb, std::integral_constant<int, 2>{}); break;
      case 1: run(cb, std::integral_constant<int, 1>{}); break;
      default: break;
    }
  } else {
    // two row sets: two chunks at a time (their activation operands fill the registers)
    for (; cb + 2 <= c_end; cb += 2) run(cb, std::integral_constant<int, 2>{});
    if (cb < c_end) run(cb, std::integral_constant<int, 1>{});
  }
  if (tail) {
    // 32-element chunks: lane group g holds elements K0 + 8g .. K0 + 8g + 7
    for (int K0 = (K / 128) * 128; K0 < K; K0 += 32) {
      u32x4 xv[RS];
#pragma unroll
      for (int r = 0; r < RS; ++r) xv[r] = act_load(ars, aoff[r], K0 + 8 * grp);
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq[i] + (size_t)col * wstride + K0 / 2 + 4 * grp);
        const E4M3Split s = e4m3_split(wsc[i][K0 / 16 + (grp >> 1)]);
        const bf16x8 wv = nvfp4x8_to_bf16(q, s);
#pragma unroll
        for (int r = 0; r < RS; ++r) acc[i][r] = mfma16(wv, u32x4_as_bf16x8(xv[r]), acc[i][r]);
      }
    }
  }
}

// The experts of each row-set count, in index order: list 0 holds the experts of
// 1..16 rows, list 1 those of 17..32. LDS layout of the streaming phase (kSkLdsBytes):
// partial sums of two items [2][waves][4][64] floatx4, the waves' rearrangement
// scratch, then the two lists (expert, first row, row count) and two item slots.
constexpr int kSkRedBytes = 2 * kSkWaves * 4 * 64 * 16;
constexpr int kSkScrOff = kSkRedBytes;
constexpr int kSkListOff = kSkScrOff + kSkWaves * kSkScr;
constexpr int kSkSlotOff = kSkListOff + 2 * kSkMaxE * (4 + 4 + 2);  // row counts 16-bit
constexpr int kSkLdsBytes = kSkSlotOff + 64;

struct SkLds {
  floatx4* red;
  unsigned char* scr;
  int* e[2];
  int* r0[2];
  uint16_t* n[2];
  int* slot;  // [0..1] item slots, [2..3] list lengths
  __device__ explicit SkLds(unsigned char* base) {
    red = reinterpret_cast<floatx4*>(base);
    scr = base + kSkScrOff;
    int* l = reinterpret_cast<int*>(base + kSkListOff);
    uint16_t* ln = reinterpret_cast<uint16_t*>(base + kSkListOff + 2 * 2 * kSkMaxE * 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      e[s] = l + (2 * s + 0) * kSkMaxE;
      r0[s] = l + (2 * s + 1) * kSkMaxE;
      n[s] = ln + s * kSkMaxE;
    }
    slot = reinterpret_cast<int*>(base + kSkSlotOff);
  }
};

// Builds both lists (one wave, offsets read from memory); every thread of the block
// reaches the barrier at the end.
__device__ __forceinline__ void skinny_lists(const int32_t* __restrict__ offsets, int E, const SkLds& L) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int seen[2] = {0, 0};
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int o0 = 0, c = 0;
      if (e < E) {
        o0 = offsets[e];
        c = offsets[e + 1] - o0;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bool pick = c >= 16 * s + 1 && c <= 16 * (s + 1);
        const uint64_t m = __ballot(pick);
        if (pick) {
          const int r = seen[s] + __popcll(m & ((1ull << lane) - 1ull));
          L.e[s][r] = e;
          L.r0[s][r] = o0;
          L.n[s][r] = (uint16_t)c;
        }
        seen[s] += __popcll(m);
      }
    }
    if (lane == 0) {
      L.slot[2] = seen[0];
      L.slot[3] = seen[1];
    }
  }
  __syncthreads();
}

// Tiles of an item: gate/up items hold gu_tiles(RS) 16-feature tiles of gate and of up,
// down items dn_tiles(RS) 16-column tiles, so that an item holds four tile-by-set
// accumulators a wave at RS = 1 and at RS = 2 alike.
constexpr int gu_tiles(int RS) { return RS == 1 ? 2 : 1; }
constexpr int dn_tiles(int RS) { return RS == 1 ? 4 : 2; }
template <int MODE, int RS>
__device__ __forceinline__ int items_per_expert(const FFNArgs& a) {
  return MODE == 0 ? a.f / (16 * gu_tiles(RS)) : (a.d / 16 + dn_tiles(RS) - 1) / dn_tiles(RS);
}

// Partial sums of unit u (tile-by-set) of wave w, item buffer buf, lane `lane`.
__device__ __forceinline__ floatx4& red_at(const SkLds& L, int buf, int w, int u, int lane) {
  return L.red[((buf * kSkWaves + w) * 4 + u) * 64 + lane];
}

// One gate/up item (expert list index u = i / items_per_expert, 16 gu_tiles(RS)
// features): H = bf16_rne(silu(ts_g G) (ts_u U)) for the expert's rows. Ends with the
// block's one barrier of the item: the next item writes the other half of red, and the
// one after it is written only after the next item's barrier, which the summing waves
// reach once their sums here are done.
template <int RS>
__device__ __forceinline__ void skinny_gateup_item(const FFNArgs& a, __amdgpu_buffer_rsrc_t xrs, const SkLds& L,
                                                   int i, int buf) {
  constexpr int FT = gu_tiles(RS), NW = 2 * FT, NU = FT * RS;  // NU: (tile, set) units of the sums
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nfg = items_per_expert<0, RS>(a);
  const int nch = a.d / 128;
  const int u = i / nfg, fg = i - u * nfg;
  const int e = L.e[RS - 1][u], r0 = L.r0[RS - 1][u], ne = L.n[RS - 1][u];
  // tiles: gate features 16t.., t < FT, then up
  const size_t wrow0 = (size_t)e * a.f + (size_t)fg * (16 * FT);
  const uint8_t* wq[NW];
  const uint8_t* wsc[NW];
#pragma unroll
  for (int t = 0; t < FT; ++t) {
    wq[t] = a.gate_q + (wrow0 + 16 * t) * (a.d / 2);
    wq[FT + t] = a.up_q + (wrow0 + 16 * t) * (a.d / 2);
    wsc[t] = a.gate_s + (wrow0 + 16 * t + col) * (a.d / 16);
    wsc[FT + t] = a.up_s + (wrow0 + 16 * t + col) * (a.d / 16);
  }
  // one row set of at most 8 (4) rows, K a multiple of 256: rows packed 2 (4) to a lane row
  const int pk = RS == 1 && a.d % 256 == 0 ? (ne <= 4 ? 4 : ne <= 8 ? 2 : 1) : 1;
  // the activation rows of routed rows 16 r + col (x row sorted_rows[..] / k); packed:
  // row col mod (16 / pk)
  uint32_t aoff[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int row = 16 * r + (col & (16 / pk - 1));
    aoff[r] = row < ne ? (uint32_t)(a.sorted_rows[r0 + row] / a.k) * (uint32_t)(a.d * 2) : kSkOOB;
  }
  // the tensor scales, loaded with the weights (the epilogue needs them)
  const float tg = a.gate_ts[e], tu = a.up_ts[e];
  floatx4 acc[NW][RS];
#pragma unroll
  for (int t = 0; t < NW; ++t)
#pragma unroll
    for (int r = 0; r < RS; ++r) acc[t][r] = floatx4{0.f, 0.f, 0.f, 0.f};
  unsigned char* const scr = L.scr + wave * kSkScr;
  // the scale-load role of this lane (16-byte scale loads): tile (lane / 16) mod NW, row lane mod 16
  const int lt = (lane >> 4) % NW, lr = lane & 15;
  const uint8_t* wsl = (lt < FT ? a.gate_s : a.up_s) + (wrow0 + 16 * (lt % FT) + lr) * (a.d / 16);
  // the two-pair scale loads of the line path: row 32h + lane / 2 of the NW tiles
  const uint8_t* wsl2[NW / 2];
#pragma unroll
  for (int h = 0; h < NW / 2; ++h) {
    const int t = (32 * h + (lane >> 1)) >> 4, rr = (lane >> 1) & 15;
    wsl2[h] = (t < FT ? a.gate_s : a.up_s) + (wrow0 + 16 * (t % FT) + rr) * (a.d / 16);
  }
  const int c_begin = nch * wave / kSkWaves, c_end = nch * (wave + 1) / kSkWaves;
  auto stream = [&](auto pk_c) {
    constexpr int PK = decltype(pk_c)::value;
    if (nch >= 4 * kSkWaves) decode_accumulate<NW, RS, PK>(wq, NW, a.d / 2, wsl2, xrs, aoff, c_begin, c_end, acc, scr);
    else decode_accumulate_lanes<NW, RS, true, PK>(wq, NW, a.d / 2, wsc, wsl, xrs, aoff, a.d, c_begin, c_end, false, acc, scr);
  };
  if (a.d % 256 == 0) {
    if constexpr (RS == 1) {
      if (pk == 4) stream(std::integral_constant<int, 4>{});
      else if (pk == 2) stream(std::integral_constant<int, 2>{});
      else stream(std::integral_constant<int, 1>{});
    } else {
      stream(std::integral_constant<int, 1>{});
    }
  } else {
    decode_accumulate_lanes<NW, RS, false>(wq, NW, a.d / 2, wsc, wsl, xrs, aoff, a.d, c_begin, c_end,
                                           wave == kSkWaves - 1, acc, scr);
  }
#pragma unroll
  for (int t = 0; t < NW; ++t)
#pragma unroll
    for (int r = 0; r < RS; ++r) red_at(L, buf, wave, t * RS + r, lane) = acc[t][r];
  __syncthreads();
  if (wave < NU) {
    // wave w sums unit (feature tile t, row set r): gate partials [t], up [FT + t]
    const int t = wave / RS, r = wave - t * RS;
    if (16 * r + col < ne) {
      floatx4 G = red_at(L, buf, 0, t * RS + r, lane), Uv = red_at(L, buf, 0, (FT + t) * RS + r, lane);
#pragma unroll
      for (int w = 1; w < kSkWaves; ++w) {
        G += red_at(L, buf, w, t * RS + r, lane);
        Uv += red_at(L, buf, w, (FT + t) * RS + r, lane);
      }
      uint32_t hb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hb[q] = bf16_rne(silu_f32(tg * G[q]) * (tu * Uv[q]));
      // lane holds routed row 16 r + col, features 4*grp .. 4*grp + 3 of tile t
      uint2 v;
      v.x = hb[0] | (hb[1] << 16);
      v.y = hb[2] | (hb[3] << 16);
      *reinterpret_cast<uint2*>(a.h + (size_t)(r0 + 16 * r + col) * a.f + (size_t)fg * (16 * FT) + 16 * t + 4 * grp) = v;
    }
  }
}

// One down item (expert list index u = i / items_per_expert, 16 dn_tiles(RS) columns of
// d; the last group of a row may be short): y rows = ts_d (H W_d^T) for the expert's
// rows. Ends with the item's one barrier, as the gate/up item.
template <int RS>
__device__ __forceinline__ void skinny_down_item(const FFNArgs& a, __amdgpu_buffer_rsrc_t hrs, const SkLds& L,
                                                 int i, int buf) {
  constexpr int NW = dn_tiles(RS), NU = NW * RS;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int ndt = a.d / 16;
  const int ndg = items_per_expert<1, RS>(a);
  const int nch = a.f / 128;
  const int u = i / ndg, dg = i - u * ndg;
  const int e = L.e[RS - 1][u], r0 = L.r0[RS - 1][u], ne = L.n[RS - 1][u];
  const int nt = min(NW, ndt - dg * NW);  // tiles of this group
  const uint8_t* wq[NW];
  const uint8_t* wsc[NW];
#pragma unroll
  for (int t = 0; t < NW; ++t) {
    // absent tiles (t >= nt) point at tile 0 and read zeros
    const size_t wrow0 = (size_t)e * a.d + (size_t)(dg * NW + (t < nt ? t : 0)) * 16;
    wq[t] = a.down_q + wrow0 * (a.f / 2);
    wsc[t] = a.down_s + (wrow0 + col) * (a.f / 16);
  }
  // one row set of at most 8 (4) rows, K a multiple of 256: rows packed 2 (4) to a lane row
  const int pk = RS == 1 && a.f % 256 == 0 ? (ne <= 4 ? 4 : ne <= 8 ? 2 : 1) : 1;
  // H rows r0 + 16 r + col; packed: row col mod (16 / pk)
  uint32_t aoff[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int row = 16 * r + (col & (16 / pk - 1));
    aoff[r] = row < ne ? (uint32_t)(r0 + row) * (uint32_t)(a.f * 2) : kSkOOB;
  }
  const float td = a.down_ts[e];  // loaded with the weights (the epilogue needs it)
  floatx4 acc[NW][RS];
#pragma unroll
  for (int t = 0; t < NW; ++t)
#pragma unroll
    for (int r = 0; r < RS; ++r) acc[t][r] = floatx4{0.f, 0.f, 0.f, 0.f};
  unsigned char* const scr = L.scr + wave * kSkScr;
  // the scale-load role of this lane (16-byte scale loads): tile (lane / 16) mod NW
  // (absent tiles: tile 0), row lane mod 16
  const int lt = (lane >> 4) % NW, lr = lane & 15;
  const uint8_t* wsl = a.down_s + ((size_t)e * a.d + (size_t)(dg * NW + (lt < nt ? lt : 0)) * 16 + lr) * (a.f / 16);
  // the two-pair scale loads of the line path: row 32h + lane / 2 of the NW tiles
  const uint8_t* wsl2[NW / 2];
#pragma unroll
  for (int h = 0; h < NW / 2; ++h) {
    const int t = (32 * h + (lane >> 1)) >> 4, rr = (lane >> 1) & 15;
    wsl2[h] = a.down_s + ((size_t)e * a.d + (size_t)(dg * NW + (t < nt ? t : 0)) * 16 + rr) * (a.f / 16);
  }
  const int c_begin = nch * wave / kSkWaves, c_end = nch * (wave + 1) / kSkWaves;
  auto stream = [&](auto pk_c) {
    constexpr int PK = decltype(pk_c)::value;
    if (nch >= 4 * kSkWaves) decode_accumulate<NW, RS, PK>(wq, nt, a.f / 2, wsl2, hrs, aoff, c_begin, c_end, acc, scr);
    else decode_accumulate_lanes<NW, RS, true, PK>(wq, nt, a.f / 2, wsc, wsl, hrs, aoff, a.f, c_begin, c_end, false, acc, scr);
  };
  if (a.f % 256 == 0) {
    if constexpr (RS == 1) {
      if (pk == 4) stream(std::integral_constant<int, 4>{});
      else if (pk == 2) stream(std::integral_constant<int, 2>{});
      else stream(std::integral_constant<int, 1>{});
    } else {
      stream(std::integral_constant<int, 1>{});
    }
  } else {
    decode_accumulate_lanes<NW, RS, false>(wq, nt, a.f / 2, wsc, wsl, hrs, aoff, a.f, c_begin, c_end,
                                           wave == kSkWaves - 1, acc, scr);
  }
#pragma unroll
  for (int t = 0; t < NW; ++t)
#pragma unroll
    for (int r = 0; r < RS; ++r) red_at(L, buf, wave, t * RS + r, lane) = acc[t][r];
  __syncthreads();
  if (wave < NU) {
    // wave w sums unit (column tile t, row set r)
    const int t = wave / RS, r = wave - t * RS;
    if (t < nt && 16 * r + col < ne) {
      floatx4 O = red_at(L, buf, 0, t * RS + r, lane);
#pragma unroll
      for (int w = 1; w < kSkWaves; ++w) O += red_at(L, buf, w, t * RS + r, lane);
      float4 v;
      v.x = td * O[0];
      v.y = td * O[1];
      v.z = td * O[2];
      v.w = td * O[3];
      *reinterpret_cast<float4*>(a.y_rows + (size_t)(r0 + 16 * r + col) * a.d + (size_t)(dg * NW + t) * 16 + 4 * grp) = v;
    }
  }
}

// The streaming phase of a block (MODE 0: gate/up items, 1: down items), the LDS at
// `lds` (kSkLdsBytes, free for this phase). Items of the two-set experts come first
// (the heavier ones), then the one-set experts. With `ctr` set the block takes items
// from that counter (zero when the launch starts; a vector atomic of thread 0, its
// result passed on through an LDS slot that the item's barrier publishes); else it
// takes items blockIdx.x, blockIdx.x + gridDim.x, ...
template <int MODE>
__device__ __forceinline__ void skinny_phase(const FFNArgs& a, unsigned char* lds, uint32_t* ctr) {
  const SkLds L(lds);
  skinny_lists(a.offsets, a.E, L);
  const int n2 = L.slot[3] * items_per_expert<MODE, 2>(a);
  const int total = n2 + L.slot[2] * items_per_expert<MODE, 1>(a);
  // the activation operand as one buffer: x (T d 2 < 2^31 bytes) for gate/up, H
  // (T k f 2 < 2^31 bytes) for down, both checked by the entry points
  const __amdgpu_buffer_rsrc_t ars =
      MODE == 0 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0,
                                                    (int)((uint32_t)a.T * (uint32_t)a.d * 2u), 0x00020000)
                : __builtin_amdgcn_make_buffer_rsrc(a.h, 0, (int)((uint32_t)a.T * (uint32_t)a.k * (uint32_t)a.f * 2u),
                                                    0x00020000);
  auto take = [&]() -> int {
    return (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int it;
  if (ctr) {
    if (threadIdx.x == 0) L.slot[0] = take();
    __syncthreads();
    it = L.slot[0];
  } else {
    it = blockIdx.x;
  }
  int buf = 0;
  while (it < total) {
    if (ctr && threadIdx.x == 0) L.slot[buf ^ 1] = take();  // the next item, read after this item's barrier
    if constexpr (MODE == 0) {
      if (it < n2) skinny_gateup_item<2>(a, ars, L, it, buf);
      else skinny_gateup_item<1>(a, ars, L, it - n2, buf);
    } else {
      if (it < n2) skinny_down_item<2>(a, ars, L, it, buf);
      else skinny_down_item<1>(a, ars, L, it - n2, buf);
    }
    it = ctr ? L.slot[buf ^ 1] : it + (int)gridDim.x;
    buf ^= 1;
  }
}

}  // namespace moe
