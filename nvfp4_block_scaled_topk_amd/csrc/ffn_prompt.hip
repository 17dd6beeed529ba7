// ffn_prompt.hip -- the expert FFN for many tokens (prompt): a grouped GEMM over the
// per-expert row lists.
//
// The pages' prompt path admits routed NVFP4 experts into a grouped GEMM whose store
// scales each row by its expert's tensor scale [FP4-Local checkpoints on DGX Spark,
// §4 Round 1, #545], runs gate, up and SwiGLU as one launch (#766) and copies its
// operands through a multi-stage pipeline in fixed K steps (§4 remaining items, #822).
// Here, on gfx950:
//
//   tile    = (expert e, 128 routed rows of e, 128 features of f)   [gate/up launch:
//             weight rows 0..127 are gate rows, 128..255 the up rows of the same features]
//             (expert e, 128 routed rows of e, 256 columns of d)    [down launch]
//   waves   = 4 (one per SIMD), two workgroups a CU (72 KB of LDS each), so the two
//             workgroups' barriers are independent; wave w owns two 32-row weight
//             fragments (gate and up of the same 32 features, or two 32-column slices
//             of d) over all 128 routed rows
//   MFMA    = v_mfma_f32_32x32x16_bf16, weights as the A operand, activations as B
//   staging = buffer->LDS DMA only (no register staging; out-of-range lanes read zeros,
//             which also pads ragged rows and K tails): activations in double-buffered
//             stages of 64 K elements; packed weight codes in double-buffered
//             blocks of 128 K elements (two activation stages), 64 bytes of codes a
//             weight row; block scales with them (2 bytes a lane), or, when K is a
//             multiple of 256, 16 bytes a lane for 256 K elements (four stages)
//
// Work: one flat list of tiles (row tiles that use all four 32-row fragments first, in
// expert order, then experts' partly filled last tiles by fragments descending; column
// tile fastest) walked by a persistent grid; each block derives the list from
// expert_offsets. Block b works on
// the list positions of "lane" (b mod 8) * (grid / 8) + b / 8, so the blocks a chip's
// XCD receives (round-robin by block index) take consecutive tiles, which share
// activation rows and weight columns in that XCD's L2.
#include "device.hpp"
#include "internal.hpp"
#include "skinny_device.hpp"

#include <type_traits>

namespace moe {

constexpr int kPromptRows = 128;        // routed rows per tile
constexpr int kPromptKC = 64;           // K elements per activation stage
constexpr int kBlockStages = 2;         // weight / scale block = 2 stages = 128 K elements
constexpr int kXStageBytes = 128 * 128;     // 16 KB: 128 rows x 64 bf16
constexpr int kWRowBytes = 64;              // a weight row's codes in one block
constexpr int kWBlockBytes = 256 * kWRowBytes;  // 16 KB: 256 weight rows x 128 codes
// a weight row's block scales in LDS: the 4 scale pairs of one weight block in dword slots, or
// (16-byte scale copies) the 16 scale bytes of 256 K elements, four stages
constexpr int kSRowBytes = 16;
constexpr int kSBlockBytes = 256 * kSRowBytes;  // 4 KB
constexpr int kXOff = 0;
constexpr int kWOff = 2 * kXStageBytes;
constexpr int kSOff = kWOff + 2 * kWBlockBytes;
constexpr int kPromptLdsBytes = kSOff + 2 * kSBlockBytes;  // 72 KB: two workgroups a CU
constexpr int kPromptThreads = 256;     // 4 waves, one per SIMD (two workgroups a CU)
constexpr int kPromptBlocksPerCu = 2;
constexpr int kXDma = 4;                // activation DMA instructions per wave per stage
constexpr int kWSDma = 8;               // weight + scale DMA instructions per wave per block
constexpr int kWDma = 4;                // weight DMA instructions per wave per block
constexpr int kMaxE = 1024;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every record: reads zeros
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One buffer->LDS DMA instruction: lane l writes `size` bytes read at byte offset
// voff + soff of the buffer to LDS address lds_base + l * max(size, 4). soff is a
// wave-uniform offset (the K step); lanes whose voff is kOOB read zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char* lds_base, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma2(__amdgpu_buffer_rsrc_t rs, unsigned char* lds_base, uint32_t voff,
                                     uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)lds_base, 2, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Per-block tile table, heaviest row tiles first. A row tile's cost grows with the
// 32-row activation fragments it uses (1..4); ordering the list by that, so that the
// last, partly filled round of the persistent grid gets the lightest tiles, shortens the
// longest block. Experts with at most kSkinnyRows rows have no tiles (they go to the
// weight-streaming kernels).
//   s_pref[e]: the four-fragment row tiles of experts < e (an expert's full 128-row
//              tiles, and its last tile when it holds more than 96 rows), in expert order;
//   s_part[i]: then the experts whose last tile has 1..96 rows, by fragments descending
//              (3, 2, 1), each in expert order; returns their number.
__device__ int build_tile_table(const int32_t* __restrict__ offsets, int E, int* s_pref, uint16_t* s_part) {
  __shared__ int s_np;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
      const int rem = cnt % kPromptRows;
      const int v = cnt > kSkinnyRows ? cnt / kPromptRows + (rem > 3 * 32 ? 1 : 0) : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (e < E) s_pref[e] = run + incl - v;
      run += __shfl(incl, 63);
    }
    if (lane == 0) s_pref[E] = run;
    int np = 0;
    for (int frags = 3; frags >= 1; --frags) {
      for (int base = 0; base < E; base += 64) {
        const int e = base + lane;
        const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
        const int rem = cnt % kPromptRows;
        const bool pick = cnt > kSkinnyRows && rem > 0 && (rem + 31) / 32 == frags;
        const uint64_t m = __ballot(pick);
        if (pick) s_part[np + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)e;
        np += __popcll(m);
      }
    }
    if (lane == 0) s_np = np;
  }
  __syncthreads();
  return s_np;
}

// largest e with s_pref[e] <= t (s_pref non-decreasing, s_pref[0] = 0)
__device__ __forceinline__ int find_tile_expert(const int* s_pref, int E, int t) {
  int lo = 0, hi = E;  // invariant: s_pref[lo] <= t < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <int MODE>  // 0: gate/up/SwiGLU -> H (bf16); 1: down -> y_rows (fp32)
__global__ __launch_bounds__(kPromptThreads, 2) void ffn_prompt_kernel(FFNArgs a, int n_col_tiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_pref[kMaxE + 1];
  __shared__ uint16_t s_part[kMaxE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int wcol = wave;  // weight-row group of this wave (all 128 routed rows)
  const int l32 = lane & 31, g = lane >> 5;
  const int K = MODE == 0 ? a.d : a.f;  // contraction length
  const int N = MODE == 0 ? a.f : a.d;  // weight rows per matrix
  const int nch = (K + kPromptKC - 1) / kPromptKC;
  // DMA slot -> 16-byte segment: slot s of a 128-byte activation row r holds logical
  // segment s ^ (r & 7); for the 8-lanes-a-row DMA pattern, r & 7 = lane >> 3 and
  // s = lane & 7. Slot s of a 64-byte weight row r holds logical segment
  // s ^ ((r >> 1) & 3); for the 4-lanes-a-row pattern, (r >> 1) & 3 = (lane >> 3) & 3.
  const int dseg = (lane & 7) ^ (lane >> 3);
  const int wseg = (lane & 3) ^ ((lane >> 3) & 3);

  const int n_part = build_tile_table(a.offsets, a.E, s_pref, s_part);
  const int n_full = s_pref[a.E];
  const int total_tiles = (n_full + n_part) * n_col_tiles;
  const int G = gridDim.x;
  const int lid = (G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds : blockIdx.x;

  // Block scales copied 16 bytes a lane (one DMA instruction a wave brings 256 K elements'
  // scales of 64 weight rows, in place of eight 2-byte copies over the same four stages)
  // when K is a multiple of 256 and the scale tensors are 16-byte aligned (then so is
  // every row's 256-K piece).
  const bool sc16 =
      K % 256 == 0 &&
      ((MODE == 0 ? (reinterpret_cast<uintptr_t>(a.gate_s) | reinterpret_cast<uintptr_t>(a.up_s))
                  : reinterpret_cast<uintptr_t>(a.down_s)) & 15) == 0;

  for (int item = lid; item < total_tiles; item += G) {
    const int mt_all = item / n_col_tiles;
    const int ct = item - mt_all * n_col_tiles;
    int e, mt;
    if (mt_all < n_full) {
      e = find_tile_expert(s_pref, a.E, mt_all);
      mt = mt_all - s_pref[e];
    } else {  // an expert's last, partly filled tile
      e = s_part[mt_all - n_full];
      mt = (a.offsets[e + 1] - a.offsets[e]) / kPromptRows;
    }
    const int p0 = a.offsets[e] + mt * kPromptRows;
    const int nrows = min(kPromptRows, a.offsets[e + 1] - p0);
    // 32-row activation fragments in use (0..4)
    const int ntf = min(4, (nrows + 31) >> 5);

    // ---- buffer descriptors (wave-uniform). Weight rows 0..127 of the tile are gate
    // rows and 128..255 up rows (gate/up launch).
    __amdgpu_buffer_rsrc_t xrs, wrs, srs;
    const size_t wslab = (size_t)N * (K / 2), sslab = (size_t)N * (K / 16);
    if (MODE == 0) {
      xrs = make_rsrc(a.x, (uint32_t)((size_t)a.T * a.d * 2));
      const bool up = wave >= 2;  // waves 0-1 stage the gate rows, waves 2-3 the up rows
      wrs = make_rsrc((up ? a.up_q : a.gate_q) + (size_t)e * wslab, (uint32_t)wslab);
      srs = make_rsrc((up ? a.up_s : a.gate_s) + (size_t)e * sslab, (uint32_t)sslab);
    } else {
      xrs = make_rsrc(a.h + (size_t)p0 * a.f, (uint32_t)((size_t)nrows * a.f * 2));
      wrs = make_rsrc(a.down_q + (size_t)e * wslab, (uint32_t)wslab);
      srs = make_rsrc(a.down_s + (size_t)e * sslab, (uint32_t)sslab);
    }

    // ---- per-lane DMA sources. Activation instruction i of wave w covers LDS rows
    // 32w + 8i + lane/8, 8 lanes a row; weight / scale instruction i covers tile rows
    // 64w + 16i + lane/4, 4 lanes a row.
    uint32_t xoff[4], woff[4], soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 32 + i * 8 + (lane >> 3);
      if (r < nrows) {
        const uint32_t rb = MODE == 0 ? (uint32_t)(a.sorted_rows[p0 + r] / a.k) * (uint32_t)(a.d * 2)
                                      : (uint32_t)(r * a.f * 2);
        xoff[i] = rb + dseg * 16;
      } else {
        xoff[i] = kOOB;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 64 + i * 16 + (lane >> 2);
      const int n = MODE == 0 ? ct * 128 + (r & 127) : ct * 256 + r;
      if (n < N) {
        woff[i] = (uint32_t)n * (uint32_t)(K / 2) + wseg * 16;        // 16 B = 32 codes of a block
        soff[i] = (uint32_t)n * (uint32_t)(K / 16) + (lane & 3) * 2;  // scale pair u = lane & 3
      } else {
        woff[i] = soff[i] = kOOB;
      }
    }
    // 16-byte scale copies: lane l of wave w copies tile row 64w + l
    uint32_t soff16;
    {
      const int r = wave * 64 + lane;
      const int n = MODE == 0 ? ct * 128 + (r & 127) : ct * 256 + r;
      soff16 = n < N ? (uint32_t)n * (uint32_t)(K / 16) : kOOB;
    }
    // A stage or block that lies wholly inside K (a wave-uniform test) copies with the
    // lanes' offsets as they are; only a last, half stage (K % 64 == 32) selects per lane.
    auto issue_x = [&](int c) {
      const int K0 = c * kPromptKC;
      unsigned char* buf = smem + kXOff + (c & 1) * kXStageBytes + wave * 32 * 128;
      if (K0 + kPromptKC <= K) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(xrs, buf + i * 1024, xoff[i], K0 * 2);
      } else {
        const bool tail = K0 + 8 * dseg >= K;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(xrs, buf + i * 1024, tail ? kOOB : xoff[i], K0 * 2);
      }
    };
    auto issue_ws = [&](int b) {
      const int K0 = b * kBlockStages * kPromptKC;
      unsigned char* wbuf = smem + kWOff + (b & 1) * kWBlockBytes + wave * 64 * kWRowBytes;
      unsigned char* sbuf = smem + kSOff + (b & 1) * kSBlockBytes + wave * 64 * kSRowBytes;
      if (K0 + kBlockStages * kPromptKC <= K) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(wrs, wbuf + i * 1024, woff[i], K0 / 2);
        if (sc16) {
          // with the first weight block of each pair: the scales of stages 2b .. 2b + 3
          if ((b & 1) == 0)
            dma16(srs, smem + kSOff + ((b >> 1) & 1) * kSBlockBytes + wave * 64 * kSRowBytes, soff16, K0 / 16);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) dma2(srs, sbuf + i * 256, soff[i], K0 / 16);
        }
      } else {  // K is not a multiple of 256 here, so no 16-byte scale copies
        const bool wtail = K0 + 32 * wseg >= K;
        const bool stail = K0 + 32 * (lane & 3) >= K;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(wrs, wbuf + i * 1024, wtail ? kOOB : woff[i], K0 / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma2(srs, sbuf + i * 256, stail ? kOOB : soff[i], K0 / 16);
      }
    };

    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.0f;

    // this wave's weight rows inside the staged 256-row weight tile
    int wrow[2];
    if (MODE == 0) {
      wrow[0] = wcol * 32 + l32;        // gate features ct*128 + wcol*32 + l32
      wrow[1] = 128 + wcol * 32 + l32;  // up rows of the same features
    } else {
      wrow[0] = wcol * 64 + l32;
      wrow[1] = wcol * 64 + 32 + l32;
    }
    const int fbase = MODE == 0 ? ct * 128 + wcol * 32 : ct * 256 + wcol * 64;
    const bool fvalid[2] = {fbase < N, MODE == 0 ? fbase < N : fbase + 32 < N};
    const int nblk = (nch + kBlockStages - 1) / kBlockStages;

    // previous tile: stores drained and every wave done with the LDS buffers
    wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue_ws(0);
    issue_x(0);

    // The K loop, specialised on the number of 32-row activation fragments in use so
    // the MFMA sequence is branch-free (rows past nrows are zeros; weight rows past N
    // decode to zeros and are not stored). Stage c: wait for its activations (and, at a
    // block start, its weight block: issued earlier, so complete too), barrier, issue the
    // next stage's activations and, at a block start, the next weight / scale block;
    // then decode + MFMA. The MFMA step s + 1 operands are read and decoded alongside
    // step s's MFMAs (ping-pong registers).
    auto k_loop = [&](auto ntf_c) {
      constexpr int NTF = decltype(ntf_c)::value;
      for (int c = 0; c < nch; ++c) {
        // loads issued after stage c's activations: the block issued in stage c - 1
        const bool blk_after = c >= 1 && ((c - 1) % kBlockStages) == 0 && (c - 1) / kBlockStages + 1 < nblk;
        // (the block issued then, (c - 1) / 2 + 1, brought 16-byte scale copies if even)
        if (blk_after) {
          if (!sc16) wait_vm<kWSDma>();
          else if ((((c - 1) / kBlockStages + 1) & 1) == 0) wait_vm<kWDma + 1>();
          else wait_vm<kWDma>();
        } else {
          wait_vm<0>();
        }
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        if (c + 1 < nch) issue_x(c + 1);
        if (c % kBlockStages == 0 && c / kBlockStages + 1 < nblk) issue_ws(c / kBlockStages + 1);

        if (NTF == 0) continue;
        const unsigned char* xb = smem + kXOff + (c & 1) * kXStageBytes + l32 * 128;
        const int cs = c % kBlockStages;
        const int blk = (c / kBlockStages) & 1;
        const unsigned char* wb = smem + kWOff + blk * kWBlockBytes;
        // this stage's two scale bytes of lane group g: dword slot 2cs + g of the block's
        // scale pairs, or bytes 4 (c mod 4) + 2g of the 16-byte scale copy
        const unsigned char* sb = smem + kSOff + (sc16 ? ((c >> 2) & 1) : blk) * kSBlockBytes +
                                  (sc16 ? 4 * (c & 3) + 2 * g : (2 * cs + g) * 4);
        // weights of this stage: logical 16-byte segment 2cs + g of the row's 64 bytes
        u32x4 q[2];
        uint32_t sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wrow[i];
          q[i] = *reinterpret_cast<const u32x4*>(wb + r * kWRowBytes + (((2 * cs + g) ^ ((r >> 1) & 3)) * 16));
          sc[i] = *reinterpret_cast<const uint16_t*>(sb + r * kSRowBytes);
        }
        // activation fragment t of MFMA step s: row 32t + l32, logical segment 4g + s
        constexpr int NB = NTF > 0 ? NTF : 1;
        auto read_b = [&](int s, u32x4 (&bv)[NB]) {
          const int off = ((4 * g + s) ^ (l32 & 7)) * 16;
#pragma unroll
          for (int t = 0; t < NTF; ++t) bv[t] = *reinterpret_cast<const u32x4*>(xb + t * 4096 + off);
        };
        auto mfma_step = [&](const u32x4 (&bv)[NB], const bf16x8 (&w)[2]) {
#pragma unroll
          for (int t = 0; t < NTF; ++t) {
            const bf16x8 b = u32x4_as_bf16x8(bv[t]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i][t] = mfma32(w[i], b, acc[i][t]);
          }
        };
        u32x4 x0[NB], x1[NB];
        read_b(0, x0);
        E4M3Split sp[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sp[i][0] = e4m3_split_b<0>(sc[i]);
          sp[i][1] = e4m3_split_b<1>(sc[i]);
        }
        bf16x8 w0[2], w1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) w0[i] = nvfp4x8_to_bf16(q[i].x, sp[i][0]);
        read_b(1, x1);
#pragma unroll
        for (int i = 0; i < 2; ++i) w1[i] = nvfp4x8_to_bf16(q[i].y, sp[i][0]);
        mfma_step(x0, w0);
        read_b(2, x0);
#pragma unroll
        for (int i = 0; i < 2; ++i) w0[i] = nvfp4x8_to_bf16(q[i].z, sp[i][1]);
        mfma_step(x1, w1);
        read_b(3, x1);
#pragma unroll
        for (int i = 0; i < 2; ++i) w1[i] = nvfp4x8_to_bf16(q[i].w, sp[i][1]);
        mfma_step(x0, w0);
        mfma_step(x1, w1);
      }
    };
    switch (ntf) {
      case 0: k_loop(std::integral_constant<int, 0>()); break;
      case 1: k_loop(std::integral_constant<int, 1>()); break;
      case 2: k_loop(std::integral_constant<int, 2>()); break;
      case 3: k_loop(std::integral_constant<int, 3>()); break;
      default: k_loop(std::integral_constant<int, 4>()); break;
    }

    // ---- epilogue. Accumulator r of fragment (i, t): weight row 8*(r/4) + 4*g + r%4 of
    // the fragment, activation row 32t + l32 of the tile.
    if (MODE == 0) {
      if (fvalid[0]) {
        const float tg = a.gate_ts[e], tu = a.up_ts[e];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = t * 32 + l32;
          if (t < ntf && row < nrows) {
            uint16_t* hp = a.h + (size_t)(p0 + row) * a.f + fbase + 4 * g;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              uint32_t hb[4];
#pragma unroll
              for (int r = 0; r < 4; ++r)
                hb[r] = bf16_rne(silu_f32(tg * acc[0][t][4 * qd + r]) * (tu * acc[1][t][4 * qd + r]));
              uint2 v;
              v.x = hb[0] | (hb[1] << 16);
              v.y = hb[2] | (hb[3] << 16);
              *reinterpret_cast<uint2*>(hp + 8 * qd) = v;
            }
          }
        }
      }
    } else {
      const float td = a.down_ts[e];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (!fvalid[i]) continue;
        const int c0 = fbase + 32 * i;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = t * 32 + l32;
          if (t < ntf && row < nrows) {
            float* yp = a.y_rows + (size_t)(p0 + row) * a.d + c0 + 4 * g;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              float4 v;
              v.x = td * acc[i][t][4 * qd + 0];
              v.y = td * acc[i][t][4 * qd + 1];
              v.z = td * acc[i][t][4 * qd + 2];
              v.w = td * acc[i][t][4 * qd + 3];
              *reinterpret_cast<float4*>(yp + 8 * qd) = v;
            }
          }
        }
      }
    }
  }
  // Then the weight-streaming items of the experts with at most kSkinnyRows rows, from
  // the launch's counter: a block that runs out of tiles early (the last round of
  // tiles is partly filled) starts on them at once. The LDS is theirs once every wave
  // is done with the last tile.
  __syncthreads();
  static_assert(kSkLdsBytes <= kPromptLdsBytes, "the streaming items reuse the tiles' LDS");
  skinny_phase<MODE>(a, smem, a.work_ctr + MODE);
}

__global__ void zero_words_kernel(uint32_t* w, int n) {
  if ((int)threadIdx.x < n) w[threadIdx.x] = 0u;
}

hipError_t launch_ffn_prompt(const FFNArgs& a, hipStream_t stream) {
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&ffn_prompt_kernel<0>), kPromptLdsBytes);
  if (err == hipSuccess) err = ensure_dynamic_lds(reinterpret_cast<const void*>(&ffn_prompt_kernel<1>), kPromptLdsBytes);
  if (err != hipSuccess) return err;
  int ncu = 0;
  err = device_cu_count(ncu);
  if (err != hipSuccess) return err;
  // a persistent grid of two blocks a CU: tiles first, then the streaming items
  const int grid = kPromptBlocksPerCu * ncu;
  const int ct_gu = (a.f + 127) / 128;
  const int ct_dn = (a.d + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, a.work_ctr, 2);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_prompt_kernel<0>, dim3(grid), dim3(kPromptThreads), kPromptLdsBytes, stream, a, ct_gu);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ffn_prompt_kernel<1>, dim3(grid), dim3(kPromptThreads), kPromptLdsBytes, stream, a, ct_dn);
  return hipGetLastError();
}

}  // namespace moe
