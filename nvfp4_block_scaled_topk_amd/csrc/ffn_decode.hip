// ffn_decode.hip -- the expert FFN for a few tokens (decode): weight streaming.
//
// With a few tokens every selected expert has at most a handful of rows, and the
// layer's time is the time to read the selected experts' weight bytes once. The pages
// read each selected expert once for all of its rows [FP4-Local checkpoints on DGX
// Spark, §4 Round 1, #808]; here one 16x16x32 bf16 MFMA tile covers all of an
// expert's rows (<= 16), so each weight byte is read once whatever the row count.
//
// MFMA mapping (per wave and 16-row weight tile): 16 weight rows (output features) x
// up to 16 routed rows. In the MFMA operand a lane holds 32 E2M1 codes of one weight
// row: within a 128-element chunk, lane group g (lane / 16) holds elements
// [32g, 32g + 32) and MFMA step s takes elements 32g + 8s .. 32g + 8s + 7 of every
// group -- a permutation of the contraction index, applied identically to the
// activation operand, so the sums are unchanged. The codes are not loaded in that
// layout, which would make every load touch 64 bytes of 16 rows: a load covers a pair
// of chunks (128 bytes, one cache line) of 8 rows, and the wave rearranges each pair
// through its LDS scratch into the operand layout. Block scales come in whole rows too:
// a gate/up item's 32 scale rows of each matrix (contiguous in memory) by DMA into
// LDS, a down tile's 16 scale rows with one 16-byte load a lane.
//
// One launch does gate, up, SwiGLU [same page, §4 Round 1, #766] and the down product,
// with 8-wave blocks and two kinds of work item:
//   gate/up item (touched expert u, 32 features): waves 0-3 take the gate and up tiles
//     of features 0..15, waves 4-7 those of 16..31, each wave a quarter of K = d. A wave
//     issues every code load of its share at once, while the block copies the item's
//     scale rows into LDS by buffer->LDS DMA (every token's activation row came into
//     LDS the same way at the start of the launch). Waves 0 and 4 add the four K
//     quarters of their half in LDS in order, form H = bf16_rne(silu(ts_g * G) *
//     (ts_u * U)) and store it;
//   down item (u, 128 columns of d): wave w owns a 16-column tile over all of K = f.
//     A block loads the weight codes and scales of its first down item into registers
//     as soon as its last gate/up item is done (or at the start, if it has none), so
//     those bytes are in flight while the other gate/up items finish. It then copies H's rows of u
//     into LDS, waiting until all of them are there, and finishes the products with the
//     weights already in hand.
// H in the workspace is self-validating: every 64-bit word holds two bf16 values and
// the call's 32-bit tag, written and read as one device-scope atomic access. A reader
// that sees the current tag sees the values stored with it, so the producer never
// waits for its stores and there are no separate completion flags. Every call writes
// every H word it reads, so words left from earlier calls carry older tags.
// Block b takes gate/up items b, b + G, ... and then down items G-1-b, 2G-1-b, ... (the
// blocks without a gate/up item take the extra down items); every block finishes its
// gate/up items before it waits, and the grid is sized to what the device holds at once,
// so normally every awaited H word belongs to a running block. Correctness does not rest
// on that: a down item whose H slices are still missing after `steal_after` polls
// computes the missing gate/up items of its expert itself (the same code on the same
// inputs, so the same bits; a word written twice is written with the same value), so no
// wait depends on a block that has not started (other work on the GPU, another stream).
// As a last guard the full read gives up after `give_up` polls: the block then writes
// NaN rows and raises the library's asynchronous status flag (moe_async_status).
#include "device.hpp"
#include "internal.hpp"
#include "route_device.hpp"

namespace moe {

constexpr int kDecThreads = 512;               // 8 waves
constexpr int kDecWaves = 8;
constexpr int kDecMaxE = 1024;
constexpr int kDecMaxAssign = kDecodeMaxRows * 32;  // T * k
constexpr int kDecMaxTouched = kDecMaxAssign;      // min(E, T * k)
constexpr int kGUFeat = 32;                     // features of a gate/up item
constexpr int kDCols = 16 * kDecWaves;          // columns of d in a down item
constexpr int kDownPairs = 3;                   // W_down chunk pairs (2 x 128 K) a wave holds before its wait
constexpr int kScrWave = 4096;                  // LDS a wave uses to rearrange its weight codes
constexpr int kDecMaxDeferred = 64;             // down items a block may take (the grid is sized for it)
constexpr int kLayerMaxAssign = kDecodeMaxRows * kFusedRouteMaxK;  // T * k of a launch that routes
constexpr int kCtrWords = kLayerCounterBytes / 8;                  // arrival counters: one a 128-byte line

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every record: reads zeros
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dec_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Workgroup barrier without the memory fence of __syncthreads() (which waits for every
// outstanding load); the empty asm keeps the compiler from moving memory accesses
// across it. LDS written before it (stores, or DMA covered by an explicit vmcnt wait)
// is visible after it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS stores done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// H word: bf16 values of features 2i, 2i+1 and the call's tag
__device__ __forceinline__ unsigned long long h_word(uint32_t lo, uint32_t hi, uint32_t tag) {
  return (unsigned long long)(lo | (hi << 16)) | ((unsigned long long)tag << 32);
}

// Set (atomic or, vector memory) when a wait of a few-token launch gives up; read and
// cleared by moe_async_status.
__device__ unsigned int g_async_status;

struct DownPrefetch {
  u32x4 q[kDownPairs][2];  // [pair][rows 0-7 / 8-15], as loaded
  u32x4 sc;                // 16 bytes of the wave's 16 scale rows (f bytes, contiguous)
};

// Dynamic LDS: the activation rows of one expert (gate/up phase; row stride
// xstride bytes) and later its H rows (down phase; row stride (f + 8) bf16), then
// kScrWave bytes per wave for rearranging weight codes (which also hold the gate/up
// partial sums and, at the start, the expert offsets). Both row strides are 16 bytes
// past a multiple of the bank period, which staggers the banks of the 16 rows an MFMA
// operand read touches.
__device__ __forceinline__ int dec_xstride(int d) { return (d * 2 + 1023) / 1024 * 1024 + 16; }
__host__ __device__ __forceinline__ size_t dec_row_region(int T, int d, int f) {
  const size_t xs = (size_t)((d * 2 + 1023) / 1024 * 1024 + 16);
  const size_t hs = (size_t)(f + 8) * sizeof(uint16_t);
  const size_t r = (size_t)T * (xs > hs ? xs : hs);
  return (r + 15) / 16 * 16;
}

// Expert e's slab of a weight tensor and its tensor scale: e < E a routed expert, e == E
// the shared expert (a one-launch layer with a shared expert)
__device__ __forceinline__ const uint8_t* eslab(const uint8_t* routed, const uint8_t* shared, int e, int E,
                                                size_t slab) {
  return e < E ? routed + (size_t)e * slab : shared;
}
__device__ __forceinline__ float ets(const float* routed, const float* shared, int e, int E) {
  return e < E ? routed[e] : shared[0];
}

// Everything a gate/up item needs besides the kernel arguments: the block's LDS regions
// and index lists, the H words and the call's tag.
struct GateUpCtx {
  unsigned char* s_dyn;      // the activation rows (row t at t * xstride)
  unsigned char* s_scr;      // kScrWave bytes a wave
  unsigned char* s_sc;       // the item's block scales
  const int* s_tok;          // token of each routed row
  const int* s_e;            // touched experts: id, first row, row count
  const int* s_r0;
  const int* s_n;
  unsigned long long* hw;    // H as tagged words
  uint32_t tag;
};

// One gate/up item (touched expert u = i / nfg, features 32 (i % nfg) ..): the block's
// 8 waves compute the gate and up tiles, wave pairs of K quarters are summed in a fixed
// order, and H = bf16_rne(silu(ts_g G) (ts_u U)) is stored as tagged words. Ends after
// the H stores (the caller places the barrier). The kernel inlines it where a block does
// its own items and where it computes a missing item of another block: the same code, so
// the same bits.
__device__ __forceinline__ void gate_up_item(const FFNArgs& a, const GateUpCtx& cx, int i) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nfg = a.f / kGUFeat;
  const int nchG = a.d / 128;
  const int half = wave >> 2, kq = wave & 3;  // 16-feature half of the item, quarter of K
  const int kc0 = nchG * kq / 4, kc1 = nchG * (kq + 1) / 4;
  const bool gtail = kq == 3;
  const int xstride = dec_xstride(a.d);
  constexpr int kB = 4;  // chunks a wave loads at once
  unsigned char* const s_dyn = cx.s_dyn;
  unsigned char* const s_scr = cx.s_scr;
  unsigned char* const s_sc = cx.s_sc;
  const int* const s_tok = cx.s_tok;
  const int* const s_e = cx.s_e;
  const int* const s_r0 = cx.s_r0;
  const int* const s_n = cx.s_n;
  unsigned long long* const hw = cx.hw;
  const uint32_t tag = cx.tag;
  const int u = i / nfg, fg = i - u * nfg;
  const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
  // weight rows through buffer descriptors (expert slab base in scalar registers,
  // a 32-bit row offset per lane)
  const size_t slab = (size_t)a.f * (a.d / 2), sslab = (size_t)a.f * (a.d / 16);
  const __amdgpu_buffer_rsrc_t qrs[2] = {dec_rsrc(eslab(a.gate_q, a.sh_gate_q, e, a.E, slab), (uint32_t)slab),
                                         dec_rsrc(eslab(a.up_q, a.sh_up_q, e, a.E, slab), (uint32_t)slab)};
  const __amdgpu_buffer_rsrc_t srs[2] = {dec_rsrc(eslab(a.gate_s, a.sh_gate_s, e, a.E, sslab), (uint32_t)sslab),
                                         dec_rsrc(eslab(a.up_s, a.sh_up_s, e, a.E, sslab), (uint32_t)sslab)};
  // MFMA layout: lane (grp, col) works on weight row `frow` of the item
  const uint32_t frow = (uint32_t)(fg * kGUFeat + half * 16 + col);
  // the item's scales in LDS: [gate / up][32 rows][d / 16 bytes]
  const int srow = a.d / 16, sbytes = kGUFeat * srow;
  const unsigned char* const my_sc = s_sc + (half * 16 + col) * srow;
  // Code loads run along the rows instead: a load covers a pair of chunks (128 bytes,
  // one cache line) of 8 rows -- lane group grp8 = lane / 8 takes row 8i + grp8 and
  // lane lane % 8 its 16-byte segment -- rather than 64 bytes of 16 rows. The wave
  // rearranges each pair into the MFMA layout through its LDS scratch.
  const int grp8 = lane >> 3, seg8 = lane & 7;
  const uint32_t qoff = (uint32_t)(fg * kGUFeat + half * 16 + grp8) * (uint32_t)(a.d / 2);
  unsigned char* const scr = s_scr + wave * kScrWave;
  floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  u32x4 lq[2][2][2];  // [pair][gate / up][rows 0-7 / 8-15], as loaded
  // A batch always issues kB chunks of loads (a chunk past the wave's range repeats
  // chunk c), so the number of loads in flight is a constant and every wait below is
  // exact. Per pair: gate codes, then up.
  auto load_batch = [&](int c) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int lc = c + 2 * pr + (seg8 >> 2) < kc1 ? c + 2 * pr + (seg8 >> 2) : c;  // this lane's chunk
      const int lb = (int)qoff + lc * 64 + 16 * (seg8 & 3);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(qrs[m], lb, i * 8 * (a.d / 2), kWeightAux);
          lq[pr][m][i] = u32x4{v.x, v.y, v.z, v.w};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the item's scales (32 whole scale rows of gate and of up, contiguous in memory)
  // and the activation rows of expert u by DMA first, then the first batch of
  // weights; waiting for all but the weight loads leaves those in flight, and each
  // pair of chunks is decoded as soon as its own loads have landed
  for (int qi = (int)threadIdx.x; qi < 2 * sbytes / 16; qi += kDecThreads) {
    const int m = qi >= sbytes / 16;
    const uint32_t off = (uint32_t)(fg * kGUFeat) * (uint32_t)srow + (uint32_t)(qi * 16 - m * sbytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs[m], (lds_void_ptr)(s_sc + (qi - lane) * 16), 16, off, 0, 0, kWeightAux);
  }
  load_batch(kc0);
  wait_vm<8>();  // the scale DMA has landed; the batch's 8 code loads may still be in flight
  // a bare barrier: __syncthreads() would also wait for the weight loads
  lds_barrier();
  const bool valid = col < ne;
  // Lanes of routed rows >= ne read whatever the LDS row holds: MFMA output column j
  // depends only on operand column j, and those columns are never stored.
  // the activation row of routed row col (rows >= ne: the expert's last row's token)
  const unsigned char* xrow = s_dyn + s_tok[r0 + min(col, ne - 1)] * xstride;
  auto xop = [&](int k0) -> bf16x8 { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4v*>(xrow + k0 * 2)); };
  // Rearrange a pair: piece (row r, 16-byte segment s) of matrix m sits at
  // m * 2048 + r * 128 + ((s + r / 2) mod 8) * 16 in the wave's scratch, so the stores
  // (two rows per 16 lanes) and the loads (a segment of 16 rows per 16 lanes) each hit
  // 16 distinct 16-byte bank groups. LDS operations of one wave complete in order.
  auto compute_pair = [&](int c, int pr) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * i + grp8;
        *reinterpret_cast<u32x4v*>(scr + m * 2048 + r * 128 + ((seg8 + (r >> 1)) & 7) * 16) =
            u32x4v{lq[pr][m][i].x, lq[pr][m][i].y, lq[pr][m][i].z, lq[pr][m][i].w};
      }
    }
    __builtin_amdgcn_wave_barrier();
    u32x4 q[2][2];  // [gate / up][chunk of the pair], MFMA layout
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // chunk j of the pair, row col: segments 4j .. 4j + 3, lane group grp takes 4j + grp
        const u32x4v v =
            *reinterpret_cast<const u32x4v*>(scr + m * 2048 + col * 128 + ((4 * j + grp + (col >> 1)) & 7) * 16);
        q[m][j] = u32x4{v.x, v.y, v.z, v.w};
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int h = 2 * pr + j;
      if (c + h < kc1) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t sc = *reinterpret_cast<const uint16_t*>(my_sc + m * sbytes + (c + h) * 8 + 2 * grp);
          const E4M3Split s0 = e4m3_split_b<0>(sc);
          const E4M3Split s1 = e4m3_split_b<1>(sc);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[m] = mfma16(nvfp4x8_to_bf16(word_of(q[m][j], s), s < 2 ? s0 : s1),
                                xop((c + h) * 128 + 32 * grp + 8 * s), acc[m]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_batch = [&](int c) {
    compute_pair(c, 0);
    compute_pair(c, 1);
  };
  // the first batch straight after its loads (a separate copy keeps the compiler's
  // per-load waits exact), then any further batches
  compute_batch(kc0);
  for (int c = kc0 + kB; c < kc1; c += kB) {
    load_batch(c);
    compute_batch(c);
  }
  if (gtail) {
    // 32-element chunks past the last full 128: lane group g holds K0 + 8g .. K0 + 8g + 7
    for (int K0 = nchG * 128; K0 < a.d; K0 += 32) {
      const bf16x8 xv = xop(K0 + 8 * grp);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t qq = __builtin_amdgcn_raw_buffer_load_b32(qrs[m], (int)(frow * (uint32_t)(a.d / 2) + 4 * grp),
                                                               K0 / 2, kWeightAux);
        const uint32_t sv = my_sc[m * sbytes + K0 / 16 + (grp >> 1)];
        acc[m] = mfma16(nvfp4x8_to_bf16(qq, e4m3_split(sv)), xv, acc[m]);
      }
    }
  }
  // partial sums through the waves' scratch: [wave][gate / up][lane]
  floatx4* const red = reinterpret_cast<floatx4*>(s_scr);
  constexpr int kRedWave = kScrWave / (int)sizeof(floatx4);
  red[wave * kRedWave + lane] = acc[0];
  red[wave * kRedWave + 64 + lane] = acc[1];
  __syncthreads();
  if (kq == 0) {
    if (valid) {
      floatx4 Gs = red[wave * kRedWave + lane], Us = red[wave * kRedWave + 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        Gs += red[(wave + w) * kRedWave + lane];
        Us += red[(wave + w) * kRedWave + 64 + lane];
      }
      const float tg = ets(a.gate_ts, a.sh_gate_ts, e, a.E), tu = ets(a.up_ts, a.sh_up_ts, e, a.E);
      uint32_t hb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(silu_f32(tg * Gs[r]) * (tu * Us[r]));
      // lane holds routed row `col`, features 4*grp .. 4*grp + 3 of the half
      unsigned long long* dst = hw + ((size_t)(r0 + col) * a.f + fg * kGUFeat + half * 16 + 4 * grp) / 2;
      __hip_atomic_store(dst, h_word(hb[0], hb[1], tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1, h_word(hb[2], hb[3], tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The same gate/up item with plain loads: every operand loaded in the MFMA layout
// straight from memory (codes 16 bytes a lane, scales 2 bytes a lane) instead of whole
// cache lines rearranged in LDS, no batching. Slower, and much lighter on registers; the
// MFMA sequence, its operands and the reduction are those of gate_up_item, so the H bits
// are the same. Used only by a down item that computes a missing item of another block.
__device__ __forceinline__ void gate_up_item_plain(const FFNArgs& a, const GateUpCtx& cx, int i) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nfg = a.f / kGUFeat;
  const int nchG = a.d / 128;
  const int half = wave >> 2, kq = wave & 3;
  const int kc0 = nchG * kq / 4, kc1 = nchG * (kq + 1) / 4;
  const int u = i / nfg, fg = i - u * nfg;
  const int e = cx.s_e[u], r0 = cx.s_r0[u], ne = cx.s_n[u];
  const int frow = fg * kGUFeat + half * 16 + col;  // this lane's weight row
  const size_t slab = (size_t)a.f * (a.d / 2), sslab = (size_t)a.f * (a.d / 16);
  const uint8_t* const q[2] = {eslab(a.gate_q, a.sh_gate_q, e, a.E, slab) + (size_t)frow * (a.d / 2),
                               eslab(a.up_q, a.sh_up_q, e, a.E, slab) + (size_t)frow * (a.d / 2)};
  const uint8_t* const sc[2] = {eslab(a.gate_s, a.sh_gate_s, e, a.E, sslab) + (size_t)frow * (a.d / 16),
                                eslab(a.up_s, a.sh_up_s, e, a.E, sslab) + (size_t)frow * (a.d / 16)};
  const unsigned char* xrow = cx.s_dyn + cx.s_tok[r0 + min(col, ne - 1)] * dec_xstride(a.d);
  auto xop = [&](int k0) -> bf16x8 { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4v*>(xrow + k0 * 2)); };
  floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int c = kc0; c < kc1; ++c) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4 w = ldg_u32x4(q[m] + c * 64 + 16 * grp);
      const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sc[m] + c * 8 + 2 * grp);
      const E4M3Split s0 = e4m3_split_b<0>(s2);
      const E4M3Split s1 = e4m3_split_b<1>(s2);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[m] = mfma16(nvfp4x8_to_bf16(word_of(w, s), s < 2 ? s0 : s1), xop(c * 128 + 32 * grp + 8 * s), acc[m]);
    }
  }
  if (kq == 3) {
    for (int K0 = nchG * 128; K0 < a.d; K0 += 32) {
      const bf16x8 xv = xop(K0 + 8 * grp);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t qq = *reinterpret_cast<const uint32_t*>(q[m] + K0 / 2 + 4 * grp);
        const uint32_t sv = sc[m][K0 / 16 + (grp >> 1)];
        acc[m] = mfma16(nvfp4x8_to_bf16(qq, e4m3_split(sv)), xv, acc[m]);
      }
    }
  }
  floatx4* const red = reinterpret_cast<floatx4*>(cx.s_scr);
  constexpr int kRedWave = kScrWave / (int)sizeof(floatx4);
  red[wave * kRedWave + lane] = acc[0];
  red[wave * kRedWave + 64 + lane] = acc[1];
  __syncthreads();
  if (kq == 0 && col < ne) {
    floatx4 Gs = red[wave * kRedWave + lane], Us = red[wave * kRedWave + 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      Gs += red[(wave + w) * kRedWave + lane];
      Us += red[(wave + w) * kRedWave + 64 + lane];
    }
    const float tg = ets(a.gate_ts, a.sh_gate_ts, e, a.E), tu = ets(a.up_ts, a.sh_up_ts, e, a.E);
    uint32_t hb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(silu_f32(tg * Gs[r]) * (tu * Us[r]));
    unsigned long long* dst = cx.hw + ((size_t)(r0 + col) * a.f + fg * kGUFeat + half * 16 + 4 * grp) / 2;
    __hip_atomic_store(dst, h_word(hb[0], hb[1], cx.tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 1, h_word(hb[2], hb[3], cx.tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Under HIP graph capture a kernel argument is frozen for every replay, so a captured
// call takes its tag from the workspace instead: this one-thread kernel, captured just
// before the FFN launch, advances the word there (tags of captured calls have the top bit
// set, those of direct calls clear, so the two never meet; never 0).
__global__ void advance_epoch_kernel(uint32_t* epoch) {
  if (threadIdx.x == 0) {
    const uint32_t e = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t n = 0x80000000u | ((e + 1u) & 0x7FFFFFFFu);
    if (n == 0x80000000u) n = 0x80000001u;
    __hip_atomic_store(epoch, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ __launch_bounds__(kDecThreads, 4) void ffn_decode_kernel(FFNArgs a, uint32_t tag_arg, uint32_t steal_after,
                                                                    uint32_t give_up) {
  // this call's tag: the argument, or under graph capture the word the epoch kernel wrote
  const uint32_t tag = a.epoch ? __builtin_amdgcn_readfirstlane(
                                     __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                               : tag_arg;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  __shared__ int s_tok[kDecMaxAssign];
  __shared__ int s_e[kDecMaxTouched], s_r0[kDecMaxTouched], s_n[kDecMaxTouched];
  __shared__ int s_U, s_timeout;
  __shared__ uint32_t s_missing;   // a down item's H slices still missing (bit g: slice g)
  __shared__ int s_def[kDecMaxDeferred];  // down items left for the end (their H not all there)
  // one-launch layer: each assignment's row and weight (from the routing), and the tokens
  // whose column tile the block combines after a down item
  __shared__ int s_rowof[kLayerMaxAssign];
  __shared__ float s_wt[kLayerMaxAssign];
  __shared__ int s_done[kDecodeMaxRows];
  __shared__ int s_ndone;
  unsigned char* const s_scr = s_dyn + dec_row_region(a.T, a.d, a.f);
  unsigned char* const s_sc = s_scr + kDecWaves * kScrWave;  // a gate/up item's block scales
  int* s_off = reinterpret_cast<int*>(s_scr);
  static_assert(kDecWaves * kScrWave >= (int)sizeof(int) * (kDecMaxE + 1), "offsets fit the scratch");
  static_assert(kScrWave >= 2 * 64 * (int)sizeof(floatx4), "partial sums fit a wave's scratch");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;

  // ---- every token's activation row into LDS (row t at t * xstride; used by all of the
  // block's gate/up items), the touched experts and the token of every routed row: one
  // round trip
  const __amdgpu_buffer_rsrc_t xrs = dec_rsrc(a.x, (uint32_t)(a.T * a.d * 2));
  // the activation rows by buffer->LDS DMA, issued by waves first_wave.. (a 1 KB copy
  // an instruction); the caller waits for them
  auto copy_x_rows = [&](int first_wave) {
    const int xs = dec_xstride(a.d), ipr = (a.d * 2 + 1023) / 1024;  // 1 KB DMA instructions a row
    const int nw = kDecWaves - first_wave;
    for (int qi = wave - first_wave; qi < a.T * ipr; qi += nw) {
      if (qi < 0) break;
      const int r = qi / ipr, jj = qi - r * ipr;
      const int within = jj * 1024 + lane * 16;
      const uint32_t voff = within < a.d * 2 ? (uint32_t)r * (uint32_t)(a.d * 2) + within : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void_ptr)(s_dyn + r * xs + jj * 1024), 16, voff, 0, 0, 0);
    }
  };
  // waves 0-3 load the routing inputs (or route the tokens: a 16-lane row a token) and
  // waves 4-7 issue these copies, so that the loads the prologue waits on do not queue
  // behind them (a wave's loads complete in order)
  copy_x_rows(kDecWaves / 2);
  const int nA = a.T * a.k;
  const bool fold = a.out != nullptr;             // the launch also combines (with routing only)
  const bool has_sh = a.sh_gate_q != nullptr;     // a shared expert: touched expert U, rows nA ..
  bool listed = false;  // the touched experts (s_e, s_r0, s_n, s_U) already listed; block-uniform
  if (a.logits) {
    // Route the tokens here (every block, redundantly: T <= 16 tokens of E <= 256 logits):
    // the same top-k and weights as the routing kernel (one 16-lane row a token, waves
    // 0-3), then the stable row lists. Block 0 writes the routing outputs. Work arrays
    // live in the waves' scratch (free until the gate/up items start): offsets at 0,
    // counts at 1028, experts of the assignments at 1288, ranks at 1800 (ints).
    int* const s_cnt = s_off + 1028;
    int* const s_aid = s_off + 1288;
    int* const s_rnk = s_off + 1800;
    static_assert(kDecWaves * kScrWave >= (int)sizeof(int) * (1800 + kDecMaxAssign), "routing arrays fit the scratch");
    const bool one_wave = nA <= 64;  // the row lists from one wave's ballots (below)
    if (!one_wave)
      for (int e = threadIdx.x; e < a.E; e += kDecThreads) s_cnt[e] = 0;
    {
      // up to 4 tokens: one wave a token (waves 0-3); more: a 16-lane row a token, four
      // tokens a wave
      const bool by_wave = a.T <= 4;
      const int gl = by_wave ? lane : lane & 15;
      const int t = by_wave ? wave : wave * 4 + (lane >> 4);
      const size_t ld = a.logits_ld > 0 ? (size_t)a.logits_ld : (size_t)a.E;
      if (t < a.T && (!by_wave || wave < 4)) {
        float my_w;
        int my_i;
        const float* const lrow = a.logits + (size_t)t * ld;
        if (by_wave) {
          if (a.E <= 64) wave_topk<1>(lrow, a.E, a.k, lane, my_i, my_w);
          else if (a.E <= 128) wave_topk<2>(lrow, a.E, a.k, lane, my_i, my_w);
          else wave_topk<4>(lrow, a.E, a.k, lane, my_i, my_w);
        } else if (a.E <= 128) {
          row_topk<8>(lrow, nullptr, a.E, a.k, gl, 0, my_i, my_w);
        } else {
          row_topk<16>(lrow, nullptr, a.E, a.k, gl, 0, my_i, my_w);
        }
        if (gl < a.k) {
          s_aid[t * a.k + gl] = my_i;
          s_rnk[t * a.k + gl] = t;  // the assignment's token (the one-wave lists below; else overwritten)
          if (fold) s_wt[t * a.k + gl] = my_w;
          if (blockIdx.x == 0) {
            if (a.ids_out) a.ids_out[t * a.k + gl] = my_i;
            if (a.w_out) a.w_out[t * a.k + gl] = my_w;
          }
        }
      }
    }
    // LDS-only barriers inside the routing (the copies and the first block's stores are
    // covered by the full barrier that ends the prologue)
    lds_barrier();
    if (one_wave) {
      // At most 64 assignments: lane a of wave 0 holds assignment a (expert e) and finds,
      // by one ballot per bit of the expert index from the top, the lanes holding the same
      // expert and those holding a smaller one. Its row in the expert-grouped order is
      // (assignments of smaller experts) + (earlier assignments of its own): the stable row
      // lists. The first assignment of each expert lists it among the touched experts, at
      // the number of distinct smaller experts.
      if (wave == 0) {
        const int e = lane < nA ? s_aid[lane] : -1;
        const int tok = lane < nA ? s_rnk[lane] : 0;
        const bool valid = e >= 0;
        // the ballots first (independent of each other), then each lane's masks from the
        // top bit down (expert indices < 256 on this path: 8 bits)
        uint64_t bal[8];
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) bal[bit] = __ballot(valid && ((e >> bit) & 1));
        uint64_t same = __ballot(valid), less = 0ull;
#pragma unroll
        for (int bit = 7; bit >= 0; --bit) {
          const bool one = valid && ((e >> bit) & 1);
          less |= one ? (same & ~bal[bit]) : 0ull;
          same &= one ? bal[bit] : ~bal[bit];
        }
        const int before = __popcll(same & ((1ull << lane) - 1ull));
        const int nless = __popcll(less);
        const int p = nless + before;
        const bool first = valid && before == 0;
        const uint64_t firsts = __ballot(first);
        if (valid) {
          s_tok[p] = tok;
          if (fold) s_rowof[lane] = p;
          if (blockIdx.x == 0) {
            if (a.sorted_rows_out) a.sorted_rows_out[p] = lane;
            if (a.row_of_out) a.row_of_out[lane] = p;
          }
        }
        if (first) {
          const int u = __popcll(firsts & less);
          s_e[u] = e;
          s_r0[u] = nless;
          s_n[u] = __popcll(same);
        }
        const int U0 = __popcll(firsts);
        if (has_sh)  // the shared expert: one more touched expert, every token a row (nA + t)
          for (int t = lane; t < a.T; t += 64) s_tok[nA + t] = t;
        if (lane == 0) {
          if (has_sh) {
            s_e[U0] = a.E;
            s_r0[U0] = nA;
            s_n[U0] = a.T;
          }
          s_U = U0 + (has_sh ? 1 : 0);
          s_timeout = 0;
        }
      }
      if (blockIdx.x == 0 && a.offsets_out)
        for (int e2 = threadIdx.x; e2 <= a.E; e2 += kDecThreads) {
          int c = 0;
          for (int i = 0; i < nA; ++i) c += s_aid[i] < e2 ? 1 : 0;
          a.offsets_out[e2] = c;
        }
      listed = true;
    } else {
    // the rank of each assignment among the earlier ones of its expert (ballots, as the
    // routing kernel), the per-expert counts and their exclusive scan
    if (wave == 0) wave_rank_assignments(s_aid, nA, s_rnk, s_cnt, lane);
    lds_barrier();
    block_exclusive_scan(s_cnt, s_off, a.E);  // ends with a barrier
    for (int i = threadIdx.x; i < nA; i += kDecThreads) {
      const int p = s_off[s_aid[i]] + s_rnk[i];
      s_tok[p] = i / a.k;
      if (fold) s_rowof[i] = p;
      if (blockIdx.x == 0) {
        if (a.sorted_rows_out) a.sorted_rows_out[p] = i;
        if (a.row_of_out) a.row_of_out[i] = p;
      }
    }
    if (blockIdx.x == 0 && a.offsets_out)
      for (int e = threadIdx.x; e <= a.E; e += kDecThreads) a.offsets_out[e] = s_off[e];
    // the shared expert's rows: row nA + t is token t
    if (has_sh)
      for (int t = threadIdx.x; t < a.T; t += kDecThreads) s_tok[nA + t] = t;
    }
  } else {
    constexpr int kHalf = kDecThreads / 2;  // waves 0-3
    if (threadIdx.x < kHalf) {
      for (int i = threadIdx.x; i <= a.E; i += kHalf) s_off[i] = a.offsets[i];
      for (int i = threadIdx.x; i < nA; i += kHalf) s_tok[i] = a.sorted_rows[i] / a.k;
    }
  }
  // LDS only: the copies (and the first block's routing stores) are covered by the full
  // barrier that ends the prologue
  if (!listed) lds_barrier();
  if (wave == 0 && !listed) {
    int seen = 0;
    for (int base = 0; base < a.E; base += 64) {
      const int e = base + lane;
      int o0 = 0, c = 0;
      if (e < a.E) {
        o0 = s_off[e];
        c = s_off[e + 1] - o0;
      }
      const uint64_t nz = __ballot(c > 0);
      if (c > 0) {
        const int r = seen + __popcll(nz & ((1ull << lane) - 1ull));
        s_e[r] = e;
        s_r0[r] = o0;
        s_n[r] = c;
      }
      seen += __popcll(nz);
    }
    if (lane == 0) {
      if (has_sh) {  // the shared expert: one more touched expert, every token a row
        s_e[seen] = a.E;
        s_r0[seen] = nA;
        s_n[seen] = a.T;
      }
      s_U = seen + (has_sh ? 1 : 0);
      s_timeout = 0;
    }
  }
  __syncthreads();
  const int U = s_U;
  const int G = gridDim.x;
  const int nfg = a.f / kGUFeat;                  // gate/up items per expert (f % 32 == 0)
  const int ndt = (a.d + kDCols - 1) / kDCols;    // down items per expert
  const int nGU = U * nfg, nD = U * ndt;
  unsigned long long* const hw = reinterpret_cast<unsigned long long*>(a.h);  // [T*k][f/2] tagged words
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // ---- this wave's share of a down item: a 16-column tile over all of K = f. Its 16
  // code rows are loaded a chunk pair at a time (8 rows x 128 bytes a load, as for
  // gate/up) and its 16 scale rows (f bytes, contiguous) 16 bytes a lane.
  const int nchD = a.f / 128, npD = (nchD + 1) / 2;
  const int grp8 = lane >> 3, seg8 = lane & 7;
  DownPrefetch pf;
  const size_t dslab = (size_t)a.d * (a.f / 2), dsslab = (size_t)a.d * (a.f / 16);
  auto down_rsrc = [&](int e) { return dec_rsrc(eslab(a.down_q, a.sh_down_q, e, a.E, dslab), (uint32_t)dslab); };
  auto down_pair = [&](__amdgpu_buffer_rsrc_t rs, int ct, int pr, u32x4 (&dst)[2]) {
    const int lc = 2 * pr + (seg8 >> 2) < nchD ? 2 * pr + (seg8 >> 2) : 2 * pr;  // this lane's chunk
    const int lb = (ct * 16 + grp8) * (a.f / 2) + lc * 64 + 16 * (seg8 & 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, lb, i * 8 * (a.f / 2), kWeightAux);
      dst[i] = u32x4{v.x, v.y, v.z, v.w};
    }
  };
  auto prefetch = [&](int j) {
    const int u = j / ndt;
    const int ct = (j - u * ndt) * kDecWaves + wave;
    if (ct * 16 >= a.d) return;
    const int e = s_e[u];
    const __amdgpu_buffer_rsrc_t rs = down_rsrc(e);
#pragma unroll
    for (int pr = 0; pr < kDownPairs; ++pr)
      if (pr < npD) down_pair(rs, ct, pr, pf.q[pr]);
    if (lane * 16 < a.f)
      pf.sc = ldg_nt_u32x4(eslab(a.down_s, a.sh_down_s, e, a.E, dsslab) + (size_t)(ct * 16) * (a.f / 16) + lane * 16);
  };
  int j = G - 1 - (int)blockIdx.x;

  // ---- gate / up / SwiGLU items
  const GateUpCtx gcx = {s_dyn, s_scr, s_sc, s_tok, s_e, s_r0, s_n, hw, tag};
  auto gu_item = [&](int i, bool last) {
    gate_up_item(a, gcx, i);
    if (last && j < nD) prefetch(j);
    __syncthreads();
  };
  // Blocks with gate/up work prefetch once their last gate/up item is done (the gate/up
  // operand registers are free by then; that item is peeled so the prefetched registers
  // are live only from there on); the others right away.
  if ((int)blockIdx.x >= nGU) {
    if (j < nD) prefetch(j);
  } else {
    int i = blockIdx.x;
    for (; i + G < nGU; i += G) gu_item(i, false);
    gu_item(i, true);
  }

  // ---- down items
  const int hstride = a.f + 8;
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_dyn);
  const int nsl = a.f / 32;  // 32-feature slices of H = gate/up items an expert (slice g is item u * nfg + g)
  // Probes: one word of each 32-feature slice of expert u's H rows (the last word the
  // slice's gate/up item writes), polled up to `polls` times. missing_mask looks once at
  // every probe of expert u and returns the slices still missing (bit g: slice g),
  // block-uniform.
  auto probe = [&](int r0, int r, int g, uint32_t polls) -> bool {
    const unsigned long long* src = hw + ((size_t)(r0 + r) * a.f) / 2 + 16 * g + 15;
    for (uint32_t it = 0;; ++it) {
      const unsigned long long w0 = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)(w0 >> 32) == tag) return true;
      if (it >= polls) return false;
      __builtin_amdgcn_s_sleep(1);
    }
  };
  auto missing_mask = [&](int u) -> uint32_t {
    const int r0 = s_r0[u], ne = s_n[u];
    if (threadIdx.x == 0) s_missing = 0;
    __syncthreads();
    for (int idx = threadIdx.x; idx < ne * nsl; idx += kDecThreads) {
      const int r = idx / nsl, g = idx - r * nsl;
      if (!probe(r0, r, g, 0)) atomicOr(&s_missing, 1u << g);  // LDS atomic
    }
    __syncthreads();
    return s_missing;
  };
  // One-launch layer: after a down item (column tile jt of the expert whose rows are
  // r0 .. r0 + ne - 1) has issued its row stores, it counts its arrival at each of those
  // rows' tokens' (token, jt) counters (one 128-byte line each, so that arrivals at
  // different counters do not queue behind each other). A counter is zero when a call
  // starts, and the arrival that completes it (k routed rows, plus the shared row) sets it
  // back to zero and combines that token's columns of the tile. Every row it reads had
  // its stores issued before its writer arrived, so its only wait is for those stores to
  // become visible (the row words' tags tell). The sum is the combining kernel's: fp32
  // fmaf in top-k order, then the gated shared row, then the residual, one rounding.
  const int arrivals = a.k + (has_sh ? 1 : 0);
  auto arrive_and_combine = [&](int jt, int r0, int ne) {
    if (threadIdx.x == 0) s_ndone = 0;
    __syncthreads();
    if ((int)threadIdx.x < ne) {
      const int t = s_tok[r0 + threadIdx.x];
      unsigned long long* const cw = a.ctr + ((size_t)t * ndt + jt) * kCtrWords;
      const unsigned long long old = __hip_atomic_fetch_add(cw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((old >> 32) != 0ull || old >= (unsigned long long)arrivals) {
        // a value no call leaves (the workspace was not zero-filled before its first use):
        // this arrival combines nothing; reported, as a wait that gave up
        __hip_atomic_fetch_or(&g_async_status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (old + 1ull == (unsigned long long)arrivals) {
        __hip_atomic_store(cw, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_done[atomicAdd(&s_ndone, 1)] = t;  // LDS atomic
      }
    }
    __syncthreads();
    const int nd = s_ndone;
    for (int q = threadIdx.x; q < nd * kDCols; q += kDecThreads) {
      const int t = s_done[q / kDCols], c = jt * kDCols + q % kDCols;
      if (c >= a.d) continue;
      const int* const ro = s_rowof + t * a.k;
      const float* const wt = s_wt + t * a.k;
      float acc;
      for (uint32_t it = 0;; ++it) {
        acc = 0.f;
        bool ok = true;
        for (int j0 = 0; j0 < a.k; j0 += 8) {  // eight rows' loads in flight at once
          unsigned long long v[8];
#pragma unroll
          for (int uu = 0; uu < 8; ++uu)
            v[uu] = __hip_atomic_load(a.yw + (size_t)ro[min(j0 + uu, a.k - 1)] * a.d + c, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int uu = 0; uu < 8; ++uu) {
            if (j0 + uu < a.k) {
              ok = ok && (uint32_t)(v[uu] >> 32) == tag;
              acc = fmaf(wt[j0 + uu], __uint_as_float((uint32_t)v[uu]), acc);
            }
          }
        }
        if (has_sh) {
          const unsigned long long sv =
              __hip_atomic_load(a.yw + (size_t)(nA + t) * a.d + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = ok && (uint32_t)(sv >> 32) == tag;
          const float g = a.gate_logit ? 1.0f / (1.0f + expf(-a.gate_logit[(size_t)t * a.gate_ld])) : 1.0f;
          acc = fmaf(g, __uint_as_float((uint32_t)sv), acc);
        }
        if (ok) break;
        if (it >= give_up) {
          acc = __builtin_nanf("");
          __hip_atomic_fetch_or(&g_async_status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (a.resid) acc += bf16_to_f32(a.resid[(size_t)t * a.d + c]);
      a.out[(size_t)t * a.d + c] = (uint16_t)bf16_rne(acc);
    }
  };
  // Down item j, its weights already in `pf`: H rows of its expert into LDS (bf16, row
  // stride hstride) once every word carries this call's tag, then the products. With
  // allow_defer, an item whose H slices are not all there after steal_after polls is
  // left (returns true) for the block to finish after computing those slices itself.
  auto down_item = [&](int j, bool allow_defer) -> bool {
    const int u = j / ndt;
    const int ct = (j - u * ndt) * kDecWaves + wave;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    // H rows of expert u -> LDS (bf16, row stride hstride), polling until every word
    // carries this call's tag
    const int npair = a.f / 4;  // pairs of H words (4 features) a row
    // first wait on one word of each 32-feature slice of each row (the last word its
    // gate/up item writes: 16x fewer device-scope loads while the producers finish, which
    // eases the hot spot of many pollers on the same few KB); the full read below still
    // validates every word
    const bool may_defer = allow_defer && steal_after < give_up;
    {
      const uint32_t polls = may_defer ? steal_after : give_up;
      for (int idx = threadIdx.x; idx < ne * nsl; idx += kDecThreads) probe(r0, idx / nsl, idx % nsl, polls);
      __syncthreads();
    }
    for (uint32_t it = 0;; ++it) {
      int bad = 0;
      for (int idx = threadIdx.x; idx < ne * npair; idx += kDecThreads) {
        const int r = idx / npair, sg = idx - r * npair;
        const unsigned long long* src = hw + ((size_t)(r0 + r) * a.f) / 2 + 2 * sg;
        const unsigned long long w0 = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long w1 = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w0 >> 32) != tag || (uint32_t)(w1 >> 32) != tag) {
          bad = 1;
        } else {
          const u32x2v v = {(uint32_t)w0, (uint32_t)w1};
          *reinterpret_cast<u32x2v*>(s_h + r * hstride + 4 * sg) = v;
        }
      }
      if (__syncthreads_or(bad) == 0) break;
      // some producer has not written its slice yet: leave the item for later
      if (may_defer && it >= steal_after) return true;
      if (it >= give_up) {
        if (threadIdx.x == 0) {
          s_timeout = 1;
          __hip_atomic_fetch_or(&g_async_status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    const bool valid = col < ne;
    if (ct * 16 < a.d) {
      unsigned char* const scr = s_scr + wave * kScrWave;
      unsigned char* const dsc = scr + 2048;  // the wave's scale rows: [16][f / 16]
      const int srowD = a.f / 16;
      const uint16_t* hrow = s_h + col * hstride;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      // rows >= ne: stale LDS, confined to output columns that are not stored
      auto hv = [&](int k0) -> bf16x8 { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4v*>(hrow + k0)); };
      if (lane * 16 < a.f) *reinterpret_cast<u32x4v*>(dsc + lane * 16) = u32x4v{pf.sc.x, pf.sc.y, pf.sc.z, pf.sc.w};
      const __amdgpu_buffer_rsrc_t rs = down_rsrc(e);
      // a pair of chunks: rearranged through the scratch (layout as for gate/up), then
      // two chunks of MFMAs
      auto down_compute = [&](int pr, const u32x4 (&lq)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 8 * i + grp8;
          *reinterpret_cast<u32x4v*>(scr + r * 128 + ((seg8 + (r >> 1)) & 7) * 16) =
              u32x4v{lq[i].x, lq[i].y, lq[i].z, lq[i].w};
        }
        __builtin_amdgcn_wave_barrier();
        u32x4 q[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const u32x4v v = *reinterpret_cast<const u32x4v*>(scr + col * 128 + ((4 * jj + grp + (col >> 1)) & 7) * 16);
          q[jj] = u32x4{v.x, v.y, v.z, v.w};
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int c = 2 * pr + jj;
          if (c < nchD) {
            const uint32_t sc = *reinterpret_cast<const uint16_t*>(dsc + col * srowD + c * 8 + 2 * grp);
            const E4M3Split s0 = e4m3_split_b<0>(sc);
            const E4M3Split s1 = e4m3_split_b<1>(sc);
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc = mfma16(nvfp4x8_to_bf16(word_of(q[jj], s), s < 2 ? s0 : s1), hv(c * 128 + 32 * grp + 8 * s), acc);
          }
        }
      };
#pragma unroll
      for (int pr = 0; pr < kDownPairs; ++pr)
        if (pr < npD) down_compute(pr, pf.q[pr]);
      // pairs past the prefetch depth (f > 2 * kDownPairs * 128)
      for (int pr = kDownPairs; pr < npD; ++pr) {
        u32x4 lq[2];
        down_pair(rs, ct, pr, lq);
        down_compute(pr, lq);
      }
      // the 32-element chunks past the last full 128: lane group g holds K0 + 8g .. K0 + 8g + 7
      const uint8_t* const wq = eslab(a.down_q, a.sh_down_q, e, a.E, dslab) + (size_t)(ct * 16 + col) * (a.f / 2);
      for (int K0 = nchD * 128; K0 < a.f; K0 += 32) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq + K0 / 2 + 4 * grp);
        const E4M3Split sp = e4m3_split(dsc[col * srowD + K0 / 16 + (grp >> 1)]);
        acc = mfma16(nvfp4x8_to_bf16(q, sp), hv(K0 + 8 * grp), acc);
      }
      if (valid) {
        const float td = ets(a.down_ts, a.sh_down_ts, e, a.E);
        const float nanv = __builtin_nanf("");
        const bool bad = s_timeout != 0;
        float4 v;
        v.x = bad ? nanv : td * acc[0];
        v.y = bad ? nanv : td * acc[1];
        v.z = bad ? nanv : td * acc[2];
        v.w = bad ? nanv : td * acc[3];
        if (fold) {
          // tagged words for the combining block (value, tag), as H
          unsigned long long* dst = a.yw + (size_t)(r0 + col) * a.d + ct * 16 + 4 * grp;
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __hip_atomic_store(dst + r, ((unsigned long long)tag << 32) | __float_as_uint(vv[r]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *reinterpret_cast<float4*>(a.y_rows + (size_t)(r0 + col) * a.d + ct * 16 + 4 * grp) = v;
        }
      }
    }
    if (fold) arrive_and_combine(j - u * ndt, r0, ne);
    __syncthreads();  // before the next item overwrites s_h
    return false;
  };
  // The block's own down items (G - 1 - b, 2G - 1 - b, ...), then the ones it deferred.
  // A deferred item's missing gate/up items are computed first (gate_up_item_plain: the
  // same bits as their own blocks would give; a word written twice is written with the
  // same value), on the activation rows copied into LDS again (H rows of down items
  // replaced them); then the deferred items, whose waits now end. (Separate loops, and
  // the plain item code: in one loop, or with the batched item code, the kernel spilled.)
  int ndef = 0;  // deferred down items (their ids in s_def), block-uniform
  bool first = true;
  for (; j < nD; j += G) {
    if (!first) prefetch(j);
    first = false;
    if (down_item(j, true)) {
      if (threadIdx.x == 0) s_def[ndef] = j;
      ++ndef;
    }
  }
  if (ndef == 0) return;
  __syncthreads();
  for (int di = 0; di < ndef; ++di) {
    const int u = s_def[di] / ndt;
    const uint32_t missing = missing_mask(u);
    if (missing != 0u) {
      copy_x_rows(0);
      __syncthreads();
      for (int g = 0; g < nsl; ++g) {
        if ((missing >> g) & 1u) {
          gate_up_item_plain(a, gcx, u * nfg + g);
          __syncthreads();
        }
      }
    }
  }
  for (int di = 0; di < ndef; ++di) {
    const int jd = s_def[di];
    prefetch(jd);
    down_item(jd, false);
  }
}

size_t ffn_decode_lds_bytes(int T, int d, int f) { return dec_row_region(T, d, f); }

hipError_t launch_ffn_decode(const FFNArgs& a, uint32_t tag, uint32_t steal_after, uint32_t give_up,
                             hipStream_t stream) {
  const int lds = (int)(dec_row_region(a.T, a.d, a.f) + (size_t)kDecWaves * kScrWave + (size_t)4 * a.d);
  // as many blocks as the device holds at once for this LDS size (so normally every
  // block starts at once; the waits do not depend on it)
  int capacity = 0;
  hipError_t err = resident_blocks(reinterpret_cast<const void*>(&ffn_decode_kernel), kDecThreads, lds, capacity);
  if (err != hipSuccess) return err;
  const long long touched = std::min<long long>(a.E, (long long)a.T * a.k) + (a.sh_gate_q ? 1 : 0);
  const long long down_items = touched * ((a.d + kDCols - 1) / kDCols);
  const long long items = touched * std::max<long long>(a.f / kGUFeat, (a.d + kDCols - 1) / kDCols);
  // no block may take more down items than it can defer
  const long long grid_min = (down_items + kDecMaxDeferred - 1) / kDecMaxDeferred;
  const int grid = (int)std::max<long long>(std::min<long long>(items, capacity), grid_min);
  // Under graph capture: a fresh tag for every replay from the workspace's epoch word
  // (a direct call passes its own and leaves `epoch` unused).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  err = hipStreamIsCapturing(stream, &cap);
  if (err != hipSuccess) return err;
  FFNArgs b = a;
  b.epoch = nullptr;
  if (cap == hipStreamCaptureStatusActive) {
    if (a.epoch == nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL(advance_epoch_kernel, dim3(1), dim3(64), 0, stream, a.epoch);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    b.epoch = a.epoch;
  }
  hipLaunchKernelGGL(ffn_decode_kernel, dim3(grid), dim3(kDecThreads), lds, stream, b, tag, steal_after, give_up);
  return hipGetLastError();
}

hipError_t read_and_clear_async_status(unsigned int& status) {
  hipError_t err = hipMemcpyFromSymbol(&status, HIP_SYMBOL(g_async_status), sizeof(status), 0, hipMemcpyDeviceToHost);
  if (err != hipSuccess || status == 0) return err;
  const unsigned int zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_async_status), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
}

}  // namespace moe
