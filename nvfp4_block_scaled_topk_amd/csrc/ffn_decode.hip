// ffn_decode.hip -- the expert FFN for a few tokens (decode): weight streaming.
//
// With a few tokens every selected expert has at most a handful of rows, and the
// layer's time is the time to read the selected experts' weight bytes once. The pages
// read each selected expert once for all of its rows [FP4-Local checkpoints on DGX
// Spark, §4 Round 1, #808]; here one 16x16x32 bf16 MFMA tile covers all of an
// expert's rows (<= 16), so each weight byte is read once whatever the row count.
//
// MFMA mapping (per wave and 16-row weight tile): 16 weight rows (output features) x
// up to 16 routed rows. Each lane streams one weight row's packed codes with 128-bit
// loads (32 E2M1 codes = two scale blocks) and decodes them in registers into four
// MFMA operands. Within a 128-element chunk, lane group g (lane / 16) holds elements
// [32g, 32g + 32) and MFMA step s takes elements 32g + 8s .. 32g + 8s + 7 of every
// group -- a permutation of the contraction index, applied identically to the
// activation operand, so the sums are unchanged.
//
// One launch does gate, up, SwiGLU [same page, §4 Round 1, #766] and the down product,
// with 8-wave blocks and two kinds of work item:
//   gate/up item (touched expert u, 32 features): waves 0-3 take the gate and up tiles
//     of features 0..15, waves 4-7 those of 16..31, each wave a quarter of K = d. A wave
//     issues every code and scale load of its share at once, while the block copies u's
//     activation rows into LDS by buffer->LDS DMA. Waves 0 and 4 add the four K
//     quarters of their half in LDS in order, form H = bf16_rne(silu(ts_g * G) *
//     (ts_u * U)) and store it;
//   down item (u, 128 columns of d): wave w owns a 16-column tile over all of K = f.
//     A block loads the weight codes of its first down item into registers as soon as
//     its last gate/up item is done (or at the start, if it has none), so those bytes
//     are in flight while the other gate/up items finish. It then copies H's rows of u
//     into LDS, waiting until all of them are there, and finishes the products with the
//     weights already in hand.
// H in the workspace is self-validating: every 64-bit word holds two bf16 values and
// the call's 32-bit tag, written and read as one device-scope atomic access. A reader
// that sees the current tag sees the values stored with it, so the producer never
// waits for its stores and there are no separate completion flags. Every call writes
// every H word it reads, so words left from earlier calls carry older tags.
// Block b takes gate/up items b, b + G, ... and then down items G-1-b, 2G-1-b, ... (the
// blocks without a gate/up item take the extra down items). Every block finishes its
// gate/up items before it waits, and the grid never exceeds the number of blocks the
// device holds at once, so every awaited H word belongs to a running block. A wait is
// bounded: past kSpinLimit polls the block writes NaN rows instead of hanging.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kDecThreads = 512;               // 8 waves
constexpr int kDecWaves = 8;
constexpr int kDecMaxE = 1024;
constexpr int kDecMaxAssign = kDecodeMaxRows * 32;  // T * k
constexpr int kDecMaxTouched = kDecMaxAssign;      // min(E, T * k)
constexpr int kGUFeat = 32;                     // features of a gate/up item
constexpr int kDCols = 16 * kDecWaves;          // columns of d in a down item
constexpr int kDownPrefetch = 6;                // W_down chunks (128 K) a wave holds before its wait
constexpr uint32_t kSpinLimit = 1u << 20;       // polls (each followed by s_sleep) before giving up

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

struct DownPrefetch {
  u32x4 q[kDownPrefetch];
  uint32_t sc[kDownPrefetch];
};

// Dynamic LDS: the activation rows of one expert (gate/up phase; row stride
// xstride bytes) and later its H rows (down phase; row stride (f + 8) bf16). Both
// strides are 16 bytes past a multiple of the bank period, which staggers the banks of
// the 16 rows an MFMA operand read touches.
__device__ __forceinline__ int dec_xstride(int d) { return (d * 2 + 1023) / 1024 * 1024 + 16; }

__global__ __launch_bounds__(kDecThreads, 4) void ffn_decode_kernel(FFNArgs a, uint32_t tag) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  __shared__ floatx4 red[kDecWaves][2][64];  // gate/up partial sums (16 KB); the offsets before that
  __shared__ int s_tok[kDecMaxAssign];
  __shared__ int s_e[kDecMaxTouched], s_r0[kDecMaxTouched], s_n[kDecMaxTouched];
  __shared__ int s_U, s_timeout;
  int* s_off = reinterpret_cast<int*>(&red[0][0][0]);
  static_assert(sizeof(red) >= sizeof(int) * (kDecMaxE + 1), "offsets fit the reduction buffer");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;

  // ---- touched experts and the token of every routed row (one round trip)
  const int nA = a.T * a.k;
  for (int i = threadIdx.x; i <= a.E; i += kDecThreads) s_off[i] = a.offsets[i];
  for (int i = threadIdx.x; i < nA; i += kDecThreads) s_tok[i] = a.sorted_rows[i] / a.k;
  __syncthreads();
  if (wave == 0) {
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
      s_U = seen;
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
  const __amdgpu_buffer_rsrc_t xrs = dec_rsrc(a.x, (uint32_t)(a.T * a.d * 2));
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // ---- this wave's share of a down item: a 16-column tile over all of K = f
  const int nchD = a.f / 128;
  DownPrefetch pf;
  auto prefetch = [&](int j) {
    const int u = j / ndt;
    const int ct = (j - u * ndt) * kDecWaves + wave;
    if (ct * 16 >= a.d) return;
    const size_t wrow = (size_t)s_e[u] * a.d + ct * 16 + col;
    const uint8_t* wq = a.down_q + wrow * (a.f / 2);
    const uint8_t* ws = a.down_s + wrow * (a.f / 16);
#pragma unroll
    for (int p = 0; p < kDownPrefetch; ++p) {
      if (p < nchD) {
        pf.q[p] = ldg_u32x4(wq + p * 64 + 16 * grp);
        pf.sc[p] = *reinterpret_cast<const uint16_t*>(ws + p * 8 + 2 * grp);
      }
    }
  };
  int j = G - 1 - (int)blockIdx.x;

  // ---- gate / up / SwiGLU items
  const int nchG = a.d / 128;
  const int half = wave >> 2, kq = wave & 3;  // 16-feature half of the item, quarter of K
  const int kc0 = nchG * kq / 4, kc1 = nchG * (kq + 1) / 4;
  const bool gtail = kq == 3;
  const int xstride = dec_xstride(a.d);
  const int ipr = (a.d * 2 + 1023) / 1024;  // 1 KB DMA instructions per activation row
  constexpr int kB = 4;                     // chunks a wave loads at once
  auto gu_item = [&](int i, bool last) {
    const int u = i / nfg, fg = i - u * nfg;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    // weight rows through buffer descriptors (expert slab base in scalar registers,
    // a 32-bit row offset per lane)
    const size_t slab = (size_t)a.f * (a.d / 2), sslab = (size_t)a.f * (a.d / 16);
    const __amdgpu_buffer_rsrc_t qrs[2] = {dec_rsrc(a.gate_q + (size_t)e * slab, (uint32_t)slab),
                                           dec_rsrc(a.up_q + (size_t)e * slab, (uint32_t)slab)};
    const __amdgpu_buffer_rsrc_t srs[2] = {dec_rsrc(a.gate_s + (size_t)e * sslab, (uint32_t)sslab),
                                           dec_rsrc(a.up_s + (size_t)e * sslab, (uint32_t)sslab)};
    const uint32_t frow = (uint32_t)(fg * kGUFeat + half * 16 + col);
    const uint32_t qoff = frow * (uint32_t)(a.d / 2) + 16 * grp, soff = frow * (uint32_t)(a.d / 16) + 2 * grp;
    floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    u32x4 q[kB][2];
    uint32_t sc[kB][2];
    // A batch always issues kB chunks of loads (a chunk past the wave's range repeats
    // chunk c), so the number of loads in flight is a constant and every wait below is
    // exact.
    auto load_batch = [&](int c) {
#pragma unroll
      for (int h = 0; h < kB; ++h) {
        const int cc = c + h < kc1 ? c + h : c;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(qrs[m], (int)qoff, cc * 64, 0);
          q[h][m] = u32x4{v.x, v.y, v.z, v.w};
          sc[h][m] = __builtin_amdgcn_raw_buffer_load_b16(srs[m], (int)soff, cc * 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the chunks in issue order
      }
    };
    // the activation rows of expert u by DMA first, then the first batch of weights;
    // waiting for all but the weight loads leaves those in flight, and each chunk is
    // decoded as soon as its own loads have landed
    for (int qi = wave; qi < ne * ipr; qi += kDecWaves) {
      const int r = qi / ipr, jj = qi - r * ipr;
      const int within = jj * 1024 + lane * 16;
      const uint32_t voff = within < a.d * 2 ? (uint32_t)s_tok[r0 + r] * (uint32_t)(a.d * 2) + within : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void_ptr)(s_dyn + r * xstride + jj * 1024), 16, voff, 0,
                                               0, 0);
    }
    load_batch(kc0);
    wait_vm<4 * kB>();  // the DMA has landed; the weight loads may still be in flight
    // a bare barrier: __syncthreads() would also wait for the weight loads
    lds_barrier();
    const bool valid = col < ne;
    // Lanes of routed rows >= ne read whatever the LDS row holds: MFMA output column j
    // depends only on operand column j, and those columns are never stored.
    const unsigned char* xrow = s_dyn + col * xstride;
    auto xop = [&](int k0) -> bf16x8 { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4v*>(xrow + k0 * 2)); };
    auto compute_batch = [&](int c) {
#pragma unroll
      for (int h = 0; h < kB; ++h) {
        if (c + h < kc1) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const E4M3Split s0 = e4m3_split(sc[h][m] & 0xFFu);
            const E4M3Split s1 = e4m3_split(sc[h][m] >> 8);
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc[m] = mfma16(nvfp4x8_to_bf16(word_of(q[h][m], s), s < 2 ? s0 : s1),
                              xop((c + h) * 128 + 32 * grp + 8 * s), acc[m]);
          }
        }
        // chunk by chunk, so each waits only for its own loads
        __builtin_amdgcn_sched_barrier(0);
      }
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
                                                                 K0 / 2, 0);
          const uint32_t sv = __builtin_amdgcn_raw_buffer_load_b8(
              srs[m], (int)(frow * (uint32_t)(a.d / 16) + (grp >> 1)), K0 / 16, 0);
          acc[m] = mfma16(nvfp4x8_to_bf16(qq, e4m3_split(sv)), xv, acc[m]);
        }
      }
    }
    red[wave][0][lane] = acc[0];
    red[wave][1][lane] = acc[1];
    __syncthreads();
    if (kq == 0) {
      if (valid) {
        floatx4 Gs = red[wave][0][lane], Us = red[wave][1][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          Gs += red[wave + w][0][lane];
          Us += red[wave + w][1][lane];
        }
        const float tg = a.gate_ts[e], tu = a.up_ts[e];
        uint32_t hb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(silu_f32(tg * Gs[r]) * (tu * Us[r]));
        // lane holds routed row `col`, features 4*grp .. 4*grp + 3 of the half
        unsigned long long* dst = hw + ((size_t)(r0 + col) * a.f + fg * kGUFeat + half * 16 + 4 * grp) / 2;
        __hip_atomic_store(dst, h_word(hb[0], hb[1], tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, h_word(hb[2], hb[3], tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
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
  bool first = true;
  for (; j < nD; j += G) {
    if (!first) prefetch(j);
    first = false;
    const int u = j / ndt;
    const int ct = (j - u * ndt) * kDecWaves + wave;
    const int e = s_e[u], r0 = s_r0[u], ne = s_n[u];
    // H rows of expert u -> LDS (bf16, row stride hstride), polling until every word
    // carries this call's tag
    const int npair = a.f / 4;  // pairs of H words (4 features) a row
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
      if (it >= kSpinLimit) {
        if (threadIdx.x == 0) s_timeout = 1;
        __syncthreads();
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    const bool valid = col < ne;
    if (ct * 16 < a.d) {
      const size_t wrow = (size_t)e * a.d + ct * 16 + col;
      const uint8_t* const wq = a.down_q + wrow * (a.f / 2);
      const uint8_t* const ws = a.down_s + wrow * (a.f / 16);
      const uint16_t* hrow = s_h + col * hstride;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      // rows >= ne: stale LDS, confined to output columns that are not stored
      auto hv = [&](int k0) -> bf16x8 { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4v*>(hrow + k0)); };
#pragma unroll
      for (int p = 0; p < kDownPrefetch; ++p) {
        if (p < nchD) {
          const E4M3Split s0 = e4m3_split(pf.sc[p] & 0xFFu);
          const E4M3Split s1 = e4m3_split(pf.sc[p] >> 8);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = mfma16(nvfp4x8_to_bf16(word_of(pf.q[p], s), s < 2 ? s0 : s1), hv(p * 128 + 32 * grp + 8 * s), acc);
        }
      }
      // chunks past the prefetch depth (f > kDownPrefetch * 128)
      for (int c = kDownPrefetch; c < nchD; ++c) {
        const u32x4 q = ldg_u32x4(wq + c * 64 + 16 * grp);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(ws + c * 8 + 2 * grp);
        const E4M3Split s0 = e4m3_split(sc & 0xFFu);
        const E4M3Split s1 = e4m3_split(sc >> 8);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = mfma16(nvfp4x8_to_bf16(word_of(q, s), s < 2 ? s0 : s1), hv(c * 128 + 32 * grp + 8 * s), acc);
      }
      // the 32-element chunks past the last full 128: lane group g holds K0 + 8g .. K0 + 8g + 7
      for (int K0 = nchD * 128; K0 < a.f; K0 += 32) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(wq + K0 / 2 + 4 * grp);
        const E4M3Split sp = e4m3_split(ws[K0 / 16 + (grp >> 1)]);
        acc = mfma16(nvfp4x8_to_bf16(q, sp), hv(K0 + 8 * grp), acc);
      }
      if (valid) {
        const float td = a.down_ts[e];
        const float nanv = __builtin_nanf("");
        const bool bad = s_timeout != 0;
        float4 v;
        v.x = bad ? nanv : td * acc[0];
        v.y = bad ? nanv : td * acc[1];
        v.z = bad ? nanv : td * acc[2];
        v.w = bad ? nanv : td * acc[3];
        *reinterpret_cast<float4*>(a.y_rows + (size_t)(r0 + col) * a.d + ct * 16 + 4 * grp) = v;
      }
    }
    __syncthreads();  // before the next item overwrites s_h
  }
}

size_t ffn_decode_lds_bytes(int T, int d, int f) {
  const size_t xs = (size_t)((d * 2 + 1023) / 1024 * 1024 + 16);
  const size_t hs = (size_t)(f + 8) * sizeof(uint16_t);
  return (size_t)T * std::max(xs, hs);
}

hipError_t launch_ffn_decode(const FFNArgs& a, uint32_t tag, hipStream_t stream) {
  // co-resident blocks for this dynamic LDS size (cached per size)
  static int cached_lds = -1, cached_capacity = 0;
  const int lds = (int)ffn_decode_lds_bytes(a.T, a.d, a.f);
  if (lds != cached_lds) {
    int dev = 0, ncu = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess)
      err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&ffn_decode_kernel),
                                                         kDecThreads, lds);
    if (err != hipSuccess) return err;
    if (ncu < 1 || per_cu < 1) return hipErrorInvalidConfiguration;
    cached_capacity = ncu * per_cu;
    cached_lds = lds;
  }
  const long long touched = std::min<long long>(a.E, (long long)a.T * a.k);
  const long long items = touched * std::max(a.f / kGUFeat, (a.d + kDCols - 1) / kDCols);
  const int grid = (int)std::min<long long>(items, cached_capacity);
  hipLaunchKernelGGL(ffn_decode_kernel, dim3(grid), dim3(kDecThreads), lds, stream, a, tag);
  return hipGetLastError();
}

}  // namespace moe
