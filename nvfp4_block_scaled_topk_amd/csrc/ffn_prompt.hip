// ffn_prompt.hip -- the expert FFN for many tokens (prompt): a grouped GEMM over the
// per-expert row lists.
//
// The pages' prompt path admits routed NVFP4 experts into a grouped GEMM whose store
// scales each row by its expert's tensor scale [FP4-Local checkpoints on DGX Spark,
// §4 Round 1, #545], runs gate, up and SwiGLU as one launch (#766) and copies its
// operands through a multi-stage pipeline in fixed K steps (§4 remaining items, #822).
// Here, on gfx950:
//
//   tile    = (expert e, 128 routed rows of e, 128 features of f)   [gate/up launch]
//             (expert e, 128 routed rows of e, 256 columns of d)    [down launch]
//   waves   = 4; wave w owns two 32-row weight fragments (gate and up of the same 32
//             features, or two 32-column slices of d) and all 128 routed rows
//   MFMA    = v_mfma_f32_32x32x16_bf16, weights as the A operand, activations as B
//   stages  = 4 LDS stages of 64 K elements: activations (bf16), packed weight codes
//             and block scales, each filled by buffer->LDS DMA (no register staging;
//             out-of-range lanes read zeros, which also pads ragged rows and K tails)
//
// Each wave decodes its weight fragments from LDS into bf16 MFMA operands (exact, see
// device.hpp); the activation tile is shared by the four waves. Activation rows sit in
// LDS as 128-byte rows of eight 16-byte segments, segment j of row r stored at slot
// j ^ (r & 7), so the MFMA operand reads (32 rows, same segment) hit distinct banks.
// The fp32 tensor scale multiplies the accumulator in the epilogue; gate/up's
// epilogue forms H = bf16_rne(silu(G) * U), down's writes fp32 rows.
//
// Work: one flat list of tiles (expert-major, column tile fastest) walked by a
// persistent grid; each block derives the list from expert_offsets. Block b works on
// the list positions of "lane" (b mod 8) * (grid / 8) + b / 8, so the blocks a chip's
// XCD receives (round-robin by block index) take consecutive tiles, which share
// activation rows and weight columns in that XCD's L2.
#include "device.hpp"
#include "internal.hpp"

#include <type_traits>

namespace moe {

constexpr int kPromptRows = 128;                      // routed rows per tile
constexpr int kPromptKC = 64;                         // K elements per stage
constexpr int kPromptStages = 4;
constexpr int kPromptXBytes = kPromptRows * kPromptKC * 2;  // 16 KB
constexpr int kPromptWBytes = 256 * (kPromptKC / 2);        // 8 KB: 256 weight rows
constexpr int kPromptSBytes = 256 * 2 * 4;                  // 2 KB: 2 scale pairs a row, dword slots
constexpr int kPromptStageBytes = kPromptXBytes + kPromptWBytes + kPromptSBytes;
constexpr int kPromptLdsBytes = kPromptStages * kPromptStageBytes;
constexpr int kPromptThreads = 256;
constexpr int kMaxE = 1024;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every record: reads zeros
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word4(const u32x4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One buffer->LDS DMA instruction: lane l writes `size` bytes read at byte offset
// voff of the buffer to LDS address lds_base + l * max(size, 4).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma2(__amdgpu_buffer_rsrc_t rs, unsigned char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)lds_base, 2, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Per-block tile table: s_pref[e] = number of 128-row tiles of experts < e.
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int* s_pref) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      const int v = e < E ? (offsets[e + 1] - offsets[e] + kPromptRows - 1) / kPromptRows : 0;
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
  }
  __syncthreads();
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
__global__ __launch_bounds__(kPromptThreads, 1) void ffn_prompt_kernel(FFNArgs a, int n_col_tiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_pref[kMaxE + 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int l32 = lane & 31, g = lane >> 5;
  const int K = MODE == 0 ? a.d : a.f;  // contraction length
  const int N = MODE == 0 ? a.f : a.d;  // weight rows per matrix
  const int nch = (K + kPromptKC - 1) / kPromptKC;

  build_tile_prefix(a.offsets, a.E, s_pref);
  const int total_tiles = s_pref[a.E] * n_col_tiles;
  const int G = gridDim.x;
  const int lid = (G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds : blockIdx.x;

  for (int item = lid; item < total_tiles; item += G) {
    const int mt_all = item / n_col_tiles;
    const int ct = item - mt_all * n_col_tiles;
    const int e = find_tile_expert(s_pref, a.E, mt_all);
    const int mt = mt_all - s_pref[e];
    const int p0 = a.offsets[e] + mt * kPromptRows;
    const int nrows = min(kPromptRows, a.offsets[e + 1] - p0);
    const int ntf = (nrows + 31) >> 5;  // 32-row activation fragments in use

    // ---- buffer descriptors (wave-uniform)
    __amdgpu_buffer_rsrc_t xrs, wrs, srs;
    const size_t wslab = (size_t)N * (K / 2), sslab = (size_t)N * (K / 16);
    if (MODE == 0) {
      xrs = make_rsrc(a.x, (uint32_t)((size_t)a.T * a.d * 2));
      const bool up = wave >= 2;  // waves 0,1 stage the gate rows, waves 2,3 the up rows
      wrs = make_rsrc((up ? a.up_q : a.gate_q) + (size_t)e * wslab, (uint32_t)wslab);
      srs = make_rsrc((up ? a.up_s : a.gate_s) + (size_t)e * sslab, (uint32_t)sslab);
    } else {
      xrs = make_rsrc(a.h + (size_t)p0 * a.f, (uint32_t)((size_t)nrows * a.f * 2));
      wrs = make_rsrc(a.down_q + (size_t)e * wslab, (uint32_t)wslab);
      srs = make_rsrc(a.down_s + (size_t)e * sslab, (uint32_t)sslab);
    }

    // ---- per-lane DMA sources for this tile (byte offsets at K0 = 0)
    // activations: 4 instructions, slot s = wave*256 + i*64 + lane -> row s/8, slot s%8
    uint32_t xoff[4];
    int xseg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = wave * 256 + i * 64 + lane;
      const int r = s >> 3;
      const int j = (s & 7) ^ (r & 7);  // logical 16-byte segment held by this slot
      xseg[i] = j;
      if (r < nrows) {
        const uint32_t rb = MODE == 0 ? (uint32_t)(a.sorted_rows[p0 + r] / a.k) * (uint32_t)(a.d * 2)
                                      : (uint32_t)(r * a.f * 2);
        xoff[i] = rb + j * 16;
      } else {
        xoff[i] = kOOB;
      }
    }
    // weights / scales: 2 instructions each, slot s = wave*128 + i*64 + lane -> row s/2, half s%2
    uint32_t woff[2], soff[2];
    int whalf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = wave * 128 + i * 64 + lane;
      const int row = s >> 1, h = s & 1;
      const int n = MODE == 0 ? ct * 128 + (row & 127) : ct * 256 + row;
      whalf[i] = h;
      if (n < N) {
        woff[i] = (uint32_t)n * (uint32_t)(K / 2) + 16 * h;
        soff[i] = (uint32_t)n * (uint32_t)(K / 16) + 2 * h;
      } else {
        woff[i] = soff[i] = kOOB;
      }
    }

    auto issue = [&](int c) {
      const int K0 = c * kPromptKC;
      unsigned char* buf = smem + (c % kPromptStages) * kPromptStageBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = xoff[i] != kOOB && K0 + 8 * xseg[i] < K;
        dma16(xrs, buf + (wave * 256 + i * 64) * 16, ok ? xoff[i] + K0 * 2 : kOOB);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = woff[i] != kOOB && K0 + 32 * whalf[i] < K;
        dma16(wrs, buf + kPromptXBytes + (wave * 128 + i * 64) * 16, ok ? woff[i] + K0 / 2 : kOOB);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = soff[i] != kOOB && K0 + 32 * whalf[i] < K;
        dma2(srs, buf + kPromptXBytes + kPromptWBytes + (wave * 128 + i * 64) * 4, ok ? soff[i] + K0 / 16 : kOOB);
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
      wrow[0] = wave * 32 + l32;        // gate features ct*128 + wave*32 + l32
      wrow[1] = 128 + wave * 32 + l32;  // up rows of the same features
    } else {
      wrow[0] = wave * 64 + l32;
      wrow[1] = wave * 64 + 32 + l32;
    }
    const bool fvalid[2] = {MODE == 0 ? ct * 128 + wave * 32 < N : ct * 256 + wave * 64 < N,
                            MODE == 0 ? ct * 128 + wave * 32 < N : ct * 256 + wave * 64 + 32 < N};

    // previous tile: stores drained and every wave done with the stage buffers
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int c = 0; c < kPromptStages - 1; ++c)
      if (c < nch) issue(c);

    // The K loop, specialised on the number of 32-row activation fragments in use so
    // the MFMA sequence is branch-free (rows past nrows are zeros; weight rows past N
    // decode to zeros and are not stored).
    auto k_loop = [&](auto ntf_c) {
      constexpr int NTF = decltype(ntf_c)::value;
      for (int c = 0; c < nch; ++c) {
        // stages issued after c still in flight: min(kPromptStages - 2, nch - 1 - c)
        const int after = min(kPromptStages - 2, nch - 1 - c);
        if (after >= 2) wait_vm<16>();
        else if (after == 1) wait_vm<8>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (c + kPromptStages - 1 < nch) issue(c + kPromptStages - 1);

        const unsigned char* buf = smem + (c % kPromptStages) * kPromptStageBytes;
        const unsigned char* xb = buf;
        const unsigned char* wb = buf + kPromptXBytes;
        const unsigned char* sb = buf + kPromptXBytes + kPromptWBytes;
        // all operand reads of the stage first (weights first: their decode starts
        // while the activation reads are in flight), then decode + MFMA
        u32x4 q[2];
        uint32_t sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          q[i] = *reinterpret_cast<const u32x4*>(wb + wrow[i] * 32 + 16 * g);
          sc[i] = *reinterpret_cast<const uint32_t*>(sb + (wrow[i] * 2 + g) * 4);
        }
        u32x4 bq[4][NTF];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int t = 0; t < NTF; ++t) {
            const int row = t * 32 + l32;
            const int slot = (4 * g + s) ^ (row & 7);
            bq[s][t] = *reinterpret_cast<const u32x4*>(xb + row * 128 + slot * 16);
          }
        // keep the reads above this point: the scheduler would otherwise sink each read
        // next to its MFMA and expose the LDS latency once per operand
        __builtin_amdgcn_sched_barrier(0);
        E4M3Split sp[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sp[i][0] = e4m3_split(sc[i] & 0xFFu);
          sp[i][1] = e4m3_split((sc[i] >> 8) & 0xFFu);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8 wa[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) wa[i] = nvfp4x8_to_bf16(word4(q[i], s), sp[i][s >> 1]);
#pragma unroll
          for (int t = 0; t < NTF; ++t) {
            const bf16x8 b = u32x4_as_bf16x8(bq[s][t]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i][t] = mfma32(wa[i], b, acc[i][t]);
          }
        }
      }
    };
    switch (ntf) {
      case 1: k_loop(std::integral_constant<int, 1>()); break;
      case 2: k_loop(std::integral_constant<int, 2>()); break;
      case 3: k_loop(std::integral_constant<int, 3>()); break;
      default: k_loop(std::integral_constant<int, 4>()); break;
    }

    // ---- epilogue. Accumulator r of fragment (i, t): weight row 8*(r/4) + 4*g + r%4 of
    // the fragment, activation row t*32 + l32 of the tile.
    if (MODE == 0) {
      const int f0 = ct * 128 + wave * 32;
      if (fvalid[0]) {
        const float tg = a.gate_ts[e], tu = a.up_ts[e];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = t * 32 + l32;
          if (t < ntf && row < nrows) {
            uint16_t* hp = a.h + (size_t)(p0 + row) * a.f + f0 + 4 * g;
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
        const int c0 = ct * 256 + wave * 64 + 32 * i;
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
}

static int device_cu_count() {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ncu = v;
  }
  return ncu;
}

hipError_t launch_ffn_prompt(const FFNArgs& a, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e0 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_prompt_kernel<0>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, kPromptLdsBytes);
    hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_prompt_kernel<1>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, kPromptLdsBytes);
    if (e0 != hipSuccess) return e0;
    if (e1 != hipSuccess) return e1;
    attr_set = true;
  }
  const long long rows = (long long)a.T * a.k;
  const long long max_tiles = rows / kPromptRows + std::min<long long>(a.E, rows);
  const int ncu = device_cu_count();
  const int ct_gu = (a.f + 127) / 128;
  const int grid_gu = (int)std::min<long long>(max_tiles * ct_gu, ncu);
  hipLaunchKernelGGL(ffn_prompt_kernel<0>, dim3(grid_gu), dim3(kPromptThreads), kPromptLdsBytes, stream, a, ct_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ct_dn = (a.d + 255) / 256;
  const int grid_dn = (int)std::min<long long>(max_tiles * ct_dn, ncu);
  hipLaunchKernelGGL(ffn_prompt_kernel<1>, dim3(grid_dn), dim3(kPromptThreads), kPromptLdsBytes, stream, a, ct_dn);
  return hipGetLastError();
}

}  // namespace moe
