// ffn_prompt.hip -- the expert FFN for many tokens (prompt): a grouped GEMM over the
// per-expert row lists.
//
// The pages' prompt path admits routed NVFP4 experts into a grouped GEMM whose store
// scales each row by its expert's tensor scale [FP4-Local checkpoints on DGX Spark,
// §4 Round 1, #545], runs gate, up and SwiGLU as one launch (#766) and walks K in
// 128-element steps with a three-stage operand copy (§4 remaining items, #822). Here:
//
//   tile    = (expert e, 128 routed rows of e, 128 features of f)   [gate/up launch]
//             (expert e, 128 routed rows of e, 256 columns of d)    [down launch]
//   waves   = 4; wave w owns two 32-row weight fragments (gate and up of the same 32
//             features, or two 32-column slices of d) and all 128 routed rows
//   MFMA    = v_mfma_f32_32x32x16_bf16, weights as the A operand, activations as B
//   K step  = 64 elements per LDS stage, two stages (global -> registers -> LDS)
//
// Weights never touch LDS: each weight row belongs to exactly one wave, which loads
// its packed codes with 128-bit loads (32 codes = two scale blocks per lane) and
// decodes them in registers (exact, see device.hpp). The activation tile (gathered
// through the row list for gate/up, contiguous H rows for down) is shared by the four
// waves through LDS. The fp32 tensor scale multiplies the accumulator in the epilogue;
// gate/up's epilogue forms H = bf16_rne(silu(G) * U), down's writes fp32 rows.
//
// Work: one flat list of tiles (expert-major, column tile fastest) walked by a
// persistent grid; each block derives the list from expert_offsets in LDS.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kPromptRows = 128;                 // routed rows per tile
constexpr int kPromptKC = 64;                    // K per LDS stage
constexpr int kPromptLdsRow = kPromptKC * 2 + 16;  // bytes per LDS activation row (padded)
constexpr int kPromptStage = kPromptRows * kPromptLdsRow;
constexpr int kPromptThreads = 256;
constexpr int kMaxE = 1024;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word4(const u32x4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Per-block tile table: s_pref[e] = number of 128-row tiles of experts < e.
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int* s_cnt,
                                  int* s_pref) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int n = offsets[e + 1] - offsets[e];
    s_cnt[e] = (n + kPromptRows - 1) / kPromptRows;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // one wave scans E entries, 64 at a time
    const int lane = threadIdx.x;
    int run = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int v = e < E ? s_cnt[e] : 0;
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
__global__ __launch_bounds__(kPromptThreads) void ffn_prompt_kernel(FFNArgs a, int n_col_tiles) {
  __shared__ __attribute__((aligned(16))) unsigned char s_x[2][kPromptStage];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_pref[kMaxE + 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int K = MODE == 0 ? a.d : a.f;       // contraction length
  const int N = MODE == 0 ? a.f : a.d;       // weight rows per matrix
  const int nch = (K + kPromptKC - 1) / kPromptKC;

  build_tile_prefix(a.offsets, a.E, s_cnt, s_pref);
  const int total_tiles = s_pref[a.E] * n_col_tiles;

  for (int item = blockIdx.x; item < total_tiles; item += gridDim.x) {
    const int mt_all = item / n_col_tiles;
    const int ct = item - mt_all * n_col_tiles;
    const int e = find_tile_expert(s_pref, a.E, mt_all);
    const int mt = mt_all - s_pref[e];
    const int p0 = a.offsets[e] + mt * kPromptRows;
    const int nrows = min(kPromptRows, a.offsets[e + 1] - p0);
    const int ntf = (nrows + 31) >> 5;  // 32-row activation fragments in use

    // ---- this wave's two weight fragments
    int frow[2];
    if (MODE == 0) {
      frow[0] = frow[1] = ct * 128 + wave * 32;  // gate and up rows of the same features
    } else {
      frow[0] = ct * 256 + wave * 64;
      frow[1] = frow[0] + 32;
    }
    const bool fvalid[2] = {frow[0] < N, frow[1] < N};
    const uint8_t* wq[2];
    const uint8_t* wsc[2];
    {
      const uint8_t* q0 = MODE == 0 ? a.gate_q : a.down_q;
      const uint8_t* s0 = MODE == 0 ? a.gate_s : a.down_s;
      const uint8_t* q1 = MODE == 0 ? a.up_q : a.down_q;
      const uint8_t* s1 = MODE == 0 ? a.up_s : a.down_s;
      const size_t r0 = (size_t)e * N + (fvalid[0] ? frow[0] + l32 : 0);
      const size_t r1 = (size_t)e * N + (fvalid[1] ? frow[1] + l32 : 0);
      wq[0] = q0 + r0 * (K / 2);
      wsc[0] = s0 + r0 * (K / 16);
      wq[1] = q1 + r1 * (K / 2);
      wsc[1] = s1 + r1 * (K / 16);
    }

    // ---- the activation rows this thread stages: row = tid / 2, 32 elements a chunk
    const int srow = threadIdx.x >> 1, shalf = threadIdx.x & 1;
    const bool svalid = srow < nrows;
    const uint16_t* sact;
    if (MODE == 0) {
      const int tok = svalid ? a.sorted_rows[p0 + srow] / a.k : 0;
      sact = a.x + (size_t)tok * a.d;
    } else {
      sact = a.h + (size_t)(svalid ? p0 + srow : 0) * a.f;
    }

    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.0f;

    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 xs[4];
    u32x4 q[2];
    uint32_t sc[2];
    auto load_chunk = [&](int c, u32x4 (&xr)[4], u32x4 (&qr)[2], uint32_t (&sr)[2]) {
      const int K0 = c * kPromptKC;
      const bool kv = K0 + 32 * shalf < K;
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[j] = (svalid && kv) ? ldg_u32x4(sact + K0 + 32 * shalf + 8 * j) : zero;
      const bool wk = K0 + 32 * g < K;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = fvalid[i] && wk;
        qr[i] = ok ? ldg_u32x4(wq[i] + K0 / 2 + 16 * g) : zero;
        sr[i] = ok ? (uint32_t)(*reinterpret_cast<const uint16_t*>(wsc[i] + K0 / 16 + 2 * g)) : 0u;
      }
    };
    auto store_stage = [&](int stage, const u32x4 (&xr)[4]) {
      unsigned char* dst = &s_x[stage][srow * kPromptLdsRow + shalf * 64];
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(dst + 16 * j) = xr[j];
    };

    load_chunk(0, xs, q, sc);
    store_stage(0, xs);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const bool more = c + 1 < nch;
      u32x4 qn[2];
      uint32_t scn[2];
      if (more) load_chunk(c + 1, xs, qn, scn);
      const unsigned char* src = &s_x[c & 1][0];
      E4M3Split sp[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        sp[i][0] = e4m3_split(sc[i] & 0xFFu);
        sp[i][1] = e4m3_split(sc[i] >> 8);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 wa[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) wa[i] = nvfp4x8_to_bf16(word4(q[i], s), sp[i][s >> 1]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < ntf) {
            const u32x4 bv =
                *reinterpret_cast<const u32x4*>(src + (t * 32 + l32) * kPromptLdsRow + 64 * g + 16 * s);
            const bf16x8 b = u32x4_as_bf16x8(bv);
#pragma unroll
            for (int i = 0; i < 2; ++i)
              if (fvalid[i]) acc[i][t] = mfma32(wa[i], b, acc[i][t]);
          }
        }
      }
      if (more) store_stage((c + 1) & 1, xs);
      __syncthreads();
      if (more) {
        q[0] = qn[0];
        q[1] = qn[1];
        sc[0] = scn[0];
        sc[1] = scn[1];
      }
    }

    // ---- epilogue. Accumulator r of fragment (i, t): weight row 8*(r/4) + 4*g + r%4 of
    // the fragment, activation row t*32 + l32 of the tile.
    if (MODE == 0) {
      if (fvalid[0]) {
        const float tg = a.gate_ts[e], tu = a.up_ts[e];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = t * 32 + l32;
          if (t < ntf && row < nrows) {
            uint16_t* hp = a.h + (size_t)(p0 + row) * a.f + frow[0] + 4 * g;
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
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = t * 32 + l32;
          if (t < ntf && row < nrows) {
            float* yp = a.y_rows + (size_t)(p0 + row) * a.d + frow[i] + 4 * g;
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

hipError_t launch_ffn_prompt(const FFNArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.T * a.k;
  const long long max_tiles = rows / kPromptRows + std::min<long long>(a.E, rows);
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ncu = v;
  }
  const int ct_gu = (a.f + 127) / 128;
  const long long items_gu = max_tiles * ct_gu;
  const int grid_gu = (int)std::min<long long>(items_gu, 2LL * ncu);
  hipLaunchKernelGGL(ffn_prompt_kernel<0>, dim3(grid_gu), dim3(kPromptThreads), 0, stream, a, ct_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ct_dn = (a.d + 255) / 256;
  const long long items_dn = max_tiles * ct_dn;
  const int grid_dn = (int)std::min<long long>(items_dn, 2LL * ncu);
  hipLaunchKernelGGL(ffn_prompt_kernel<1>, dim3(grid_dn), dim3(kPromptThreads), 0, stream, a, ct_dn);
  return hipGetLastError();
}

}  // namespace moe
