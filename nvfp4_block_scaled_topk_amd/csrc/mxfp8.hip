// mxfp8.hip -- y = x . W^T for MXFP8 weights: E4M3 elements in blocks of 32 along K
// with one E8M0 scale a block, as a gemv for a few rows and a wide GEMM for many
// [FP4-Local checkpoints on DGX Spark, §4 Round 1, #521].
//
// The decoded weight E4M3 * 2^(s - 127) has 4 significant bits, so it is exact in
// bf16 for the scales in use; the activations stay bf16 and the products accumulate
// in fp32 on bf16 MFMA, rounded once to bf16 at the store. gfx950's scaled FP8
// conversion applies the power-of-two block scale while decoding (one instruction
// per two weights).
//
// gemv (M <= 16): one 16x16x32 MFMA tile covers every activation row; a wave owns 16
//   weight rows and streams them with 128-bit loads (16 elements a lane, half of a
//   scale block); KSPLIT waves split K and reduce in LDS in wave order.
// GEMM: 128 weight rows x 128 activation rows per block, 32x32x16 MFMA, weights from
//   registers (decoded in place), activations staged through LDS in 64-element steps.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kMxGemvKsplit = 4;
constexpr int kMxRows = 128;
constexpr int kMxKC = 64;
constexpr int kMxLdsRow = kMxKC * 2 + 16;

__device__ __forceinline__ floatx4 mx_mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mx_mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const uint32_t (&hb)[4], int nleft, bool vec) {
  if (vec && nleft >= 4) {
    uint2 v;
    v.x = hb[0] | (hb[1] << 16);
    v.y = hb[2] | (hb[3] << 16);
    *reinterpret_cast<uint2*>(p) = v;
  } else {
    for (int r = 0; r < 4 && r < nleft; ++r) p[r] = (uint16_t)hb[r];
  }
}

template <int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void mxfp8_gemv_kernel(const uint16_t* __restrict__ x, int M,
                                                                 int N, int K,
                                                                 const uint8_t* __restrict__ w,
                                                                 const uint8_t* __restrict__ s,
                                                                 uint16_t* __restrict__ y) {
  __shared__ floatx4 red[KSPLIT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + col;
  const bool nvalid = n < N;
  const uint8_t* wr = w + (size_t)(nvalid ? n : 0) * K;
  const uint8_t* sr = s + (size_t)(nvalid ? n : 0) * (K / 32);
  const bool mvalid = col < M;
  const uint16_t* xr = x + (size_t)(mvalid ? col : 0) * K;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nch = K / 64;
  const int c0 = nch * wave / KSPLIT, c1 = nch * (wave + 1) / KSPLIT;
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    u32x4 wv[2], xa[2], xb[2];
    uint32_t sb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int K0 = (c + h) * 64;
      wv[h] = nvalid ? ldg_u32x4(wr + K0 + 16 * grp) : zero;
      sb[h] = nvalid ? sr[K0 / 32 + (grp >> 1)] : 127u;
      xa[h] = mvalid ? ldg_u32x4(xr + K0 + 16 * grp) : zero;
      xb[h] = mvalid ? ldg_u32x4(xr + K0 + 16 * grp + 8) : zero;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float p2 = e8m0_pow2(sb[h]);
      acc = mx_mfma16(mxfp8x8_to_bf16(wv[h].x, wv[h].y, p2), u32x4_as_bf16x8(xa[h]), acc);
      acc = mx_mfma16(mxfp8x8_to_bf16(wv[h].z, wv[h].w, p2), u32x4_as_bf16x8(xb[h]), acc);
    }
  }
  for (; c < c1; ++c) {
    const int K0 = c * 64;
    const u32x4 wv = nvalid ? ldg_u32x4(wr + K0 + 16 * grp) : zero;
    const uint32_t sb = nvalid ? sr[K0 / 32 + (grp >> 1)] : 127u;
    const u32x4 xa = mvalid ? ldg_u32x4(xr + K0 + 16 * grp) : zero;
    const u32x4 xb = mvalid ? ldg_u32x4(xr + K0 + 16 * grp + 8) : zero;
    const float p2 = e8m0_pow2(sb);
    acc = mx_mfma16(mxfp8x8_to_bf16(wv.x, wv.y, p2), u32x4_as_bf16x8(xa), acc);
    acc = mx_mfma16(mxfp8x8_to_bf16(wv.z, wv.w, p2), u32x4_as_bf16x8(xb), acc);
  }
  if (wave == KSPLIT - 1 && (K & 63)) {
    // last 32 elements: lane group g holds elements K0 + 8g .. K0 + 8g + 7
    const int K0 = nch * 64;
    uint2 wv = make_uint2(0u, 0u);
    if (nvalid) wv = *reinterpret_cast<const uint2*>(wr + K0 + 8 * grp);
    const uint32_t sb = nvalid ? sr[K0 / 32] : 127u;
    const u32x4 xa = mvalid ? ldg_u32x4(xr + K0 + 8 * grp) : zero;
    acc = mx_mfma16(mxfp8x8_to_bf16(wv.x, wv.y, e8m0_pow2(sb)), u32x4_as_bf16x8(xa), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || !mvalid) return;
  floatx4 o = red[0][lane];
#pragma unroll
  for (int v = 1; v < KSPLIT; ++v) o += red[v][lane];
  const int nb = n0 + 4 * grp;  // lane holds activation row `col`, weight rows nb .. nb+3
  if (nb >= N) return;
  uint32_t hb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(o[r]);
  store_bf16x4(y + (size_t)col * N + nb, hb, N - nb, (N & 3) == 0);
}

__global__ __launch_bounds__(256) void mxfp8_gemm_kernel(const uint16_t* __restrict__ x, int M, int N,
                                                         int K, const uint8_t* __restrict__ w,
                                                         const uint8_t* __restrict__ s,
                                                         uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) unsigned char s_x[2][kMxRows * kMxLdsRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * 128 + wave * 32;  // this wave's 32 weight rows
  const int m0 = blockIdx.y * kMxRows;
  const int nrows = min(kMxRows, M - m0);
  const int ntf = (nrows + 31) >> 5;
  const bool nvalid = n0 + l32 < N;
  const bool wave_has_rows = n0 < N;
  const uint8_t* wr = w + (size_t)(nvalid ? n0 + l32 : 0) * K;
  const uint8_t* sr = s + (size_t)(nvalid ? n0 + l32 : 0) * (K / 32);
  const int srow = threadIdx.x >> 1, shalf = threadIdx.x & 1;
  const bool svalid = srow < nrows;
  const uint16_t* xr = x + (size_t)(svalid ? m0 + srow : 0) * K;
  const int nch = (K + kMxKC - 1) / kMxKC;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  floatx16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  u32x4 xs[4], wq[2];
  uint32_t sb;
  auto load_chunk = [&](int c, u32x4 (&xr4)[4], u32x4 (&wr2)[2], uint32_t& sbr) {
    const int K0 = c * kMxKC;
    const bool kv = K0 + 32 * shalf < K;
#pragma unroll
    for (int j = 0; j < 4; ++j) xr4[j] = (svalid && kv) ? ldg_u32x4(xr + K0 + 32 * shalf + 8 * j) : zero;
    const bool ok = nvalid && (K0 + 32 * g < K);
    wr2[0] = ok ? ldg_u32x4(wr + K0 + 32 * g) : zero;
    wr2[1] = ok ? ldg_u32x4(wr + K0 + 32 * g + 16) : zero;
    sbr = ok ? (uint32_t)sr[K0 / 32 + g] : 127u;
  };
  auto store_stage = [&](int stage, const u32x4 (&xr4)[4]) {
    unsigned char* dst = &s_x[stage][srow * kMxLdsRow + shalf * 64];
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(dst + 16 * j) = xr4[j];
  };

  load_chunk(0, xs, wq, sb);
  store_stage(0, xs);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const bool more = c + 1 < nch;
    u32x4 wn[2];
    uint32_t sbn;
    if (more) load_chunk(c + 1, xs, wn, sbn);
    const unsigned char* src = &s_x[c & 1][0];
    const float p2 = e8m0_pow2(sb);
    if (wave_has_rows) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4& wv = wq[st >> 1];
        const uint32_t lo = (st & 1) ? wv.z : wv.x;
        const uint32_t hi = (st & 1) ? wv.w : wv.y;
        const bf16x8 a = mxfp8x8_to_bf16(lo, hi, p2);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < ntf) {
            const u32x4 bv = *reinterpret_cast<const u32x4*>(src + (t * 32 + l32) * kMxLdsRow + 64 * g + 16 * st);
            acc[t] = mx_mfma32(a, u32x4_as_bf16x8(bv), acc[t]);
          }
        }
      }
    }
    if (more) store_stage((c + 1) & 1, xs);
    __syncthreads();
    if (more) {
      wq[0] = wn[0];
      wq[1] = wn[1];
      sb = sbn;
    }
  }
  if (!wave_has_rows) return;
  // accumulator r of fragment t: weight row n0 + 8*(r/4) + 4*g + r%4, activation row t*32 + l32
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = t * 32 + l32;
    if (t < ntf && m < nrows) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int nb = n0 + 8 * qd + 4 * g;
        if (nb < N) {
          uint32_t hb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(acc[t][4 * qd + r]);
          store_bf16x4(y + (size_t)(m0 + m) * N + nb, hb, N - nb, (N & 3) == 0);
        }
      }
    }
  }
}

hipError_t launch_mxfp8(const uint16_t* x, int M, int N, int K, const uint8_t* w, const uint8_t* s,
                        uint16_t* y, hipStream_t stream) {
  if (M <= 16) {
    hipLaunchKernelGGL(mxfp8_gemv_kernel<kMxGemvKsplit>, dim3((N + 15) / 16), dim3(64 * kMxGemvKsplit), 0,
                       stream, x, M, N, K, w, s, y);
  } else {
    hipLaunchKernelGGL(mxfp8_gemm_kernel, dim3((N + 127) / 128, (M + kMxRows - 1) / kMxRows), dim3(256), 0,
                       stream, x, M, N, K, w, s, y);
  }
  return hipGetLastError();
}

}  // namespace moe
