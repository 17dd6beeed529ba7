// mxfp8_w8a8.hip -- MXFP8 activations and the W8A8 MXFP8 projection.
//
// The pages run an MXFP8 projection with 8-bit activations beside the bf16-activation one
// [FP4-Local checkpoints on DGX Spark, §4 Round 1, #769]. Here the activations are
// quantized once to MXFP8 (E4M3 elements in blocks of 32 along K, one E8M0 scale a
// block, by the OCP MX v1.0 conversion) and the product runs on gfx950's block-scaled
// matrix instruction, v_mfma_scale_f32_32x32x64_f8f6f4: both operands stay 8-bit and the
// two E8M0 block scales are applied by the matrix core itself, so nothing is decoded in
// registers.
//
// mx_quantize_kernel: a thread per block of 32 bf16 values. The block scale exponent is
//   floor(log2 max|v|) - 8 (8: the largest exponent of E4M3), clamped to the E8M0 code
//   range (an all-zero block gets code 0); elements are v / scale (exact: a power of two),
//   saturated to +-448, rounded to nearest even by the hardware's FP8 conversion.
// mx_gemm_kernel: the tiling of the bf16-activation MXFP8 GEMM (mxfp8.hip): a tile of 128
//   activation rows x 192 weight rows per block of 8 waves, each wave 32 activation rows
//   x 96 weight rows (three 32x32 fragments); activation and weight codes reach LDS by
//   buffer->LDS DMA in four stages of 64 K elements, three ahead; both operands' scale
//   rows come in once before the K loop (K a multiple of 512, at most 4096). A stage is
//   one scaled MFMA a fragment. Its operand layout (checked on the device with
//   controlled inputs): lane group g (lane / 32) holds K elements 16g .. 16g + 15 of the
//   row in its bytes 0-15 and 32 + 16g .. 32 + 16g + 15 in bytes 16-31; bytes 0-15 of
//   both lane groups form the first block of 32, scaled by the scale the g = 0 lane
//   supplies for its row, bytes 16-31 the second, scaled by the g = 1 lane's.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void mx_quantize_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                                uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const long long b = (long long)blockIdx.x * kQThreads + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 32);
  uint32_t h[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = src[i];
    h[4 * i] = v.x;
    h[4 * i + 1] = v.y;
    h[4 * i + 2] = v.z;
    h[4 * i + 3] = v.w;
  }
  // largest magnitude: bf16 magnitudes order as integers
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(h[i] & 0x7FFFu, (h[i] >> 16) & 0x7FFFu));
  int code = 0;
  if (amax != 0) {
    const int e = __builtin_amdgcn_frexp_expf(bf16_to_f32((uint16_t)amax));  // amax = m 2^e, m in [0.5, 1)
    code = min(max((e - 1) - 8 + 127, 0), 254);
  }
  const float inv = __builtin_ldexpf(1.0f, 127 - code);  // 1 / scale, a power of two
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = h[2 * i + (j >> 1)];
      const float v = bf16_to_f32((uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu))) * inv;
      f[j] = fminf(fmaxf(v, -448.0f), 448.0f);
    }
    uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], p, true);
    out[i] = p;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(xq + b * 32);
  dst[0] = u32x4{out[0], out[1], out[2], out[3]};
  dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  xs[b] = (uint8_t)code;
}

hipError_t launch_mx_quantize(const uint16_t* x, int M, int K, uint8_t* xq, uint8_t* xs, hipStream_t stream) {
  const long long nb = (long long)M * (K / 32);
  const long long grid = (nb + kQThreads - 1) / kQThreads;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream, x, nb, xq, xs);
  return hipGetLastError();
}

constexpr int kWM = 128;                 // activation rows per tile
constexpr int kWN = 192;                 // weight rows per tile
constexpr int kWK = 64;                  // K elements per stage
constexpr int kWStages = 4;
constexpr int kWXBytes = kWM * kWK;      // 8 KB: 128 rows x 64 bytes
constexpr int kWWBytes = kWN * kWK;      // 12 KB: 192 rows x 64 bytes
constexpr int kWStage = kWXBytes + kWWBytes;
constexpr int kWSRow = 128;              // preloaded scale bytes a row (K <= 4096)
constexpr int kWLds = kWStages * kWStage + 1024 + (kWN + kWM) * kWSRow;
constexpr int kWThreads = 512;
constexpr int kWOps = 3;                 // DMA instructions a wave issues per stage
constexpr uint32_t kWOOB = 0x80000000u;  // a buffer offset past every record: reads zeros

typedef __attribute__((address_space(3))) void* w8_lds_ptr;
typedef uint32_t w8u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w8_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
template <int N>
__device__ __forceinline__ void w8_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void w8_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS layout: a stage holds the activation codes (row r: 64 bytes = 4 slots of 16, logical
// segment j in slot j ^ ((r >> 2) & 3): the 16 rows that 16 lanes of an operand read
// then fall on 16 distinct 16-byte bank groups) then the weight codes (same layout); after
// the stages a 1 KB sink, then the tile's scale rows (weights, then activations; row r's
// logical 16-byte segment j in slot j ^ (r & 7) of its 128 bytes). A lane reads the
// 16-byte segment of its rows' scales once per 8 stages (16 blocks) and takes a byte a
// stage from registers.
__global__ __launch_bounds__(kWThreads, 1) void mx_gemm_kernel(const uint8_t* __restrict__ xq,
                                                             const uint8_t* __restrict__ xs, int M, int N, int K,
                                                             const uint8_t* __restrict__ w,
                                                             const uint8_t* __restrict__ s,
                                                             uint16_t* __restrict__ y, int mtiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int ma = wave >> 1;  // 32-row quarter of the activation tile
  const int nb = wave & 1;   // 96-row half of the weight tile (three 32-row fragments)

  // tile of this block: XCD-aware order, neighbouring tiles share weight rows
  const int G = gridDim.x;
  const int lid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const int nt = lid / mtiles, mt = lid - nt * mtiles;
  const int m0 = mt * kWM, n0 = nt * kWN;

  const __amdgpu_buffer_rsrc_t xrs = w8_rsrc(xq, (uint32_t)((size_t)M * K));
  const __amdgpu_buffer_rsrc_t xsrs = w8_rsrc(xs, (uint32_t)((size_t)M * (K / 32)));
  const __amdgpu_buffer_rsrc_t wrs = w8_rsrc(w, (uint32_t)((size_t)N * K));
  const __amdgpu_buffer_rsrc_t srs = w8_rsrc(s, (uint32_t)((size_t)N * (K / 32)));

  // per-lane DMA sources: one activation instruction (16 rows x 64 bytes) and two weight
  // instructions a wave per stage; the stage's K offset goes in soffset
  const int xr = wave * 16 + (lane >> 2);
  const int xseg = (lane & 3) ^ ((xr >> 2) & 3);
  const uint32_t xoff = (m0 + xr < M) ? (uint32_t)(m0 + xr) * (uint32_t)K + xseg * 16 : kWOOB;
  uint32_t woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int wr = (wave * 2 + i) * 16 + (lane >> 2);  // weight row in the tile (past kWN: no row)
    const int wseg = (lane & 3) ^ ((wr >> 2) & 3);
    woff[i] = (wr < kWN && n0 + wr < N) ? (uint32_t)(n0 + wr) * (uint32_t)K + wseg * 16 : kWOOB;
  }
  const int nst = K / kWK;
  unsigned char* const sink = smem + kWStages * kWStage;
  unsigned char* const wscl = sink + 1024;
  unsigned char* const xscl = wscl + kWN * kWSRow;

  // the tile's scale rows: 24 weight and 16 activation instructions of 8 rows x 128 bytes
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int ins = wave * 5 + j;  // 0..39
    if (ins < 24) {
      const int r = ins * 8 + (lane >> 3);
      const int seg = (lane & 7) ^ (r & 7);
      const uint32_t off = (n0 + r < N && seg * 16 < K / 32) ? (uint32_t)(n0 + r) * (uint32_t)(K / 32) + seg * 16 : kWOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (w8_lds_ptr)(wscl + ins * 1024), 16, off, 0, 0, 0);
    } else {
      const int r = (ins - 24) * 8 + (lane >> 3);
      const int seg = (lane & 7) ^ (r & 7);
      const uint32_t off = (m0 + r < M && seg * 16 < K / 32) ? (uint32_t)(m0 + r) * (uint32_t)(K / 32) + seg * 16 : kWOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrs, (w8_lds_ptr)(xscl + (ins - 24) * 1024), 16, off, 0, 0, 0);
    }
  }

  auto issue = [&](int c) {
    unsigned char* st = smem + (c % kWStages) * kWStage;
    const int K0 = c * kWK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (w8_lds_ptr)(st + wave * 1024), 16, xoff, K0, 0, 0);
    // 12 weight instructions a stage; the waves past them issue theirs too (every wave
    // has the same number of loads in flight, so the waits stay exact), reading zeros
    // into a 1 KB sink past the stages
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ins = wave * 2 + i;
      unsigned char* dst = ins * 16 < kWN ? st + kWXBytes + ins * 1024 : sink;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (w8_lds_ptr)dst, 16, woff[i], K0, 0, 0);
    }
  };

  floatx16 acc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  for (int c = 0; c < kWStages - 1 && c < nst; ++c) issue(c);
  const int rx = ma * 32 + l32;  // this lane's activation row of the tile
  int rw[3];                      // and its weight rows
#pragma unroll
  for (int i = 0; i < 3; ++i) rw[i] = nb * 96 + i * 32 + l32;
  // stages in groups of 8 (nst is a multiple of 8: K % 512 == 0): the group's 16 scale
  // blocks of each of the lane's rows are one 16-byte segment of the scale rows
  for (int c8 = 0; c8 < nst; c8 += 8) {
    const int seg = c8 >> 3;  // segment of blocks 16 seg .. 16 seg + 15
    w8u32x4 xsv, wsv[3];
#pragma unroll 1
    for (int cc = 0; cc < 8; ++cc) {
      const int c = c8 + cc;
      // stage c's loads are the oldest in flight (the scale rows before them); later
      // stages may still be outstanding
      if (c + 2 < nst) w8_wait_vm<2 * kWOps>();
      else if (c + 1 < nst) w8_wait_vm<kWOps>();
      else w8_wait_vm<0>();
      w8_barrier();  // every wave's part of stage c is in LDS; stage c - 1 is consumed
      if (c + kWStages - 1 < nst) issue(c + kWStages - 1);
      if (cc == 0) {
        xsv = *reinterpret_cast<const w8u32x4*>(xscl + rx * kWSRow + ((seg ^ (rx & 7)) * 16));
#pragma unroll
        for (int i = 0; i < 3; ++i)
          wsv[i] = *reinterpret_cast<const w8u32x4*>(wscl + rw[i] * kWSRow + ((seg ^ (rw[i] & 7)) * 16));
      }
      // the scale block this lane supplies: 2c + g, byte 2 cc + g of the segment, in
      // dword cc / 2 at bit 8 (2 (cc % 2) + g)
      const int sh = 8 * (2 * (cc & 1) + g);
      auto pick = [&](const w8u32x4& v) -> int {
        const uint32_t d = (cc >> 1) == 0 ? v.x : (cc >> 1) == 1 ? v.y : (cc >> 1) == 2 ? v.z : v.w;
        return (int)((d >> sh) & 0xFFu);
      };

      const unsigned char* st = smem + (c % kWStages) * kWStage;
      const unsigned char* xsm = st;
      const unsigned char* wsm = st + kWXBytes;
      // activation operand: row rx; lane group g holds the stage's K elements 16g .. 16g + 15
      // (of scale block 2c) and 32 + 16g .. 32 + 16g + 15 (of block 2c + 1)
      const w8u32x4 x0 = *reinterpret_cast<const w8u32x4*>(xsm + rx * 64 + ((g ^ ((rx >> 2) & 3)) * 16));
      const w8u32x4 x1 = *reinterpret_cast<const w8u32x4*>(xsm + rx * 64 + (((g + 2) ^ ((rx >> 2) & 3)) * 16));
      const i32x8 bop = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      const int xsc = pick(xsv);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int r = rw[i];
        const w8u32x4 w0 = *reinterpret_cast<const w8u32x4*>(wsm + r * 64 + ((g ^ ((r >> 2) & 3)) * 16));
        const w8u32x4 w1 = *reinterpret_cast<const w8u32x4*>(wsm + r * 64 + (((g + 2) ^ ((r >> 2) & 3)) * 16));
        const i32x8 aop = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc[i], 0, 0, 0, pick(wsv[i]), 0, xsc);
      }
    }
  }

  // accumulator r of fragment i: weight row 8 * (r / 4) + 4 * g + r % 4 of the
  // fragment, activation row l32 of the wave's 32 rows
  const int m = m0 + ma * 32 + l32;
  if (m < M) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int n = n0 + nb * 96 + i * 32 + 8 * qd + 4 * g;
        if (n < N) {
          uint32_t hb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hb[r] = bf16_rne(acc[i][4 * qd + r]);
          uint16_t* p = y + (size_t)m * N + n;
          if ((N & 3) == 0 && N - n >= 4) {
            uint2 v;
            v.x = hb[0] | (hb[1] << 16);
            v.y = hb[2] | (hb[3] << 16);
            *reinterpret_cast<uint2*>(p) = v;
          } else {
            for (int r = 0; r < 4 && r < N - n; ++r) p[r] = (uint16_t)hb[r];
          }
        }
      }
    }
  }
}

hipError_t launch_mx_gemm(const uint8_t* xq, const uint8_t* xs, int M, int N, int K, const uint8_t* w,
                          const uint8_t* s, uint16_t* y, hipStream_t stream) {
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&mx_gemm_kernel), kWLds);
  if (err != hipSuccess) return err;
  const int mtiles = (M + kWM - 1) / kWM, ntiles = (N + kWN - 1) / kWN;
  hipLaunchKernelGGL(mx_gemm_kernel, dim3(mtiles * ntiles), dim3(kWThreads), kWLds, stream, xq, xs, M, N, K, w, s, y,
                     mtiles);
  return hipGetLastError();
}

}  // namespace moe
