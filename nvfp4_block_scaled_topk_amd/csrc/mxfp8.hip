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
// gemv (M <= 4): vector ALUs, see mxfp8_gemv_valu_kernel.
// gemv (M <= 16): one 16x16x32 MFMA tile covers every activation row; a wave owns 16
//   weight rows and streams them with 128-bit loads (16 elements a lane, half of a
//   scale block); KSPLIT waves split K and reduce in LDS in wave order.
// GEMM: a tile of 128 activation rows x 192 weight rows per block of 8 waves (each wave
//   1 x 3 32x32x16 MFMA fragments: 32 activation rows x 96 weight rows; 512 x 12288 makes
//   256 tiles, one per CU). Activations
//   (bf16), weight codes (E4M3) and block scales (E8M0) reach LDS by buffer->LDS DMA in
//   four stages of 64 K elements, three stages ahead of the products, with no register
//   staging; out-of-range lanes read zeros, which also pads ragged tiles and the K
//   tail. Both operands sit in LDS in swizzled 16-byte slots so the MFMA operand reads
//   are free of bank conflicts. Blocks on one XCD take neighbouring tiles (same weight
//   rows), which then share that XCD's L2.
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kMxGemvKsplit = 4;

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
      wv[h] = nvalid ? ldg_nt_u32x4(wr + K0 + 16 * grp) : zero;
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
    const u32x4 wv = nvalid ? ldg_nt_u32x4(wr + K0 + 16 * grp) : zero;
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

// gemv for 1..4 activation rows on the vector ALUs: with so few rows the matrix cores
// add nothing, and plain per-row reads let each wave load 1 KB contiguous runs of a weight
// row (full cache lines, HBM bursts) instead of 64-byte pieces of 16 rows. A wave owns
// kVRows weight rows; lane l covers bytes [1024 i + 16 l, + 16) of each row in step i,
// decodes its 16 E4M3 codes with the scaled FP8 -> fp32 conversion (the block's E8M0
// scale applied on the way) and accumulates x . w in fp32; the wave then sums its lanes.
constexpr int kVRows = 2;        // weight rows a wave (measured: 2 beats 1, 4 and 8)
constexpr int kVThreads = 256;   // 4 waves

template <int MM>
__global__ __launch_bounds__(kVThreads) void mxfp8_gemv_valu_kernel(const uint16_t* __restrict__ x, int N, int K,
                                                                    const uint8_t* __restrict__ w,
                                                                    const uint8_t* __restrict__ s,
                                                                    uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * (kVThreads / 64) + wave) * kVRows;
  if (n0 >= N) return;
  float acc[kVRows][MM];
#pragma unroll
  for (int r = 0; r < kVRows; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[r][m] = 0.0f;
  const int nstep = (K + 1023) / 1024;
  for (int i = 0; i < nstep; ++i) {
    const int k0 = i * 1024 + lane * 16;  // this lane's 16 codes
    if (k0 >= K) break;                    // K is a multiple of 32: a lane's 16 codes are all in range or none
    // activations of this lane's 16 elements, as fp32
    float xf[MM][16];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const u32x4 xa = ldg_u32x4(x + (size_t)m * K + k0);
      const u32x4 xb = ldg_u32x4(x + (size_t)m * K + k0 + 8);
      const uint32_t wd[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xf[m][2 * j] = bits_f32(wd[j] << 16);
        xf[m][2 * j + 1] = bits_f32(wd[j] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int r = 0; r < kVRows; ++r) {
      const int n = n0 + r;
      if (n < N) {
        const u32x4 q = ldg_nt_u32x4(w + (size_t)n * K + k0);
        const float p2 = e8m0_pow2(s[(size_t)n * (K / 32) + k0 / 32]);
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(qw[j], p2, false);
          const floatx2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(qw[j], p2, true);
#pragma unroll
          for (int m = 0; m < MM; ++m) {
            acc[r][m] = fmaf(lo.x, xf[m][4 * j + 0], acc[r][m]);
            acc[r][m] = fmaf(lo.y, xf[m][4 * j + 1], acc[r][m]);
            acc[r][m] = fmaf(hi.x, xf[m][4 * j + 2], acc[r][m]);
            acc[r][m] = fmaf(hi.y, xf[m][4 * j + 3], acc[r][m]);
          }
        }
      }
    }
  }
  // sum over the wave's lanes (fixed order: the result is the same on every run)
#pragma unroll
  for (int r = 0; r < kVRows; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      acc[r][m] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kVRows; ++r)
      if (n0 + r < N)
#pragma unroll
        for (int m = 0; m < MM; ++m) y[(size_t)m * N + n0 + r] = bf16_rne(acc[r][m]);
  }
}

constexpr int kGM = 128;                        // activation rows per tile
constexpr int kGN = 192;                        // weight rows per tile
constexpr int kGK = 64;                         // K elements per stage
constexpr int kGStages = 4;
constexpr int kGXBytes = kGM * kGK * 2;         // 16 KB: 128 rows x 128 bytes
constexpr int kGWBytes = kGN * kGK;             // 12 KB: 192 rows x 64 bytes
constexpr int kGSBytes = 8 * 64 * 4;            // 2 KB: a dword slot per (row, block)
constexpr int kGSRow = 128;                     // preloaded scale bytes a weight row (K <= 4096)
// a stage holds activations, weight codes and (without the scale preload) scales
template <bool PRE>
constexpr int gemm_stage_bytes() { return kGXBytes + kGWBytes + (PRE ? 0 : kGSBytes); }
// the stages, a 1 KB sink (see issue()) and, with the preload, the tile's scale rows
template <bool PRE>
constexpr int gemm_lds_bytes() { return kGStages * gemm_stage_bytes<PRE>() + 1024 + (PRE ? kGN * kGSRow : 0); }
constexpr int kGThreads = 512;
constexpr int kGOps = 5;                        // DMA instructions a wave issues per stage
constexpr uint32_t kGOOB = 0x80000000u;         // a buffer offset past every record: reads zeros

typedef __attribute__((address_space(3))) void* gemm_lds_ptr;
typedef uint32_t gu32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
template <int N>
__device__ __forceinline__ void gemm_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void gemm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS layout of a stage (the slot patterns give the 16 rows that 16 lanes read 16
// distinct 16-byte bank groups):
//   x: row r (128 bytes = 8 slots of 16 bytes), logical segment j in slot j ^ ((r >> 1) & 7);
//   W: row r (64 bytes = 4 slots), logical segment j in slot j ^ ((r >> 2) & 3);
//   scales: wave w's region holds rows 32w .. 32w + 31, (row, block b) in dword slot
//   2 * (row & 31) + b -- or, when K is a multiple of 512 and at most 4096, all of the
//   tile's scale rows come in once before the K loop, in whole 128-byte rows (a DMA
//   instruction reads 8 full cache lines instead of one byte of 32 rows every stage):
//   row r's logical 16-byte segment j in slot j ^ ((r >> 1) & 7) of its 128 bytes.
// MFMA K order within a stage (a permutation of K applied to both operands): lane group
// g (lane / 32) at step 2p + h takes W bytes 8h .. 8h + 7 of segment 2p + g, i.e. K
// elements 16 * (2p + g) + 8h .. + 7, which are activation segment 4p + 2g + h.
template <bool PRE>
__global__ __launch_bounds__(kGThreads, 1) void mxfp8_gemm_kernel(const uint16_t* __restrict__ x, int M, int N,
                                                                  int K, const uint8_t* __restrict__ w,
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
  const int m0 = mt * kGM, n0 = nt * kGN;

  const __amdgpu_buffer_rsrc_t xrs = gemm_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t wrs = gemm_rsrc(w, (uint32_t)((size_t)N * K));
  const __amdgpu_buffer_rsrc_t srs = gemm_rsrc(s, (uint32_t)((size_t)N * (K / 32)));

  // per-lane DMA sources (byte offsets; the stage's K offset goes in soffset)
  uint32_t xoff[2], woff[2];
  int xseg[2], wseg[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ins = wave * 2 + i;
    const int xr = ins * 8 + (lane >> 3);           // activation row in the tile
    xseg[i] = (lane & 7) ^ ((xr >> 1) & 7);          // logical segment this lane fetches
    xoff[i] = (m0 + xr < M) ? (uint32_t)(m0 + xr) * (uint32_t)(K * 2) + xseg[i] * 16 : kGOOB;
    const int wr = ins * 16 + (lane >> 2);           // weight row in the tile (past kGN: no row)
    wseg[i] = (lane & 3) ^ ((wr >> 2) & 3);
    woff[i] = (wr < kGN && n0 + wr < N) ? (uint32_t)(n0 + wr) * (uint32_t)K + wseg[i] * 16 : kGOOB;
  }
  const int srow = wave * 32 + (lane >> 1), sblk = lane & 1;
  const uint32_t soff = (srow < kGN && n0 + srow < N) ? (uint32_t)(n0 + srow) * (uint32_t)(K / 32) + sblk : kGOOB;
  const int nst = (K + kGK - 1) / kGK;
  constexpr int kStage = gemm_stage_bytes<PRE>();
  constexpr int kOps = PRE ? 4 : kGOps;  // DMA instructions a wave issues per stage
  unsigned char* const sink = smem + kGStages * kStage;
  unsigned char* const scl = sink + 1024;  // preloaded scale rows

  if (PRE) {
    // the tile's scale rows: 24 instructions of 8 rows x 128 bytes, 3 a wave
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int ins = wave * 3 + j;
      const int r = ins * 8 + (lane >> 3);
      const int seg = (lane & 7) ^ ((r >> 1) & 7);
      const uint32_t off = (n0 + r < N && seg * 16 < K / 32) ? (uint32_t)(n0 + r) * (uint32_t)(K / 32) + seg * 16 : kGOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (gemm_lds_ptr)(scl + ins * 1024), 16, off, 0, 0, 0);
    }
  }

  auto issue = [&](int c) {
    unsigned char* st = smem + (c % kGStages) * kStage;
    const int K0 = c * kGK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool xin = K0 + 8 * xseg[i] < K;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (gemm_lds_ptr)(st + (wave * 2 + i) * 1024), 16,
                                               xin ? xoff[i] : kGOOB, K0 * 2, 0, 0);
    }
    // 12 weight instructions a stage; the waves past them issue theirs too (every wave
    // has the same number of loads in flight, so the waits stay exact), reading zeros
    // into a 1 KB sink past the stages
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ins = wave * 2 + i;
      const bool win = K0 + 16 * wseg[i] < K;
      unsigned char* dst = ins * 16 < kGN ? st + kGXBytes + ins * 1024 : sink;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (gemm_lds_ptr)dst, 16, win ? woff[i] : kGOOB, K0, 0, 0);
    }
    if (!PRE) {
      const bool sin = K0 + 32 * sblk < K;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (gemm_lds_ptr)(st + kGXBytes + kGWBytes + wave * 256), 1,
                                               sin ? soff : kGOOB, K0 / 32, 0, 0);
    }
  };

  floatx16 acc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  for (int c = 0; c < kGStages - 1 && c < nst; ++c) issue(c);
  for (int c = 0; c < nst; ++c) {
    // stage c's loads are the oldest in flight; later stages may still be outstanding
    if (c + 2 < nst) gemm_wait_vm<2 * kOps>();
    else if (c + 1 < nst) gemm_wait_vm<kOps>();
    else gemm_wait_vm<0>();
    gemm_barrier();  // every wave's part of stage c is in LDS; stage c - 1 is consumed
    if (c + kGStages - 1 < nst) issue(c + kGStages - 1);

    const unsigned char* st = smem + (c % kGStages) * kStage;
    const unsigned char* xs = st;
    const unsigned char* ws = st + kGXBytes;
    const unsigned char* ss = st + kGXBytes + kGWBytes;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      gu32x4v wv[3];
      float p2[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int r = nb * 96 + i * 32 + l32;
        const int slot = (2 * p + g) ^ ((r >> 2) & 3);
        wv[i] = *reinterpret_cast<const gu32x4v*>(ws + r * 64 + slot * 16);
        uint32_t code;
        if (PRE) {
          const int b = 2 * c + p;  // scale block of this half stage
          code = *(scl + r * kGSRow + (((b >> 4) ^ ((r >> 1) & 7)) * 16) + (b & 15));
        } else {
          code = *(ss + (r >> 5) * 256 + ((r & 31) * 2 + p) * 4);
        }
        p2[i] = e8m0_pow2(code);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 a[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) a[i] = mxfp8x8_to_bf16(wv[i][2 * h], wv[i][2 * h + 1], p2[i]);
        const int r = ma * 32 + l32;
        const int j = 4 * p + 2 * g + h;
        const gu32x4v bv = *reinterpret_cast<const gu32x4v*>(xs + r * 128 + ((j ^ ((r >> 1) & 7)) * 16));
        const bf16x8 b = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
        for (int i = 0; i < 3; ++i) acc[i] = mx_mfma32(a[i], b, acc[i]);
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
          store_bf16x4(y + (size_t)m * N + n, hb, N - n, (N & 3) == 0);
        }
      }
    }
  }
}

// The few-row kernels, by id: the vector-ALU gemv (M <= 8), the MFMA gemv (M <= 16) and
// the tiled GEMM (any M). Which is fastest for M = 1..16 depends on the card (clocks, HBM,
// cache sizes); mxfp8_autotune times them on the caller's operands and records the pick
// per (device, M, N, K). Without a record: vector ALUs for M <= 4, the MFMA gemv up to 16.
hipError_t launch_mxfp8_kernel(int kernel, const uint16_t* x, int M, int N, int K, const uint8_t* w, const uint8_t* s,
                               uint16_t* y, hipStream_t stream) {
  if (kernel == kMxValuGemv && M >= 1 && M <= 8) {
    const dim3 grid((N + kVRows * (kVThreads / 64) - 1) / (kVRows * (kVThreads / 64)));
    switch (M) {
      case 1: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<1>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      case 2: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<2>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      case 3: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<3>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      case 4: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<4>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      case 5: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<5>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      case 6: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<6>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      case 7: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<7>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
      default: hipLaunchKernelGGL(mxfp8_gemv_valu_kernel<8>, grid, dim3(kVThreads), 0, stream, x, N, K, w, s, y); break;
    }
    return hipGetLastError();
  }
  if (kernel == kMxMfmaGemv && M >= 1 && M <= 16) {
    hipLaunchKernelGGL(mxfp8_gemv_kernel<kMxGemvKsplit>, dim3((N + 15) / 16), dim3(64 * kMxGemvKsplit), 0,
                       stream, x, M, N, K, w, s, y);
    return hipGetLastError();
  }
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&mxfp8_gemm_kernel<true>), gemm_lds_bytes<true>());
  if (e == hipSuccess)
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(&mxfp8_gemm_kernel<false>), gemm_lds_bytes<false>());
  if (e != hipSuccess) return e;
  const int mtiles = (M + kGM - 1) / kGM, ntiles = (N + kGN - 1) / kGN;
  if (K % 512 == 0 && K / 32 <= kGSRow)
    hipLaunchKernelGGL(mxfp8_gemm_kernel<true>, dim3(mtiles * ntiles), dim3(kGThreads), gemm_lds_bytes<true>(),
                       stream, x, M, N, K, w, s, y, mtiles);
  else
    hipLaunchKernelGGL(mxfp8_gemm_kernel<false>, dim3(mtiles * ntiles), dim3(kGThreads), gemm_lds_bytes<false>(),
                       stream, x, M, N, K, w, s, y, mtiles);
  return hipGetLastError();
}

int mxfp8_default_kernel(int M) { return M <= 4 ? kMxValuGemv : M <= 16 ? kMxMfmaGemv : kMxTiledGemm; }

hipError_t launch_mxfp8(const uint16_t* x, int M, int N, int K, const uint8_t* w, const uint8_t* s,
                        uint16_t* y, hipStream_t stream) {
  int kernel = mxfp8_default_kernel(M);
  if (M <= 16) {
    const int forced = mxfp8_forced_kernel();
    int picked = -1;
    if (forced >= 0) kernel = forced;
    else if (mxfp8_recorded_kernel(M, N, K, picked) == hipSuccess && picked >= 0) kernel = picked;
  }
  return launch_mxfp8_kernel(kernel, x, M, N, K, w, s, y, stream);
}

}  // namespace moe
