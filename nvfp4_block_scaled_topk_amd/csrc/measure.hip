// measure.hip -- a plain streaming read of given byte ranges: the ceiling the benchmark
// reports beside the expert kernels (how fast this part reads the same bytes with nothing
// else to do), as the pages report results against a measured baseline [FP4-Local
// checkpoints on DGX Spark, §3 How results are measured].
//
// The ranges (device address, bytes; both multiples of 16) come as a table in device
// memory. Every workgroup owns 32 KB pieces of the concatenated ranges, grid-stride; a
// thread reads 16 bytes at a time with the non-temporal hint of the weight streams, eight
// loads in flight (a whole piece per round, also where a piece straddles two ranges), and
// folds them with xor; a workgroup writes one word to `sink` (so the loads are not dead
// code). Measured on the decode layer's 45 MB (17 experts' codes and scales, 24 rotating
// weight copies), when parts shorter than eight rounds still took one load at a time:
// the 102 ranges of the stored layout 15.7 us, the same bytes as 17 contiguous ranges
// 12.2 us and as one flat buffer 11.8 us (so the range count, not the addresses, set the
// difference).
#include "device.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kReadThreads = 256;
constexpr int kReadPiece = 32768;
constexpr int kReadMaxRanges = 1024;

__global__ __launch_bounds__(kReadThreads) void read_ranges_kernel(const unsigned long long* __restrict__ table,
                                                                   int n, unsigned long long total,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ unsigned long long s_start[kReadMaxRanges + 1];
  __shared__ unsigned long long s_addr[kReadMaxRanges];
  // the table into LDS by every thread at once (one memory round trip whatever n is),
  // then exclusive prefix sums of the range lengths (n <= kReadMaxRanges): wave 0, 64
  // ranges at a time from LDS, a shuffle scan each
  for (int i = threadIdx.x; i < n; i += kReadThreads) {
    s_addr[i] = table[2 * i];
    s_start[i] = table[2 * i + 1];  // the length, until the scan replaces it
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    unsigned long long carry = 0;
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      const unsigned long long len = i < n ? s_start[i] : 0ull;
      unsigned long long v = len;  // inclusive scan across the wave
      for (int off = 1; off < 64; off *= 2) {
        const unsigned long long t = __shfl_up(v, off);
        if (lane >= off) v += t;
      }
      if (i < n) s_start[i] = carry + v - len;
      carry += __shfl(v, 63);
    }
    if (lane == 0) s_start[n] = carry;
  }
  __syncthreads();
  uint32_t x = 0;
  const unsigned long long npieces = (total + kReadPiece - 1) / kReadPiece;
  __shared__ int s_r;
  for (unsigned long long pc = blockIdx.x; pc < npieces; pc += gridDim.x) {
    const unsigned long long p0 = pc * kReadPiece;
    const unsigned long long p1 = p0 + kReadPiece < total ? p0 + kReadPiece : total;
    // the range holding the piece's first byte, found by every thread testing its own
    // ranges at once (a walk from the first range cost one dependent LDS read a range)
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kReadThreads)
      if (s_start[i] <= p0 && p0 < s_start[i + 1]) s_r = i;
    __syncthreads();
    const int r = s_r;
    // the piece may span ranges
    for (int rr = r; rr < n && s_start[rr] < p1; ++rr) {
      const unsigned long long a = p0 > s_start[rr] ? p0 : s_start[rr];
      const unsigned long long b = p1 < s_start[rr + 1] ? p1 : s_start[rr + 1];
      const unsigned char* base = reinterpret_cast<const unsigned char*>(s_addr[rr]) + (a - s_start[rr]);
      const long long len = (long long)(b - a);
      // eight loads in flight however short the part (a part of a piece that straddles
      // two ranges): the loads past its end are switched off, not serialized
      for (long long off = (long long)threadIdx.x * 16; off < len; off += 8 * kReadThreads * 16) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const long long o = off + (long long)u * kReadThreads * 16;
          v[u] = o < len ? ldg_nt_u32x4(base + o) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      }
    }
  }
  // one word a workgroup
  __shared__ uint32_t s_x;
  if (threadIdx.x == 0) s_x = 0;
  __syncthreads();
  atomicXor(&s_x, x);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_x;
}

int read_ranges_max() { return kReadMaxRanges; }
int read_piece_bytes() { return kReadPiece; }

hipError_t launch_read_ranges(const unsigned long long* table, int n, unsigned long long total, uint32_t* sink,
                              int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(read_ranges_kernel, dim3(blocks), dim3(kReadThreads), 0, stream, table, n, total, sink);
  return hipGetLastError();
}

}  // namespace moe
