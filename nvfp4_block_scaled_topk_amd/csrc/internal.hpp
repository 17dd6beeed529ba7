// internal.hpp -- launchers behind the C ABI (host side). Every launcher assumes its
// arguments were validated by abi.cpp and only enqueues kernels on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

struct moe_nvfp4_experts;

namespace moe {

// routing
size_t route_workspace_bytes(int T, int E, int k);
hipError_t launch_route(const float* logits, const float* bias, int policy, int T, int E, int k, int32_t* ids,
                        float* w,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* row_of, void* ws,
                        hipStream_t stream);

// expert FFN: H ([T*k][f]) lives in the caller's workspace
struct FFNArgs {
  const uint16_t* x;
  int T, d, f, E, k;
  const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
  const float *gate_ts, *up_ts, *down_ts;
  const int32_t* offsets;
  const int32_t* sorted_rows;
  float* y_rows;
  uint16_t* h;
  // few-token path only: when `logits` is set the launch routes its tokens itself
  // (default policy, no bias; E <= 256, k <= 16) instead of reading offsets and
  // sorted_rows, and its first block writes the routing outputs
  const float* logits = nullptr;
  int logits_ld = 0;  // row stride of logits (0: E)
  int32_t* ids_out = nullptr;
  float* w_out = nullptr;
  int32_t* offsets_out = nullptr;
  int32_t* sorted_rows_out = nullptr;
  int32_t* row_of_out = nullptr;
  // few-token path with routing in the launch only: the whole layer. With `out` set the
  // launch also combines: the down items write their rows as tagged words `yw`
  // ([rows][d], value and tag), count arrivals per (token, 128 columns) in `ctr`
  // ([T][ceil(d / 128)] counters), and the block that completes a token's column
  // tile writes out = bf16_rne(sum_j w_j y_j (+ g S) (+ resid)). A shared expert (the
  // sh_* pointers, one expert of the same d and f) is one more touched expert with T
  // rows after the routed ones, its add gated by sigmoid(gate_logit[t * gate_ld]).
  uint16_t* out = nullptr;
  unsigned long long* yw = nullptr;
  unsigned long long* ctr = nullptr;  // kLayerCounterBytes apart, zero when a call starts
  const uint16_t* resid = nullptr;
  const uint8_t *sh_gate_q = nullptr, *sh_gate_s = nullptr, *sh_up_q = nullptr, *sh_up_s = nullptr,
                *sh_down_q = nullptr, *sh_down_s = nullptr;
  const float *sh_gate_ts = nullptr, *sh_up_ts = nullptr, *sh_down_ts = nullptr;
  const float* gate_logit = nullptr;
  int gate_ld = 1;
  // few-token path: a 32-bit word in the workspace holding the tag of the latest call made
  // under HIP graph capture (see launch_ffn_decode)
  uint32_t* epoch = nullptr;
  // prompt path: two 32-bit work counters in the workspace (gate/up, down), zeroed by
  // the launch itself before its kernels take items from them
  uint32_t* work_ctr = nullptr;
};
// Bytes a few-token workspace keeps for that word (at its end).
constexpr size_t kEpochBytes = 256;

constexpr int kLayerCounterBytes = 128;  // one arrival counter a cache line
constexpr int kFusedRouteMaxE = 256;
constexpr int kFusedRouteMaxK = 16;
// The decode path keeps every expert's rows in one 16-row MFMA tile (T <= 16).
constexpr int kDecodeMaxRows = 16;
size_t ffn_workspace_bytes(int T, int d, int f, int E, int k);
// The decode path keeps H in the workspace as 64-bit words (two bf16 values and a
// 32-bit tag that differs between calls): T * k * f * 4 bytes.
// The decode path stages one expert's activation rows, then its H rows, in LDS.
size_t ffn_decode_lds_bytes(int T, int d, int f);
constexpr size_t kDecodeMaxLds = 64 * 1024;
constexpr int kDecodeMaxD = 4096;  // a gate/up item keeps all its block scales (4d bytes) in LDS
constexpr int kDecodeMaxF = 1024;  // a down tile's 16 scale rows (f bytes) fit one 16-byte load a lane
inline bool use_decode_path(int T, int d, int f) {
  return T <= kDecodeMaxRows && d <= kDecodeMaxD && f <= kDecodeMaxF &&
         ffn_decode_lds_bytes(T, d, f) <= kDecodeMaxLds;
}
// `steal_after`: polls of a missing H slice before a down item computes the missing
// gate/up items itself; `give_up`: polls of the full H read before it writes NaN rows and
// raises the asynchronous status flag (see ffn_decode.hip)
hipError_t launch_ffn_decode(const FFNArgs& a, uint32_t tag, uint32_t steal_after, uint32_t give_up,
                             hipStream_t stream);
constexpr uint32_t kDefaultStealAfter = 256;
constexpr uint32_t kDefaultGiveUp = 1u << 20;
// the few-token launch's flag of a wait that gave up: read and cleared (synchronous)
hipError_t read_and_clear_async_status(unsigned int& status);
hipError_t launch_ffn_prompt(const FFNArgs& a, hipStream_t stream);
// The two paths of a few-token call (T <= kDecodeMaxRows: no expert has more rows than
// one streaming tile): the one-launch decode kernel, or the two weight-streaming kernels
// (no grouped-GEMM launch: it would have no tiles). Which is faster depends on the card
// and the shape; moe_ffn_autotune records the pick per (device, T, d, f, E, k).
constexpr int kFfnDecodeLaunch = 0;
constexpr int kFfnStreaming = 1;
int ffn_forced_path();  // -1: none
void ffn_force_path(int path);
hipError_t ffn_recorded_path(int T, int d, int f, int E, int k, int& path);  // -1 when none is recorded
hipError_t ffn_record_path(int T, int d, int f, int E, int k, int path);
// Prompt batches: experts with at most kSkinnyRows rows take the weight-streaming
// kernels (ffn_skinny.hip: 1..16 rows as one 16-row set, 17..32 as two); the grouped
// GEMM takes the others.
constexpr int kSkinnyRows = 32;
hipError_t launch_ffn_skinny_gateup(const FFNArgs& a, hipStream_t stream);
hipError_t launch_ffn_skinny_down(const FFNArgs& a, hipStream_t stream);

// device properties, cached per device (host_util.cpp; thread-safe)
hipError_t device_cu_count(int& ncu);
hipError_t resident_blocks(const void* kernel, int threads, int lds, int& blocks);
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);

// combine
hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* w, int T,
                          int k, int d, const float* s_rows, const float* s_gate, const uint16_t* resid,
                          uint16_t* out, hipStream_t stream);

// router projection
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_r, int T, int d, int E, float* logits,
                                hipStream_t stream);

// a plain streaming read of byte ranges (measure.hip): the benchmark's ceiling
int read_ranges_max();
int read_piece_bytes();
hipError_t launch_read_ranges(const unsigned long long* table, int n, unsigned long long total, uint32_t* sink,
                              int blocks, hipStream_t stream);

// MXFP8
hipError_t launch_mxfp8(const uint16_t* x, int M, int N, int K, const uint8_t* w,
                        const uint8_t* s, uint16_t* y, hipStream_t stream);
// the few-row MXFP8 kernels by id, and their pick per card (mxfp8_autotune)
constexpr int kMxValuGemv = 0;   // M <= 8
constexpr int kMxMfmaGemv = 1;   // M <= 16
constexpr int kMxTiledGemm = 2;  // any M
hipError_t launch_mxfp8_kernel(int kernel, const uint16_t* x, int M, int N, int K, const uint8_t* w,
                               const uint8_t* s, uint16_t* y, hipStream_t stream);
int mxfp8_default_kernel(int M);
int mxfp8_forced_kernel();                                        // -1: none
void mxfp8_force_kernel(int kernel);
hipError_t mxfp8_recorded_kernel(int M, int N, int K, int& kernel);  // -1 when none is recorded
hipError_t mxfp8_record_kernel(int M, int N, int K, int kernel);

// MXFP8 activations and the W8A8 projection (mxfp8_w8a8.hip)
hipError_t launch_mx_quantize(const uint16_t* x, int M, int K, uint8_t* xq, uint8_t* xs, hipStream_t stream);
hipError_t launch_mx_gemm(const uint8_t* xq, const uint8_t* xs, int M, int N, int K, const uint8_t* w,
                          const uint8_t* s, uint16_t* y, hipStream_t stream);

}  // namespace moe
