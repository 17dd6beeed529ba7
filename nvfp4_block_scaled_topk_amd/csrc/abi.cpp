// abi.cpp -- the C ABI: argument checks on the host (no HIP call before they pass),
// path choice, launches. See include/moe_nvfp4.h for the contract of each entry point.
#include "moe_nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <random>

#include "internal.hpp"

namespace {

thread_local char g_last_error[256] = "";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(hipError_t err) {
  if (err == hipSuccess) return MOE_OK;
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", hipGetErrorString(err));
  return MOE_E_LAUNCH;
}

bool route_shape_ok(int T, int E, int k) {
  return T >= 1 && E >= 1 && E <= 1024 && k >= 1 && k <= 32 && k <= E &&
         (long long)T * k < (1LL << 31);
}

// The kernels address activations and one expert's weight matrix through 32-bit
// buffer offsets: x (T*d bf16), one projection (f*d/2 bytes) and H (T*k*f bf16) must
// each stay below 2 GiB.
bool ffn_shape_ok(int T, int d, int f, int E, int k) {
  return route_shape_ok(T, E, k) && d >= 32 && f >= 32 && d % 32 == 0 && f % 32 == 0 &&
         (long long)T * d * 2 < (1LL << 31) && (long long)f * d / 2 < (1LL << 31) &&
         (long long)T * k * f * 2 < (1LL << 31) && (long long)T * k * d * 4 < (1LL << 40);
}

constexpr size_t kWsAlign = 256;
size_t round_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Tags of the decode path's H words: a different value on every call, never 0 (freshly
// cleared memory), starting from a random point so that words a workspace still holds
// from earlier use cannot match.
// Tags of calls made under graph capture come from the device and have the top bit set
// (ffn_decode.hip); these have it clear.
uint32_t next_call_tag() {
  static std::atomic<uint32_t> counter{static_cast<uint32_t>(std::random_device{}())};
  uint32_t t = (counter.fetch_add(1, std::memory_order_relaxed) + 1u) & 0x7FFFFFFFu;
  while (t == 0) t = (counter.fetch_add(1, std::memory_order_relaxed) + 1u) & 0x7FFFFFFFu;
  return t;
}

// H: bf16 for the prompt path, bf16 + tag (4 bytes an element) for the decode path; after
// H the decode path keeps its epoch word (graph capture), the prompt path its two work
// counters (kEpochBytes either way)
size_t h_bytes(int T, int d, int f, int k) {
  const bool dec = moe::use_decode_path(T, d, f);
  return round_up((size_t)T * k * f * (dec ? 4 : 2)) + moe::kEpochBytes;
}
uint32_t* epoch_word(void* workspace, int T, int d, int f, int k) {
  return reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) + h_bytes(T, d, f, k) - moe::kEpochBytes);
}

// Workspace of the one-launch layer (moe_layer_nvfp4), in 256-byte aligned parts: the
// arrival counters first ([T][ceil(d / 128)], one 128-byte line each; zero before the
// first call, and every call leaves them zero), then H as tagged words ([rows][f / 2]
// 8-byte words) and the expert rows as tagged words ([rows][d] 8-byte words); rows = T * k,
// plus T with a shared expert.
void layer_workspace_parts(int T, int d, int f, int k, bool shared, size_t& y_off, size_t& c_off, size_t& total) {
  const size_t rows = (size_t)T * k + (shared ? (size_t)T : 0);
  c_off = 0;
  const size_t h_off = round_up((size_t)T * (size_t)((d + 127) / 128) * moe::kLayerCounterBytes);
  y_off = h_off + round_up(rows * (size_t)f * 4);
  total = y_off + round_up(rows * (size_t)d * 8) + moe::kEpochBytes;  // the epoch word last
}
size_t layer_counter_bytes(int T, int d) {
  return round_up((size_t)T * (size_t)((d + 127) / 128) * moe::kLayerCounterBytes);
}

// polls of the few-token launch's waits (moe_set_wait_limits)
std::atomic<uint32_t> g_steal_after{moe::kDefaultStealAfter};
std::atomic<uint32_t> g_give_up{moe::kDefaultGiveUp};

}  // namespace

namespace moe {
size_t ffn_workspace_bytes(int T, int d, int f, int E, int k) {
  (void)E;
  return h_bytes(T, d, f, k);
}
}  // namespace moe

extern "C" {

size_t moe_route_topk_workspace(int T, int E, int k) {
  if (!route_shape_ok(T, E, k)) return 0;
  const size_t b = moe::route_workspace_bytes(T, E, k);
  return b ? round_up(b) : 0;
}

int moe_route_topk_policy(const float* logits, int T, int E, int k, int policy, const float* bias,
                          int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_rows,
                          int32_t* row_of, void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !topk_ids || !topk_w || !expert_offsets || !sorted_rows || !row_of) return MOE_E_NULL;
  if (!route_shape_ok(T, E, k)) return MOE_E_SHAPE;
  if (policy < MOE_ROUTE_SOFTMAX_RENORM || policy > MOE_ROUTE_SIGMOID) return MOE_E_POLICY;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(expert_offsets) ||
      !aligned16(sorted_rows) || !aligned16(row_of) || (bias && !aligned16(bias)))
    return MOE_E_ALIGN;
  const size_t need = moe_route_topk_workspace(T, E, k);
  if (need) {
    if (!workspace || workspace_bytes < need) return MOE_E_WORKSPACE;
    if (!aligned16(workspace)) return MOE_E_ALIGN;
  }
  return launch_status(moe::launch_route(logits, bias, policy, T, E, k, topk_ids, topk_w, expert_offsets,
                                         sorted_rows, row_of, need ? workspace : nullptr,
                                         static_cast<hipStream_t>(stream)));
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                   int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_of, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return moe_route_topk_policy(logits, T, E, k, MOE_ROUTE_SOFTMAX_RENORM, nullptr, topk_ids, topk_w,
                               expert_offsets, sorted_rows, row_of, workspace, workspace_bytes, stream);
}

size_t moe_expert_ffn_nvfp4_workspace(int T, int d, int f, int E, int k) {
  if (!ffn_shape_ok(T, d, f, E, k)) return 0;
  return moe::ffn_workspace_bytes(T, d, f, E, k);
}

}  // extern "C"

namespace {

// Checks and argument block shared by the two FFN entry points (routing lists given or
// made by the launch itself); returns MOE_OK and fills `a`, or a refusal status.
int ffn_setup(const uint16_t* x, int T, int d, int f, int E, int k, const moe_nvfp4_experts* w, float* y_rows,
              void* workspace, size_t workspace_bytes, moe::FFNArgs& a) {
  if (!x || !w || !y_rows) return MOE_E_NULL;
  if (!w->gate_q || !w->gate_s || !w->gate_ts || !w->up_q || !w->up_s || !w->up_ts || !w->down_q ||
      !w->down_s || !w->down_ts)
    return MOE_E_NULL;
  if (!ffn_shape_ok(T, d, f, E, k)) return MOE_E_SHAPE;
  const void* ptrs[] = {x, y_rows, w->gate_q, w->gate_s, w->gate_ts, w->up_q, w->up_s, w->up_ts, w->down_q,
                        w->down_s, w->down_ts};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  const size_t need = moe_expert_ffn_nvfp4_workspace(T, d, f, E, k);
  if (!workspace || workspace_bytes < need) return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  a.x = x;
  a.T = T;
  a.d = d;
  a.f = f;
  a.E = E;
  a.k = k;
  a.gate_q = w->gate_q;
  a.gate_s = w->gate_s;
  a.up_q = w->up_q;
  a.up_s = w->up_s;
  a.down_q = w->down_q;
  a.down_s = w->down_s;
  a.gate_ts = w->gate_ts;
  a.up_ts = w->up_ts;
  a.down_ts = w->down_ts;
  a.y_rows = y_rows;
  a.h = static_cast<uint16_t*>(workspace);
  if (moe::use_decode_path(T, d, f)) a.epoch = epoch_word(workspace, T, d, f, k);
  else a.work_ctr = epoch_word(workspace, T, d, f, k);  // the same slot after H
  return MOE_OK;
}

// The path of a few-token call (a token routes to k distinct experts, so with T <= 16 an
// expert has at most 16 rows: one decode or streaming tile): the forced one, else the
// recorded pick, else the one-launch decode kernel when its size limits allow it.
hipError_t few_token_path(int T, int d, int f, int E, int k, int& path) {
  path = moe::ffn_forced_path();
  if (path < 0) {
    const hipError_t err = moe::ffn_recorded_path(T, d, f, E, k, path);
    if (err != hipSuccess) return err;
  }
  if (path < 0) path = moe::kFfnDecodeLaunch;
  if (path == moe::kFfnDecodeLaunch && !moe::use_decode_path(T, d, f)) path = moe::kFfnStreaming;
  return hipSuccess;
}

// path: -1 for a batch (grouped GEMM and streaming kernels), else a few-token path
hipError_t launch_ffn_path(const moe::FFNArgs& a, int path, hipStream_t st) {
  if (path == moe::kFfnDecodeLaunch)
    return moe::launch_ffn_decode(a, next_call_tag(), g_steal_after.load(), g_give_up.load(), st);
  if (path == moe::kFfnStreaming) {
    hipError_t err = moe::launch_ffn_skinny_gateup(a, st);
    return err == hipSuccess ? moe::launch_ffn_skinny_down(a, st) : err;
  }
  return moe::launch_ffn_prompt(a, st);
}

}  // namespace

extern "C" {

int moe_expert_ffn_nvfp4(const uint16_t* x, int T, int d, int f, int E, int k, const moe_nvfp4_experts* w,
                         const int32_t* expert_offsets, const int32_t* sorted_rows, float* y_rows,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!expert_offsets || !sorted_rows) return MOE_E_NULL;
  moe::FFNArgs a;
  const int st0 = ffn_setup(x, T, d, f, E, k, w, y_rows, workspace, workspace_bytes, a);
  if (st0 != MOE_OK) return st0;
  if (!aligned16(expert_offsets) || !aligned16(sorted_rows)) return MOE_E_ALIGN;
  a.offsets = expert_offsets;
  a.sorted_rows = sorted_rows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int path = -1;
  if (T <= moe::kDecodeMaxRows) {
    const hipError_t err = few_token_path(T, d, f, E, k, path);
    if (err != hipSuccess) return launch_status(err);
  }
  return launch_status(launch_ffn_path(a, path, st));
}

}  // extern "C"

namespace {

// The scratch of moe_expert_ffn_nvfp4_scratch: H lives here instead of in a caller
// workspace. One array per device (each device holds its own copy for the life of the
// process); host code never uses the array's name as an address, only the device address
// hipGetSymbolAddress gives for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> address of its scratch

hipError_t scratch_address(void*& ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess) return err;
  if (p == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = p;
  ptr = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int moe_expert_ffn_nvfp4_scratch(const uint16_t* x, int T, int d, int f, int E, int k, const moe_nvfp4_experts* w,
                                 const int32_t* expert_offsets, const int32_t* sorted_rows, float* y_rows,
                                 void* stream) {
  const size_t need = moe_expert_ffn_nvfp4_workspace(T, d, f, E, k);
  if (need > MOE_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "moe_expert_ffn_nvfp4_scratch: H needs %zu bytes, the static scratch holds %zu", need,
                  (size_t)MOE_SCRATCH_BYTES);
    return MOE_E_WORKSPACE;
  }
  if (need == 0) return moe_expert_ffn_nvfp4(x, T, d, f, E, k, w, expert_offsets, sorted_rows, y_rows, nullptr, 0,
                                             stream);  // a refused shape: named by the workspace entry point
  void* ptr = nullptr;
  const hipError_t err = scratch_address(ptr);
  if (err != hipSuccess) return launch_status(err);
  return moe_expert_ffn_nvfp4(x, T, d, f, E, k, w, expert_offsets, sorted_rows, y_rows, ptr, MOE_SCRATCH_BYTES,
                              stream);
}

int moe_route_expert_ffn_nvfp4(const float* logits, const uint16_t* x, int T, int d, int f, int E, int k,
                               const moe_nvfp4_experts* w, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                               int32_t* sorted_rows, int32_t* row_of, float* y_rows, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!logits || !topk_ids || !topk_w || !expert_offsets || !sorted_rows || !row_of) return MOE_E_NULL;
  moe::FFNArgs a;
  const int st0 = ffn_setup(x, T, d, f, E, k, w, y_rows, workspace, workspace_bytes, a);
  if (st0 != MOE_OK) return st0;
  if (!moe::use_decode_path(T, d, f) || E > moe::kFusedRouteMaxE || k > moe::kFusedRouteMaxK) return MOE_E_SHAPE;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(expert_offsets) ||
      !aligned16(sorted_rows) || !aligned16(row_of))
    return MOE_E_ALIGN;
  a.logits = logits;
  a.ids_out = topk_ids;
  a.w_out = topk_w;
  a.offsets_out = expert_offsets;
  a.sorted_rows_out = sorted_rows;
  a.row_of_out = row_of;
  return launch_status(
      moe::launch_ffn_decode(a, next_call_tag(), g_steal_after.load(), g_give_up.load(), static_cast<hipStream_t>(stream)));
}

size_t moe_layer_nvfp4_workspace(int T, int d, int f, int E, int k, int with_shared) {
  if (!ffn_shape_ok(T, d, f, E, k) || !moe::use_decode_path(T, d, f) || E > moe::kFusedRouteMaxE ||
      k > moe::kFusedRouteMaxK)
    return 0;
  size_t y_off, c_off, total;
  layer_workspace_parts(T, d, f, k, with_shared != 0, y_off, c_off, total);
  return total;
}

int moe_layer_nvfp4(const float* logits, int logits_ld, const uint16_t* x, int T, int d, int f, int E, int k,
                    const moe_nvfp4_experts* w, const moe_nvfp4_experts* shared, const float* shared_gate_logit,
                    int gate_ld, const uint16_t* residual, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                    int32_t* sorted_rows, int32_t* row_of, uint16_t* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!logits || !x || !w || !out || !workspace) return MOE_E_NULL;
  if (!w->gate_q || !w->gate_s || !w->gate_ts || !w->up_q || !w->up_s || !w->up_ts || !w->down_q ||
      !w->down_s || !w->down_ts)
    return MOE_E_NULL;
  if (shared && (!shared->gate_q || !shared->gate_s || !shared->gate_ts || !shared->up_q || !shared->up_s ||
                 !shared->up_ts || !shared->down_q || !shared->down_s || !shared->down_ts))
    return MOE_E_NULL;
  if (shared_gate_logit && !shared) return MOE_E_NULL;
  const size_t need = moe_layer_nvfp4_workspace(T, d, f, E, k, shared != nullptr);
  if (need == 0) return MOE_E_SHAPE;
  if (logits_ld == 0) logits_ld = E;
  if (logits_ld < E || (long long)T * logits_ld >= (1LL << 31)) return MOE_E_SHAPE;
  if (shared_gate_logit && (gate_ld < 1 || (long long)T * gate_ld >= (1LL << 31))) return MOE_E_SHAPE;
  if (workspace_bytes < need) return MOE_E_WORKSPACE;
  const void* ptrs[] = {logits, x, out, workspace, w->gate_q, w->gate_s, w->gate_ts, w->up_q, w->up_s, w->up_ts,
                        w->down_q, w->down_s, w->down_ts};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  if (shared) {
    const void* sp[] = {shared->gate_q, shared->gate_s, shared->gate_ts, shared->up_q, shared->up_s, shared->up_ts,
                        shared->down_q, shared->down_s, shared->down_ts};
    for (const void* p : sp)
      if (!aligned16(p)) return MOE_E_ALIGN;
  }
  const void* opt[] = {residual, topk_ids, topk_w, expert_offsets, sorted_rows, row_of};
  for (const void* p : opt)
    if (p && !aligned16(p)) return MOE_E_ALIGN;
  moe::FFNArgs a;
  a.x = x;
  a.T = T;
  a.d = d;
  a.f = f;
  a.E = E;
  a.k = k;
  a.gate_q = w->gate_q;
  a.gate_s = w->gate_s;
  a.up_q = w->up_q;
  a.up_s = w->up_s;
  a.down_q = w->down_q;
  a.down_s = w->down_s;
  a.gate_ts = w->gate_ts;
  a.up_ts = w->up_ts;
  a.down_ts = w->down_ts;
  size_t y_off, c_off, total;
  layer_workspace_parts(T, d, f, k, shared != nullptr, y_off, c_off, total);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.ctr = reinterpret_cast<unsigned long long*>(ws + c_off);
  a.h = reinterpret_cast<uint16_t*>(ws + layer_counter_bytes(T, d));
  a.yw = reinterpret_cast<unsigned long long*>(ws + y_off);
  a.epoch = reinterpret_cast<uint32_t*>(ws + total - moe::kEpochBytes);
  a.out = out;
  a.resid = residual;
  a.logits = logits;
  a.logits_ld = logits_ld;
  a.ids_out = topk_ids;
  a.w_out = topk_w;
  a.offsets_out = expert_offsets;
  a.sorted_rows_out = sorted_rows;
  a.row_of_out = row_of;
  if (shared) {
    a.sh_gate_q = shared->gate_q;
    a.sh_gate_s = shared->gate_s;
    a.sh_up_q = shared->up_q;
    a.sh_up_s = shared->up_s;
    a.sh_down_q = shared->down_q;
    a.sh_down_s = shared->down_s;
    a.sh_gate_ts = shared->gate_ts;
    a.sh_up_ts = shared->up_ts;
    a.sh_down_ts = shared->down_ts;
    a.gate_logit = shared_gate_logit;
    a.gate_ld = gate_ld;
  }
  return launch_status(
      moe::launch_ffn_decode(a, next_call_tag(), g_steal_after.load(), g_give_up.load(), static_cast<hipStream_t>(stream)));
}

int moe_combine(const float* y_rows, const int32_t* row_of, const float* topk_w, int T, int k, int d,
                uint16_t* out, void* stream) {
  if (!y_rows || !row_of || !topk_w || !out) return MOE_E_NULL;
  if (T < 1 || k < 1 || k > 32 || d < 32 || d % 32 != 0 || (long long)T * k >= (1LL << 31)) return MOE_E_SHAPE;
  if (!aligned16(y_rows) || !aligned16(row_of) || !aligned16(topk_w) || !aligned16(out)) return MOE_E_ALIGN;
  return launch_status(
      moe::launch_combine(y_rows, row_of, topk_w, T, k, d, nullptr, nullptr, nullptr, out,
                          static_cast<hipStream_t>(stream)));
}

int moe_combine_shared(const float* y_rows, const int32_t* row_of, const float* topk_w, int T, int k, int d,
                       const float* shared_rows, const float* shared_gate_logit, uint16_t* out, void* stream) {
  if (!y_rows || !row_of || !topk_w || !shared_rows || !out) return MOE_E_NULL;
  if (T < 1 || k < 1 || k > 32 || d < 32 || d % 32 != 0 || (long long)T * k >= (1LL << 31)) return MOE_E_SHAPE;
  if (!aligned16(y_rows) || !aligned16(row_of) || !aligned16(topk_w) || !aligned16(shared_rows) ||
      (shared_gate_logit && !aligned16(shared_gate_logit)) || !aligned16(out))
    return MOE_E_ALIGN;
  return launch_status(moe::launch_combine(y_rows, row_of, topk_w, T, k, d, shared_rows, shared_gate_logit, nullptr,
                                           out, static_cast<hipStream_t>(stream)));
}

int moe_combine_residual(const float* y_rows, const int32_t* row_of, const float* topk_w, int T, int k, int d,
                         const float* shared_rows, const float* shared_gate_logit, const uint16_t* residual,
                         uint16_t* out, void* stream) {
  if (!y_rows || !row_of || !topk_w || !residual || !out) return MOE_E_NULL;
  if (shared_gate_logit && !shared_rows) return MOE_E_NULL;
  if (T < 1 || k < 1 || k > 32 || d < 32 || d % 32 != 0 || (long long)T * k >= (1LL << 31)) return MOE_E_SHAPE;
  if (!aligned16(y_rows) || !aligned16(row_of) || !aligned16(topk_w) || (shared_rows && !aligned16(shared_rows)) ||
      (shared_gate_logit && !aligned16(shared_gate_logit)) || !aligned16(residual) || !aligned16(out))
    return MOE_E_ALIGN;
  return launch_status(moe::launch_combine(y_rows, row_of, topk_w, T, k, d, shared_rows, shared_gate_logit, residual,
                                           out, static_cast<hipStream_t>(stream)));
}

int moe_router_logits(const uint16_t* x, const uint16_t* w_r, int T, int d, int E, float* logits, void* stream) {
  if (!x || !w_r || !logits) return MOE_E_NULL;
  // x (T * d bf16) and W_r (E * d bf16) are addressed through 32-bit buffer offsets;
  // the grid has ceil(E / 32) rows
  if (T < 1 || E < 1 || d < 32 || d % 32 != 0 || (long long)T * d * 2 >= (1LL << 31) ||
      (long long)E * d * 2 >= (1LL << 31) || E > (1 << 20))
    return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(w_r) || !aligned16(logits)) return MOE_E_ALIGN;
  return launch_status(moe::launch_router_logits(x, w_r, T, d, E, logits, static_cast<hipStream_t>(stream)));
}

int mxfp8_gemm(const uint16_t* x, int M, int N, int K, const uint8_t* w, const uint8_t* s, uint16_t* y,
               void* stream) {
  if (!x || !w || !s || !y) return MOE_E_NULL;
  // x (M * K bf16) and W (N * K bytes) are addressed through 32-bit buffer offsets
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || (long long)M * K * 2 >= (1LL << 31) ||
      (long long)N * K >= (1LL << 31))
    return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return MOE_E_ALIGN;
  return launch_status(moe::launch_mxfp8(x, M, N, K, w, s, y, static_cast<hipStream_t>(stream)));
}

int moe_async_status(void* stream) {
  hipError_t err = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  unsigned int flag = 0;
  if (err == hipSuccess) err = moe::read_and_clear_async_status(flag);
  if (err != hipSuccess) return launch_status(err);
  return flag ? MOE_E_WAIT_EXPIRED : MOE_OK;
}

void moe_set_wait_limits(uint32_t steal_after, uint32_t give_up) {
  g_steal_after.store(steal_after);
  g_give_up.store(give_up);
}

void moe_get_wait_limits(uint32_t* steal_after, uint32_t* give_up) {
  if (steal_after) *steal_after = g_steal_after.load();
  if (give_up) *give_up = g_give_up.load();
}

int mxfp8_autotune(const uint16_t* x, int M_max, int N, int K, const uint8_t* w, const uint8_t* s, uint16_t* y,
                   int reps, int* picks, float* us, void* stream) {
  if (!x || !w || !s || !y) return MOE_E_NULL;
  if (M_max < 1 || M_max > 16 || N < 1 || K < 32 || K % 32 != 0 || reps < 1 || (long long)M_max * K * 2 >= (1LL << 31) ||
      (long long)N * K >= (1LL << 31))
    return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return MOE_E_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t ev[2];
  hipError_t err = hipEventCreate(&ev[0]);
  if (err != hipSuccess) return launch_status(err);
  err = hipEventCreate(&ev[1]);
  if (err != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return launch_status(err);
  }
  for (int M = 1; M <= M_max && err == hipSuccess; ++M) {
    float best = 0.f;
    int pick = moe::mxfp8_default_kernel(M);
    for (int kernel = moe::kMxValuGemv; kernel <= moe::kMxTiledGemm && err == hipSuccess; ++kernel) {
      if (kernel == moe::kMxValuGemv && M > 8) continue;
      err = moe::launch_mxfp8_kernel(kernel, x, M, N, K, w, s, y, st);  // warm-up
      if (err == hipSuccess) err = hipEventRecord(ev[0], st);
      for (int r = 0; r < reps && err == hipSuccess; ++r) err = moe::launch_mxfp8_kernel(kernel, x, M, N, K, w, s, y, st);
      if (err == hipSuccess) err = hipEventRecord(ev[1], st);
      if (err == hipSuccess) err = hipEventSynchronize(ev[1]);
      float ms = 0.f;
      if (err == hipSuccess) err = hipEventElapsedTime(&ms, ev[0], ev[1]);
      if (err != hipSuccess) break;
      const float t = ms * 1000.f / reps;
      if (us) us[(M - 1) * 3 + kernel] = t;
      if (best == 0.f || t < best) {
        best = t;
        pick = kernel;
      }
    }
    if (err == hipSuccess) err = moe::mxfp8_record_kernel(M, N, K, pick);
    if (picks) picks[M - 1] = pick;
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  return launch_status(err);
}

int moe_ffn_autotune(const uint16_t* x, int T, int d, int f, int E, int k, const moe_nvfp4_experts* w,
                     const int32_t* expert_offsets, const int32_t* sorted_rows, float* y_rows, void* workspace,
                     size_t workspace_bytes, int reps, int* pick, float* us, void* stream) {
  if (!expert_offsets || !sorted_rows) return MOE_E_NULL;
  moe::FFNArgs a;
  const int st0 = ffn_setup(x, T, d, f, E, k, w, y_rows, workspace, workspace_bytes, a);
  if (st0 != MOE_OK) return st0;
  if (T > moe::kDecodeMaxRows || reps < 1) return MOE_E_SHAPE;
  if (!aligned16(expert_offsets) || !aligned16(sorted_rows)) return MOE_E_ALIGN;
  a.offsets = expert_offsets;
  a.sorted_rows = sorted_rows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t ev[2];
  hipError_t err = hipEventCreate(&ev[0]);
  if (err != hipSuccess) return launch_status(err);
  err = hipEventCreate(&ev[1]);
  if (err != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return launch_status(err);
  }
  float best = 0.f;
  int choice = moe::kFfnStreaming;
  for (int path = moe::kFfnDecodeLaunch; path <= moe::kFfnStreaming && err == hipSuccess; ++path) {
    if (path == moe::kFfnDecodeLaunch && !moe::use_decode_path(T, d, f)) continue;
    err = launch_ffn_path(a, path, st);  // warm-up
    if (err == hipSuccess) err = hipEventRecord(ev[0], st);
    for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch_ffn_path(a, path, st);
    if (err == hipSuccess) err = hipEventRecord(ev[1], st);
    if (err == hipSuccess) err = hipEventSynchronize(ev[1]);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, ev[0], ev[1]);
    if (err != hipSuccess) break;
    const float t = ms * 1000.f / reps;
    if (us) us[path] = t;
    if (best == 0.f || t < best) {
      best = t;
      choice = path;
    }
  }
  if (err == hipSuccess) err = moe::ffn_record_path(T, d, f, E, k, choice);
  if (pick) *pick = choice;
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  return launch_status(err);
}

int moe_ffn_force_path(int path) {
  if (path < -1 || path > moe::kFfnStreaming) return MOE_E_SHAPE;
  moe::ffn_force_path(path);
  return MOE_OK;
}

int mxfp8_force_kernel(int kernel) {
  if (kernel < -1 || kernel > moe::kMxTiledGemm) return MOE_E_SHAPE;
  moe::mxfp8_force_kernel(kernel);
  return MOE_OK;
}

int mxfp8_quantize(const uint16_t* x, int M, int K, uint8_t* xq, uint8_t* xs, void* stream) {
  if (!x || !xq || !xs) return MOE_E_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || (long long)M * K * 2 >= (1LL << 31)) return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(xs)) return MOE_E_ALIGN;
  return launch_status(moe::launch_mx_quantize(x, M, K, xq, xs, static_cast<hipStream_t>(stream)));
}

int mxfp8_gemm_mx(const uint8_t* xq, const uint8_t* xs, int M, int N, int K, const uint8_t* w, const uint8_t* s,
                  uint16_t* y, void* stream) {
  if (!xq || !xs || !w || !s || !y) return MOE_E_NULL;
  // the tile's scale rows are loaded whole (K / 32 a multiple of 16, at most 128 bytes)
  if (M < 1 || N < 1 || K < 512 || K % 512 != 0 || K > 4096 || (long long)M * K >= (1LL << 31) ||
      (long long)N * K >= (1LL << 31))
    return MOE_E_SHAPE;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return MOE_E_ALIGN;
  return launch_status(moe::launch_mx_gemm(xq, xs, M, N, K, w, s, y, static_cast<hipStream_t>(stream)));
}

int moe_read_ceiling(const uint64_t* ranges, int n, uint64_t total_bytes, uint32_t* sink, int sink_words,
                     void* stream) {
  if (!ranges || !sink) return MOE_E_NULL;
  if (n < 1 || n > moe::read_ranges_max() || total_bytes == 0 || sink_words < 1) return MOE_E_SHAPE;
  if (!aligned16(ranges) || !aligned16(sink)) return MOE_E_ALIGN;
  int ncu = 0;
  hipError_t err = moe::device_cu_count(ncu);
  if (err != hipSuccess) return launch_status(err);
  const long long pieces = (long long)((total_bytes + moe::read_piece_bytes() - 1) / moe::read_piece_bytes());
  const int blocks = (int)std::min<long long>(std::min<long long>(pieces, 16LL * ncu), sink_words);
  return launch_status(moe::launch_read_ranges(reinterpret_cast<const unsigned long long*>(ranges), n,
                                               (unsigned long long)total_bytes, sink, blocks,
                                               static_cast<hipStream_t>(stream)));
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_NULL: return "MOE_E_NULL";
    case MOE_E_SHAPE: return "MOE_E_SHAPE";
    case MOE_E_ALIGN: return "MOE_E_ALIGN";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE";
    case MOE_E_LAUNCH: return "MOE_E_LAUNCH";
    case MOE_E_POLICY: return "MOE_E_POLICY";
    case MOE_E_WAIT_EXPIRED: return "MOE_E_WAIT_EXPIRED";
    default: return "MOE_E_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error; }

}  // extern "C"
