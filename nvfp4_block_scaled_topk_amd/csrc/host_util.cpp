// host_util.cpp -- device properties the launchers need, cached per device and safe to
// call from several host threads at once.
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "internal.hpp"

namespace moe {

namespace {
std::mutex g_mu;
std::map<int, int> g_cu;                                           // device -> compute units
std::map<std::tuple<int, const void*, int, int>, int> g_resident;  // (device, kernel, threads, lds) -> blocks
std::map<std::pair<int, const void*>, int> g_lds_attr;             // (device, kernel) -> bytes set
std::map<std::tuple<int, int, int, int>, int> g_mx_pick;           // (device, M, N, K) -> MXFP8 kernel
std::atomic<int> g_mx_forced{-1};
std::map<std::tuple<int, int, int, int, int, int>, int> g_ffn_pick;  // (device, T, d, f, E, k) -> few-token path
std::atomic<int> g_ffn_forced{-1};
}  // namespace

int ffn_forced_path() { return g_ffn_forced.load(); }
void ffn_force_path(int path) { g_ffn_forced.store(path); }

hipError_t ffn_recorded_path(int T, int d, int f, int E, int k, int& path) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_ffn_pick.find(std::make_tuple(dev, T, d, f, E, k));
  path = it == g_ffn_pick.end() ? -1 : it->second;
  return hipSuccess;
}

hipError_t ffn_record_path(int T, int d, int f, int E, int k, int path) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_mu);
  g_ffn_pick[std::make_tuple(dev, T, d, f, E, k)] = path;
  return hipSuccess;
}

int mxfp8_forced_kernel() { return g_mx_forced.load(); }
void mxfp8_force_kernel(int kernel) { g_mx_forced.store(kernel); }

hipError_t mxfp8_recorded_kernel(int M, int N, int K, int& kernel) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_mx_pick.find(std::make_tuple(dev, M, N, K));
  kernel = it == g_mx_pick.end() ? -1 : it->second;
  return hipSuccess;
}

hipError_t mxfp8_record_kernel(int M, int N, int K, int kernel) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_mu);
  g_mx_pick[std::make_tuple(dev, M, N, K)] = kernel;
  return hipSuccess;
}

hipError_t device_cu_count(int& ncu) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_cu.find(dev);
  if (it != g_cu.end()) {
    ncu = it->second;
    return hipSuccess;
  }
  int v = 0;
  err = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (v < 1) return hipErrorInvalidDevice;
  g_cu[dev] = v;
  ncu = v;
  return hipSuccess;
}

hipError_t resident_blocks(const void* kernel, int threads, int lds, int& blocks) {
  int ncu = 0;
  hipError_t err = device_cu_count(ncu);
  if (err != hipSuccess) return err;
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const auto key = std::make_tuple(dev, kernel, threads, lds);
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_resident.find(key);
  if (it != g_resident.end()) {
    blocks = it->second;
    return hipSuccess;
  }
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  g_resident[key] = per_cu * ncu;
  blocks = per_cu * ncu;
  return hipSuccess;
}

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_mu);
  const auto key = std::make_pair(dev, kernel);
  auto it = g_lds_attr.find(key);
  if (it != g_lds_attr.end() && it->second >= bytes) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err != hipSuccess) return err;
  g_lds_attr[key] = bytes;
  return hipSuccess;
}

}  // namespace moe
