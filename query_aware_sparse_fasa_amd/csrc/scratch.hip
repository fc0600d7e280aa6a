// fasa_decode_scratch: fasa_decode with its workspace in memory the library
// owns, for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The workspace is `scratch`, a file-scope device array of kScratchBytes.
// Every device the library runs on gets its own copy when this code object is
// loaded there, and keeps it until the process ends.  In host code the array's
// name only stands for the symbol: its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept; only that address is ever passed to kernels.
//
// What the workspace holds between calls never changes a result: the one
// region carried from call to call (the select's per-unit coarse histograms)
// only sends the select to its slower path once when it is not zero, and the
// FAC arrival counters are zeroed by the launch before the one that counts on
// them, inside the same call.  So nothing is cleared here.  Calls that overlap
// on one device (different streams, no ordering) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fasa.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's `scratch`, or nullptr if it cannot be had.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" size_t fasa_scratch_capacity(void) { return kScratchBytes; }

extern "C" fasa_status fasa_decode_scratch(const fasa_shape* shape, const void* q, const void* k_pool,
                                           const void* v_pool, const void* slab, const int32_t* block_table,
                                           const int32_t* seq_lens, int32_t max_t, const int32_t* fc_idx,
                                           float* out, int32_t* sel_idx, int32_t* sel_count, hipStream_t stream) {
  size_t need = 0;
  fasa_status st = fasa_workspace_size(shape, max_t, &need);
  if (st != FASA_OK) return st;
  if (need > kScratchBytes) return FASA_ERR_SCRATCH;
  // The scratch of the stream's device (the current device for the null stream).
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return FASA_ERR_HIP;
  }
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return FASA_ERR_INVALID_ARG;
    }
    if (int(sdev) != dev) return FASA_ERR_INVALID_ARG;
  }
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return FASA_ERR_HIP;
  return fasa_decode(shape, q, k_pool, v_pool, slab, block_table, seq_lens, max_t, fc_idx, out, sel_idx,
                     sel_count, ws, kScratchBytes, stream);
}
