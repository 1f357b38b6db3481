// Allocation-free variant of sw_chunk_attend, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The only scratch memory of the attention is the split workspace: the partial outputs and
// log-sum-exps of the query tiles the dense launch cuts into key ranges (the last, partial round
// of its grid), combined afterwards by the merge kernel.  sw_chunk_attend takes it from the
// cache's pool; this entry point takes it from `scratch`, a static device array of the library
// (one per GPU, held until the process ends), so the call allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "swattn.h"
#include "launch.h"

namespace {

constexpr int kScratchRows = 256 * 256;   // 256 pieces of a 256-query tile (or 512 of a 128-query tile)
constexpr int kScratchD = 128;             // head_dim of the split kernels
// [kScratchRows][kScratchD] partial outputs, then [kScratchRows] log2 sum-exps: 33.8 MB per GPU
static __device__ __align__(256) float scratch[(size_t)kScratchRows * (kScratchD + 1)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each GPU (nullptr: not looked up yet)

// Device address of `scratch` on device `dev`, looked up once per device with that device current.
// In host code the array's name stands for a host-side shadow, not device memory: only this
// address may be handed to kernels.
hipError_t scratch_on(int dev, float** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t er = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (er != hipSuccess) return er;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" sw_status sw_chunk_attend_noalloc(sw_cache* c, const void* q_raw, sw_step_kind step,
                                             const int32_t* tile_idx, int32_t k_row, void* out, float* lse_out) {
  if (!c) return static_cast<sw_status>(swhost::chunk_attend_scratch(nullptr, q_raw, step, tile_idx, k_row, out,
                                                                     lse_out, nullptr, nullptr, 0));
  const int dev = swhost::cache_device(c);
  if (dev < 0)   // a metadata-only cache: the call reports that it cannot launch
    return static_cast<sw_status>(swhost::chunk_attend_scratch(c, q_raw, step, tile_idx, k_row, out, lse_out,
                                                               nullptr, nullptr, 0));
  if (dev >= kMaxDevices) return static_cast<sw_status>(swhost::hip_error(hipErrorInvalidDevice, "scratch lookup"));
  float* base = nullptr;
  const hipError_t e = scratch_on(dev, &base);
  if (e != hipSuccess) return static_cast<sw_status>(swhost::hip_error(e, "scratch lookup (hipGetSymbolAddress)"));
  return static_cast<sw_status>(swhost::chunk_attend_scratch(c, q_raw, step, tile_idx, k_row, out, lse_out, base,
                                                             base + (size_t)kScratchRows * kScratchD, kScratchRows));
}
