// Measurement aid, not a step of the method: the matrix-core rate this device actually sustains,
// so that attention throughput can be given as a fraction of a measured peak beside the
// datasheet one.  Every wave runs four independent accumulator chains of one MFMA shape with
// operands in registers (no memory traffic inside the loop), 8 waves per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swattn.h"
#include "device_common.h"

namespace swattn {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

template <bool FP8>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // operand values depend on the lane, so nothing folds at compile time
  const float x = 1.0f / (float)(lane + 3);
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
  if (FP8) {
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // scattered finite E4M3 bytes (exponent field <= 14), as varied as real data: a constant
      // operand toggles fewer bits and lets the clock run higher than attention ever sees
      const uint32_t ha = (uint32_t)(lane * 8 + i + 1) * 2654435761u, hb = (uint32_t)(lane * 8 + i + 7) * 2246822519u;
      a[i] = (int)((ha ^ (ha >> 15)) & 0x77777777u);
      b[i] = (int)((hb ^ (hb >> 13)) & 0x77777777u);
    }
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // varied values (see the fp8 operands)
      a[i] = (__bf16)(x * (float)(i + 1));
      b[i] = (__bf16)(x - 0.01f * (float)i);
    }
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  // one value per wave keeps every chain live
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace swattn

extern "C" sw_status sw_probe_mfma(void* hip_stream, sw_dtype dtype, int32_t iters, float* sink, int32_t sink_floats,
                                   double* flops_out) {
  using namespace swattn;
  if (!sink || !flops_out || iters < 1 || (dtype != SW_BF16 && dtype != SW_FP8)) return SW_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SW_ERR_HIP;
  const int grid = 2 * cus;   // 2 workgroups x 4 waves = 8 waves per CU, 2 per SIMD
  if (sink_floats < 4 * grid) return SW_ERR_CAPACITY;
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (dtype == SW_FP8)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(grid), dim3(256), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(grid), dim3(256), 0, st, iters, sink);
  if (hipGetLastError() != hipSuccess) return SW_ERR_HIP;
  // 2 * 32 * 32 * K flops per MFMA (K = 16 for bf16, 64 for fp8), 4 per iteration, 4 waves per group
  *flops_out = (double)grid * 4 * iters * 4 * 2.0 * 32 * 32 * (dtype == SW_FP8 ? 64 : 16);
  return SW_OK;
}
