// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace swattn {

typedef uint16_t u16;
typedef uint32_t u32;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }

// 16-byte load through the global address space.  Pointers fetched from LDS or
// computed at run time are otherwise generic (flat) loads, which also count on the
// LDS counter: waiting for an LDS operand would then wait for the HBM prefetch too.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const void* p) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
      reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ u16 f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(u16, h);
}

// cos/sin of RoPE pair p for a token at (t, h, w).  Branch-free: the table and the index are
// selected and one load is issued, so the loads of several pairs can be in flight together
// (lanes of one wave often hold pairs of different axes; with a branch per axis every branch's
// load would be issued and waited for on its own).
// The three tables lie back to back (time, height, width), so one uniform base and a 32-bit
// index address them: a per-lane choice of 64-bit table pointers costs twice the registers.
__device__ __forceinline__ void rope_cs(const RopeTab rt, int p, int t, int h, int w, float& c,
                                        float& s) {
  const bool on_t = p < rt.pt, on_h = p < rt.pt + rt.ph;
  const int h0 = (int)(rt.h - rt.t), w0 = (int)(rt.w - rt.t);
  const int idx = on_t ? t * rt.pt + p
                       : (on_h ? h0 + h * rt.ph + (p - rt.pt) : w0 + w * rt.pw + (p - rt.pt - rt.ph));
  const CosSin v = rt.t[idx];
  c = v.c;
  s = v.s;
}

// Position of key c inside a 16-key group of the bf16 V^T cache layout.
// Column c of a group holds key perm16(c): [0..3, 8..11, 4..7, 12..15]; the map is
// its own inverse.  With it, the 8 keys one half-wave needs as the A operand of a
// 32x32x16 MFMA (the rows of the 32x32 score tile it holds) are contiguous.
__host__ __device__ __forceinline__ int perm16(int c) {
  return (c >= 4 && c < 8) ? c + 4 : ((c >= 8 && c < 12) ? c - 4 : c);
}

// blockIdx -> task id so that consecutive tasks run on the same XCD (workgroups
// are dealt to the 8 XCDs round-robin); keeps one head's K/V reads in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, x = bid & 7, loc = bid >> 3;
  return (x < r) ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
}

}  // namespace swattn
