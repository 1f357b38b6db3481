// K1 for fp8 caches: rotate K at block-local positions, quantise K and V to OCP E4M3 with
// power-of-two (E8M0) scales per group of 32 values, store them in the layout the fp8
// attention kernel's scaled MFMAs read; and the read-back (dequantise to fp32).
//
// Quantised attention is chosen per layer in the pages' stack (Vidu S2 paper read, section
// 2.4); the scheme is this library's own, built for CDNA4's scaled fp8 matrix instructions:
//   * a group of 32 values shares 2^e, e = ceil(log2(amax / 448)) (-127 for an all-zero
//     group); an element is the E4M3 rounding (to nearest, ties to even) of x / 2^e;
//   * K [H][n_pad][128] bytes, groups = 32 consecutive channels of a key; its scale bytes
//     (e + 127) follow all K data as [H][n_pad][4];
//   * V^T [H][n_pad / 64][128][64] bytes (block-major: one 64-key block of a head is one
//     contiguous 8 KB run); inside each block, storage position 32 * s + j holds
//     key 32 * (j / 16) + 8 * (j / 4 % 4) + 4 * s + j % 4 -- the order in which one lane of the
//     attention kernel holds 32 probabilities of its query; the groups are the block's first
//     and last 32 keys (positions [0, 16) + [32, 48) and [16, 32) + [48, 64)), per channel; the
//     scale bytes follow all V data as [H][n_pad / 64][2][32][4] (block, group, channel % 32,
//     channel / 32).  (The scaled MFMA applies the scale of lane half 0 to operand bytes 0-15
//     of both lane halves and that of half 1 to bytes 16-31.)
// One workgroup per (128-token tile, head); HBM-bound.
#include "device_common.h"

namespace swattn {

namespace {

struct Fp8Args {
  const u16* k_raw;
  const u16* v_raw;
  uint8_t* k_dst;   // data, then the scale bytes
  uint8_t* v_dst;
  int B, H, n_pad, hw, lat_w;
  RopeTab rt;
};

// key index (inside a 64-key block) stored at position 32 * half + j of a V^T row
__host__ __device__ __forceinline__ int v_key_of(int half, int j) {
  return 32 * (j >> 4) + 8 * ((j >> 2) & 3) + 4 * half + (j & 3);
}

__device__ __forceinline__ int e8m0_of(float amax) {   // smallest e with amax / 2^e <= 448
  const uint32_t b = __float_as_uint(amax);
  const int E = (b >> 23) & 255;
  if (E == 0) return -127;                              // zero (or subnormal): the smallest scale
  const int e = E - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float pow2_neg(int e) {      // 2^-e for e in [-127, 126]
  return __uint_as_float((uint32_t)(127 - e) << 23);
}
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__global__ __launch_bounds__(256) void append_fp8_kernel(Fp8Args a) {
  constexpr int D = 128, GPR = 16;
  __shared__ __attribute__((aligned(16))) u16 vl[kTile][D + 8];
  const int tid = threadIdx.x, j = blockIdx.x, h = blockIdx.y;
  const int grp = tid % GPR;
  const RopeTab rt = a.rt;
  uint8_t* kd = a.k_dst + (size_t)h * a.n_pad * D;
  uint8_t* ksc = a.k_dst + (size_t)a.H * a.n_pad * D + (size_t)h * a.n_pad * 4;

  // loads are unconditional (a pad row reads row 0, always valid, and is zeroed by select), so a
  // row's K, V and table loads are in flight together instead of one branch at a time
#pragma unroll 2
  for (int it = 0; it < kTile * GPR / 256; ++it) {
    const int row = (tid + 256 * it) / GPR;
    const int r = j * kTile + row;
    const bool ok = r < a.B;
    const int rc = ok ? r : 0;
    const uint4 raw = ldg16(a.k_raw + ((size_t)rc * a.H + h) * D + grp * 8);
    const uint4 v = ldg16(a.v_raw + ((size_t)rc * a.H + h) * D + grp * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const int f = rc / a.hw, rem = rc - f * a.hw, hh = rem / a.lat_w, ww = rem - hh * a.lat_w;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c, s;
      rope_cs(rt, grp * 4 + i, f, hh, ww, c, s);
      const float x0 = __uint_as_float(w[i] << 16), x1 = __uint_as_float(w[i] & 0xffff0000u);
      x[2 * i] = ok ? x0 * c - x1 * s : 0.f;
      x[2 * i + 1] = ok ? x0 * s + x1 * c : 0.f;
    }
    // group of 32 channels = 4 neighbouring lanes of the row
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int e = e8m0_of(amax);
    const float sc = pow2_neg(e);
    uint2 q;
    q.x = pack4_fp8(x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc);
    q.y = pack4_fp8(x[4] * sc, x[5] * sc, x[6] * sc, x[7] * sc);
    *reinterpret_cast<uint2*>(kd + (size_t)r * D + grp * 8) = q;
    if ((grp & 3) == 0) ksc[(size_t)r * 4 + (grp >> 2)] = (uint8_t)(e + 127);
    *reinterpret_cast<uint4*>(&vl[row][grp * 8]) = ok ? v : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // V^T: (channel, 64-key block, group) items; group g (keys 32g..32g+31) sits at storage
  // positions [16g, 16g + 16) and [32 + 16g, 32 + 16g + 16)
  uint8_t* vd = a.v_dst + ((size_t)h * (a.n_pad / 64) + 2 * j) * D * 64;   // block 2j of head h
  uint8_t* vsc = a.v_dst + (size_t)a.H * D * a.n_pad + (size_t)h * a.n_pad * 4;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = tid + 256 * it;
    const int dd = item & 127, bg = item >> 7, blk = bg >> 1, g = bg & 1;
    float x[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int pos = (i < 16 ? 16 * g : 32 + 16 * g) + (i & 15);
      x[i] = bf2f(vl[blk * 64 + v_key_of(pos >> 5, pos & 31)][dd]);
      amax = fmaxf(amax, fabsf(x[i]));
    }
    const int e = e8m0_of(amax);
    const float sc = pow2_neg(e);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack4_fp8(x[4 * i] * sc, x[4 * i + 1] * sc, x[4 * i + 2] * sc, x[4 * i + 3] * sc);
    uint8_t* row = vd + ((size_t)blk * D + dd) * 64;
    *reinterpret_cast<uint4*>(row + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(row + 32 + 16 * g) = make_uint4(w[4], w[5], w[6], w[7]);
    const int gblk = j * 2 + blk;
    vsc[((size_t)(gblk * 2 + g) * 32 + (dd & 31)) * 4 + (dd >> 5)] = (uint8_t)(e + 127);
  }
}

__device__ __forceinline__ float fp8_decode(uint32_t c) {   // OCP E4M3
  const int e = (c >> 3) & 15, m = c & 7;
  const float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float((uint32_t)(e + 120) << 23) * (1.f + m * 0.125f);
  return (c & 0x80) ? -v : v;
}
__device__ __forceinline__ float pow2(int byte) { return __uint_as_float((uint32_t)byte << 23); }   // 2^(byte-127)

__global__ __launch_bounds__(256) void unpack_fp8_kernel(const uint8_t* k_src, const uint8_t* v_src, float* k_out,
                                                          float* v_out, int B, int H, int n_pad) {
  constexpr int D = 128;
  const size_t total = (size_t)B * H * D;
  const uint8_t* ksc = k_src + (size_t)H * n_pad * D;
  const uint8_t* vsc = v_src + (size_t)H * D * n_pad;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (size_t)gridDim.x * 256) {
    const int dd = idx % D;
    const int h = (idx / D) % H;
    const int r = idx / ((size_t)H * D);
    const int kbyte = ksc[((size_t)h * n_pad + r) * 4 + (dd >> 5)];
    k_out[idx] = fp8_decode(k_src[((size_t)h * n_pad + r) * D + dd]) * pow2(kbyte);
    const int gblk = r >> 6, k = r & 63, half = (k >> 2) & 1, grp = k >> 5;
    const int jj = 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3);    // inverse of v_key_of
    const int vbyte = vsc[((size_t)h * n_pad * 4) + ((size_t)(gblk * 2 + grp) * 32 + (dd & 31)) * 4 + (dd >> 5)];
    v_out[idx] = fp8_decode(v_src[(((size_t)h * (n_pad / 64) + gblk) * D + dd) * 64 + 32 * half + jj]) * pow2(vbyte);
  }
}

}  // namespace

hipError_t launch_append_fp8(const Geometry& g, const RopeTab& rt, const void* k_raw, const void* v_raw, void* k_dst,
                             void* v_dst, hipStream_t stream) {
  if (g.d != 128) return hipErrorInvalidValue;
  Fp8Args a{static_cast<const u16*>(k_raw), static_cast<const u16*>(v_raw), static_cast<uint8_t*>(k_dst),
            static_cast<uint8_t*>(v_dst), g.B, g.H, g.n_pad, g.lat_h * g.lat_w, g.lat_w, rt};
  hipLaunchKernelGGL(append_fp8_kernel, dim3(g.nt, g.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_unpack_fp8(const Geometry& g, const void* k_src, const void* v_src, void* k_out, void* v_out,
                             hipStream_t stream) {
  if (g.d != 128) return hipErrorInvalidValue;
  const size_t total = (size_t)g.B * g.H * g.d;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  hipLaunchKernelGGL(unpack_fp8_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint8_t*>(k_src),
                     static_cast<const uint8_t*>(v_src), static_cast<float*>(k_out), static_cast<float*>(v_out), g.B,
                     g.H, g.n_pad);
  return hipGetLastError();
}

}  // namespace swattn
