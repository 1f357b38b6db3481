// K1: fused RoPE + KV append, and the cache read-back kernel.
//
// A block's raw K/V arrive token-major [B][H][d] (what a QKV projection writes).
// The kernel rotates K at block-local positions (t = frame within the block, h,
// w) -- the time relocation of each block is applied later to the queries, so a
// stored block never has to be rewritten when the window slides (Vidu S2 vs
// PixVerse R2 blog, section "Choice 3: bounded memory": RoPE relocation keeps
// positions in the trained range) -- and stores K and V head-major so every
// attention tile is one contiguous run of HBM.  bf16 V is stored transposed
// and tile-major (V^T [H][n_pad / 128][d][128]: one 128-key tile of a head is one
// contiguous 32 KB run, which also keeps the block-sparse kernel's scattered tile
// reads inside few DRAM pages) with keys permuted inside groups of 16 (perm16), the
// operand order of the attention kernel's P.V MFMA.  Pad rows are zero.  For
// block-sparse caches it also writes the fp32 mean of the rotated K of every
// 128-token tile (valid tokens only), the pooled keys the tile mask scores.
//
// One workgroup per (128-token tile, head); HBM-bound: reads B*H*d raw K and V
// once, writes them once.
//
// The fused QKV epilogue (NORM) reads the packed output of a QKV projection
// ([B][3][H][d]: q, k, v of a token side by side), normalises q and k per head
// (RMSNorm over d with per-channel weights: x / sqrt(mean(x^2) + eps) * g),
// writes the normalised q token-major for the attention call, and stores the
// normalised, rotated k and the v like the plain append -- one pass over HBM for
// what would otherwise be two norm kernels and the append (Vidu S2 paper read,
// section 2.4: adjacent operators such as RMSNorm and elementwise work fused
// into one kernel).
#include "device_common.h"

namespace swattn {

namespace {

struct AppendArgs {
  const void* k_raw;
  const void* v_raw;
  void* k_dst;
  void* v_dst;
  float* pooled;
  int B, H, n_pad, nt, hw, lat_w;
  RopeTab rt;
  size_t row_stride;    // elements from one token's k (or v) to the next: H*d, or 3*H*d packed
  const void* q_raw;    // NORM only: q of the packed projection output, normalised into q_out
  void* q_out;          // [B][H][d]
  const float* gq;      // [d] RMSNorm weights of q and k
  const float* gk;
  float eps;
};

// sum over the 16 lanes that hold one row (aligned groups of 16 within the wave)
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// x[0..8) of a row (this lane's 8 channels starting at c0) *= rsqrt(mean over the row of x^2 + eps) * g
__device__ __forceinline__ void rms_scale8(float* x, const float* g, int c0, int D, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = row16_sum(ss);
  const float inv = 1.0f / __builtin_sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x[i] * inv * g[c0 + i];
}

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  typedef u16 T;
  static __device__ __forceinline__ void load8(const u16* p, float* x) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store8(u16* p, const float* x) {
    uint4 v;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(x[2 * i]) | ((uint32_t)f2bf(x[2 * i + 1]) << 16);
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    *reinterpret_cast<uint4*>(p) = v;
  }
};
template <>
struct Elem<false> {
  typedef float T;
  static __device__ __forceinline__ void load8(const float* p, float* x) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void store8(float* p, const float* x) {
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
};

template <int D, bool BF16, bool NORM>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  static_assert(!NORM || D / 8 == 16, "the row reduction assumes 16 lanes per row");
  typedef typename Elem<BF16>::T T;
  constexpr int GPR = D / 8;              // 8-element groups per row
  constexpr int ITEMS = kTile * GPR / 256;
  constexpr int SUB = 256 / GPR;          // row sub-groups in the pooled reduction
  constexpr int VROWS = kTile / 2;        // V rows staged in LDS at a time (bf16 transpose)
  // one LDS buffer: first the pooled partial sums, then (bf16) half a tile of V rows; small
  // enough for 8 workgroups per CU, so a whole 540p launch is resident at once
  // V rows staged with a stride of D + 2 elements (an odd number of 4-byte words): the transpose
  // reads rows 0, 4, 16, 20, ... of one column in a single instruction, and an odd stride sends
  // them to distinct banks (a 16-byte-aligned stride cannot)
  constexpr int VST = D + 2;
  constexpr int SMEM = SUB * D * 4 > VROWS * VST * 2 ? SUB * D * 4 : VROWS * VST * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  float (*red)[D] = reinterpret_cast<float (*)[D]>(smem);
  u16 (*vl)[VST] = reinterpret_cast<u16 (*)[VST]>(smem);

  const int tid = threadIdx.x, j = blockIdx.x, h = blockIdx.y;
  const int grp = tid % GPR;
  const RopeTab rt = a.rt;
  const T* kr = static_cast<const T*>(a.k_raw);
  const T* vr = static_cast<const T*>(a.v_raw);
  T* kd = static_cast<T*>(a.k_dst) + (size_t)h * a.n_pad * D;

  float pacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pacc[i] = 0.f;

  // Loads are unconditional (a pad row reads row 0, always valid, and its values are replaced
  // by zeros), so the compiler can keep the loads of several rows in flight: behind a branch
  // each load was issued and waited for on its own.
#pragma unroll 2
  for (int it = 0; it < ITEMS; ++it) {
    const int row = (tid + 256 * it) / GPR;
    const int r = j * kTile + row;
    const bool ok = r < a.B;
    const int rc = ok ? r : 0;
    float x[8];
    if (NORM) {   // q: normalise, store token-major (the attention call rotates it)
      float y[8];
      Elem<BF16>::load8(static_cast<const T*>(a.q_raw) + (size_t)rc * a.row_stride + (size_t)h * D + grp * 8, y);
      rms_scale8(y, a.gq, grp * 8, D, a.eps);
      if (ok) Elem<BF16>::store8(static_cast<T*>(a.q_out) + ((size_t)r * a.H + h) * D + grp * 8, y);
    }
    Elem<BF16>::load8(kr + (size_t)rc * a.row_stride + (size_t)h * D + grp * 8, x);
    if (NORM) rms_scale8(x, a.gk, grp * 8, D, a.eps);
    const int f = rc / a.hw, rem = rc - f * a.hw, hh = rem / a.lat_w, ww = rem - hh * a.lat_w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c, s;
      rope_cs(rt, grp * 4 + i, f, hh, ww, c, s);
      const float x0 = x[2 * i], x1 = x[2 * i + 1];
      x[2 * i] = ok ? x0 * c - x1 * s : 0.f;
      x[2 * i + 1] = ok ? x0 * s + x1 * c : 0.f;
      pacc[2 * i] += x[2 * i];
      pacc[2 * i + 1] += x[2 * i + 1];
    }
    Elem<BF16>::store8(kd + (size_t)r * D + grp * 8, x);

    if (!BF16) {   // fp32 V: a straight copy, head-major
      float y[8];
      Elem<BF16>::load8(vr + (size_t)rc * a.row_stride + (size_t)h * D + grp * 8, y);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ok ? y[i] : 0.f;
      T* vd = static_cast<T*>(a.v_dst) + ((size_t)h * a.n_pad + r) * D + grp * 8;
      Elem<BF16>::store8(vd, y);
    }
  }

  if (a.pooled) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[tid / GPR][grp * 8 + i] = pacc[i];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < SUB; ++i) s += red[i][tid];
      const int cnt = min(kTile, a.B - j * kTile);
      a.pooled[((size_t)h * D + tid) * a.nt + j] = s / (float)cnt;   // [H][d][nt]: tiles contiguous
    }
  }

  if (BF16) {
    // V^T rows: dd = feature, 16 chunks of 8 keys (perm16 order) per 128-key tile, written in two
    // halves of 64 keys through LDS
    u16* vt = static_cast<u16*>(a.v_dst) + ((size_t)h * (a.n_pad / kTile) + j) * D * kTile;   // slot's full stride
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      __syncthreads();   // the buffer's previous use (pooled sums or the other half) is finished
      constexpr int NV = VROWS * GPR / 256;
      uint4 v[NV];
#pragma unroll
      for (int it = 0; it < NV; ++it) {   // all loads first (unconditional, see above)
        const int r = j * kTile + VROWS * hv + (tid + 256 * it) / GPR;
        v[it] = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(vr) + (size_t)(r < a.B ? r : 0) * a.row_stride +
                                                (size_t)h * D + grp * 8);
      }
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int row = (tid + 256 * it) / GPR;
        const bool ok = j * kTile + VROWS * hv + row < a.B;
        const uint4 x = ok ? v[it] : make_uint4(0, 0, 0, 0);
        uint32_t* dst = reinterpret_cast<uint32_t*>(&vl[row][grp * 8]);   // 4-byte aligned rows
        dst[0] = x.x;
        dst[1] = x.y;
        dst[2] = x.z;
        dst[3] = x.w;
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < D * 8 / 256; ++it) {
        const int c = tid + 256 * it;
        const int dd = c >> 3, cc = 8 * hv + (c & 7);
        const int g = cc >> 1, half = cc & 1;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = 16 * g + perm16(8 * half + 2 * i) - VROWS * hv;
          const int k1 = 16 * g + perm16(8 * half + 2 * i + 1) - VROWS * hv;
          w[i] = (uint32_t)vl[k0][dd] | ((uint32_t)vl[k1][dd] << 16);
        }
        *reinterpret_cast<uint4*>(vt + (size_t)dd * kTile + 8 * cc) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void unpack_kernel(const void* k_src, const void* v_src,
                                                     void* k_out, void* v_out, int B, int H,
                                                     int n_pad) {
  typedef typename Elem<BF16>::T T;
  const size_t total = (size_t)B * H * D;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * 256) {
    const int dd = idx % D;
    const int h = (idx / D) % H;
    const int r = idx / ((size_t)H * D);
    static_cast<T*>(k_out)[idx] = static_cast<const T*>(k_src)[((size_t)h * n_pad + r) * D + dd];
    if (BF16) {
      const int tile = r / kTile, in = r % kTile, g = in >> 4, c = perm16(in & 15);
      static_cast<T*>(v_out)[idx] = static_cast<const T*>(
          v_src)[(((size_t)h * (n_pad / kTile) + tile) * D + dd) * kTile + 16 * g + c];
    } else {
      static_cast<T*>(v_out)[idx] = static_cast<const T*>(v_src)[((size_t)h * n_pad + r) * D + dd];
    }
  }
}

}  // namespace

hipError_t launch_append(const Geometry& g, const RopeTab& rt, bool bf16, const void* k_raw,
                         const void* v_raw, void* k_dst, void* v_dst, float* pooled_dst,
                         hipStream_t stream) {
  AppendArgs a{k_raw, v_raw, k_dst, v_dst, pooled_dst, g.B, g.H, g.n_pad, g.nt,
               g.lat_h * g.lat_w, g.lat_w, rt, (size_t)g.H * g.d, nullptr, nullptr, nullptr, nullptr, 0.f};
  const dim3 grid(g.nt, g.H), block(256);
  if (bf16 && g.d == 128) {
    hipLaunchKernelGGL((append_kernel<128, true, false>), grid, block, 0, stream, a);
  } else if (!bf16 && g.d == 128) {
    hipLaunchKernelGGL((append_kernel<128, false, false>), grid, block, 0, stream, a);
  } else if (!bf16 && g.d == 64) {
    hipLaunchKernelGGL((append_kernel<64, false, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append_qkv(const Geometry& g, const RopeTab& rt, bool bf16, const void* qkv,
                             const float* gamma_q, const float* gamma_k, float eps, void* q_out,
                             void* k_dst, void* v_dst, float* pooled_dst, hipStream_t stream) {
  const size_t hd = (size_t)g.H * g.d;
  const size_t esz = bf16 ? 2 : 4;
  const char* base = static_cast<const char*>(qkv);
  AppendArgs a{base + hd * esz, base + 2 * hd * esz, k_dst, v_dst, pooled_dst, g.B, g.H, g.n_pad, g.nt,
               g.lat_h * g.lat_w, g.lat_w, rt, 3 * hd, base, q_out, gamma_q, gamma_k, eps};
  const dim3 grid(g.nt, g.H), block(256);
  if (bf16 && g.d == 128) {
    hipLaunchKernelGGL((append_kernel<128, true, true>), grid, block, 0, stream, a);
  } else if (!bf16 && g.d == 128) {
    hipLaunchKernelGGL((append_kernel<128, false, true>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;   // the row reduction is built for d = 128
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const Geometry& g, bool bf16, const void* k_src, const void* v_src,
                         void* k_out, void* v_out, hipStream_t stream) {
  const size_t total = (size_t)g.B * g.H * g.d;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (bf16 && g.d == 128) {
    hipLaunchKernelGGL((unpack_kernel<128, true>), dim3(blocks), dim3(256), 0, stream, k_src,
                       v_src, k_out, v_out, g.B, g.H, g.n_pad);
  } else if (!bf16 && g.d == 128) {
    hipLaunchKernelGGL((unpack_kernel<128, false>), dim3(blocks), dim3(256), 0, stream, k_src,
                       v_src, k_out, v_out, g.B, g.H, g.n_pad);
  } else if (!bf16 && g.d == 64) {
    hipLaunchKernelGGL((unpack_kernel<64, false>), dim3(blocks), dim3(256), 0, stream, k_src,
                       v_src, k_out, v_out, g.B, g.H, g.n_pad);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swattn
