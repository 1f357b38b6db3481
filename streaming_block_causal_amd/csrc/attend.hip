// K2 / K3: one denoising step's chunk attention over the bounded KV cache.
//
// For head h and query n of the current block:
//   O[n] = softmax_k( <R(p_n) q_n, R(p_k) k> / sqrt(d) ) V
// over the keys of [sinks, window oldest->newest, current] (Vidu S2 vs PixVerse
// R2 blog, sections "What real-time changes" and "Choice 3: bounded memory";
// block-wise causal attention, Vidu S2 paper read, section 2.2).  The current
// block sees itself in full; older blocks are visible through the cache, later
// ones do not exist yet.
//
// Relocation without moving data: K is stored rotated at block-local positions
// (t = frame in block).  Pairs of different axes commute, so rotating the query
// at time (frame + delta_l), delta_l = base(current) - base(slot l), gives every
// score the relocated relative angle.  The query tile is re-rotated (fp32 ->
// bf16) each time the key loop enters a new slot; stored keys are never touched
// again, which also makes the result independent of where the ring sits.
//
// bf16 path (d = 128): one workgroup = 4 waves = 128 queries of one head; each
// wave owns 32 queries.  Keys stream through LDS 64 at a time.  A wave computes
// the transposed score tile S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so every
// lane holds 16 keys of ONE query: the softmax row max and sum are in-register
// plus one cross-half exchange (v_permlane32_swap).  P^T stays in registers as
// the B operand of O^T += V^T P^T; the V^T cache layout (keys permuted in groups
// of 16) makes the matching A operand one 16-byte LDS read.  Online softmax runs
// in the log2 domain with the 1/sqrt(d) scale folded into one FMA before v_exp.
// Block-sparse (K3): the same loop, over the listed 128-key tiles only.
//
// fp32 path (d = 64 or 128): one thread per query, keys broadcast from LDS;
// exact-ish reference-grade arithmetic for the small fp32 workload.
#include "device_common.h"

namespace swattn {

namespace {

constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const void* q;
  void* o;
  float* lse;
  const int32_t* tile_idx;
  int k_row;
  int B, H, n_pad, nt, hw, lat_w;
  int n_slots;
  float scale_log2;   // log2(e) / sqrt(d)
  RopeTab rt;
  SlotPtrs slot[kMaxSlots];
};

__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------------------------
// bf16 MFMA kernel
// ------------------------------------------------------------------------------------
constexpr int D = 128;
constexpr int QW = 32;          // queries per wave
constexpr int KB = 64;          // keys per LDS block
constexpr int KS = D + 8;       // LDS row stride of K (bf16 elements)
constexpr int VS = KB + 8;      // LDS row stride of V^T

template <bool SPARSE>
__global__ __launch_bounds__(256) void attend_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) u16 ks[KB * KS];
  __shared__ __attribute__((aligned(16))) u16 vs[D * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, ln = lane & 31;
  const int task = xcd_remap(blockIdx.x, gridDim.x);
  const int h = task / a.nt, qt = task - h * a.nt;
  const int qrow = qt * kTile + wave * QW + ln;
  const bool qvalid = qrow < a.B;
  const int qf = qrow / a.hw, qrem = qrow - qf * a.hw;
  const int qh = qrem / a.lat_w, qw = qrem - qh * a.lat_w;
  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)qrow * a.H + h) * D;

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  bf16x8 qb[8];

  // Q^T operand for slot delta: lane (hf, ln) holds q[ln][16j + 8hf + 0..7], rotated.
  auto load_q = [&](int delta) {
    const int t = qf + delta;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!qvalid) {   // rows past the block: zero operand, no table reads
#pragma unroll
        for (int i = 0; i < 8; ++i) qb[j][i] = (__bf16)0.f;
        continue;
      }
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * j + 8 * hf);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float c, s;
        rope_cs(a.rt, 8 * j + 4 * hf + i, t, qh, qw, c, s);
        const float x0 = __uint_as_float(w[i] << 16), x1 = __uint_as_float(w[i] & 0xffff0000u);
        qb[j][2 * i] = (__bf16)(x0 * c - x1 * s);
        qb[j][2 * i + 1] = (__bf16)(x0 * s + x1 * c);
      }
    }
  };

  auto do_block = [&](const u16* kbase, const u16* vbase, int kb) {
    __syncthreads();   // previous block fully consumed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = c & 15;
      *reinterpret_cast<uint4*>(&ks[row * KS + col * 8]) =
          *reinterpret_cast<const uint4*>(kbase + (size_t)(kb * KB + row) * D + col * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, dd = c >> 3, col = c & 7;
      *reinterpret_cast<uint4*>(&vs[dd * VS + col * 8]) =
          *reinterpret_cast<const uint4*>(vbase + (size_t)dd * a.n_pad + kb * KB + col * 8);
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&ks[(kt * 32 + ln) * KS + 16 * j + 8 * hf]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qb[j], s[kt], 0, 0, 0);
      }
    }
    const int kvalid = a.B - kb * KB;
    if (kvalid < KB) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= kvalid) s[kt][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = swap_halves_max(mx);
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], a.scale_log2, -m_new));
        s[kt][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
    bf16x8 pb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[g][i] = (__bf16)s[g >> 1][8 * (g & 1) + i];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(&vs[(32 * t + ln) * VS + 16 * g + 8 * hf]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[g], acc[t], 0, 0, 0);
      }
  };

  const int nkb = (a.B + KB - 1) / KB;
  const size_t kstride = (size_t)a.n_pad * D;   // per head, K and V^T alike
  if (!SPARSE) {
    for (int sl = 0; sl < a.n_slots; ++sl) {
      load_q(a.slot[sl].delta);
      const u16* kbase = static_cast<const u16*>(a.slot[sl].k) + h * kstride;
      const u16* vbase = static_cast<const u16*>(a.slot[sl].v) + h * kstride;
      for (int kb = 0; kb < nkb; ++kb) do_block(kbase, vbase, kb);
    }
  } else {
    const int32_t* list = a.tile_idx + ((size_t)h * a.nt + qt) * a.k_row;
    int cur = -1;
    const u16 *kbase = nullptr, *vbase = nullptr;
    for (int i = 0; i < a.k_row; ++i) {
      const int tix = list[i];
      if (tix < 0 || tix >= a.n_slots * a.nt) continue;   // never read outside the cache
      const int sl = tix / a.nt, jt = tix - sl * a.nt;
      if (sl != cur) {
        cur = sl;
        load_q(a.slot[sl].delta);
        kbase = static_cast<const u16*>(a.slot[sl].k) + h * kstride;
        vbase = static_cast<const u16*>(a.slot[sl].v) + h * kstride;
      }
      do_block(kbase, vbase, 2 * jt);
      if (2 * jt + 1 < nkb) do_block(kbase, vbase, 2 * jt + 1);
    }
  }

  const float l_tot = swap_halves_sum(l_run);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    u16* op = static_cast<u16*>(a.o) + ((size_t)qrow * a.H + h) * D;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * t + 8 * rg + 4 * hf;
        uint2 w;
        w.x = (uint32_t)f2bf(acc[t][4 * rg] * inv) | ((uint32_t)f2bf(acc[t][4 * rg + 1] * inv) << 16);
        w.y = (uint32_t)f2bf(acc[t][4 * rg + 2] * inv) | ((uint32_t)f2bf(acc[t][4 * rg + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (a.lse && hf == 0) a.lse[(size_t)h * a.B + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------------------------------
// fp32 kernel: one thread per query, keys broadcast from LDS, 16-key sub-blocks
// ------------------------------------------------------------------------------------
template <int DD>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttnArgs a) {
  constexpr int KBF = 32;
  __shared__ float kl[KBF][DD];
  __shared__ float vl[KBF][DD];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int qrow = blockIdx.x * 64 + tid;
  const bool qvalid = qrow < a.B;
  const int qf = qrow / a.hw, qrem = qrow - qf * a.hw;
  const int qh = qrem / a.lat_w, qw = qrem - qh * a.lat_w;
  const float* qp = static_cast<const float*>(a.q) + ((size_t)qrow * a.H + h) * DD;
  float qr[DD], acc[DD];
#pragma unroll
  for (int i = 0; i < DD; ++i) acc[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = a.scale_log2;

  for (int sl = 0; sl < a.n_slots; ++sl) {
    const int t = qf + a.slot[sl].delta;
#pragma unroll
    for (int p = 0; p < DD / 2; ++p) {
      float c = 1.f, s = 0.f, x0 = 0.f, x1 = 0.f;
      if (qvalid) {
        rope_cs(a.rt, p, t, qh, qw, c, s);
        x0 = qp[2 * p];
        x1 = qp[2 * p + 1];
      }
      qr[2 * p] = x0 * c - x1 * s;
      qr[2 * p + 1] = x0 * s + x1 * c;
    }
    const float* kbase = static_cast<const float*>(a.slot[sl].k) + (size_t)h * a.n_pad * DD;
    const float* vbase = static_cast<const float*>(a.slot[sl].v) + (size_t)h * a.n_pad * DD;
    for (int k0 = 0; k0 < a.B; k0 += KBF) {
      __syncthreads();
      for (int i = tid; i < KBF * DD; i += 64) {
        kl[i / DD][i % DD] = kbase[(size_t)k0 * DD + i];
        vl[i / DD][i % DD] = vbase[(size_t)k0 * DD + i];
      }
      __syncthreads();
      const int nk = min(KBF, a.B - k0);
      float sc[KBF];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KBF; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DD; ++i) dot = fmaf(qr[i], kl[j][i], dot);
        sc[j] = j < nk ? dot * scale : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DD; ++i) acc[i] *= alpha;
#pragma unroll
      for (int j = 0; j < KBF; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[j] - m_new);
        l_run += p;
#pragma unroll
        for (int i = 0; i < DD; ++i) acc[i] = fmaf(p, vl[j][i], acc[i]);
      }
    }
  }
  if (qvalid) {
    float* op = static_cast<float*>(a.o) + ((size_t)qrow * a.H + h) * DD;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int i = 0; i < DD; ++i) op[i] = acc[i] * inv;
    if (a.lse) a.lse[(size_t)h * a.B + qrow] = (m_run + __log2f(l_run)) * kLn2;
  }
}

}  // namespace

hipError_t launch_attend(const Geometry& g, const RopeTab& rt, bool bf16, const void* q,
                         const SlotPtrs* slots, int n_slots, const int32_t* tile_idx, int k_row,
                         void* out, float* lse, hipStream_t stream) {
  if (n_slots < 1 || n_slots > kMaxSlots) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q;
  a.o = out;
  a.lse = lse;
  a.tile_idx = tile_idx;
  a.k_row = k_row;
  a.B = g.B;
  a.H = g.H;
  a.n_pad = g.n_pad;
  a.nt = g.nt;
  a.hw = g.lat_h * g.lat_w;
  a.lat_w = g.lat_w;
  a.n_slots = n_slots;
  a.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)g.d));
  a.rt = rt;
  for (int i = 0; i < kMaxSlots; ++i) a.slot[i] = i < n_slots ? slots[i] : SlotPtrs{nullptr, nullptr, 0};
  if (bf16) {
    if (g.d != 128) return hipErrorInvalidValue;
    const dim3 grid(g.nt * g.H), block(256);
    if (tile_idx)
      hipLaunchKernelGGL((attend_bf16_kernel<true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attend_bf16_kernel<false>), grid, block, 0, stream, a);
  } else {
    if (tile_idx) return hipErrorInvalidValue;
    const dim3 grid((g.B + 63) / 64, g.H), block(64);
    if (g.d == 64)
      hipLaunchKernelGGL((attend_f32_kernel<64>), grid, block, 0, stream, a);
    else if (g.d == 128)
      hipLaunchKernelGGL((attend_f32_kernel<128>), grid, block, 0, stream, a);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swattn
