// K4: block-sparse tile mask for one attention call (bf16, d = 128).
//
// R2 reaches >90% attention sparsity with block-sparse attention learned in
// training (Vidu S2 vs PixVerse R2 blog, section "Choice 4: where the speed comes
// from").  Without trained weights the mask is built from the data: per head and
// 128-query tile, every 128-key tile of every cached block is scored by the dot
// product of the mean relocated query and the mean relocated key / sqrt(d); key
// tile 0 of the first sink (when there is a sink) and the diagonal current tile
// are always kept, the remaining budget goes to the highest scores, ties to the
// lower linear index.  Rotation is linear and the time rotation of a slot is the
// same for all its tokens, so the relocated pooled query is the block-local
// pooled query turned by R_t(delta_l) -- the pooled keys come from the append
// kernel, rotated at block-local positions.
//
// One workgroup per (query tile, head): it reads the query tile once and the small
// pooled-key tables.  The selection is a per-wave radix search for the budget's
// threshold score (32 ballot rounds): linear in the number of key tiles, where an
// all-pairs rank is quadratic (4096 key tiles at the largest shapes).
#include "device_common.h"

#include <type_traits>

namespace swattn {

namespace {

// query tiles per workgroup (one wave selects for each): 1 measured fastest at 540p, where
// 4 (each pooled key read once for four tiles) leaves too few workgroups to hide latency
constexpr int kQT = 1;

struct MaskArgs {
  const u16* q;
  int32_t* out;
  int k_row, k_cap;
  int B, H, nt, hw, lat_w;
  int n_slots, has_sink;
  float inv_sqrt_d;
  float inv_hw, inv_lat_w;   // 1 / (lat_h * lat_w), 1 / lat_w in fp32 (positions by multiplication)
  RopeTab rt;
  const float* pooled[kMaxSlots];
  int delta[kMaxSlots];
};

// order-preserving map of a finite score to an unsigned key >= 1 (-0 and +0 map alike);
// key 0 marks a tile that does not compete (forced, or past the end)
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t b = __float_as_uint(s + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(256) void tile_mask_kernel(MaskArgs a) {
  constexpr int D = 128;
  // dynamic LDS: first the partial sums of step 1 ([kQT][16][D] floats), then, reusing it, the
  // relocated pooled queries ([kQT][n_slots][D] floats) and the score keys ([kQT][n_kv64])
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  __shared__ float2 xm[kQT][D / 2];
  __shared__ const float* spooled[kMaxSlots];
  __shared__ CosSin relrow[kMaxSlots][32];   // each slot's time row of the relocation

  const int tid = threadIdx.x, qt0 = blockIdx.x * kQT, h = blockIdx.y;
  const int n_qt = min(kQT, a.nt - qt0);
  const int n_kv = a.n_slots * a.nt;
  const int n_kv64 = (n_kv + 63) & ~63;
  float* red = dyn;
  float* qs = dyn;
  uint32_t* keys = reinterpret_cast<uint32_t*>(dyn + kQT * a.n_slots * D);
  // the argument struct is never addressed (that would copy it to scratch): static indices only
#pragma unroll
  for (int q = 0; q < kMaxSlots; ++q)
    if (tid == q) spooled[q] = a.pooled[q];
  const RopeTab rt = a.rt;
  // the time rows of the relocation (step 2), one per slot, go straight into LDS now (load-to-LDS,
  // no registers held), so their latency passes under step 1.  A row is pt <= 32 entries (256
  // bytes, one 4-byte word per lane); lanes past its end re-read its last word, and a row of no
  // entries reads the first word of the (back-to-back, never empty) tables: all in bounds.
  {
    // the wave index made uniform: slot loop, delta and LDS row address stay scalar
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
    const int off = min(4 * ln, max(8 * rt.pt - 4, 0));
    for (int sl = w; sl < a.n_slots; sl += 4) {
      int dl = 0;
#pragma unroll
      for (int q = 0; q < kMaxSlots; ++q) dl = q == sl ? a.delta[q] : dl;
      const char* row = reinterpret_cast<const char*>(rt.t + dl * rt.pt) + off;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const __attribute__((address_space(1))) void*>(reinterpret_cast<uintptr_t>(row)),
          reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&relrow[sl][0])), 4, 0,
          0);
    }
  }

  // 1. per query tile, the sum over its valid queries of q rotated at block-local positions.
  //    Thread t takes 4 pairs (16 bytes) of 8 rows (16 apart) of every tile.  Positions come from
  //    reciprocal multiplications (exact below 2^16 tokens), and every Q load and every cos/sin
  //    gather of the thread is issued before the first is used: rows past the block read row 0
  //    and are dropped by a select, so no branch splits the loads into dependent groups.
  {
    const int pg = tid & 15, rg = tid >> 4;   // pair group (4 pairs), row group
    // the axis, row stride and first entry of each of the thread's 4 pairs (fixed for all its
    // rows); the three tables lie back to back, so one uniform base and 32-bit indices address them
    const CosSin* tab = rt.t;
    const int h0 = (int)(rt.h - rt.t), w0 = (int)(rt.w - rt.t);
    int axis[4], stride[4], col[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * pg + e;
      axis[e] = p < rt.pt ? 0 : (p < rt.pt + rt.ph ? 1 : 2);
      stride[e] = axis[e] == 0 ? rt.pt : (axis[e] == 1 ? rt.ph : rt.pw);
      col[e] = axis[e] == 0 ? p : (axis[e] == 1 ? h0 + p - rt.pt : w0 + p - rt.pt - rt.ph);
    }
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      uint4 raw[8];
      CosSin cs[8][4];
      bool ok[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (qt0 + t) * kTile + rg + 16 * i;
        ok[i] = t < n_qt && r < a.B;
        const int rr = ok[i] ? r : 0;
        raw[i] = ldg16(a.q + ((size_t)rr * a.H + h) * D + 8 * pg);
        const int f = (int)(((float)rr + 0.5f) * a.inv_hw);
        const int rem = rr - f * a.hw;
        const int hh = (int)(((float)rem + 0.5f) * a.inv_lat_w);
        const int ww = rem - hh * a.lat_w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = axis[e] == 0 ? f : (axis[e] == 1 ? hh : ww);
          cs[i][e] = tab[pos * stride[e] + col[e]];
        }
      }
      float acc8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // a row past the block contributes zeros (its loaded row-0 values are dropped)
        const uint32_t w[4] = {ok[i] ? raw[i].x : 0u, ok[i] ? raw[i].y : 0u, ok[i] ? raw[i].z : 0u,
                               ok[i] ? raw[i].w : 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = cs[i][e].c, sn = cs[i][e].s;
          const float x0 = __uint_as_float(w[e] << 16), x1 = __uint_as_float(w[e] & 0xffff0000u);
          acc8[2 * e] += x0 * c - x1 * sn;
          acc8[2 * e + 1] += x0 * sn + x1 * c;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(t * 16 + rg) * D + 8 * pg + e] = acc8[e];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the relocation rows are in LDS
  __syncthreads();
  // 2. means (thread = (tile, pair)), then the relocation per slot: the time pairs are turned by
  //    delta_l; the shared array is overwritten with the relocated queries only after the barrier
  {
    const int t = tid >> 6, p = tid & 63;
    if (t < n_qt) {
      const float cnt = (float)min(kTile, a.B - (qt0 + t) * kTile);
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        x0 += red[(t * 16 + g) * D + 2 * p];
        x1 += red[(t * 16 + g) * D + 2 * p + 1];
      }
      xm[t][p] = make_float2(x0 / cnt, x1 / cnt);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < n_qt * a.n_slots * (D / 2); idx += 256) {
    const int pp = idx & (D / 2 - 1), ts = idx / (D / 2), sl = ts % a.n_slots, t = ts / a.n_slots;
    const CosSin v = pp < rt.pt ? relrow[sl][pp] : CosSin{1.f, 0.f};
    const float2 m = xm[t][pp];
    qs[(t * a.n_slots + sl) * D + 2 * pp] = m.x * v.c - m.y * v.s;
    qs[(t * a.n_slots + sl) * D + 2 * pp + 1] = m.x * v.s + m.y * v.c;
  }
  __syncthreads();
  // 3. scores of every key tile against every query tile of the group: lane per key tile, the
  //    pooled keys are stored dimension-major so a wave's loads of one dimension are contiguous,
  //    and each pooled key is read once for the whole group.  Forced tiles (tile 0 of the first
  //    sink, the query tile's own diagonal tile) do not compete: key 0.
  const int f_sink = a.has_sink ? 0 : -1;
  const int f_diag0 = (a.n_slots - 1) * a.nt + qt0;
  for (int u = tid; u < n_kv64; u += 256) {
    // four partial sums over interleaved dimensions: four dependent chains of 32 FMAs instead of
    // one of 128
    float dot[kQT][4];
#pragma unroll
    for (int t = 0; t < kQT; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) dot[t][c] = 0.f;
    if (u < n_kv) {
      const int sl = u / a.nt, jt = u - sl * a.nt;
      const float* kp = spooled[sl] + (size_t)h * D * a.nt + jt;
      const float* qp = qs + sl * D;
#pragma unroll 32
      for (int i = 0; i < D; ++i) {
        const float kv = kp[(size_t)i * a.nt];
#pragma unroll
        for (int t = 0; t < kQT; ++t) dot[t][i & 3] = fmaf(qp[t * a.n_slots * D + i], kv, dot[t][i & 3]);
      }
    }
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      const bool cand = u < n_kv && u != f_sink && u != f_diag0 + t;
      const float d = (dot[t][0] + dot[t][1]) + (dot[t][2] + dot[t][3]);
      keys[t * n_kv64 + u] = cand ? score_key(d * a.inv_sqrt_d) : 0u;
    }
  }
  __syncthreads();
  // 4. selection, one wave per query tile: the kept competitors are the `need` highest scores,
  //    ties to the lower index.  T = the need-th highest key, found bit by bit from the top
  //    (largest T with #(key >= T) >= need); then every key above T is kept and, of the keys
  //    equal to T, the first need - #(key > T) in index order.
  const int t = tid >> 6, lane = tid & 63;
  if (t >= n_qt) return;
  const uint32_t* kt = keys + t * n_kv64;
  const int nch = n_kv64 >> 6;
  uint32_t kr[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) kr[c] = c < nch ? kt[64 * c + lane] : 0u;
  // keys >= K, for K >= 1: the register chunks past n_kv64 hold 0 and never count, so they need
  // no branch (a uniform branch per chunk and round cost more than the compares themselves)
  auto count_reg = [&](uint32_t K, auto NC) {
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < decltype(NC)::value; ++c) cnt += __popcll(__ballot(kr[c] >= K));
    return cnt;
  };
  using C4 = std::integral_constant<int, 4>;
  using C8 = std::integral_constant<int, 8>;
  auto count_ge = [&](uint32_t K) {
    int cnt = count_reg(K, C8{});
    for (int c = 8; c < nch; ++c) cnt += __popcll(__ballot(kt[64 * c + lane] >= K));
    return cnt;
  };
  const int n_forced = 1 + (f_sink >= 0 ? 1 : 0);
  const int need = a.k_row - n_forced;
  const int n_cand = count_ge(1u);
  uint32_t T;
  int take_eq;
  if (need <= 0) {               // forced tiles only
    T = 0xffffffffu;
    take_eq = 0;
  } else if (need >= n_cand) {   // every competitor
    T = 0u;
    take_eq = 0;
  } else {
    T = 0u;
    // every key in registers: 32 straight rounds over the chunks that can hold keys
    if (nch <= 4) {
#pragma unroll
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        if (count_reg(cand, C4{}) >= need) T = cand;
      }
    } else if (nch <= 8) {
#pragma unroll
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        if (count_reg(cand, C8{}) >= need) T = cand;
      }
    } else {
      for (int b = 31; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        if (count_ge(cand) >= need) T = cand;
      }
    }
    take_eq = need - (T == 0xffffffffu ? 0 : count_ge(T + 1u));
  }
  // 5. ascending compaction of forced + kept tiles
  int32_t* dst = a.out + ((size_t)h * a.nt + qt0 + t) * a.k_cap;
  const int diag = f_diag0 + t;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int count = 0, eq_seen = 0;
  auto emit = [&](int c, uint32_t k) {
    const int u = 64 * c + lane;
    const unsigned long long meq = __ballot(k != 0u && k == T);
    const bool keep = u < n_kv && (u == f_sink || u == diag || (k != 0u && k > T) ||
                                   (k != 0u && k == T && eq_seen + __popcll(meq & lt) < take_eq));
    eq_seen += __popcll(meq);
    const unsigned long long m = __ballot(keep);
    const int pos = count + __popcll(m & lt);
    if (keep && pos < a.k_cap) dst[pos] = u;
    count += __popcll(m);
  };
  // chunks past n_kv64 keep nothing
  if (nch <= 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) emit(c, kr[c]);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) emit(c, kr[c]);
  }
  for (int c = 8; c < nch; ++c) emit(c, kt[64 * c + lane]);
  for (int pos = count + lane; pos < a.k_cap; pos += 64) dst[pos] = -1;
}

}  // namespace

hipError_t launch_tile_mask(const Geometry& g, const RopeTab& rt, const void* q,
                            const float* const* pooled, const int* deltas, int n_slots,
                            bool has_sink, int k_row, int k_cap, int32_t* out, hipStream_t stream) {
  if (g.d != 128 || n_slots < 1 || n_slots > kMaxSlots || n_slots * g.nt > kMaxKeyTiles || rt.pt > 32)
    return hipErrorInvalidValue;   // (a slot's time row is staged as at most 32 entries)
  MaskArgs a;
  a.q = static_cast<const u16*>(q);
  a.out = out;
  a.k_row = k_row;
  a.k_cap = k_cap;
  a.B = g.B;
  a.H = g.H;
  a.nt = g.nt;
  a.hw = g.lat_h * g.lat_w;
  a.lat_w = g.lat_w;
  a.n_slots = n_slots;
  a.has_sink = has_sink ? 1 : 0;
  a.inv_sqrt_d = (float)(1.0 / __builtin_sqrt((double)g.d));
  a.inv_hw = 1.0f / (float)(g.lat_h * g.lat_w);
  a.inv_lat_w = 1.0f / (float)g.lat_w;
  a.rt = rt;
  for (int i = 0; i < kMaxSlots; ++i) {
    a.pooled[i] = i < n_slots ? pooled[i] : nullptr;
    a.delta[i] = i < n_slots ? deltas[i] : 0;
  }
  const int n_kv64 = (n_slots * g.nt + 63) & ~63;
  const size_t red = (size_t)kQT * 16 * g.d * sizeof(float);
  const size_t sel = ((size_t)kQT * n_slots * g.d + (size_t)kQT * n_kv64) * sizeof(float);
  const size_t lds = red > sel ? red : sel;   // <= 24 KB at the largest shapes
  int dev = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      lds > (size_t)lds_max)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_mask_kernel, dim3((g.nt + kQT - 1) / kQT, g.H), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace swattn
