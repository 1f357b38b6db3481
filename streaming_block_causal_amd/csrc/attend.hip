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
// bf16 path (d = 128): one workgroup = 8 waves = 256 queries of one head (dense; the
// block-sparse launch uses 4 waves = 128 queries, two workgroups per CU); each wave
// owns 32 queries.  Keys stream through LDS 64 at a time.  A wave computes
// the transposed score tile S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so every
// lane holds 16 keys of ONE query: the softmax row max and sum are in-register
// plus one cross-half exchange (v_permlane32_swap).  P^T stays in registers as
// the B operand of O^T += V^T P^T; the V^T cache layout (keys permuted in groups
// of 16) makes the matching A operand one 16-byte LDS read.  Online softmax runs
// in the log2 domain with the 1/sqrt(d) scale folded into one FMA before v_exp.
// Block-sparse (K3): the same loop, over the listed 128-key tiles only.
//
// fp8 path (d = 128, E4M3 cache with power-of-two scales per 32 values): the same
// structure with v_mfma_scale_f32_32x32x64_f8f6f4 (64-deep contractions, the scale
// bytes applied by the instruction); the probabilities are rounded to E4M3 and
// their row sums come from one more scaled MFMA with an all-ones operand.
//
// fp32 path (d = 64 or 128): four lanes per query (a quarter of the dimensions each,
// scores reduced with two lane exchanges), keys broadcast from LDS; plain fp32
// arithmetic for the small fp32 workload.
#include <algorithm>

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
  int aligned_last;   // 1: the last slot is frame-aligned (editing source frames)
  float scale_log2;   // log2(e) / sqrt(d)
  float inv_hw;       // 1 / (lat_h * lat_w), rounded to fp32 on the host
  int n_qt;           // query tiles per head of this launch
  int n_full;         // workgroups that own a whole query tile
  int n_split;        // key-range pieces of each remaining tile (0: none)
  float* part_o;      // [piece][rows of a tile][d] normalised partial outputs of split tiles
  float* part_lse;    // [piece][rows of a tile] their log2 sum-exp
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

// With 4-wave workgroups two of them share a CU, so each SIMD runs one wave of each and no
// barrier ties the two together.  Each wave alternates its MFMAs and its softmax, each waiting on
// the other's results, and the pair tends to run the same phase at the same time.  A fixed issue
// priority for the wave in the even slot of its SIMD (HW_ID wave id, bits 3:0) lets that one run
// ahead: about 3% faster for the block-sparse and fp8 launches (with one 8-wave workgroup per CU,
// whose waves meet at every block's barrier, it changes nothing).
__device__ __forceinline__ void favour_even_slot() {
  const uint32_t slot = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 4);
  if ((slot & 1) == 0) __builtin_amdgcn_s_setprio(1);
}

// Largest of a lane's 32 scores (two 32x32 score tiles): a tree of max3 steps, depth 4, rather
// than a chain of 16 dependent ones.
__device__ __forceinline__ float max_of_32(const f32x16& s0, const f32x16& s1) {
  float m8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m8[i] = fmaxf(fmaxf(s0[2 * i], s0[2 * i + 1]), s1[2 * i]);
  const float a = fmaxf(fmaxf(m8[0], m8[1]), m8[2]), b = fmaxf(fmaxf(m8[3], m8[4]), m8[5]);
  const float c = fmaxf(fmaxf(m8[6], m8[7]), s1[1]), d = fmaxf(fmaxf(s1[3], s1[5]), s1[7]);
  const float e = fmaxf(fmaxf(s1[9], s1[11]), s1[13]);
  return fmaxf(fmaxf(a, b), fmaxf(fmaxf(c, d), fmaxf(e, s1[15])));
}

// ------------------------------------------------------------------------------------
// bf16 MFMA kernel
// ------------------------------------------------------------------------------------
constexpr int D = 128;
constexpr int KB = 64;          // keys per LDS block
constexpr float kRescaleSlack = 8.0f;   // log2 units: exp2 arguments stay <= 8 between rescales

#ifndef QK_AHEAD
#define QK_AHEAD 1   // K operands read this many MFMA pairs ahead
#endif
#ifndef PV_AHEAD
#define PV_AHEAD 8   // V^T operands of the P.V MFMAs read before the softmax
#endif

// Q^T operand of one wave: lane (hf, ln) holds q[row][16j + 8hf + 0..7] for j in [J0, J1), rotated
// at time frame + delta (fp32 math, bf16 result).  Rows past the block give a zero operand.
// Every Q load and cos/sin gather is issued before the first is used (one memory round trip, not
// one per operand group): qp must point at a readable row -- a row past the block passes row 0's,
// whose values a select drops -- and such a row's positions are taken as 0 (table entries exist).
// Only the first kTimeJ operand groups hold time pairs (d = 128: 22 time pairs = dims 0..43), so a
// new slot re-rotates those and the spatial groups are computed once per workgroup.
constexpr int kTimeJ = 3;
constexpr int kTimeTabLds = 1024;   // time-table entries the block-sparse kernel copies to LDS
template <int J0, int J1>
__device__ __forceinline__ void load_q(const RopeTab rt, const u16* qp, bool valid, int qf, int qh, int qw,
                                       int hf, int delta, bf16x8 (&qb)[8]) {
  constexpr int NJ = J1 - J0;
  const int t = valid ? qf + delta : 0, ph = valid ? qh : 0, pw = valid ? qw : 0;
  uint4 raw[NJ];
  float c[NJ][4], s[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j) raw[j] = ldg16(qp + 16 * (J0 + j) + 8 * hf);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) rope_cs(rt, 8 * (J0 + j) + 4 * hf + i, t, ph, pw, c[j][i], s[j][i]);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = valid ? __uint_as_float(w[i] << 16) : 0.f;
      const float x1 = valid ? __uint_as_float(w[i] & 0xffff0000u) : 0.f;
      qb[J0 + j][2 * i] = (__bf16)(x0 * c[j][i] - x1 * s[j][i]);
      qb[J0 + j][2 * i + 1] = (__bf16)(x0 * s[j][i] + x1 * c[j][i]);
    }
  }
}

// Slot entry: the time pairs among the first kTimeJ operand groups re-rotated at time t from the
// raw query (raw[j]: q[16j + 8hf .. +8) as loaded, zero for rows past the block); the other pairs
// of these groups keep the values load_q gave them (their angles do not depend on the slot).
// cs(idx) returns the cos/sin of time-table entry idx.  Same arithmetic as load_q.
template <typename CS>
__device__ __forceinline__ void retime_q(const uint4 (&raw)[kTimeJ], int pt, int t, int hf, CS cs, bf16x8 (&qb)[8]) {
#pragma unroll
  for (int j = 0; j < kTimeJ; ++j) {
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 8 * j + 4 * hf + i;
      const bool on_t = p < pt;
      const CosSin v = cs(t * pt + (on_t ? p : 0));
      const float x0 = __uint_as_float(w[i] << 16), x1 = __uint_as_float(w[i] & 0xffff0000u);
      const __bf16 r0 = (__bf16)(x0 * v.c - x1 * v.s), r1 = (__bf16)(x0 * v.s + x1 * v.c);
      qb[j][2 * i] = on_t ? r0 : qb[j][2 * i];
      qb[j][2 * i + 1] = on_t ? r1 : qb[j][2 * i + 1];
    }
  }
}

// Sparse schedule: position i -> (slot, 64-key block, keys in the block) from the two halves of
// each listed 128-key tile (every slot holds B keys).  Returns false for entries to skip: half of
// a short last tile, a tile index outside the cache, or one not above the last tile taken from the
// row (`last`, updated after a tile's second half) -- so a repeated tile never counts twice.
__device__ __forceinline__ bool block_at(const int32_t* list, int B, int n_slots, int nt, int nkb, int i, int& last,
                                         int& sl, int& kb, int& kvalid) {
  // the list is read-only during the launch and its address is uniform: a scalar (constant
  // address space) load, counted on lgkmcnt.  A vector load here would be waited for with
  // vmcnt(0), which also waits for the staging loads of the next block issued just before.
  const int tix = *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(list + (i >> 1)));
  if (tix < 0 || tix >= n_slots * nt || tix <= last) return false;   // never read outside the cache
  if (i & 1) last = tix;
  sl = tix / nt;
  kb = 2 * (tix - sl * nt) + (i & 1);
  kvalid = B - kb * KB;
  return kb < nkb;
}

// Direct global -> LDS staging of one 64-key block (gfx950 global_load_lds_dwordx4: each lane
// moves 16 bytes into LDS at base + 16 * lane, no registers involved).  LDS rows are unpadded and
// XOR-swizzled so the MFMA operand reads are bank-conflict free:
//   K  [64 keys][128 dims]: row r at r * 256 B, 16-byte chunk c at slot c ^ (r & 15)
//   V^T[128 dims][64 keys]: row d at d * 128 B, 16-byte chunk c at slot c ^ ((d >> 1) & 7)
// A workgroup's NW waves each issue 16/NW K and 16/NW V loads (1 KB each) per block: load p of a
// wave is K chunk NW * (p / 2) + wave for even p, the V^T chunk for odd p.  st[p] is the lane's
// element offset inside the block (K: row-major, V^T: row stride 128 inside its tile).
__device__ __forceinline__ const u16* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const u16*>(((uint64_t)hi << 32) | lo);
}
template <int NW>
__device__ __forceinline__ void stage_load(int p, const u16* kbase, const u16* vbase, const int (&st)[32 / NW],
                                           int wave, u16* kdst, u16* vdst) {
  const int C = NW * (p >> 1) + wave;   // 1 KB chunk of the block
  const u16* src = ((p & 1) ? vbase : kbase) + (uint32_t)st[p];
  u16* dst = ((p & 1) ? vdst : kdst) + C * 512;
  __builtin_amdgcn_global_load_lds(
      reinterpret_cast<const __attribute__((address_space(1))) void*>(reinterpret_cast<uintptr_t>(src)),
      reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(dst)), 16, 0, 0);
}

// One workgroup = NW waves = 32 * NW queries of one head (32 per wave), two waves per SIMD:
// NW = 4 -> two workgroups per CU, NW = 8 -> one.  The K/V blocks a workgroup streams are shared
// by its waves through two LDS buffers: block n + 1 is requested while block n is computed; one
// barrier per block.
// Workgroups past n_full each take 1/n_split of the key blocks of one of the remaining tiles
// and write a normalised partial result; merge_kernel combines them.  This fills the last,
// partial round of the grid instead of leaving most CUs idle.
// ALIGN: the last slot is frame-aligned (editing source frames): per tile only the key blocks of
// the frames its queries belong to, and a key is masked for the queries of other frames.
template <bool SPARSE, int NW, bool ALIGN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attend_bf16_kernel(AttnArgs a) {
  constexpr int ROWS = 32 * NW;
  constexpr int NBUF = 2;
  __shared__ __attribute__((aligned(1024))) u16 kbuf[NBUF][KB * D];
  __shared__ __attribute__((aligned(1024))) u16 vbuf[NBUF][D * KB];
  __shared__ SlotPtrs sslot[kMaxSlots];
  // block-sparse: tile lists change slot every few blocks, so the time rotation of the queries is
  // redone often; its cos/sin come from an LDS copy of the time table (when it fits) and the raw
  // time part of the query stays in registers, so a slot entry waits on no global load
  __shared__ CosSin ttab[SPARSE ? kTimeTabLds : 1];

  // wave index made explicitly uniform: the LDS destinations of the staging loads (M0) then stay
  // in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, ln = lane & 31;
  if (NW == 4) favour_even_slot();   // two workgroups per CU
  // the argument struct is never addressed (that would copy it to scratch): static indices only,
  // and every field the lambdas below need is copied to a local first
#pragma unroll
  for (int q = 0; q < kMaxSlots; ++q)
    if (tid == q) sslot[q] = a.slot[q];
  // dense schedule: every 64-key block of every slot in logical order (slots may hold blocks of
  // different lengths); a frame-aligned last slot contributes only the blocks of the frames this
  // tile's queries belong to (below)
  int dense_total = 0, aligned_count = 0;
#pragma unroll
  for (int q = 0; q < kMaxSlots; ++q) {
    if (q < a.n_slots && !(ALIGN && q == a.n_slots - 1)) dense_total += (a.slot[q].count + KB - 1) / KB;
    if (q == a.n_slots - 1) aligned_count = a.slot[q].count;
  }
  const RopeTab rt = a.rt;
  const int B = a.B, n_pad = a.n_pad, n_slots = a.n_slots, nt = a.nt;
  const float scale_log2 = a.scale_log2;
  const int tt_n = rt.t_len * rt.pt;
  const bool tt_lds = SPARSE && tt_n <= kTimeTabLds;
  if (tt_lds)
    for (int i = tid; i < tt_n; i += NW * 64) ttab[i] = rt.t[i];
  __syncthreads();

  const int nkb = (B + KB - 1) / KB;   // sparse: every slot holds B keys
  int tile, part = 0, piece = -1;
  if ((int)blockIdx.x < a.n_full) {
    tile = xcd_remap(blockIdx.x, a.n_full);
  } else {
    piece = xcd_remap(blockIdx.x - a.n_full, gridDim.x - a.n_full);
    part = piece % a.n_split;
    tile = a.n_full + piece / a.n_split;
  }
  const int h = tile / a.n_qt, qt = tile - h * a.n_qt;
  // frame-aligned slot: key blocks [al_lo, al_hi) cover the frames of rows qt*ROWS .. (last row)
  int al_lo = 0, al_hi = 0;
  if (ALIGN) {
    const int r0 = qt * ROWS, r1 = min(B, r0 + ROWS);
    al_lo = (r0 / a.hw) * a.hw / KB;
    al_hi = (min(aligned_count, ((r1 - 1) / a.hw + 1) * a.hw) + KB - 1) / KB;
    dense_total += al_hi - al_lo;
  }
  const int total = SPARSE ? 2 * a.k_row : dense_total;
  int i0 = 0, i1 = total;
  if (piece >= 0) {
    i0 = part * total / a.n_split;
    i1 = (part + 1) * total / a.n_split;
  }
  const int qrow = qt * ROWS + wave * 32 + ln;
  const bool qvalid = qrow < B;
  const int qf = qrow / a.hw;
  const int qrem = qrow - qf * a.hw;
  const int qh = qrem / a.lat_w, qw = qrem - qh * a.lat_w;
  // a row past the block reads row 0 (its values are dropped): every query load is in bounds
  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)(qvalid ? qrow : 0) * a.H + h) * D;
  // frame of key j = floor((j + 0.5) / hw) in fp32: exact, since j < 65536 keeps the rounding error
  // below 0.01 / hw while (j + 0.5) / hw is at least 0.5 / hw from an integer.  A kernel argument,
  // so it stays in a scalar register: a value computed here would live in a vector register, be
  // spilled, and be reloaded in the masking branch with a wait that also waits for the staging
  // loads of the next block.
  const float inv_hw = a.inv_hw;

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  // running max starts at a finite floor, not -inf: a lane whose keys so far were all masked (a
  // frame-aligned block of another frame opening a key range) then gets alpha = 1 and p = 0
  // instead of exp2(-inf - -inf) = NaN when another lane of the wave rescales
  float m_run = -3.0e38f, l_run = 0.f;
  bf16x8 qb[8];
  // every pair rotated once here (the first slot entry re-rotates the time pairs: retime_q keeps
  // the others of the first kTimeJ groups as computed now)
  load_q<0, 8>(rt, qp, qvalid, qf, qh, qw, hf, 0, qb);
  uint4 qraw[kTimeJ];   // block-sparse: the raw time part, kept
#pragma unroll
  for (int j = 0; j < kTimeJ; ++j) {   // (a load for every row, then a select: no branch, no wait between)
    const uint4 r = SPARSE ? ldg16(qp + 16 * j + 8 * hf) : make_uint4(0, 0, 0, 0);
    qraw[j] = qvalid ? r : make_uint4(0, 0, 0, 0);
  }

  // per-lane byte offsets of the swizzled operand reads (see stage_block)
  int koff[8], voff[4];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) koff[jj] = ln * 128 + 8 * ((2 * jj + hf) ^ (ln & 15));
#pragma unroll
  for (int g = 0; g < 4; ++g) voff[g] = ln * 64 + 8 * ((2 * g + hf) ^ ((ln >> 1) & 7));

  constexpr int NST = 32 / NW;   // staging loads per wave and block
  int st[NST];
#pragma unroll
  for (int p = 0; p < NST; ++p) {
    const int C = NW * (p >> 1) + wave;
    if ((p & 1) == 0) {
      const int r = 4 * C + (lane >> 4);
      st[p] = r * D + 8 * ((lane & 15) ^ (r & 15));
    } else {
      const int d = 8 * C + (lane >> 3);
      st[p] = d * kTile + 8 * ((lane & 7) ^ ((d >> 1) & 7));
    }
  }

  const size_t kstride = (size_t)n_pad * D;   // per head, K and V^T alike
  const int32_t* list = SPARSE ? a.tile_idx + ((size_t)h * nt + qt) * a.k_row : nullptr;

  // global bases (uniform) of block kb of slot s; "no block" maps to block 0 of slot 0, a valid
  // address whose reload into an unused buffer is harmless
  auto block_base = [&](bool valid, int s, int kb, const u16*& kb_ptr, const u16*& vb_ptr) {
    if (!valid) {
      s = 0;
      kb = 0;
    }
    const SlotPtrs sp = sslot[s];
    // the slot's base made uniform first: the offsets are scalar, so the sums stay in SGPRs
    kb_ptr = uniform_ptr(sp.k) + h * kstride + (size_t)kb * KB * D;
    vb_ptr = uniform_ptr(sp.v) + h * kstride + (size_t)(kb >> 1) * D * kTile + (kb & 1) * KB;
  };

  // ---- S^T = K Q^T for 64 keys: two 32x32 tiles, lane holds 16 keys of query ln
  auto qk = [&](const u16* kl, int kvalid, int afirst, f32x16& s0, f32x16& s1, const u16* nkb, const u16* nvb, u16* kdst,
                u16* vdst) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    // operands are read QK_AHEAD steps ahead of their MFMAs; the schedule is pinned below
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 kop[QK_AHEAD + 1][2];
#pragma unroll
    for (int jj = 0; jj < QK_AHEAD; ++jj) {
      kop[jj][0] = *reinterpret_cast<const bf16x8*>(kl + koff[jj]);
      kop[jj][1] = *reinterpret_cast<const bf16x8*>(kl + 32 * D + koff[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (jj + QK_AHEAD < 8) {
        kop[(jj + QK_AHEAD) % (QK_AHEAD + 1)][0] = *reinterpret_cast<const bf16x8*>(kl + koff[jj + QK_AHEAD]);
        kop[(jj + QK_AHEAD) % (QK_AHEAD + 1)][1] =
            *reinterpret_cast<const bf16x8*>(kl + 32 * D + koff[jj + QK_AHEAD]);
      }
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[jj % (QK_AHEAD + 1)][0], qb[jj], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[jj % (QK_AHEAD + 1)][1], qb[jj], s1, 0, 0, 0);
      // the next block's staging loads ride along with the MFMAs instead of queueing up in the
      // vector memory path right after the barrier
      if (jj < NST) stage_load<NW>(jj, nkb, nvb, st, wave, kdst, vdst);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * QK_AHEAD, 0);   // the first reads
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (jj + QK_AHEAD < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // next reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                         // two MFMAs
      if (jj < NST) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);           // one staging load
    }
    __builtin_amdgcn_sched_barrier(0);
    // The masks below are taken only by a few blocks per tile.  The scheduling barrier (an
    // intrinsic with side effects) keeps the compiler from if-converting them into selects that
    // every block would execute (about 80 VALU instructions per wave and block).
    if (__builtin_expect(kvalid < KB, 0)) {   // last block of its slot: keys past its end do not exist
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= kvalid) s0[r] = -INFINITY;
        if (key + 32 >= kvalid) s1[r] = -INFINITY;
      }
    }
    if (__builtin_expect(afirst >= 0, 0)) {   // frame-aligned slot: key afirst + i is seen only by
      __builtin_amdgcn_sched_barrier(0);        // the queries of its frame
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = afirst + 8 * (r >> 2) + 4 * hf + (r & 3);
        if ((int)(((float)key + 0.5f) * inv_hw) != qf) s0[r] = -INFINITY;
        if ((int)(((float)(key + 32) + 0.5f) * inv_hw) != qf) s1[r] = -INFINITY;
      }
    }
  };
  // ---- online softmax (log2 domain, lazy rescale), then O^T += V^T P^T
  auto sm_pv = [&](const u16* vl, f32x16& s0, f32x16& s1) {
    // V^T operands of the first PV_AHEAD MFMAs are requested before the softmax, so the P.V
    // MFMAs find them in registers; MFMA i = (g, t) = (i / 4, i % 4) reads row block t, key group g
    auto vread = [&](int i) { return *reinterpret_cast<const bf16x8*>(vl + 32 * (i & 3) * KB + voff[i >> 2]); };
    constexpr int PVA = SPARSE ? 4 : PV_AHEAD;   // block-sparse: registers go to the kept raw query
    bf16x8 vop[PVA];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PVA; ++i) vop[i] = vread(i);
    __builtin_amdgcn_sched_barrier(0);
    float mx = max_of_32(s0, s1);
    mx = swap_halves_max(mx) * scale_log2;
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
    }
    const float mneg = -m_run;
    bf16x8 pb[4];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
    // row sum of the fp32 probabilities by plain adds (four chains): v_dot2c over the bf16 pairs
    // shares the matrix pipe and slows to about 13 cycles next to running MFMAs; these adds
    // measured 1-2% faster.  The sum counts each probability before its bf16 rounding for P.V (an
    // unbiased difference of at most 2^-9 per term), the same way in the dense and block-sparse
    // instantiations, so a block-sparse call keeping every tile still equals the dense one bit for bit
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s0[r], scale_log2, mneg));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s1[r], scale_log2, mneg));
      pb[r >> 3][r & 7] = (__bf16)e0;
      pb[2 + (r >> 3)][r & 7] = (__bf16)e1;
      ps[r & 1] += e0;
      ps[2 + (r & 1)] += e1;
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // ---- O^T += V^T P^T
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i % PVA], pb[i >> 2], acc[i & 3], 0, 0, 0);
      if (i + PVA < 16) vop[i % PVA] = vread(i + PVA);
    }
  };
  f32x16 s0, s1;

  // schedule positions: p[0] computed, p[1] staged, p[2] looked up ahead
  // Dense: positions are looked up once each, in increasing order, so a cursor walks the slots;
  // a slot's key count is read (from LDS, made scalar) only when the cursor enters the slot, and
  // schedule, slot and key count stay in scalar registers.
  int csl = 0, ckb = 0, ccnt = 0, cnb = 0;
  bool calign = false;
  auto enter = [&](int l) {
    csl = l;
    calign = ALIGN && l == n_slots - 1;
    ccnt = __builtin_amdgcn_readfirstlane(sslot[l].count);
    ckb = calign ? al_lo : 0;
    cnb = calign ? al_hi : (ccnt + KB - 1) / KB;
  };
  if (!SPARSE) {
    enter(0);
    int rem = i0;
    while (rem >= cnb - ckb && csl + 1 < n_slots) {
      rem -= cnb - ckb;
      enter(csl + 1);
    }
    ckb += rem;
  }
  // the schedule entry at or after position q (q is left on it): slot, block, keys in the block
  int last_tile = -1;   // sparse: the last tile taken from the row
  auto lookup = [&](int& q, int& sl, int& kb, int& kv) {
    if (SPARSE) {
      while (q < i1 && !block_at(list, B, n_slots, nt, nkb, q, last_tile, sl, kb, kv)) ++q;
    } else if (q < i1) {
      while (ckb >= cnb && csl + 1 < n_slots) enter(csl + 1);   // (skips empty slots)
      sl = csl;
      kb = ckb;
      kv = ccnt - ckb * KB;
      ++ckb;
    }
  };
  int pos[3], bsl[3], bkb[3], bkv[3];
  {
    int q = i0;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      lookup(q, bsl[u], bkb[u], bkv[u]);
      pos[u] = q;
      if (q < i1) ++q;
    }
  }
  const u16 *nk, *nv;   // bases of the block staged next
  if (pos[0] < i1) {
    block_base(true, bsl[0], bkb[0], nk, nv);
#pragma unroll
    for (int p = 0; p < NST; ++p) stage_load<NW>(p, nk, nv, st, wave, kbuf[0], vbuf[0]);
  }
  block_base(pos[1] < i1, bsl[1], bkb[1], nk, nv);
  int cur_slot = -1;
  bool pend = false;   // scores of the previous block wait for softmax and P.V
  int pend_buf = 0;

  // one pipeline step: softmax and P.V of block n - 1, the barrier of block n, then S of block n
  // from buffer cb while block n + 1 is requested into the next buffer
  auto step = [&](const int cb) {
    const int sl = bsl[0], kvalid = bkv[0];
    const int afirst = (ALIGN && sl == n_slots - 1) ? bkb[0] * KB : -1;
    auto sync = [&]() {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's part of block n has landed
      // ... and everyone's has; the buffer block n + 1 goes to (that of block n + 1 - NBUF) is
      // no longer read: its LDS reads were consumed by that block's MFMAs before this barrier.  A
      // bare s_barrier, the empty asm keeps the compiler from moving memory accesses across it.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    if (pend) sm_pv(vbuf[(cb + NBUF - 1) % NBUF], s0, s1);
    sync();
    if (sl != cur_slot) {
      cur_slot = sl;
      const int tq = qf + sslot[sl].delta;
      if (SPARSE) {
        if (tt_lds) retime_q(qraw, rt.pt, tq, hf, [&](int i) { return ttab[i]; }, qb);
        else retime_q(qraw, rt.pt, tq, hf, [&](int i) { return rt.t[i]; }, qb);
      } else {
        uint4 raw[kTimeJ];
#pragma unroll
        for (int j = 0; j < kTimeJ; ++j) raw[j] = qvalid ? ldg16(qp + 16 * j + 8 * hf) : make_uint4(0, 0, 0, 0);
        retime_q(raw, rt.pt, tq, hf, [&](int i) { return rt.t[i]; }, qb);
      }
    }
    qk(kbuf[cb], kvalid, afirst, s0, s1, nk, nv, kbuf[(cb + 1) % NBUF], vbuf[(cb + 1) % NBUF]);
    pend = true;
    pend_buf = cb;
    // look the schedule up one block further while the MFMAs drain
    int q = pos[2] < i1 ? pos[2] + 1 : i1, nsl = 0, nkb2 = 0, nkv = 0;
    if (pos[2] < i1) {
      lookup(q, nsl, nkb2, nkv);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pos[u] = pos[u + 1];
      bsl[u] = bsl[u + 1];
      bkb[u] = bkb[u + 1];
      bkv[u] = bkv[u + 1];
    }
    pos[2] = q;
    bsl[2] = nsl;
    bkb[2] = nkb2;
    bkv[2] = nkv;
    block_base(pos[1] < i1, bsl[1], bkb[1], nk, nv);
  };
  while (pos[0] < i1) {
    step(0);
    if (pos[0] >= i1) break;
    step(1);
  }
  // the last step's staging loads (of a placeholder block when the range ended) must land before
  // the workgroup's LDS can be handed to another workgroup
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // the last block's buffer is not restaged: no barrier needed before its P.V
  if (pend) sm_pv(vbuf[pend_buf], s0, s1);

  const float l_tot = swap_halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // an empty key range contributes nothing
  if (piece >= 0) {   // partial result of a split tile: fp32, normalised, plus log2 sum-exp
    const int row = wave * 32 + ln;
    float* po = a.part_o + ((size_t)piece * ROWS + row) * D;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<float4*>(po + 32 * t + 8 * rg + 4 * hf) =
            make_float4(acc[t][4 * rg] * inv, acc[t][4 * rg + 1] * inv, acc[t][4 * rg + 2] * inv,
                        acc[t][4 * rg + 3] * inv);
    if (hf == 0) a.part_lse[(size_t)piece * ROWS + row] = m_run + __log2f(l_tot);
    return;
  }
  if (qvalid) {
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
    if (a.lse && hf == 0) a.lse[(size_t)h * B + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// Combine the n_split partial results of each split tile: weights 2^(lse_p - m) / sum, m the max
// of the pieces' log2 sum-exp lse_p; the row's log2 sum-exp is m + log2(sum).  One workgroup per
// (tile, 8 rows): thread (row, d4) reads its four dims of every piece once (HBM-bound).
constexpr int kMaxSplit = 32;
constexpr int kMergeRows = 8;
template <int ROWS>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int tid = threadIdx.x, S = a.n_split;
  const int tile = a.n_full + blockIdx.x;
  const int h = tile / a.n_qt, qt = tile - h * a.n_qt;
  const int row = blockIdx.y * kMergeRows + (tid >> 5), d4 = (tid & 31) * 4;
  const int qrow = qt * ROWS + row;
  if (qrow >= a.B) return;
  const size_t p0 = (size_t)blockIdx.x * S;
  float mx = -INFINITY;
  for (int p = 0; p < S; ++p) mx = fmaxf(mx, a.part_lse[(p0 + p) * ROWS + row]);
  float sum = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  for (int p = 0; p < S; ++p) {
    const float wp = __builtin_amdgcn_exp2f(a.part_lse[(p0 + p) * ROWS + row] - mx);
    const float4 v = *reinterpret_cast<const float4*>(a.part_o + ((p0 + p) * ROWS + row) * D + d4);
    sum += wp;
    o0 = fmaf(wp, v.x, o0);
    o1 = fmaf(wp, v.y, o1);
    o2 = fmaf(wp, v.z, o2);
    o3 = fmaf(wp, v.w, o3);
  }
  const float inv = 1.f / sum;
  uint2 packed;
  packed.x = (uint32_t)f2bf(o0 * inv) | ((uint32_t)f2bf(o1 * inv) << 16);
  packed.y = (uint32_t)f2bf(o2 * inv) | ((uint32_t)f2bf(o3 * inv) << 16);
  *reinterpret_cast<uint2*>(static_cast<u16*>(a.o) + ((size_t)qrow * a.H + h) * D + d4) = packed;
  if (a.lse && d4 == 0) a.lse[(size_t)h * a.B + qrow] = (mx + __log2f(sum)) * kLn2;
}

// ------------------------------------------------------------------------------------
// fp32 kernel: four lanes per query (a quarter of the dimensions each), keys broadcast from LDS
// ------------------------------------------------------------------------------------
template <int DD>
__global__ __launch_bounds__(256) void attend_f32_kernel(AttnArgs a) {
  // 64 queries per workgroup, 4 lanes per query: lane `sub` owns dims [sub * DW, (sub + 1) * DW)
  // of the rotated query and of the accumulator; scores are reduced over the 4 lanes
  constexpr int KBF = 32, LPQ = 4, DW = DD / LPQ;
  __shared__ float kl[KBF][DD];
  __shared__ float vl[KBF][DD];
  __shared__ SlotPtrs sslot[kMaxSlots];
  const int tid = threadIdx.x, sub = tid & (LPQ - 1);
#pragma unroll
  for (int q = 0; q < kMaxSlots; ++q)
    if (tid == q) sslot[q] = a.slot[q];
  const RopeTab rt = a.rt;
  __syncthreads();
  const int h = blockIdx.y;
  const int qrow = blockIdx.x * 64 + tid / LPQ;
  const bool qvalid = qrow < a.B;
  const int qf = qrow / a.hw, qrem = qrow - qf * a.hw;
  const int qh = qrem / a.lat_w, qw = qrem - qh * a.lat_w;
  const float* qp = static_cast<const float*>(a.q) + ((size_t)qrow * a.H + h) * DD + sub * DW;
  float qr[DW], acc[DW];
#pragma unroll
  for (int i = 0; i < DW; ++i) acc[i] = 0.f;
  float m_run = -3.0e38f, l_run = 0.f;   // finite floor: a fully masked sub-block gives alpha = 1
  const float scale = a.scale_log2;

  for (int sl = 0; sl < a.n_slots; ++sl) {
    const int t = qf + sslot[sl].delta;
#pragma unroll
    for (int p = 0; p < DW / 2; ++p) {
      float c = 1.f, s = 0.f, x0 = 0.f, x1 = 0.f;
      if (qvalid) {
        rope_cs(rt, sub * (DW / 2) + p, t, qh, qw, c, s);
        x0 = qp[2 * p];
        x1 = qp[2 * p + 1];
      }
      qr[2 * p] = x0 * c - x1 * s;
      qr[2 * p + 1] = x0 * s + x1 * c;
    }
    const float* kbase = static_cast<const float*>(sslot[sl].k) + (size_t)h * a.n_pad * DD;
    const float* vbase = static_cast<const float*>(sslot[sl].v) + (size_t)h * a.n_pad * DD;
    const int count = sslot[sl].count;
    // a frame-aligned last slot: only the frames of this workgroup's rows, key by key below (the
    // range starts on a multiple of KBF so that every staged sub-block stays inside the slot)
    const bool al = a.aligned_last && sl == a.n_slots - 1;
    const int r_first = blockIdx.x * 64, r_last = min(a.B, r_first + 64) - 1;
    const int k_lo = al ? (r_first / a.hw) * a.hw / KBF * KBF : 0;
    const int k_hi = al ? min(count, (r_last / a.hw + 1) * a.hw) : count;
    for (int k0 = k_lo; k0 < k_hi; k0 += KBF) {
      __syncthreads();
      for (int i = tid; i < KBF * DD; i += 256) {
        kl[i / DD][i % DD] = kbase[(size_t)k0 * DD + i];
        vl[i / DD][i % DD] = vbase[(size_t)k0 * DD + i];
      }
      __syncthreads();
      const int nk = min(KBF, k_hi - k0);
      float sc[KBF];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KBF; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DW; ++i) dot = fmaf(qr[i], kl[j][sub * DW + i], dot);
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const bool seen = j < nk && (!al || (k0 + j) / a.hw == qf);
        sc[j] = seen ? dot * scale : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DW; ++i) acc[i] *= alpha;
#pragma unroll
      for (int j = 0; j < KBF; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[j] - m_new);
        l_run += p;
#pragma unroll
        for (int i = 0; i < DW; ++i) acc[i] = fmaf(p, vl[j][sub * DW + i], acc[i]);
      }
    }
  }
  if (qvalid) {
    float* op = static_cast<float*>(a.o) + ((size_t)qrow * a.H + h) * DD + sub * DW;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int i = 0; i < DW; ++i) op[i] = acc[i] * inv;
    if (a.lse && sub == 0) a.lse[(size_t)h * a.B + qrow] = (m_run + __log2f(l_run)) * kLn2;
  }
}


// ------------------------------------------------------------------------------------
// fp8 MFMA kernel (dense): Q, K, V in OCP E4M3 with power-of-two scales per 32 values,
// v_mfma_scale_f32_32x32x64_f8f6f4 (each lane's 32 operand bytes carry that lane's
// E8M0 scale), fp32 softmax, P rounded to E4M3 (scale 1: p <= 2^8 < 448 under the lazy
// rescale), fp32 accumulation.  Q is quantised with the softmax scale in base 2
// (log2 e / sqrt d) folded in, and each block's S accumulators start at -m_ref (the running
// max, 0 while the row has none): the MFMAs then deliver the exponents themselves, and the
// softmax spends no VALU instruction on scaling and shifting 32 scores per lane and block.
// Cache layout: see append_fp8.hip.  Same grid, split and
// pipeline as the bf16 dense kernel; per 64-key block a wave issues 4 + 4 MFMAs (64
// channels or 64 keys of contraction each) and reads 8 KB of K and 8 KB of V^T from LDS.
// The scaled MFMA applies the E8M0 scale of lane half 0 to operand bytes 0-15 of both lane
// halves (one 32-value group) and that of half 1 to bytes 16-31 (the other group).
//   QK: A = K tile t (32 keys), lane (key 32t + ln, hf) holds channels 64c + 16hf + [0, 16) in
//       bytes 0-15 and 64c + 32 + 16hf + [0, 16) in bytes 16-31, so bytes 0-15 of the two halves
//       are channel group 2c and bytes 16-31 group 2c + 1; lane half hf supplies the scale of
//       group 2c + hf.  B = Q, the same placement; S^T as in the bf16 kernel.
//   PV: A = V^T tile t (32 channels), lane (channel 32t + ln, hf) holds the stored positions
//       32hf + [0, 32) of the block (keys with index bit 2 == hf); B = P^T, lane (query ln, hf)
//       holds exactly those keys' probabilities: its 16 scores of S^T tile 0 (keys 0..31, the
//       first V group), then of tile 1 (keys 32..63, the second).
// LDS rows are XOR-swizzled by 16-byte chunks (K: 128 B rows, chunk c at c ^ (row & 7);
// V^T: 64 B rows, chunk c at c ^ ((row >> 2) & 3)) so the operand reads are conflict-free.
// ------------------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int e8m0_of(float amax) {   // smallest e with amax / 2^e <= 448
  const uint32_t b = __float_as_uint(amax);
  const int E = (b >> 23) & 255;
  if (E == 0) return -127;
  const int e = E - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  // the first conversion fills bytes 0-1 and the second bytes 2-3, so what the destination
  // held before does not matter: passing the bits of `a` (dead afterwards) lets the compiler
  // convert in place instead of first moving a zero into a fresh register
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Q operand chunks [C0, C1) of one lane: channels 64c + 16hf + [0, 16) and 64c + 32 + 16hf +
// [0, 16) of its query, rotated at time frame + delta and multiplied by qscale (the softmax
// scale in base 2); each half is quantised with the scale of
// its 32-channel group (the two lane halves exchange their partial maxima); byte c of qsc is
// the scale this lane supplies (group 2c + hf)
template <int C0, int C1>
__device__ __forceinline__ void load_q8(const RopeTab rt, const u16* qp, bool valid, int qf, int qh, int qw, int hf,
                                        int delta, float qscale, v8i (&q8)[2], uint32_t& qsc) {
  const int t = qf + delta;
#pragma unroll
  for (int c = C0; c < C1; ++c) {
    int eg[2];
    // the two 32-channel groups one after the other (16 rotated values live at a time)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int base = 64 * c + 32 * g + 16 * hf;
      float x[16];
      if (valid) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint4 raw = ldg16(qp + base + 8 * u);
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float cs, sn;
            rope_cs(rt, base / 2 + 4 * u + i, t, qh, qw, cs, sn);
            const float x0 = __uint_as_float(w[i] << 16), x1 = __uint_as_float(w[i] & 0xffff0000u);
            x[8 * u + 2 * i] = (x0 * cs - x1 * sn) * qscale;
            x[8 * u + 2 * i + 1] = (x0 * sn + x1 * cs) * qscale;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = 0.f;
      }
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
      eg[g] = e8m0_of(swap_halves_max(am));
      const float sc = __uint_as_float((uint32_t)(127 - eg[g]) << 23);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        q8[c][4 * g + i] = (int)pack4_fp8(x[4 * i] * sc, x[4 * i + 1] * sc, x[4 * i + 2] * sc, x[4 * i + 3] * sc);
    }
    const int e0 = eg[0], e1 = eg[1];
    const int e = hf ? e1 : e0;
    qsc = (qsc & ~(0xffu << (8 * c))) | ((uint32_t)(e + 127) << (8 * c));
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attend_fp8_kernel(AttnArgs a) {
  constexpr int ROWS = 32 * NW;
  constexpr int NBUF = 2;
  static_assert(NW == 4 || NW == 8, "8 / NW one-KB chunks of K and of V^T per wave and block");
  constexpr int NSTG = 8 / NW;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[NBUF][KB * D];   // 8 KB
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[NBUF][D * KB];   // 8 KB
  __shared__ SlotPtrs sslot[kMaxSlots];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, ln = lane & 31;
  if (NW == 4) favour_even_slot();
#pragma unroll
  for (int q = 0; q < kMaxSlots; ++q)
    if (tid == q) sslot[q] = a.slot[q];
  int dense_total = 0;
#pragma unroll
  for (int q = 0; q < kMaxSlots; ++q)
    if (q < a.n_slots) dense_total += (a.slot[q].count + KB - 1) / KB;
  const RopeTab rt = a.rt;
  const int B = a.B, n_pad = a.n_pad, n_slots = a.n_slots, H = a.H;
  const float scale_log2 = a.scale_log2;
  __syncthreads();

  int tile, part = 0, piece = -1;
  if ((int)blockIdx.x < a.n_full) {
    tile = xcd_remap(blockIdx.x, a.n_full);
  } else {
    piece = xcd_remap(blockIdx.x - a.n_full, gridDim.x - a.n_full);
    part = piece % a.n_split;
    tile = a.n_full + piece / a.n_split;
  }
  const int h = tile / a.n_qt, qt = tile - h * a.n_qt;
  const int total = dense_total;
  int i0 = 0, i1 = total;
  if (piece >= 0) {
    i0 = part * total / a.n_split;
    i1 = (part + 1) * total / a.n_split;
  }
  const int qrow = qt * ROWS + wave * 32 + ln;
  const bool qvalid = qrow < B;
  const int qf = qrow / a.hw;
  const int qrem = qrow - qf * a.hw;
  const int qh = qrem / a.lat_w, qw = qrem - qh * a.lat_w;
  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)qrow * a.H + h) * D;

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = -3.0e38f, l_run = 0.f;   // finite floor, as in the bf16 kernel
  v8i q8[2];
  uint32_t qsc = 0x7f7f7f7fu;
  load_q8<0, 2>(rt, qp, qvalid, qf, qh, qw, hf, 0, scale_log2, q8, qsc);

  // per-lane LDS byte offsets of the operand reads (two 16-byte chunks each).  The LDS serves a
  // 16-byte read for 16 lanes at a time from 64 four-byte banks (256 bytes): rows of 128 bytes
  // (K) put two rows in one bank line, so the chunk is swizzled with (row / 2) & 7; rows of 64
  // bytes (V^T) put four, swizzled with (row / 4) & 3.  Each group of 16 lanes then reads 16
  // different bank quads.
  int koff[2][2], voff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[c][u] = ln * 128 + 16 * ((4 * c + 2 * u + hf) ^ ((ln >> 1) & 7));
#pragma unroll
  for (int u = 0; u < 2; ++u) voff[u] = ln * 64 + 16 * ((2 * hf + u) ^ ((ln >> 2) & 3));
  // staging: chunk C = NW * p + wave moves K rows 8C..8C+7 and V^T rows 16C..16C+15 of the block,
  // into the swizzled positions the reads above expect
  int stk[NSTG], stv[NSTG];
#pragma unroll
  for (int p = 0; p < NSTG; ++p) {
    const int C = NW * p + wave;
    const int kr = 8 * C + (lane >> 3), vr = 16 * C + (lane >> 2);
    stk[p] = kr * D + 16 * ((lane & 7) ^ ((kr >> 1) & 7));
    stv[p] = vr * KB + 16 * ((lane & 3) ^ ((vr >> 2) & 3));
  }
  const size_t kstride = (size_t)n_pad * D;   // bytes per head, K and V^T alike

  // scales (E8M0 bytes) of a block: K -- the lane's key in tiles 0 and 1, shifted so that bytes 0
  // and 2 are the groups of channel chunks 0 and 1 for its half; V -- the lane's 4 channels
  auto load_scales = [&](int s, int kb, uint32_t& k0, uint32_t& k1, uint32_t& vs) {
    // block bases uniform (scalar sums), the lane's word a 32-bit offset
    const SlotPtrs sp = sslot[s];
    const size_t sc0 = (size_t)H * kstride + (size_t)h * n_pad * 4;
    const uint32_t* kp = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(uniform_ptr(sp.k)) + sc0) +
                         (size_t)kb * KB;
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(uniform_ptr(sp.v)) + sc0) +
                         (size_t)kb * 2 * 32;
    auto ld = [](const uint32_t* base, uint32_t i) {
      return *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(reinterpret_cast<uintptr_t>(base + i));
    };
    k0 = ld(kp, ln) >> (8 * hf);
    k1 = ld(kp, ln + 32) >> (8 * hf);
    vs = ld(vp, hf * 32 + ln);
  };
  auto stage = [&](int s, int kb, int buf) {
    const SlotPtrs sp = sslot[s];
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(uniform_ptr(sp.k)) + h * kstride + (size_t)kb * KB * D;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(uniform_ptr(sp.v)) + h * kstride + (size_t)kb * D * KB;
#pragma unroll
    for (int p = 0; p < NSTG; ++p) {
      const int C = NW * p + wave;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const __attribute__((address_space(1))) void*>(reinterpret_cast<uintptr_t>(kg + stk[p])),
          reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&kbuf[buf][1024 * C])),
          16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const __attribute__((address_space(1))) void*>(reinterpret_cast<uintptr_t>(vg + stv[p])),
          reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&vbuf[buf][1024 * C])),
          16, 0, 0);
    }
  };

  // ---- S^T = K Q^T for 64 keys: tiles t = 0, 1 (32 keys each), two channel chunks of 64
  auto qk = [&](const uint8_t* kl, int kvalid, uint32_t k0, uint32_t k1, f32x16& s0, f32x16& s1, bool stage_next,
                int nsl, int nkb, int nbuf) {
    // reference the scores of this block are shifted by: the running max, or 0 while it is still
    // at its floor (a shift by the floor would round the scores away)
    const float m_ref = m_run < -1.0e37f ? 0.f : m_run;
    f32x16 negm;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
    v8i kop[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kl + 4096 * t + koff[c][0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kl + 4096 * t + koff[c][1]);
        kop[c][t] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[0][0], q8[0], negm, 0, 0, 0, (int)k0, 0, (int)qsc);
    // the next block's loads ride along with the MFMAs
    if (stage_next) stage(nsl, nkb, nbuf);
    s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[0][1], q8[0], negm, 0, 0, 0, (int)k1, 0, (int)qsc);
    s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[1][0], q8[1], s0, 0, 0, 2, (int)k0, 1, (int)qsc);
    s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[1][1], q8[1], s1, 0, 0, 2, (int)k1, 1, (int)qsc);
    if (__builtin_expect(kvalid < KB, 0)) {   // last block of its slot: keys past its end do not exist
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= kvalid) s0[r] = -INFINITY;
        if (key + 32 >= kvalid) s1[r] = -INFINITY;
      }
    }
  };
  // ---- online softmax (log2 domain, lazy rescale), P -> E4M3, then O^T += V^T P^T
  auto sm_pv = [&](const uint8_t* vl, uint32_t vs, f32x16& s0, f32x16& s1) {
    v8i vop[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(vl + 2048 * t + voff[0]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(vl + 2048 * t + voff[1]);
      vop[t] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    // the scores arrive as s * scale - m_ref (base 2); m_ref as in qk
    const float m_ref = m_run < -1.0e37f ? 0.f : m_run;
    float mx = max_of_32(s0, s1);
    mx = swap_halves_max(mx) + m_ref;
    float p0[16], p1[16];
    if (__builtin_expect(__any(mx > m_run + kRescaleSlack), 0)) {
      __builtin_amdgcn_sched_barrier(0);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
      const float sh = m_ref - m_new;   // re-reference the scores to the new max
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] += sh;
        s1[r] += sh;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p0[r] = __builtin_amdgcn_exp2f(s0[r]);
      p1[r] = __builtin_amdgcn_exp2f(s1[r]);
    }
    v8i p8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p8[i] = (int)pack4_fp8(p0[4 * i], p0[4 * i + 1], p0[4 * i + 2], p0[4 * i + 3]);
      p8[4 + i] = (int)pack4_fp8(p1[4 * i], p1[4 * i + 1], p1[4 * i + 2], p1[4 * i + 3]);
    }
    // row sum of the E4M3 probabilities that multiply V, on the matrix unit: an all-ones A
    // operand (0x38 = 1.0) gives every row of the product the sum over the 64 keys
    const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838};
    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const f32x16 rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, p8, zero, 0, 0, 0, 127, 0, 127);
    l_run += rs[0];
    acc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[0], p8, acc[0], 0, 0, 0, (int)vs, 0, 127);
    acc[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[1], p8, acc[1], 0, 0, 1, (int)vs, 0, 127);
    acc[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[2], p8, acc[2], 0, 0, 2, (int)vs, 0, 127);
    acc[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[3], p8, acc[3], 0, 0, 3, (int)vs, 0, 127);
  };
  f32x16 s0, s1;

  // dense schedule cursor (as in the bf16 kernel)
  int csl = 0, ckb = 0, ccnt = 0, cnb = 0;
  auto enter = [&](int l) {
    csl = l;
    ckb = 0;
    ccnt = __builtin_amdgcn_readfirstlane(sslot[l].count);
    cnb = (ccnt + KB - 1) / KB;
  };
  enter(0);
  {
    int rem = i0;
    while (rem >= cnb && csl + 1 < n_slots) {
      rem -= cnb;
      enter(csl + 1);
    }
    ckb = rem;
  }
  auto lookup = [&](int& q, int& sl, int& kb, int& kv) {
    if (q < i1) {
      while (ckb >= cnb && csl + 1 < n_slots) enter(csl + 1);
      sl = csl;
      kb = ckb;
      kv = ccnt - ckb * KB;
      ++ckb;
    }
  };
  int pos[3], bsl[3] = {0, 0, 0}, bkb[3] = {0, 0, 0}, bkv[3] = {0, 0, 0};
  {
    int q = i0;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      lookup(q, bsl[u], bkb[u], bkv[u]);
      pos[u] = q;
      if (q < i1) ++q;
    }
  }
  uint32_t ksc0[NBUF], ksc1[NBUF], vsc[NBUF];
  // "no block" stages block 0 of slot 0 (a valid address) so that every wave's loads match
  stage(pos[0] < i1 ? bsl[0] : 0, pos[0] < i1 ? bkb[0] : 0, 0);
  load_scales(pos[0] < i1 ? bsl[0] : 0, pos[0] < i1 ? bkb[0] : 0, ksc0[0], ksc1[0], vsc[0]);
  int cur_slot = -1;   // the time channels of Q are rotated for the slot on entry
  bool pend = false;
  int pend_buf = 0;

  auto step = [&](const int cb) {
    const int sl = bsl[0], kvalid = bkv[0];
    if (pend) sm_pv(vbuf[cb ^ 1], vsc[cb ^ 1], s0, s1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's part of block n (and its scales)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (sl != cur_slot) {
      cur_slot = sl;
      load_q8<0, 1>(rt, qp, qvalid, qf, qh, qw, hf, sslot[sl].delta, scale_log2, q8, qsc);
    }
    const bool has_next = pos[1] < i1;
    const int nsl = has_next ? bsl[1] : 0, nkb = has_next ? bkb[1] : 0;
    load_scales(nsl, nkb, ksc0[cb ^ 1], ksc1[cb ^ 1], vsc[cb ^ 1]);
    qk(kbuf[cb], kvalid, ksc0[cb], ksc1[cb], s0, s1, true, nsl, nkb, cb ^ 1);
    pend = true;
    pend_buf = cb;
    int q = pos[2] < i1 ? pos[2] + 1 : i1, nsl2 = 0, nkb2 = 0, nkv = 0;
    if (pos[2] < i1) lookup(q, nsl2, nkb2, nkv);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pos[u] = pos[u + 1];
      bsl[u] = bsl[u + 1];
      bkb[u] = bkb[u + 1];
      bkv[u] = bkv[u + 1];
    }
    pos[2] = q;
    bsl[2] = nsl2;
    bkb[2] = nkb2;
    bkv[2] = nkv;
  };
  while (pos[0] < i1) {
    step(0);
    if (pos[0] >= i1) break;
    step(1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (pend) sm_pv(vbuf[pend_buf], vsc[pend_buf], s0, s1);

  const float l_tot = l_run;   // both lane halves hold the full row sum (from the matrix unit)
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (piece >= 0) {
    const int row = wave * 32 + ln;
    float* po = a.part_o + ((size_t)piece * ROWS + row) * D;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<float4*>(po + 32 * t + 8 * rg + 4 * hf) =
            make_float4(acc[t][4 * rg] * inv, acc[t][4 * rg + 1] * inv, acc[t][4 * rg + 2] * inv,
                        acc[t][4 * rg + 3] * inv);
    if (hf == 0) a.part_lse[(size_t)piece * ROWS + row] = m_run + __log2f(l_tot);
    return;
  }
  if (qvalid) {
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
    if (a.lse && hf == 0) a.lse[(size_t)h * B + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

#ifndef SWATTN_DENSE_WAVES
#define SWATTN_DENSE_WAVES 8
#endif

constexpr int kDenseWaves = SWATTN_DENSE_WAVES;

#ifndef SWATTN_FP8_WAVES
#define SWATTN_FP8_WAVES 4
#endif
constexpr int kFp8Waves = SWATTN_FP8_WAVES;



// Work split of a dense grid of `tiles` query tiles (`rows` queries each, `blocks` key blocks
// each at least) with `conc` workgroups resident at once.  Tail split: whole rounds of resident
// workgroups own whole tiles; the tiles of a last, partial round are cut into up to kMaxSplit key
// ranges (only when a whole round exists).  Fewer tiles than resident workgroups (short blocks):
// every tile is cut so that the pieces fill whole rounds (the smallest cut reaching 95% of the
// slots, if it gains 5 points).  Sets a.n_full / a.n_split; returns the number of split tiles.
int plan_split(AttnArgs& a, const SplitPlan& plan, int tiles, int conc, int rows, int blocks) {
  const int tail = conc > 0 ? tiles % conc : 0;
  const int max_pieces = plan.part_o ? plan.max_rows / rows : 0;
  int split = 0;
  if (plan.part_o && conc > 0 && tail > 0) {
    if (tiles >= conc) {
      split = std::min(std::min(kMaxSplit, conc / tail), max_pieces / tail);
      split = std::min(split, blocks);   // no empty key ranges
      if (split < 2) split = 0;
    } else {
      double best = (double)tiles / conc;
      for (int sp = 2; sp <= std::min(kMaxSplit, blocks) && tiles * sp <= max_pieces; ++sp) {
        const int pieces = tiles * sp, rounds = (pieces + conc - 1) / conc;
        const double util = (double)pieces / ((double)rounds * conc);
        if (util > best + 0.05) {
          best = util;
          split = sp;
          if (util >= 0.95) break;
        }
      }
    }
  }
  a.n_full = split ? tiles - tail : tiles;
  a.n_split = split;
  return tail;
}

hipError_t launch_attend(const Geometry& g, const RopeTab& rt, bool bf16, const void* q,
                         const SlotPtrs* slots, int n_slots, const int32_t* tile_idx, int k_row,
                         void* out, float* lse, const SplitPlan& plan, hipStream_t stream) {
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
  a.aligned_last = slots[n_slots - 1].aligned ? 1 : 0;
  for (int l = 0; l + 1 < n_slots; ++l)
    if (slots[l].aligned) return hipErrorInvalidValue;   // only the last slot may be frame-aligned
  if (a.aligned_last && (tile_idx || n_slots < 2)) return hipErrorInvalidValue;
  a.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)g.d));
  a.inv_hw = 1.0f / (float)(g.lat_h * g.lat_w);
  a.rt = rt;
  a.part_o = plan.part_o;
  a.part_lse = plan.part_lse;
  for (int i = 0; i < kMaxSlots; ++i) a.slot[i] = i < n_slots ? slots[i] : SlotPtrs{nullptr, nullptr, 0, 0, 0};
  if (bf16) {
    if (g.d != 128) return hipErrorInvalidValue;
    if (tile_idx) {   // block-sparse: 128-query tiles, 4 waves, two workgroups per CU (no split:
                      // the lists are short and the merge costs more than the tail round)
      a.n_qt = g.nt;
      a.n_full = g.nt * g.H;
      a.n_split = 0;
      hipLaunchKernelGGL((attend_bf16_kernel<true, 4, false>), dim3(a.n_full), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
    constexpr int NW = kDenseWaves;
    constexpr int ROWS = 32 * NW;
    a.n_qt = (g.B + ROWS - 1) / ROWS;
    const int conc = NW == 4 ? 2 * plan.cus : plan.cus;   // workgroups resident at once
    int blocks = 0;   // key blocks every tile has (a frame-aligned slot adds more per tile)
    for (int l = 0; l < n_slots; ++l)
      if (!slots[l].aligned) blocks += (slots[l].count + KB - 1) / KB;
    const int tail = plan_split(a, plan, a.n_qt * g.H, conc, ROWS, blocks);
    const int split = a.n_split;
    // the frame-aligned (editing) variant is its own instantiation: the plain kernel keeps its code
    if (a.aligned_last)
      hipLaunchKernelGGL((attend_bf16_kernel<false, NW, true>), dim3(a.n_full + tail * split), dim3(64 * NW), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((attend_bf16_kernel<false, NW, false>), dim3(a.n_full + tail * split), dim3(64 * NW), 0,
                         stream, a);
    if (split) hipLaunchKernelGGL((merge_kernel<ROWS>), dim3(tail, ROWS / kMergeRows), dim3(256), 0, stream, a);
  } else {
    if (tile_idx) return hipErrorInvalidValue;
    const dim3 grid((g.B + 63) / 64, g.H), block(256);
    if (g.d == 64)
      hipLaunchKernelGGL((attend_f32_kernel<64>), grid, block, 0, stream, a);
    else if (g.d == 128)
      hipLaunchKernelGGL((attend_f32_kernel<128>), grid, block, 0, stream, a);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Rows of partial results the dense bf16 or fp8 launch of these slots writes to the split
// workspace under `plan` (the same planning as the launches below; 0 when nothing is split).
int split_rows(const Geometry& g, bool fp8, const SlotPtrs* slots, int n_slots, const SplitPlan& plan) {
  if (n_slots < 1 || n_slots > kMaxSlots) return 0;
  AttnArgs a;
  const int NW = fp8 ? kFp8Waves : kDenseWaves, ROWS = 32 * NW;
  a.n_qt = (g.B + ROWS - 1) / ROWS;
  int blocks = 0;
  for (int l = 0; l < n_slots; ++l)
    if (!slots[l].aligned) blocks += (slots[l].count + KB - 1) / KB;
  const int conc = NW == 4 ? 2 * plan.cus : plan.cus;
  const int tail = plan_split(a, plan, a.n_qt * g.H, conc, ROWS, blocks);
  return tail * a.n_split * ROWS;
}

hipError_t launch_attend_fp8(const Geometry& g, const RopeTab& rt, const void* q, const SlotPtrs* slots, int n_slots,
                             void* out, float* lse, const SplitPlan& plan, hipStream_t stream) {
  if (n_slots < 1 || n_slots > kMaxSlots || g.d != 128) return hipErrorInvalidValue;
  for (int l = 0; l < n_slots; ++l)
    if (slots[l].aligned) return hipErrorInvalidValue;   // frame-aligned slots: bf16 only
  AttnArgs a;
  a.q = q;
  a.o = out;
  a.lse = lse;
  a.tile_idx = nullptr;
  a.k_row = 0;
  a.B = g.B;
  a.H = g.H;
  a.n_pad = g.n_pad;
  a.nt = g.nt;
  a.hw = g.lat_h * g.lat_w;
  a.lat_w = g.lat_w;
  a.n_slots = n_slots;
  a.aligned_last = 0;
  a.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)g.d));
  a.inv_hw = 1.0f / (float)(g.lat_h * g.lat_w);
  a.rt = rt;
  a.part_o = plan.part_o;
  a.part_lse = plan.part_lse;
  for (int i = 0; i < kMaxSlots; ++i) a.slot[i] = i < n_slots ? slots[i] : SlotPtrs{nullptr, nullptr, 0, 0, 0};
  constexpr int NW = kFp8Waves, ROWS = 32 * NW;
  a.n_qt = (g.B + ROWS - 1) / ROWS;
  int blocks = 0;
  for (int l = 0; l < n_slots; ++l) blocks += (slots[l].count + KB - 1) / KB;
  const int conc = NW == 4 ? 2 * plan.cus : plan.cus;   // workgroups resident at once
  const int tail = plan_split(a, plan, a.n_qt * g.H, conc, ROWS, blocks);
  const int split = a.n_split;
  hipLaunchKernelGGL((attend_fp8_kernel<NW>), dim3(a.n_full + tail * split), dim3(64 * NW), 0, stream, a);
  if (split) hipLaunchKernelGGL((merge_kernel<ROWS>), dim3(tail, ROWS / kMergeRows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace swattn
