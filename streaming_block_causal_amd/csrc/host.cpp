// Host side of libswattn: the ring-buffer cache bookkeeping, RoPE tables,
// argument validation and kernel dispatch behind the C ABI in include/swattn.h.
//
// Cache model ("Vidu S2 vs PixVerse R2" blog, section "Choice 3: bounded
// memory"): the first S committed blocks are permanent sinks, later blocks go to
// a window of the W most recent, older ones are evicted.  Physically there are
// P = S + W + 1 slots (plus a noisy twin of each with TwinCache): the sinks, the
// window and one staging slot the current block is written into every step.
// Committing the staged block and evicting the oldest window block are pure
// index remaps: the logical order lives in a small host table, a freed slot
// becomes the next staging slot, and no K/V byte moves.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <new>
#include <string>
#include <vector>

#include "swattn.h"
#include "launch.h"

using namespace swattn;

namespace {

thread_local std::string g_err;

sw_status fail(sw_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sw_status fail(sw_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sw_status hip_fail(hipError_t e, const char* what) {
  return fail(SW_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace swhost {

struct Entry {
  int64_t block;
  int phys;
  int frames;   // latent frames of the block (<= the configured cap)
};

struct Layout {
  Geometry g;
  size_t elem;           // bytes per stored element
  size_t kv_bytes;       // one K (or V) buffer of a slot
  size_t pooled_bytes;   // one pooled-key table of a slot (0 if not sparse)
  int P;                 // physical slots
  int t_len;             // time positions in the RoPE table
  int pt, ph, pw;
  size_t table_floats;
  size_t ws_bytes;       // partial results of split attention tiles (bf16 caches)
  size_t src_bytes;      // editing: the source-frame staging buffer (K and V of one block)
  size_t total;
};

}  // namespace swhost

using swhost::Entry;
using swhost::Layout;

namespace {

sw_status make_layout(const sw_cache_config* cfg, Layout* L) {
  if (!cfg) return fail(SW_ERR_INVALID_ARG, "config is NULL");
  const sw_cache_config& c = *cfg;
  if (c.n_heads < 1 || c.frames_per_block < 1 || c.lat_h < 1 || c.lat_w < 1)
    return fail(SW_ERR_INVALID_ARG, "n_heads, frames_per_block, lat_h, lat_w must be >= 1");
  if (c.n_sink < 0 || c.n_window < 0) return fail(SW_ERR_INVALID_ARG, "n_sink, n_window must be >= 0");
  if (c.n_heads > 65535) return fail(SW_ERR_SHAPE, "n_heads %d exceeds 65535 (a launch grid dimension)", c.n_heads);
  // 64-bit sums: n_sink and n_window are caller-controlled int32
  if ((long long)c.n_sink + c.n_window + 1 > kMaxSlots)
    return fail(SW_ERR_SHAPE, "n_sink + n_window + 1 = %lld exceeds %d", (long long)c.n_sink + c.n_window + 1,
                kMaxSlots);
  if (c.twin != 0 && c.twin != 1) return fail(SW_ERR_INVALID_ARG, "twin must be 0 or 1");
  if (c.sparse != 0 && c.sparse != 1) return fail(SW_ERR_INVALID_ARG, "sparse must be 0 or 1");
  if (c.dtype != SW_BF16 && c.dtype != SW_F32 && c.dtype != SW_FP8)
    return fail(SW_ERR_INVALID_ARG, "unknown dtype %d", (int)c.dtype);
  if (c.policy != SW_ROPE_S1_RELOCATE && c.policy != SW_ROPE_RELATIVE_TIME)
    return fail(SW_ERR_INVALID_ARG, "unknown RoPE policy %d", (int)c.policy);
  if (!(c.rope_theta > 1.0) || !std::isfinite(c.rope_theta))
    return fail(SW_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (c.tile != kTile) return fail(SW_ERR_UNSUPPORTED, "tile must be %d", kTile);
  if (c.dtype == SW_FP8 && c.head_dim != 128)
    return fail(SW_ERR_UNSUPPORTED, "fp8 kernels are built for head_dim 128 (got %d)", c.head_dim);
  if (c.dtype == SW_FP8 && (c.sparse || c.editing))
    return fail(SW_ERR_UNSUPPORTED, "fp8 attention is built for the dense stream (no sparse, no editing)");
  if (c.dtype == SW_BF16 && c.head_dim != 128)
    return fail(SW_ERR_UNSUPPORTED, "bf16 kernels are built for head_dim 128 (got %d)", c.head_dim);
  if (c.dtype == SW_F32 && c.head_dim != 64 && c.head_dim != 128)
    return fail(SW_ERR_UNSUPPORTED, "fp32 kernels are built for head_dim 64 or 128 (got %d)", c.head_dim);
  if (c.sparse && c.dtype != SW_BF16) return fail(SW_ERR_UNSUPPORTED, "block-sparse needs bf16");
  if (c.editing != 0 && c.editing != 1) return fail(SW_ERR_INVALID_ARG, "editing must be 0 or 1");
  if (c.editing && c.sparse) return fail(SW_ERR_UNSUPPORTED, "frame-aligned editing attention is dense only");
  if (c.editing && (long long)c.n_sink + c.n_window + 2 > kMaxSlots)
    return fail(SW_ERR_SHAPE, "n_sink + n_window + 2 = %d exceeds %d with editing", c.n_sink + c.n_window + 2,
                kMaxSlots);
  // RoPE split over (t, h, w): all zero = the default (time gets the remainder of thirds)
  const int pairs = c.head_dim / 2;
  int pt = pairs - 2 * (pairs / 3), ph = pairs / 3, pw = pairs / 3;
  if (c.rope_pairs_t != 0 || c.rope_pairs_h != 0 || c.rope_pairs_w != 0) {
    if (c.rope_pairs_t < 0 || c.rope_pairs_h < 0 || c.rope_pairs_w < 0 ||
        (long long)c.rope_pairs_t + c.rope_pairs_h + c.rope_pairs_w != pairs)
      return fail(SW_ERR_INVALID_ARG, "rope_pairs_t/h/w = %d/%d/%d must be >= 0 and sum to head_dim / 2 = %d",
                  c.rope_pairs_t, c.rope_pairs_h, c.rope_pairs_w, pairs);
    pt = c.rope_pairs_t;
    ph = c.rope_pairs_h;
    pw = c.rope_pairs_w;
  }
  // the bf16 and fp8 attention kernels re-rotate only the first 24 pairs of a query per slot
  if (c.dtype != SW_F32 && pt > 24)
    return fail(SW_ERR_UNSUPPORTED, "%d time RoPE pairs exceed the 24 the bf16 / fp8 kernels re-rotate", pt);
  const long long B = (long long)c.frames_per_block * c.lat_h * c.lat_w;
  if (B > 65536) return fail(SW_ERR_SHAPE, "block of %lld tokens exceeds 65536", B);
  Geometry& g = L->g;
  g.B = (int)B;
  g.H = c.n_heads;
  g.d = c.head_dim;
  g.F = c.frames_per_block;
  g.lat_h = c.lat_h;
  g.lat_w = c.lat_w;
  g.nt = (g.B + kTile - 1) / kTile;
  g.n_pad = g.nt * kTile;
  if ((long long)(c.n_sink + c.n_window + 1) * g.nt > kMaxKeyTiles && c.sparse)
    return fail(SW_ERR_SHAPE, "too many key tiles for the mask builder");
  L->elem = c.dtype == SW_BF16 ? 2 : (c.dtype == SW_FP8 ? 1 : 4);
  // fp8: E4M3 values, then one E8M0 scale byte per 32 values
  L->kv_bytes = align256((size_t)g.H * g.n_pad * g.d * L->elem + (c.dtype == SW_FP8 ? (size_t)g.H * g.n_pad * g.d / 32 : 0));
  L->pooled_bytes = c.sparse ? align256((size_t)g.H * g.nt * g.d * sizeof(float)) : 0;
  L->P = c.n_sink + c.n_window + 1;
  L->t_len = L->P * g.F;
  L->pt = pt;
  L->ph = ph;
  L->pw = pw;
  L->table_floats = 2 * ((size_t)L->t_len * L->pt + (size_t)g.lat_h * L->ph + (size_t)g.lat_w * L->pw);
  const int copies = c.twin ? 2 : 1;
  L->ws_bytes = c.dtype != SW_F32
                    ? align256((size_t)kSplitRows * g.d * sizeof(float)) +
                          align256((size_t)kSplitRows * sizeof(float))
                    : 0;
  L->src_bytes = c.editing ? 2 * L->kv_bytes : 0;
  L->total = (size_t)L->P * copies * (2 * L->kv_bytes + L->pooled_bytes) +
             align256(L->table_floats * sizeof(float)) + L->ws_bytes + L->src_bytes;
  return SW_OK;
}

}  // namespace

struct sw_cache {
  sw_cache_config cfg;
  Layout L;
  bool dry;
  hipStream_t stream;
  char* pool;
  RopeTab rt;
  std::vector<char*> kc, vc, kn, vn;     // per physical slot: clean/current and noisy copies
  std::vector<float*> pc, pn;            // pooled-key tables
  std::vector<Entry> sinks;
  std::deque<Entry> window;
  std::deque<int> free_slots;
  int staging;
  bool staged;
  int64_t staged_id;
  int staged_frames;
  bool have_commit;
  int64_t last_commit;
  bool noisy_due;
  Entry noisy_entry;
  char* ks;            // editing: source-frame K/V staging buffer (outside the ring)
  char* vs;
  bool src_staged;     // source frames of the staged block are in ks/vs
  sw_rope_policy policy;
  SplitPlan plan;
  bool capturing;      // between sw_graph_begin and sw_graph_end
  int dev;             // the device current at create
};

struct sw_graph {
  hipGraphExec_t exec;
  hipStream_t stream;   // the stream it was captured from
};

namespace {

std::vector<Entry> history(const sw_cache* c) {
  std::vector<Entry> h(c->sinks.begin(), c->sinks.end());
  h.insert(h.end(), c->window.begin(), c->window.end());
  return h;
}

// Time base of each logical slot [sinks, window oldest->newest, current]: a slot starts where
// the previous one ends (l*F when every block has F frames).  Relative time shifts the whole
// layout so that the window starts at 0 and the sinks sit just before it.
std::vector<int> bases_of(const sw_cache* c) {
  const std::vector<Entry> h = history(c);
  std::vector<int> b(h.size() + 1);
  int t = 0, sink_frames = 0;
  for (size_t l = 0; l < h.size(); ++l) {
    b[l] = t;
    t += h[l].frames;
    if (l < c->sinks.size()) sink_frames += h[l].frames;
  }
  b[h.size()] = t;
  if (c->policy == SW_ROPE_RELATIVE_TIME)
    for (int& x : b) x -= sink_frames;
  return b;
}

// tokens of a block of `frames` latent frames
int tokens_of(const sw_cache* c, int frames) { return frames * c->L.g.lat_h * c->L.g.lat_w; }

// every logical slot (and the staged block) at the full configured length
bool all_full(const sw_cache* c) {
  for (const Entry& e : history(c))
    if (e.frames != c->L.g.F) return false;
  return !c->staged || c->staged_frames == c->L.g.F;
}

void fill_tables(const Layout& L, double theta, std::vector<float>& t) {
  t.assign(L.table_floats, 0.f);
  size_t o = 0;
  auto axis = [&](int n_pos, int n_pairs) {
    for (int pos = 0; pos < n_pos; ++pos)
      for (int j = 0; j < n_pairs; ++j) {   // (cos, sin) side by side
        const double ang = (double)pos * std::pow(theta, -(double)j / (double)n_pairs);
        t[o + 2 * ((size_t)pos * n_pairs + j)] = (float)std::cos(ang);
        t[o + 2 * ((size_t)pos * n_pairs + j) + 1] = (float)std::sin(ang);
      }
    o += 2 * (size_t)n_pos * n_pairs;
  };
  axis(L.t_len, L.pt);
  axis(L.g.lat_h, L.ph);
  axis(L.g.lat_w, L.pw);
}

sw_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(SW_ERR_INVALID_ARG, "%s is NULL", name);
  return SW_OK;
}

// may block `block_id` of `n_frames` frames be staged as the current block now?
sw_status check_stage(const sw_cache* c, int64_t block_id, int n_frames) {
  if (c->noisy_due) return fail(SW_ERR_STATE, "the noisy copy of block %lld must be appended first",
                                (long long)c->noisy_entry.block);
  if (c->staged && block_id != c->staged_id)
    return fail(SW_ERR_STATE, "block %lld is staged; commit it before staging block %lld",
                (long long)c->staged_id, (long long)block_id);
  if (c->have_commit && block_id <= c->last_commit)
    return fail(SW_ERR_STATE, "block %lld is not newer than the last commit %lld", (long long)block_id,
                (long long)c->last_commit);
  if (c->staged && n_frames != c->staged_frames)
    return fail(SW_ERR_STATE, "block %lld is staged with %d frames, not %d", (long long)block_id,
                c->staged_frames, n_frames);
  return SW_OK;
}

sw_status write_block(sw_cache* c, const void* k, const void* v, char* kd, char* vd, float* pd, int frames) {
  if (c->dry) return SW_OK;
  Geometry g = c->L.g;   // the slot keeps its capped stride (n_pad); the block fills its first rows
  g.B = tokens_of(c, frames);
  g.nt = (g.B + kTile - 1) / kTile;
  const hipError_t e = c->cfg.dtype == SW_FP8
                            ? launch_append_fp8(g, c->rt, k, v, kd, vd, c->stream)
                            : launch_append(g, c->rt, c->cfg.dtype == SW_BF16, k, v, kd, vd, pd, c->stream);
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return SW_OK;
}

}  // namespace

namespace {

// One denoising step's attention (sw_chunk_attend).  part_o == nullptr: the split workspace of
// the cache pool; otherwise the caller's workspace of max_rows rows, which must hold the split the
// pool's plan makes (so that both give the same work split and the same result).
sw_status chunk_attend(sw_cache* c, const void* q_raw, sw_step_kind step, const int32_t* tile_idx, int32_t k_row,
                       void* out, float* lse_out, float* part_o, float* part_lse, int max_rows) {
  sw_status st = check_ptr(q_raw, "q_raw");
  if (st == SW_OK) st = check_ptr(out, "out");
  if (st != SW_OK) return st;
  if (step != SW_STEP_INTERMEDIATE && step != SW_STEP_FINAL)
    return fail(SW_ERR_INVALID_ARG, "unknown step kind %d", (int)step);
  if (c->dry) return fail(SW_ERR_STATE, "metadata-only cache cannot launch kernels");
  if (!c->staged) return fail(SW_ERR_STATE, "no staged current block (append SW_KV_CURRENT first)");
  if (c->noisy_due) return fail(SW_ERR_STATE, "a noisy append is due");
  if (tile_idx) {
    if (c->cfg.dtype != SW_BF16) return fail(SW_ERR_UNSUPPORTED, "block-sparse attention needs bf16");
    if (c->src_staged) return fail(SW_ERR_UNSUPPORTED, "frame-aligned editing attention is dense only");
    if (k_row < 1) return fail(SW_ERR_INVALID_ARG, "k_row must be >= 1 with a tile list");
    if (!all_full(c)) return fail(SW_ERR_UNSUPPORTED, "block-sparse attention needs full-length blocks");
  }
  const std::vector<Entry> hist = history(c);
  const std::vector<int> b = bases_of(c);
  const int n_slots = (int)hist.size() + 1;
  if (tile_idx && k_row > n_slots * c->L.g.nt)
    return fail(SW_ERR_INVALID_ARG, "k_row %d exceeds the %d key tiles", k_row, n_slots * c->L.g.nt);
  const bool noisy = c->cfg.twin && step == SW_STEP_INTERMEDIATE;
  SlotPtrs slots[kMaxSlots];
  for (int l = 0; l + 1 < n_slots; ++l) {
    const int p = hist[l].phys;
    slots[l] = SlotPtrs{noisy ? c->kn[p] : c->kc[p], noisy ? c->vn[p] : c->vc[p], b.back() - b[l],
                        tokens_of(c, hist[l].frames), 0};
  }
  slots[n_slots - 1] = SlotPtrs{c->kc[c->staging], c->vc[c->staging], 0, tokens_of(c, c->staged_frames), 0};
  int n_all = n_slots;
  if (c->src_staged)   // the source frames sit at the current block's positions, frame-aligned
    slots[n_all++] = SlotPtrs{c->ks, c->vs, 0, tokens_of(c, c->staged_frames), 1};
  Geometry gq = c->L.g;   // the queries are the staged block's tokens
  gq.B = tokens_of(c, c->staged_frames);
  SplitPlan plan = c->plan;
  if (part_o) {   // the caller's workspace: same plan as the pool's, so it must hold that split
    const int need = (tile_idx || c->cfg.dtype == SW_F32)
                         ? 0 : split_rows(gq, c->cfg.dtype == SW_FP8, slots, n_all, c->plan);
    if (need > max_rows)
      return fail(SW_ERR_CAPACITY,
                  "this call splits %d query rows into key ranges; the static scratch holds %d (fewer query tiles "
                  "than compute units: use sw_chunk_attend)", need, max_rows);
    plan.part_o = part_o;
    plan.part_lse = part_lse;
  }
  const hipError_t e = c->cfg.dtype == SW_FP8
                            ? launch_attend_fp8(gq, c->rt, q_raw, slots, n_all, out, lse_out, plan, c->stream)
                            : launch_attend(gq, c->rt, c->cfg.dtype == SW_BF16, q_raw, slots, n_all, tile_idx, k_row,
                                            out, lse_out, plan, c->stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return SW_OK;
}


}  // namespace

namespace swhost {

int cache_device(const sw_cache* c) { return c->dev; }

int chunk_attend_scratch(sw_cache* c, const void* q_raw, int step, const int32_t* tile_idx, int32_t k_row, void* out,
                         float* lse_out, float* part_o, float* part_lse, int max_rows) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (c->dry) return fail(SW_ERR_STATE, "metadata-only cache cannot launch kernels");
  if (!part_o || !part_lse || max_rows < 0) return fail(SW_ERR_INVALID_ARG, "no scratch workspace");
  return chunk_attend(c, q_raw, static_cast<sw_step_kind>(step), tile_idx, k_row, out, lse_out, part_o, part_lse,
                      max_rows);
}

int hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }

}  // namespace swhost

extern "C" {

const char* sw_last_error(void) { return g_err.c_str(); }

sw_status sw_cache_required_bytes(const sw_cache_config* cfg, size_t* bytes) {
  if (!bytes) return fail(SW_ERR_INVALID_ARG, "bytes is NULL");
  Layout L;
  const sw_status st = make_layout(cfg, &L);
  if (st != SW_OK) return st;
  *bytes = L.total;
  return SW_OK;
}

sw_status sw_cache_create(const sw_cache_config* cfg, void* device_pool, size_t pool_bytes,
                          void* hip_stream, sw_cache** out) {
  if (!out) return fail(SW_ERR_INVALID_ARG, "out is NULL");
  Layout L;
  sw_status st = make_layout(cfg, &L);
  if (st != SW_OK) return st;
  const bool dry = device_pool == nullptr && pool_bytes == 0;
  if (!dry) {
    if (!device_pool) return fail(SW_ERR_INVALID_ARG, "device_pool is NULL");
    if (((uintptr_t)device_pool & 255) != 0) return fail(SW_ERR_INVALID_ARG, "device_pool must be 256-byte aligned");
    if (pool_bytes < L.total)
      return fail(SW_ERR_CAPACITY, "pool of %zu bytes, %zu needed", pool_bytes, L.total);
  }
  sw_cache* c = new (std::nothrow) sw_cache();
  if (!c) return fail(SW_ERR_CAPACITY, "host allocation failed");
  c->cfg = *cfg;
  c->L = L;
  c->dry = dry;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->pool = static_cast<char*>(device_pool);
  const int copies = cfg->twin ? 2 : 1;
  c->kc.assign(L.P, nullptr);
  c->vc.assign(L.P, nullptr);
  c->kn.assign(L.P, nullptr);
  c->vn.assign(L.P, nullptr);
  c->pc.assign(L.P, nullptr);
  c->pn.assign(L.P, nullptr);
  if (!dry) {
    char* p = c->pool;
    for (int s = 0; s < L.P; ++s) {
      for (int cp = 0; cp < copies; ++cp) {
        char* kbuf = p; p += L.kv_bytes;
        char* vbuf = p; p += L.kv_bytes;
        float* pbuf = L.pooled_bytes ? reinterpret_cast<float*>(p) : nullptr;
        p += L.pooled_bytes;
        if (cp == 0) { c->kc[s] = kbuf; c->vc[s] = vbuf; c->pc[s] = pbuf; }
        else { c->kn[s] = kbuf; c->vn[s] = vbuf; c->pn[s] = pbuf; }
      }
    }
    float* tab = reinterpret_cast<float*>(p);
    p += align256(L.table_floats * sizeof(float));
    c->plan.part_o = L.ws_bytes ? reinterpret_cast<float*>(p) : nullptr;
    c->plan.part_lse = L.ws_bytes ? reinterpret_cast<float*>(p + align256((size_t)kSplitRows * L.g.d * sizeof(float)))
                                  : nullptr;
    c->plan.max_rows = L.ws_bytes ? kSplitRows : 0;
    p += L.ws_bytes;
    c->ks = L.src_bytes ? p : nullptr;
    c->vs = L.src_bytes ? p + L.kv_bytes : nullptr;
    int dev = 0, cus = 0;
    hipError_t de = hipGetDevice(&dev);
    if (de == hipSuccess) de = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (de != hipSuccess) {
      delete c;
      return hip_fail(de, "device query");
    }
    c->plan.cus = cus;
    c->dev = dev;
    std::vector<float> host;
    fill_tables(L, cfg->rope_theta, host);
    hipError_t e = hipMemsetAsync(c->pool, 0, L.total, c->stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(tab, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
      delete c;
      return hip_fail(e, "cache initialisation");
    }
    size_t o = 0;
    c->rt.t = reinterpret_cast<const CosSin*>(tab + o); o += 2 * (size_t)L.t_len * L.pt;
    c->rt.h = reinterpret_cast<const CosSin*>(tab + o); o += 2 * (size_t)L.g.lat_h * L.ph;
    c->rt.w = reinterpret_cast<const CosSin*>(tab + o);
  }
  c->rt.pt = L.pt;
  c->rt.ph = L.ph;
  c->rt.pw = L.pw;
  c->rt.t_len = L.t_len;
  c->staging = 0;
  for (int s = 1; s < L.P; ++s) c->free_slots.push_back(s);
  c->staged = false;
  c->staged_id = -1;
  c->staged_frames = L.g.F;
  c->have_commit = false;
  c->last_commit = -1;
  c->noisy_due = false;
  c->noisy_entry = Entry{-1, -1, 0};
  c->src_staged = false;
  c->capturing = false;
  if (dry) {
    c->ks = c->vs = nullptr;
    c->dev = -1;
  }
  c->policy = cfg->policy;
  if (dry) c->plan = SplitPlan{0, 0, nullptr, nullptr};
  *out = c;
  return SW_OK;
}

sw_status sw_cache_destroy(sw_cache* c) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (c->capturing) return fail(SW_ERR_STATE, "a graph capture is in progress; end it first");
  delete c;
  return SW_OK;
}

sw_status sw_graph_begin(sw_cache* c) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (c->dry) return fail(SW_ERR_STATE, "metadata-only cache cannot launch kernels");
  if (c->capturing) return fail(SW_ERR_STATE, "already capturing");
  const hipError_t e = hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "begin capture");
  c->capturing = true;
  return SW_OK;
}

sw_status sw_graph_end(sw_cache* c, sw_graph** out) {
  if (!c || !out) return fail(SW_ERR_INVALID_ARG, "cache or out is NULL");
  if (!c->capturing) return fail(SW_ERR_STATE, "no capture in progress");
  c->capturing = false;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(c->stream, &graph);
  if (e != hipSuccess) return hip_fail(e, "end capture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  const hipError_t ed = hipGraphDestroy(graph);   // the executable graph keeps its own copy
  if (e == hipSuccess) e = ed;
  if (e != hipSuccess) {
    if (exec) (void)hipGraphExecDestroy(exec);
    return hip_fail(e, "graph instantiation");
  }
  sw_graph* g = new (std::nothrow) sw_graph();
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    return fail(SW_ERR_CAPACITY, "host allocation failed");
  }
  g->exec = exec;
  g->stream = c->stream;
  *out = g;
  return SW_OK;
}

sw_status sw_graph_launch(sw_graph* g, void* hip_stream) {
  if (!g) return fail(SW_ERR_INVALID_ARG, "graph is NULL");
  const hipStream_t s = hip_stream ? static_cast<hipStream_t>(hip_stream) : g->stream;
  const hipError_t e = hipGraphLaunch(g->exec, s);
  if (e != hipSuccess) return hip_fail(e, "graph launch");
  return SW_OK;
}

sw_status sw_graph_destroy(sw_graph* g) {
  if (!g) return fail(SW_ERR_INVALID_ARG, "graph is NULL");
  const hipError_t e = hipGraphExecDestroy(g->exec);
  delete g;
  if (e != hipSuccess) return hip_fail(e, "graph destruction");
  return SW_OK;
}

sw_status sw_cache_ring_period(const sw_cache* c, int32_t* period) {
  if (!c || !period) return fail(SW_ERR_INVALID_ARG, "cache or period is NULL");
  *period = c->cfg.n_window + 1;
  return SW_OK;
}

sw_status sw_cache_append_block(sw_cache* c, sw_kv_kind kind, const void* k_raw, const void* v_raw,
                                int64_t block_id) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  return sw_cache_append_block_frames(c, kind, k_raw, v_raw, block_id, c->cfg.frames_per_block);
}

sw_status sw_cache_append_block_frames(sw_cache* c, sw_kv_kind kind, const void* k_raw, const void* v_raw,
                                       int64_t block_id, int32_t n_frames) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (block_id < 0) return fail(SW_ERR_INVALID_ARG, "block_id must be >= 0");
  const bool promote_call = kind == SW_KV_CLEAN && k_raw == nullptr && v_raw == nullptr;
  if (!promote_call) {
    if (n_frames < 1 || n_frames > c->cfg.frames_per_block)
      return fail(SW_ERR_INVALID_ARG, "n_frames %d outside [1, %d]", n_frames, c->cfg.frames_per_block);
    if (c->cfg.sparse && n_frames != c->cfg.frames_per_block)
      return fail(SW_ERR_UNSUPPORTED, "block-sparse caches hold full-length blocks only");
  }
  const int S = c->cfg.n_sink, W = c->cfg.n_window;
  switch (kind) {
    case SW_KV_CURRENT: {
      sw_status st = check_ptr(k_raw, "k_raw");
      if (st == SW_OK) st = check_ptr(v_raw, "v_raw");
      if (st == SW_OK) st = check_stage(c, block_id, n_frames);
      if (st != SW_OK) return st;
      const int s = c->staging;
      st = write_block(c, k_raw, v_raw, c->kc[s], c->vc[s], c->pc[s], n_frames);
      if (st != SW_OK) return st;
      c->staged = true;
      c->staged_id = block_id;
      c->staged_frames = n_frames;
      return SW_OK;
    }
    case SW_KV_CLEAN: {
      if (c->noisy_due) return fail(SW_ERR_STATE, "the noisy copy of block %lld must be appended first",
                                    (long long)c->noisy_entry.block);
      const bool promote = k_raw == nullptr && v_raw == nullptr;
      if (!promote) {
        sw_status st = check_ptr(k_raw, "k_raw");
        if (st == SW_OK) st = check_ptr(v_raw, "v_raw");
        if (st != SW_OK) return st;
        if (c->staged) return fail(SW_ERR_STATE, "a current block is staged; promote it with NULL pointers");
      } else {
        if (!c->staged) return fail(SW_ERR_STATE, "no staged current block to commit");
        if (block_id != c->staged_id)
          return fail(SW_ERR_STATE, "staged block is %lld, not %lld", (long long)c->staged_id, (long long)block_id);
      }
      if (c->have_commit && block_id <= c->last_commit)
        return fail(SW_ERR_STATE, "block %lld is not newer than the last commit %lld", (long long)block_id,
                    (long long)c->last_commit);
      const bool to_sink = (int)c->sinks.size() < S;
      if (!to_sink && W > 0 && (int)c->window.size() == W)
        return fail(SW_ERR_CAPACITY, "window is full (%d blocks); evict first", W);
      const bool dropped = !to_sink && W == 0;   // no window: the block leaves at once
      int phys = -1;
      if (!dropped) {
        if (promote) {
          if (c->free_slots.empty()) return fail(SW_ERR_STATE, "internal: no free slot for staging");
          phys = c->staging;
        } else {
          if (c->free_slots.empty()) return fail(SW_ERR_STATE, "internal: no free slot");
          phys = c->free_slots.front();
          const sw_status st = write_block(c, k_raw, v_raw, c->kc[phys], c->vc[phys], c->pc[phys], n_frames);
          if (st != SW_OK) return st;
          c->free_slots.pop_front();
        }
      }
      const int frames = promote ? c->staged_frames : n_frames;
      c->src_staged = false;   // source frames are consumed with their block, never kept
      if (promote) {
        c->staged = false;
        c->staged_id = -1;
        if (!dropped) {
          c->staging = c->free_slots.front();
          c->free_slots.pop_front();
        }
      }
      c->have_commit = true;
      c->last_commit = block_id;
      if (!dropped) {
        const Entry e{block_id, phys, frames};
        if (to_sink) c->sinks.push_back(e);
        else c->window.push_back(e);
        if (c->cfg.twin) {
          c->noisy_due = true;
          c->noisy_entry = e;
        }
      }
      return SW_OK;
    }
    case SW_KV_SOURCE: {
      if (!c->cfg.editing) return fail(SW_ERR_STATE, "source frames need an editing cache (editing = 1)");
      sw_status st = check_ptr(k_raw, "k_raw");
      if (st == SW_OK) st = check_ptr(v_raw, "v_raw");
      if (st != SW_OK) return st;
      if (c->noisy_due) return fail(SW_ERR_STATE, "the noisy copy of block %lld must be appended first",
                                    (long long)c->noisy_entry.block);
      if (!c->staged) return fail(SW_ERR_STATE, "source frames belong to the staged block: stage it first");
      if (block_id != c->staged_id)
        return fail(SW_ERR_STATE, "staged block is %lld, source frames given for %lld", (long long)c->staged_id,
                    (long long)block_id);
      if (n_frames != c->staged_frames)
        return fail(SW_ERR_STATE, "block %lld is staged with %d frames, its source with %d", (long long)block_id,
                    c->staged_frames, n_frames);
      st = write_block(c, k_raw, v_raw, c->ks, c->vs, nullptr, n_frames);
      if (st != SW_OK) return st;
      c->src_staged = true;
      return SW_OK;
    }
    case SW_KV_NOISY: {
      if (!c->cfg.twin) return fail(SW_ERR_STATE, "noisy copies need a TwinCache (twin = 1)");
      sw_status st = check_ptr(k_raw, "k_raw");
      if (st == SW_OK) st = check_ptr(v_raw, "v_raw");
      if (st != SW_OK) return st;
      if (!c->noisy_due) return fail(SW_ERR_STATE, "no committed block is waiting for its noisy copy");
      if (block_id != c->noisy_entry.block)
        return fail(SW_ERR_STATE, "noisy copy of block %lld is due, got %lld", (long long)c->noisy_entry.block,
                    (long long)block_id);
      if (n_frames != c->noisy_entry.frames)
        return fail(SW_ERR_STATE, "block %lld has %d frames, its noisy copy %d", (long long)block_id,
                    c->noisy_entry.frames, n_frames);
      const int s = c->noisy_entry.phys;
      st = write_block(c, k_raw, v_raw, c->kn[s], c->vn[s], c->pn[s], n_frames);
      if (st != SW_OK) return st;
      c->noisy_due = false;
      return SW_OK;
    }
  }
  return fail(SW_ERR_INVALID_ARG, "unknown kv kind %d", (int)kind);
}

sw_status sw_cache_append_qkv(sw_cache* c, const void* qkv_raw, const float* gamma_q, const float* gamma_k,
                              float eps, void* q_out, int64_t block_id, int32_t n_frames) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  sw_status st = check_ptr(qkv_raw, "qkv_raw");
  if (st == SW_OK) st = check_ptr(gamma_q, "gamma_q");
  if (st == SW_OK) st = check_ptr(gamma_k, "gamma_k");
  if (st == SW_OK) st = check_ptr(q_out, "q_out");
  if (st != SW_OK) return st;
  if (block_id < 0) return fail(SW_ERR_INVALID_ARG, "block_id must be >= 0");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(SW_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (n_frames < 1 || n_frames > c->cfg.frames_per_block)
    return fail(SW_ERR_INVALID_ARG, "n_frames %d outside [1, %d]", n_frames, c->cfg.frames_per_block);
  if (c->cfg.sparse && n_frames != c->cfg.frames_per_block)
    return fail(SW_ERR_UNSUPPORTED, "block-sparse caches hold full-length blocks only");
  if (c->cfg.head_dim != 128) return fail(SW_ERR_UNSUPPORTED, "the QKV epilogue is built for head_dim 128");
  if (c->cfg.dtype == SW_FP8) return fail(SW_ERR_UNSUPPORTED, "the QKV epilogue writes bf16 or fp32 caches");
  st = check_stage(c, block_id, n_frames);
  if (st != SW_OK) return st;
  const int s = c->staging;
  if (!c->dry) {
    Geometry g = c->L.g;
    g.B = tokens_of(c, n_frames);
    g.nt = (g.B + kTile - 1) / kTile;
    const hipError_t e = launch_append_qkv(g, c->rt, c->cfg.dtype == SW_BF16, qkv_raw, gamma_q, gamma_k, eps,
                                           q_out, c->kc[s], c->vc[s], c->pc[s], c->stream);
    if (e != hipSuccess) return hip_fail(e, "QKV epilogue kernel launch");
  }
  c->staged = true;
  c->staged_id = block_id;
  c->staged_frames = n_frames;
  return SW_OK;
}

sw_status sw_cache_evict(sw_cache* c) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (c->noisy_due) return fail(SW_ERR_STATE, "the noisy copy of block %lld must be appended first",
                                (long long)c->noisy_entry.block);
  if (c->window.empty()) return fail(SW_ERR_STATE, "window is empty");
  c->free_slots.push_back(c->window.front().phys);
  c->window.pop_front();
  return SW_OK;
}

sw_status sw_rope_relocate(sw_cache* c, sw_rope_policy policy) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (policy != SW_ROPE_S1_RELOCATE && policy != SW_ROPE_RELATIVE_TIME)
    return fail(SW_ERR_INVALID_ARG, "unknown RoPE policy %d", (int)policy);
  c->policy = policy;
  return SW_OK;
}

sw_status sw_tile_mask_budget(const sw_cache* c, float keep_frac, int32_t* k_row) {
  if (!c || !k_row) return fail(SW_ERR_INVALID_ARG, "cache or k_row is NULL");
  if (!(keep_frac >= 0.f && keep_frac <= 1.f)) return fail(SW_ERR_INVALID_ARG, "keep_frac must be in [0, 1]");
  const int n_slots = (int)(c->sinks.size() + c->window.size()) + 1;
  const int n_kv = n_slots * c->L.g.nt;
  const int n_forced = 1 + (c->sinks.empty() ? 0 : 1);
  const int want = (int)std::floor((double)keep_frac * n_kv + 0.5);
  *k_row = std::max(n_forced, std::min(want, n_kv));
  return SW_OK;
}

sw_status sw_build_tile_mask(sw_cache* c, const void* q_raw, sw_step_kind step, float keep_frac,
                             int32_t* tile_idx_out, int32_t k_cap, int32_t* k_row_out) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  if (step != SW_STEP_INTERMEDIATE && step != SW_STEP_FINAL)
    return fail(SW_ERR_INVALID_ARG, "unknown step kind %d", (int)step);
  sw_status st = check_ptr(q_raw, "q_raw");
  if (st == SW_OK) st = check_ptr(tile_idx_out, "tile_idx_out");
  if (st == SW_OK) st = check_ptr(k_row_out, "k_row_out");
  if (st != SW_OK) return st;
  if (!c->cfg.sparse) return fail(SW_ERR_STATE, "cache was created without sparse = 1");
  if (c->dry) return fail(SW_ERR_STATE, "metadata-only cache cannot launch kernels");
  if (!c->staged) return fail(SW_ERR_STATE, "no staged current block");
  if (c->noisy_due) return fail(SW_ERR_STATE, "a noisy append is due");
  if (!all_full(c)) return fail(SW_ERR_UNSUPPORTED, "the tile mask needs full-length blocks");
  int32_t k_row = 0;
  st = sw_tile_mask_budget(c, keep_frac, &k_row);
  if (st != SW_OK) return st;
  if (k_row > k_cap) return fail(SW_ERR_CAPACITY, "k_cap %d < budget %d", k_cap, k_row);
  const std::vector<Entry> hist = history(c);
  const std::vector<int> b = bases_of(c);
  const int n_slots = (int)hist.size() + 1;
  // score the keys this step's attention reads: the noisy history copies on intermediate TwinCache
  // steps, the clean ones otherwise; the current block has one copy
  const bool noisy = c->cfg.twin && step == SW_STEP_INTERMEDIATE;
  const float* pooled[kMaxSlots];
  int deltas[kMaxSlots];
  for (int l = 0; l < n_slots; ++l) {
    pooled[l] = l + 1 < n_slots ? (noisy ? c->pn[hist[l].phys] : c->pc[hist[l].phys]) : c->pc[c->staging];
    deltas[l] = b.back() - b[l];
  }
  const hipError_t e = launch_tile_mask(c->L.g, c->rt, q_raw, pooled, deltas, n_slots, !c->sinks.empty(),
                                        k_row, k_cap, tile_idx_out, c->stream);
  if (e != hipSuccess) return hip_fail(e, "tile mask kernel launch");
  *k_row_out = k_row;
  return SW_OK;
}

sw_status sw_chunk_attend(sw_cache* c, const void* q_raw, sw_step_kind step, const int32_t* tile_idx,
                          int32_t k_row, void* out, float* lse_out) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  return chunk_attend(c, q_raw, step, tile_idx, k_row, out, lse_out, nullptr, nullptr, 0);
}

sw_status sw_cache_inspect(const sw_cache* c, sw_slot_info* out, int32_t cap, int32_t* n) {
  if (!c || !n) return fail(SW_ERR_INVALID_ARG, "cache or n is NULL");
  if (cap > 0 && !out) return fail(SW_ERR_INVALID_ARG, "out is NULL");
  const std::vector<Entry> hist = history(c);
  const std::vector<int> b = bases_of(c);
  const int ns = (int)c->sinks.size();
  const int count = (int)hist.size() + (c->staged ? 1 : 0) + (c->src_staged ? 1 : 0);
  for (int l = 0; l < count && l < cap; ++l) {
    sw_slot_info& s = out[l];
    if (l == (int)hist.size() + 1) {   // source frames of the staged block
      s.role = 3;
      s.block_id = c->staged_id;
      s.physical_slot = -1;
      s.twin_complete = 1;
      s.frames = c->staged_frames;
      s.time_base = b.back();
      continue;
    }
    if (l < (int)hist.size()) {
      s.role = l < ns ? 0 : 1;
      s.block_id = hist[l].block;
      s.physical_slot = hist[l].phys;
      s.twin_complete = (!c->cfg.twin || !(c->noisy_due && c->noisy_entry.phys == hist[l].phys)) ? 1 : 0;
      s.frames = hist[l].frames;
    } else {
      s.role = 2;
      s.block_id = c->staged_id;
      s.physical_slot = c->staging;
      s.twin_complete = 1;
      s.frames = c->staged_frames;
    }
    s.time_base = b[l];
  }
  *n = count;
  return SW_OK;
}

sw_status sw_cache_read_slot(sw_cache* c, int32_t logical_slot, sw_kv_kind kind, void* k_out, void* v_out) {
  if (!c) return fail(SW_ERR_INVALID_ARG, "cache is NULL");
  sw_status st = check_ptr(k_out, "k_out");
  if (st == SW_OK) st = check_ptr(v_out, "v_out");
  if (st != SW_OK) return st;
  if (c->dry) return fail(SW_ERR_STATE, "metadata-only cache holds no data");
  if (c->capturing) return fail(SW_ERR_STATE, "read-back waits for the device: not while capturing a graph");
  const std::vector<Entry> hist = history(c);
  int phys, frames;
  if (kind == SW_KV_SOURCE) {
    if (!c->src_staged) return fail(SW_ERR_STATE, "no staged source frames");
    Geometry g = c->L.g;
    g.B = tokens_of(c, c->staged_frames);
    hipError_t e = launch_unpack(g, c->cfg.dtype == SW_BF16, c->ks, c->vs, k_out, v_out, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(e, "read-back");
    return SW_OK;
  }
  if (kind == SW_KV_CURRENT) {
    if (!c->staged) return fail(SW_ERR_STATE, "no staged current block");
    phys = c->staging;
    frames = c->staged_frames;
  } else {
    if (logical_slot < 0 || logical_slot >= (int)hist.size())
      return fail(SW_ERR_INVALID_ARG, "logical slot %d out of range [0, %d)", logical_slot, (int)hist.size());
    if (kind == SW_KV_NOISY && !c->cfg.twin) return fail(SW_ERR_STATE, "no noisy copies without TwinCache");
    if (kind != SW_KV_CLEAN && kind != SW_KV_NOISY) return fail(SW_ERR_INVALID_ARG, "unknown kv kind");
    phys = hist[logical_slot].phys;
    frames = hist[logical_slot].frames;
  }
  const bool noisy = kind == SW_KV_NOISY;
  Geometry g = c->L.g;
  g.B = tokens_of(c, frames);
  hipError_t e = c->cfg.dtype == SW_FP8
                    ? launch_unpack_fp8(g, noisy ? c->kn[phys] : c->kc[phys], noisy ? c->vn[phys] : c->vc[phys], k_out,
                                        v_out, c->stream)
                    : launch_unpack(g, c->cfg.dtype == SW_BF16, noisy ? c->kn[phys] : c->kc[phys],
                               noisy ? c->vn[phys] : c->vc[phys], k_out, v_out, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(e, "read-back");
  return SW_OK;
}

}  // extern "C"
