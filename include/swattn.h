/*
 * swattn.h -- C ABI of the streaming block-causal chunk-attention library
 * (libswattn.so, HIP kernels for AMD gfx950 / MI355X).
 *
 * The method (sources cited by page title and section):
 *  - Video is generated block by block in time order; a block sees only earlier
 *    content, and a denoising step of the current block attends to the cached
 *    history plus itself ("Vidu S2 vs PixVerse R2" blog, orkas.ai, section
 *    "What real-time changes"; Vidu S2 paper read, yingwang.github.io,
 *    section 2.2 on block-wise causal attention).
 *  - The history is bounded: the first blocks stay as permanent sinks, a
 *    sliding window keeps the most recent blocks, the rest is dropped; RoPE
 *    positions are relocated (S1) or made relative in time (R2) so they stay
 *    inside the trained range (blog, section "Choice 3: bounded memory").
 *  - TwinCache: each history block is kept as a noisy and a clean copy;
 *    intermediate denoising steps read the noisy copy, the final step the clean
 *    one (blog, section "Choice 3: bounded memory").
 *  - Block-sparse attention skips most key tiles (blog, section "Choice 4: where
 *    the speed comes from", >90% sparsity).
 *
 * Conventions for every call
 *  - Tensor arguments are DEVICE pointers (hipMalloc'd or torch CUDA storage),
 *    contiguous, owned by the caller, and must stay alive until the work
 *    enqueued on the cache's stream has finished.
 *  - Raw Q/K/V of a block are token-major [B][H][d]: token index in
 *    (frame, row, column) row-major order, B = frames * lat_h * lat_w, in the
 *    cache dtype (bf16 stored as raw 16-bit patterns, or fp32).
 *  - GPU work is enqueued asynchronously on the stream given at create; cache
 *    metadata (which block sits where, time bases) is updated synchronously on
 *    the host.  No call blocks on the GPU except create and read-back calls.
 *  - Every call validates its arguments and the cache state before enqueuing
 *    anything; on error it returns a status != SW_OK, leaves the cache state
 *    unchanged and sets a thread-local message readable by sw_last_error().
 *  - A handle is not thread-safe; use one handle per thread or serialise.
 *  - No call allocates device memory: the caller passes one device pool of
 *    sw_cache_required_bytes() bytes at create, which the library carves.
 *  - A handle created with device_pool == NULL and pool_bytes == 0 is
 *    metadata-only: append / evict / relocate / inspect behave as usual but
 *    touch no device (any pointers passed are only checked for NULL); calls that
 *    would launch a kernel return SW_ERR_STATE.  It lets hosts without a GPU
 *    test the cache bookkeeping.
 */
#ifndef SWATTN_H
#define SWATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sw_cache sw_cache; /* opaque, library-owned host handle */

typedef enum {
  SW_OK = 0,
  SW_ERR_INVALID_ARG = 1, /* NULL pointer, out-of-range value */
  SW_ERR_SHAPE = 2,       /* configuration the kernels do not support in size */
  SW_ERR_STATE = 3,       /* call not allowed in the current cache state */
  SW_ERR_CAPACITY = 4,    /* pool too small, window full, mask buffer too small */
  SW_ERR_UNSUPPORTED = 5, /* dtype / head_dim / variant combination not built */
  SW_ERR_HIP = 6          /* a HIP runtime call failed (message has the HIP error) */
} sw_status;

/* Storage and arithmetic of a cache.  SW_BF16 / SW_F32: inputs, stored K/V and
 * outputs in that type.  SW_FP8: bf16 inputs and outputs; K (after RoPE) and V
 * stored as OCP FP8 E4M3 with a power-of-two scale per 32 values, and the
 * attention multiplies in fp8 on the MFMA units (quantised attention chosen per
 * layer: Vidu S2 paper read, section 2.4); head_dim 128, dense stream only (no
 * block-sparse, no editing, no QKV epilogue); sw_cache_read_slot returns the
 * dequantised values as fp32. */
typedef enum { SW_BF16 = 0, SW_F32 = 1, SW_FP8 = 2 } sw_dtype;

/* What an append writes.
 *  SW_KV_CURRENT: the current (not yet committed) block's K/V for this
 *                 denoising step; overwrites the staged current block.
 *  SW_KV_CLEAN:   commit a block to the history.  With k_raw == v_raw == NULL
 *                 the staged current block is promoted (no bytes move); with
 *                 pointers, those raw K/V are written as the committed block
 *                 (used to rebuild a cache, e.g. on resume).
 *  SW_KV_NOISY:   (TwinCache only) the noisy copy of the block just committed.
 *  SW_KV_SOURCE:  (editing caches only) the source-video frames of the staged
 *                 block: block_id and n_frames must be those of the staged
 *                 current block.  Written into one staging buffer outside the
 *                 ring; the commit of the block drops it (source frames never
 *                 enter the history).  Frame-aligned editing attention: Vidu S2
 *                 paper read, section 2.6 (the editing model). */
typedef enum { SW_KV_CURRENT = 0, SW_KV_CLEAN = 1, SW_KV_NOISY = 2, SW_KV_SOURCE = 3 } sw_kv_kind;

/* Which TwinCache copy of the history a denoising step reads (blog, "Choice 3"):
 * intermediate steps read the noisy copies, the final step the clean ones.
 * Without TwinCache both read the single (clean) copy. */
typedef enum { SW_STEP_INTERMEDIATE = 0, SW_STEP_FINAL = 1 } sw_step_kind;

/* Time base of logical slot l of the materialised sequence
 * [sinks..., window oldest->newest..., current], F = frames per block:
 *  SW_ROPE_S1_RELOCATE:   base_l = l * F.
 *  SW_ROPE_RELATIVE_TIME: window j -> j * F, current -> n_window_used * F,
 *                         sink i -> (i - n_sinks_used) * F.
 * Both keep every position inside [-S*F, (S+W+1)*F) however long the stream
 * runs (blog, "Choice 3": S1 RoPE relocation, R2 relative-time RoPE). */
typedef enum { SW_ROPE_S1_RELOCATE = 0, SW_ROPE_RELATIVE_TIME = 1 } sw_rope_policy;

typedef struct {
  int32_t n_heads;          /* 1 <= H <= 65535 */
  int32_t head_dim;         /* d: 128 (bf16 or fp32) or 64 (fp32) */
  int32_t frames_per_block; /* F >= 1; the cap when blocks carry their own frame count */
  int32_t lat_h, lat_w;     /* latent grid of a frame; B = F*lat_h*lat_w <= 65536 */
  int32_t n_sink;           /* S >= 0 */
  int32_t n_window;         /* W >= 0; S + W + 1 <= 16 */
  int32_t twin;             /* 0 | 1: keep noisy + clean copies of history blocks */
  int32_t sparse;           /* 0 | 1: keep pooled key-tile means for sw_build_tile_mask (bf16 only) */
  sw_dtype dtype;           /* storage and input dtype */
  double rope_theta;        /* RoPE base, > 1 (10000 is the usual value) */
  int32_t rope_pairs_t;     /* rotation pairs of the time, height and width axes; all three 0 =  */
  int32_t rope_pairs_h;     /* the default split (see the RoPE layout below); otherwise each >= 0 */
  int32_t rope_pairs_w;     /* and t + h + w = head_dim / 2 (SW_ERR_INVALID_ARG), t <= 24 for bf16
                               and fp8 caches (SW_ERR_UNSUPPORTED: their attention re-rotates only
                               the first 48 dims of a query when it enters a slot) */
  sw_rope_policy policy;    /* initial relocation policy */
  int32_t tile;             /* block-sparse tile edge; must be 128 */
  int32_t editing;          /* 0 | 1: frame-aligned editing (a source staging buffer; dense only;
                               S + W + 2 <= 16) */
} sw_cache_config;

/* RoPE layout (pages name 3D RoPE over (t, h, w) without details -- Vidu S2
 * paper read, abbreviation table): P = d/2 pairs, pair p rotates dims
 * (2p, 2p+1); the first P_t pairs turn with time, the next P_h with the row,
 * the last P_w with the column.  Default split (rope_pairs_* all 0): P_h = P_w
 * = floor(P/3), P_t = P - 2*floor(P/3).  Inside an axis with P_a pairs, pair j
 * turns by pos * theta^(-j/P_a). */

typedef struct {
  int32_t role;          /* 0 sink, 1 window, 2 current, 3 source (editing) */
  int64_t block_id;
  int32_t physical_slot; /* ring slot holding the block (changes with eviction) */
  int32_t time_base;     /* RoPE time of the block's first frame */
  int32_t twin_complete; /* 1 if the noisy copy exists (always 1 without TwinCache) */
  int32_t frames;        /* latent frames of the block (<= frames_per_block) */
} sw_slot_info;

/* Thread-local message of the last failed call ("" if none). */
const char* sw_last_error(void);

/* Device bytes the cache needs for `cfg` (K/V slots, twin copies, pooled
 * key means, RoPE tables).  Host-only; no device call. */
sw_status sw_cache_required_bytes(const sw_cache_config* cfg, size_t* bytes);

/* Create a cache in `device_pool` (pool_bytes >= required, 256-byte aligned).
 * hip_stream: a hipStream_t (NULL = the default stream).  Uploads the RoPE
 * tables (a blocking copy) and zeroes the pool.  *out receives the handle. */
sw_status sw_cache_create(const sw_cache_config* cfg, void* device_pool, size_t pool_bytes,
                          void* hip_stream, sw_cache** out);

/* Free the host handle.  The caller frees the pool after the stream drains. */
sw_status sw_cache_destroy(sw_cache* c);

/* Append a block's raw K/V [B][H][d] (see sw_kv_kind).  The kernel rotates K
 * at block-local positions (t = frame, h, w), stores V, both head-major, and
 * (sparse caches) the per-128-token-tile means of the rotated K.
 * Rules: block ids of commits strictly increase; CURRENT may be re-appended
 * each step with the same id; CLEAN into a full window returns
 * SW_ERR_CAPACITY (evict first); with TwinCache the call after a CLEAN must be
 * the NOISY append of the same block id (else SW_ERR_STATE). */
sw_status sw_cache_append_block(sw_cache* c, sw_kv_kind kind, const void* k_raw,
                                const void* v_raw, int64_t block_id);

/* sw_cache_append_block for a block of n_frames latent frames, 1 <= n_frames
 * <= frames_per_block: K/V are [n_frames*lat_h*lat_w][H][d].  In R2 the length
 * of a block follows the active control signal up to a cap ("Vidu S2 vs
 * PixVerse R2" blog, section "Choice 5: how people control it").  The slots
 * keep their capped size; a block's time base is where the previous slot of
 * [sinks, window, current] ends (relative time: the window starts at 0, the
 * sinks sit just before it).  The queries and output of sw_chunk_attend then
 * have the staged block's length.  Re-appending CURRENT must keep the staged
 * length; CLEAN with NULL pointers commits the staged length; NOISY must match
 * the committed block.  SW_ERR_INVALID_ARG for n_frames out of range,
 * SW_ERR_UNSUPPORTED for a block shorter than the cap in a sparse cache. */
sw_status sw_cache_append_block_frames(sw_cache* c, sw_kv_kind kind, const void* k_raw,
                                       const void* v_raw, int64_t block_id, int32_t n_frames);

/* Stage the current block from the packed output of a QKV projection, with the
 * per-head RMSNorm of q and k fused into the append (Vidu S2 paper read,
 * section 2.4: adjacent operators such as RMSNorm and elementwise work fused
 * into one kernel).  qkv_raw [B][3][H][d] in the cache dtype (q, k, v of a
 * token side by side, B = n_frames*lat_h*lat_w); gamma_q, gamma_k device fp32
 * [d]; for every token and head x -> x / sqrt(mean_d(x^2) + eps) * gamma.  The
 * normalised q is written to q_out [B][H][d] (cache dtype, un-rotated: pass it
 * to sw_chunk_attend); the normalised k, rotated at block-local positions, and
 * v become the staged current block exactly as SW_KV_CURRENT stages raw K/V.
 * Same staging rules as SW_KV_CURRENT; SW_ERR_UNSUPPORTED unless head_dim is
 * 128; SW_ERR_INVALID_ARG for NULL pointers, eps < 0 or n_frames out of
 * range.  One kernel, one pass over HBM. */
sw_status sw_cache_append_qkv(sw_cache* c, const void* qkv_raw, const float* gamma_q, const float* gamma_k,
                              float eps, void* q_out, int64_t block_id, int32_t n_frames);

/* Drop the oldest window block (index remap, no bytes move).  Sinks are never
 * evicted.  SW_ERR_STATE if the window is empty or a NOISY append is due. */
sw_status sw_cache_evict(sw_cache* c);

/* Select the RoPE relocation policy and recompute the per-slot time bases
 * (also recomputed after every commit and evict).  O(S+W+1) host work. */
sw_status sw_rope_relocate(sw_cache* c, sw_rope_policy policy);

/* Number of kept key tiles per query-tile row for keep fraction `keep_frac`
 * in the current state: max(#forced, floor(keep_frac * n_key_tiles + 0.5)),
 * n_key_tiles = (#logical slots) * ceil(B/128). */
sw_status sw_tile_mask_budget(const sw_cache* c, float keep_frac, int32_t* k_row);

/* Build the block-sparse tile mask from the raw queries q_raw [B][H][d] of this
 * step (every cached block at the full frames_per_block length): per head and
 * 128-query tile, score every key tile by the dot product of
 * mean relocated rotated query and key vectors / sqrt(d), keep key tile 0 of
 * the first sink (if any) and the diagonal current tile, fill up to the budget
 * with the highest scores (ties -> lower index).  The keys scored are the ones
 * the attention of the same step reads: with TwinCache the noisy copies for
 * SW_STEP_INTERMEDIATE, the clean ones for SW_STEP_FINAL (blog, "Choice 3").
 * Writes ascending linear key tile indices (slot * ceil(B/128) + tile) to
 * tile_idx_out [H][ceil(B/128)][k_cap] (device int32); when k_cap exceeds the
 * budget the rest of each row is -1; *k_row_out (host) = budget.  Needs a
 * sparse bf16 cache with a staged current block; SW_ERR_CAPACITY if k_cap <
 * budget. */
sw_status sw_build_tile_mask(sw_cache* c, const void* q_raw, sw_step_kind step, float keep_frac,
                             int32_t* tile_idx_out, int32_t k_cap, int32_t* k_row_out);

/* One denoising step's chunk attention for the staged current block:
 *   out[n][h] = softmax_k(<R(p_n) q_n, R(p_k) k> / sqrt(d)) V
 * over keys [sinks, window oldest->newest, current], positions relocated by
 * the current policy.  Editing caches with a staged source block add, for a
 * query of frame f, the source tokens of frame f only, at the current block's
 * positions (the source frame of an instant has the target frame's (t, h, w);
 * Vidu S2 paper read, section 2.6; BloomBook Vidu S2 tutorial, section
 * "S2-Editing").  The reference image is the first committed block, a sink.  q_raw [B][H][d] raw (un-rotated) queries (B = tokens of
 * the staged block, see sw_cache_append_block_frames); out [B][H][d]
 * in the cache dtype; lse_out (nullable) [H][B] fp32 natural-log sum of
 * exp(score) per query.  tile_idx == NULL: dense; otherwise block-sparse over
 * the key tiles listed in tile_idx [H][ceil(B/128)][k_row] (as written by
 * sw_build_tile_mask).  A row is read in order and each key tile counts at
 * most once: an entry outside [0, n_key_tiles) (such as the -1 padding of a
 * mask built with k_cap > budget: pass k_row = k_cap for such a list) or not
 * above the last entry taken from its row (a repeat, or an entry out of
 * ascending order) is skipped.  step selects the TwinCache copy. */
sw_status sw_chunk_attend(sw_cache* c, const void* q_raw, sw_step_kind step,
                          const int32_t* tile_idx, int32_t k_row, void* out, float* lse_out);

/* sw_chunk_attend for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, same work split and the same result bit for bit; the only scratch
 * memory of the attention -- the partial outputs and sum-exps of the query tiles
 * the dense launch cuts into key ranges -- lives in a static device array of the
 * library instead of the cache pool's workspace: 65536 rows of 128 + 1 floats
 * (33.8 MB) per GPU, held by each GPU the library runs on until the process
 * ends.  Allocates nothing; the first call on a device looks the array up
 * (hipGetSymbolAddress) once.  The array needs no clearing (every partial row is
 * written before the merge reads it).  Every call on one GPU shares the array,
 * which keeps the last call's contents: calls that overlap on one GPU (several
 * streams or threads) race.  SW_ERR_CAPACITY, with a message, when the call's
 * split needs more rows than the array holds (fewer query tiles than the device
 * has compute units, e.g. 1-frame 540p blocks: use sw_chunk_attend); every other
 * error as sw_chunk_attend. */
sw_status sw_chunk_attend_noalloc(sw_cache* c, const void* q_raw, sw_step_kind step,
                                  const int32_t* tile_idx, int32_t k_row, void* out, float* lse_out);

/* Logical slots in attention order (sinks, window oldest->newest, staged
 * current).  Writes min(cap, count) entries; *n = count. Host-only. */
sw_status sw_cache_inspect(const sw_cache* c, sw_slot_info* out, int32_t cap, int32_t* n);

/* Copy logical slot `logical_slot`'s stored K (rotated at block-local
 * positions) and V back out as token-major [B][H][d] device arrays (cache
 * dtype).  kind: SW_KV_CLEAN or SW_KV_NOISY (history) / SW_KV_CURRENT (the
 * staged block) / SW_KV_SOURCE (the staged source frames; logical_slot is
 * ignored for these two).  For tests and debugging; blocks until copied. */
sw_status sw_cache_read_slot(sw_cache* c, int32_t logical_slot, sw_kv_kind kind, void* k_out,
                             void* v_out);

/* ---- graph replay of a chunk's launches -------------------------------------
 * The pages' stack replays fused kernels with graphs (Vidu S2 paper read, section
 * 2.4; "Vidu S2 vs PixVerse R2" blog, section "Choice 4: where the speed comes
 * from").  sw_graph_begin starts capturing the cache's stream (thread-local
 * capture mode); the append, tile-mask and attention calls that follow are
 * recorded, not run, while their host bookkeeping (commit, evict, time bases)
 * takes effect at once; sw_graph_end instantiates the recording.  A replay
 * reruns the recorded kernels with the recorded arguments: the same input and
 * output addresses, ring slots and time bases.  In steady state (full window,
 * full-length blocks) the ring layout repeats every n_window + 1 chunks, so the
 * graphs of n_window + 1 consecutive chunks, replayed in turn, continue the
 * stream; the host's block ids do not advance during replays.  Calls that wait
 * for the device (sw_cache_create, sw_cache_read_slot) fail while capturing.
 * No memory is allocated or cleared inside a recording. */
typedef struct sw_graph sw_graph; /* opaque, library-owned */

/* Start capturing the cache's stream.  SW_ERR_STATE if already capturing or
 * metadata-only; SW_ERR_HIP if the stream cannot be captured (e.g. the NULL
 * stream). */
sw_status sw_graph_begin(sw_cache* c);

/* End the capture begun by sw_graph_begin and instantiate it into *out. */
sw_status sw_graph_end(sw_cache* c, sw_graph** out);

/* Replay a graph on hip_stream (a hipStream_t; NULL = the stream it was
 * captured from).  Asynchronous, like the calls it recorded. */
sw_status sw_graph_launch(sw_graph* g, void* hip_stream);

/* Free a graph (after the replays that use it have completed). */
sw_status sw_graph_destroy(sw_graph* g);

/* Chunks after which the ring layout repeats in steady state (n_window + 1). */
sw_status sw_cache_ring_period(const sw_cache* c, int32_t* period);

/* ---- measurement aid (not a step of the method) ------------------------------
 * The sustained matrix-core rate of the device, for reporting attention throughput
 * against a measured peak beside the datasheet one.  Enqueues on hip_stream one launch
 * of 8 waves per compute unit, each running four independent chains of `iters` MFMAs
 * with operands in registers: v_mfma_f32_32x32x16_bf16 (dtype SW_BF16) or
 * v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands (SW_FP8).  sink: device buffer of
 * sink_floats >= 8 * (compute units) floats the waves write one value each into
 * (keeps the chains live).  *flops_out (host) = the launch's flops, for the caller to
 * divide by its measured duration.  SW_ERR_INVALID_ARG for NULL pointers, iters < 1 or
 * another dtype; SW_ERR_CAPACITY for a short sink; SW_ERR_HIP if the launch fails.
 * Sets no error message. */
sw_status sw_probe_mfma(void* hip_stream, sw_dtype dtype, int32_t iters, float* sink, int32_t sink_floats,
                        double* flops_out);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H */
