// Internal interface between the host library (host.cpp) and the HIP kernels.
// Not part of the public ABI (include/swattn.h is).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace swattn {

constexpr int kMaxSlots = 16;     // S + W + 1
constexpr int kTile = 128;        // block-sparse tile edge, query-tile rows
constexpr int kMaxKeyTiles = 4096;

// fp32 (cos, sin) of one RoPE angle, side by side so that one 8-byte load fetches both.
struct __attribute__((aligned(8))) CosSin {
  float c, s;
};

// cos/sin tables (computed on the host in fp64, stored fp32) for the three RoPE axes, back to
// back in one allocation (h and w follow t): time: [t_len][pt], height: [lat_h][ph], width:
// [lat_w][pw].
struct RopeTab {
  const CosSin* t;
  const CosSin* h;
  const CosSin* w;
  int pt, ph, pw, t_len;
};

struct Geometry {
  int B, H, d, F, lat_h, lat_w;
  int n_pad;   // B rounded up to a multiple of 128
  int nt;      // ceil(B / 128)
};

struct SlotPtrs {
  const void* k;   // rotated K, [H][n_pad][d]
  const void* v;   // bf16: V^T [H][n_pad/128][d][128] (keys permuted in groups of 16); fp32: V [H][n_pad][d]
  int delta;       // time base of the current block minus this slot's
  int count;       // tokens of the slot's block (<= n_pad)
  int aligned;     // 1: frame-aligned (editing source) -- key j is seen only by the queries of its
                   // frame, j / (lat_h * lat_w); must be the last slot
};

// K1: rotate K at block-local positions, store K and V head-major, pad rows zeroed,
// optional per-tile fp32 means of rotated K ([H][d][nt]).
hipError_t launch_append(const Geometry& g, const RopeTab& rt, bool bf16, const void* k_raw,
                         const void* v_raw, void* k_dst, void* v_dst, float* pooled_dst,
                         hipStream_t stream);

// K1 with the QKV epilogue: qkv [B][3][H][d] (q, k, v of a token side by side); q and k are
// RMS-normalised per head over d with weights gamma_q / gamma_k (fp32 [d]); q goes to q_out
// [B][H][d], k (then rotated) and v to the slot as in launch_append.  d = 128 only.
hipError_t launch_append_qkv(const Geometry& g, const RopeTab& rt, bool bf16, const void* qkv,
                             const float* gamma_q, const float* gamma_k, float eps, void* q_out,
                             void* k_dst, void* v_dst, float* pooled_dst, hipStream_t stream);

// Work split of the dense bf16 attention grid: the device's CU count sets how many
// workgroups are resident at once; the workspace holds max_rows partial query rows.
struct SplitPlan {
  int cus;
  int max_rows;
  float* part_o;     // [max_rows][d]
  float* part_lse;   // [max_rows]
};
constexpr int kSplitRows = 1024 * 256;   // 1024 pieces of a 256-query tile

// K2 / K3: chunk attention over the given slots (logical order); tile_idx == nullptr -> dense.
// g.B is the query count (the current block); the keys of slot l are its slots[l].count tokens
// (block-sparse: every slot holds g.B tokens).
hipError_t launch_attend(const Geometry& g, const RopeTab& rt, bool bf16, const void* q,
                         const SlotPtrs* slots, int n_slots, const int32_t* tile_idx, int k_row,
                         void* out, float* lse, const SplitPlan& plan, hipStream_t stream);

// Rows of the split workspace the dense bf16 (fp8 = false) or fp8 attention launch over these
// slots uses under `plan` (0 when no tile is split).
int split_rows(const Geometry& g, bool fp8, const SlotPtrs* slots, int n_slots, const SplitPlan& plan);

// fp8 caches (d = 128): K1 quantising K (after block-local RoPE) and V to E4M3 with power-of-two
// scales per 32 values (layout: append_fp8.hip); the fp8 attention (dense, bf16 queries and
// output); the read-back, dequantised to fp32 [B][H][d].
hipError_t launch_append_fp8(const Geometry& g, const RopeTab& rt, const void* k_raw, const void* v_raw, void* k_dst,
                             void* v_dst, hipStream_t stream);
hipError_t launch_attend_fp8(const Geometry& g, const RopeTab& rt, const void* q, const SlotPtrs* slots, int n_slots,
                             void* out, float* lse, const SplitPlan& plan, hipStream_t stream);
hipError_t launch_unpack_fp8(const Geometry& g, const void* k_src, const void* v_src, void* k_out, void* v_out,
                             hipStream_t stream);

// K4: block-sparse tile mask (bf16, d = 128).
hipError_t launch_tile_mask(const Geometry& g, const RopeTab& rt, const void* q,
                            const float* const* pooled, const int* deltas, int n_slots,
                            bool has_sink, int k_row, int k_cap, int32_t* out, hipStream_t stream);

// Read-back: cache layout -> token-major [B][H][d].
hipError_t launch_unpack(const Geometry& g, bool bf16, const void* k_src, const void* v_src,
                         void* k_out, void* v_out, hipStream_t stream);

}  // namespace swattn

// Host-library internals used by the allocation-free attention entry point (host.cpp).
struct sw_cache;
namespace swhost {
// The device the cache was created on.
int cache_device(const sw_cache* c);
// sw_chunk_attend with the split workspace at (part_o [max_rows][128], part_lse [max_rows])
// instead of the cache pool's: the same work split as sw_chunk_attend, and SW_ERR_CAPACITY when
// it needs more than max_rows rows.  Returns an sw_status.
int chunk_attend_scratch(sw_cache* c, const void* q_raw, int step, const int32_t* tile_idx, int32_t k_row, void* out,
                         float* lse_out, float* part_o, float* part_lse, int max_rows);
// Record a failed HIP call as the thread's last error; returns SW_ERR_HIP.
int hip_error(hipError_t e, const char* what);
}  // namespace swhost
