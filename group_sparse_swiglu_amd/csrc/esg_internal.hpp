// Host-side declarations shared by the esg translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace esg {

// Kernel timing: when enabled, brackets a launch with events on its stream.
struct LaunchTimer {
  LaunchTimer(const char* name, hipStream_t stream);
  ~LaunchTimer();
  const char* name_;
  hipStream_t stream_;
  void* start_;
};
bool timing_enabled();

// ---- selection -------------------------------------------------------------
// energy_ws: NULL, or an fp32 [tokens, groups] table (select_energy_bytes) that
// lets batches with fewer 32-token blocks than CUs split the groups over
// workgroups (same result).
size_t select_energy_bytes(int tokens, int groups);
hipError_t launch_select(int dtype, const void* x, const void* w_gate, int tokens, int d_model,
                         int groups, int k, const int32_t* sub, int rows_per_group, int group_size,
                         const float* bias, int32_t* idx_out, int32_t* counts_out, float* energy_ws,
                         hipStream_t stream);

// ---- bucketing ---------------------------------------------------------------
// Bucketing of (token, slot) pairs by group.  Tiles of `tile_rows` padded
// positions are laid out group after group; see esg_bucket.hip.
struct BucketOut {
  int32_t* offsets;     // [G+1] or NULL
  int32_t* perm_token;  // [T*k] (unpadded positions) or NULL
  int32_t* inv;         // [T*k] unpadded positions or NULL
  int32_t* tile_off;    // [G+1] prefix sums of tile counts, or NULL
  int32_t* tile_group;  // [max_tiles] group of each tile (-1 = unused) or NULL
  int32_t* ptoken;      // [max_tiles*tile_rows] token of each padded row (-1 = pad) or NULL
  int32_t* pinv;        // [T*k] padded position of each pair (-1 = skipped) or NULL
  int32_t* status;      // device status word or NULL
};
size_t bucket_scratch_bytes(int tokens, int groups);
// tile_pad: each group's positions are padded to a multiple of tile_pad (a
// multiple of tile_rows), so its tile count is a multiple of tile_pad/tile_rows
int max_tiles(int tokens, int k, int groups, int tile_rows, int tile_pad);
hipError_t launch_bucket(const int32_t* idx, int tokens, int k, int groups, int tile_rows,
                         const BucketOut& out, void* scratch, hipStream_t stream, int tile_pad = 0);

// ---- FFN ----------------------------------------------------------------------
struct FfnShape {
  int dtype, tokens, d_model, d_ff, group_size, k;
  int groups() const { return d_ff / group_size; }
  // neurons per kernel block: 128 for bf16, 64 for fp32 (LDS capacity); bf16
  // launches of fewer than 128 tiles of 128 neurons (decode-sized batches) take
  // 64-neuron blocks instead, which doubles their workgroups
  int gsb() const {
    const int cap = dtype == 0 ? 64 : 128;
    if (group_size < cap) return group_size;
    if (dtype == 1) {
      const long long tiles = ((long long)tokens * k + (long long)groups() * 127) / 128;
      if (tiles * (group_size / 128) < 128) return 64;
    }
    return cap;
  }
  int nsub() const { return group_size / gsb(); }                    // sub-blocks per group
  int elem_bytes() const { return dtype == 0 ? 4 : 2; }
};
constexpr int kTileRows = 128;  // bucket positions per grouped-GEMM tile
constexpr int kNominalCUs = 256;  // MI355X (see compute_units)
// Large bf16 launches with 128-neuron blocks run the forward and the dh + dx
// tiles on pairs of tiles of one group, so their training layouts pad groups
// to 2 * kTileRows positions.  "Large": at least kPairMinTiles single tiles
// (by the single-tile bound), i.e. at least four rounds of pair workgroups on
// the nominal CUs; with fewer, the coarser pair grid loses more to its last
// round than the pairs save (the 370M shape's 660 tiles: 330 pairs, 1.3
// rounds).
constexpr long long kPairMinTiles = 8ll * kNominalCUs;
inline int tile_pad(const FfnShape& s) {
  if (s.dtype != 1 || s.gsb() != 128) return kTileRows;
  const long long tiles = ((long long)s.tokens * s.k + (long long)s.groups() * (kTileRows - 1)) / kTileRows;
  return tiles * s.nsub() >= kPairMinTiles ? 2 * kTileRows : kTileRows;
}
// scratch of a routed forward with saved = NULL (no pair padding: at most the
// fwd_scratch_bytes that esg_sparse_swiglu_workspace_size reports)
size_t inference_fwd_scratch_bytes(const FfnShape& s);

// Compact per-position activations [nsub][rows/EPC][gsb][EPC]
hipError_t launch_fwd_grouped(const FfnShape& s, const void* x, const void* wg, const void* wu,
                              const void* wd, const int32_t* tile_group, const int32_t* ptoken,
                              int ntiles_max, void* hg_saved, void* hu_saved, void* partials,
                              hipStream_t stream);
hipError_t launch_rowsum(const FfnShape& s, const void* partials, size_t sub_stride_rows,
                         const int32_t* pinv, void* out, hipStream_t stream);
hipError_t launch_bwd_dh_dx(const FfnShape& s, const void* dy, const void* wg, const void* wu,
                            const void* wd, const int32_t* tile_group, const int32_t* ptoken,
                            int ntiles_max, const void* hg_saved, const void* hu_saved, void* dg,
                            void* du, void* act, void* partials, hipStream_t stream);
hipError_t launch_bwd_dw(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off,
                         const int32_t* ptoken, int rows_total, const void* dg, const void* du,
                         const void* act, void* dwg, void* dwu, void* dwd, hipStream_t stream);

// Pipelined bf16 path (group blocks of 64 or 128 neurons, buffers < 2 GiB).
// Its saved activations are row-major [sub][pos][gsb]; the generic path above
// uses [sub][pos/EPC][gsb][EPC].  Forward and backward pick the same path.
bool bf16_pipelined(const FfnShape& s, int ntiles_max);
// The bf16 forward as two launches (phase 1 over up to kFwdSplitK K ranges;
// phase 2 over d-block ranges) when the tiles of 64-neuron blocks number at
// most kFwdSplitTiles: the one-launch kernel would leave most CUs idle.  A
// shape rule (no device query), so the forward scratch holds the fp32 [hg; hu]
// partials, fwd_split_bytes, exactly when needed.
constexpr int kFwdSplitTiles = 128;
constexpr int kFwdSplitK = 4;
bool fwd_split(const FfnShape& s, int ntiles_max);
inline size_t fwd_split_bytes(const FfnShape& s, int ntiles_max) {
  return fwd_split(s, ntiles_max) ? (size_t)s.nsub() * ntiles_max * kFwdSplitK * kTileRows * 2 * s.gsb() * 4 : 0;
}
// act: the fwd_split_bytes partials for fwd_split shapes (ignored otherwise);
// pad: the bucket pad of the layout (2 * kTileRows: groups padded to tile pairs)
hipError_t launch_fwd2(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                       const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, int pad, void* hg_saved,
                       void* hu_saved, void* partials, void* act, hipStream_t stream);
hipError_t launch_dhdx2(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                        const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg_saved,
                        const void* hu_saved, void* dg, void* du, void* act, void* partials, hipStream_t stream);
// cht, slots: 128-neuron blocks cut a group's positions into chunks of cht
// tiles when its bucket holds more (0: never; dw_chunk_tiles), summing the
// chunks in fp32 slots of dw_slot_bytes (then added in chunk order)
hipError_t launch_dw2(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off, const int32_t* ptoken,
                      int rows_total, const void* dg, const void* du, const void* act, void* dwg, void* dwu, void* dwd,
                      int cht, void* slots, hipStream_t stream);
int dw_chunk_tiles(const FfnShape& s, int ntiles_max, int pad);
size_t dw_slot_bytes(const FfnShape& s, size_t rows, int cht);

// ---- dense limit (all groups active) ----------------------------------------------
constexpr int kDenseChunkTokens = 8192;  // backward token chunk (recompute workspace)
struct DenseBwdLayout {
  int tc = 0, chunks = 0, nblk = 0;      // chunk tokens (padded to 128), chunk count, 128-neuron blocks
  size_t ptoken = 0, dg = 0, du = 0, act = 0, fg = 0, fu = 0, fd = 0, bytes = 0;
};
DenseBwdLayout dense_bwd_layout(int tokens, int d_model, int d_ff);
bool dense_supported(const FfnShape& s);
hipError_t launch_dense_fwd(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd, void* y,
                            hipStream_t stream);
hipError_t launch_dense_bwd(const FfnShape& s, const void* dy, const void* x, const void* wg, const void* wu,
                            const void* wd, void* dx, void* dwg, void* dwu, void* dwd, void* scratch,
                            hipStream_t stream);

// ---- bias update / fills -------------------------------------------------------
hipError_t launch_bias_update(float* bias, float* ema, const float* freq, const int32_t* counts,
                              const int32_t* offsets, int tokens, float target, float gamma, float bias_max,
                              float momentum, int groups, hipStream_t stream);
hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t stream);
// bf16 matrix-core rate probe: blocks x 256 threads, 8 * 16*16*32 * 2 FLOPs
// per wave and iteration; out holds blocks * 256 floats
hipError_t launch_mfma_probe(int blocks, int iters, float* out, hipStream_t stream);

// ---- LeakyReLU(0.5)^2 MLP (esg_mlp.hip), bf16 ------------------------------------
size_t mlp_partial_bytes(int tokens, int d_model, int d_ff);
// bf16 buffers as void pointers (the bf16 type lives with the device code)
hipError_t launch_mlp_fwd(const void* x, const void* w_up, const void* w_down, int tokens, int d, int F, void* y,
                          void* post, void* act_grad, hipStream_t stream);
hipError_t launch_mlp_bwd(const void* dy, const void* x, const void* w_up, const void* w_down, int tokens, int d,
                          int F, const void* post, const void* act_grad, void* dx, void* dw_up, void* dw_down,
                          void* dpre, float* part, hipStream_t stream);

// ---- FlashFFN multi-head sub-network core (esg_mhffn.hip), bf16 ----------------
bool mhffn_supported(int tokens, int heads, int d_head, int subnets, int d_sub);
hipError_t launch_mhffn_fwd(const void* q, const float* r, const void* k, const void* u, const void* v, int tokens,
                            int heads, int subnets, int d_sub, void* out, hipStream_t stream);
hipError_t launch_mhffn_bwd(const void* dout, const void* q, const float* r, const void* k, const void* u,
                            const void* v, int tokens, int heads, int subnets, int d_sub, void* dq, float* dr,
                            void* dk, void* du, void* dv, hipStream_t stream);

// ---- sigmoid top-k routing (esg_route.hip) ------------------------------------
constexpr int kRouteMaxExperts = 2048;  // 32 experts per lane of one wavefront
constexpr int kRouteMaxK = 32;
bool sigmoid_topk_supported(int num_experts, int topk);
hipError_t launch_sigmoid_topk(const float* logits, const float* bias, int bias_stride, int tokens, int E, int k,
                               float scaling, int apply_scaling, float* probs, int64_t* indices,
                               hipStream_t stream);

// Compute units of the current device (cached per device): for launch sizes
// that do not change results.  Rules that decide how a sum is split (and so
// its rounding) or how buffers are laid out use kNominalCUs instead, so a
// shape rounds the same way on every device and partition mode.
int compute_units();

}  // namespace esg
