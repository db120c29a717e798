// The C ABI (include/esg.h): argument validation, workspace layout and the
// launch sequence of each entry point.  No device memory is allocated here.
#include "esg.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "esg_internal.hpp"

namespace esg {
void subsample_index(int d_ff, int group_size, int spg, uint64_t seed, int32_t* out);
void timing_set(bool on);
void timing_reset();
int timing_read(const char* name, double* total_ms, int* launches);
}  // namespace esg

using namespace esg;

namespace {

constexpr int kMaxGroups = 1024;
constexpr int kMaxK = 128;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Shape rules of the eugen_sparse README ("Parameters and how to choose
// them"): group_size a power of two >= 16; d_ff a multiple of it with at
// least two groups; d_model a multiple of 16; 1 <= k <= G; tokens*k < 2^31.
int check_shape(int dtype, int tokens, int d_model, int d_ff, int group_size, int k) {
  if (dtype != ESG_F32 && dtype != ESG_BF16) return ESG_ERR_UNSUPPORTED;
  if (tokens < 0 || d_model <= 0 || d_ff <= 0 || group_size <= 0 || k <= 0) return ESG_ERR_INVALID_ARG;
  if (!pow2(group_size) || group_size < 16) return ESG_ERR_UNSUPPORTED;
  if (d_ff % group_size != 0 || d_ff / group_size < 2) return ESG_ERR_UNSUPPORTED;
  if (d_model % 16 != 0) return ESG_ERR_UNSUPPORTED;
  const int groups = d_ff / group_size;
  if (groups > kMaxGroups || k > groups) return ESG_ERR_UNSUPPORTED;
  if ((long long)tokens * k >= (1ll << 31)) return ESG_ERR_UNSUPPORTED;
  return ESG_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ESG_OK : ESG_ERR_HIP; }

struct Layout {
  int mt = 0;            // maximum tiles
  size_t rows = 0;       // padded positions
  size_t offsets = 0, tile_off = 0, tile_group = 0, ptoken = 0, pinv = 0, hg = 0, hu = 0, saved = 0;
  size_t f_bucket = 0, f_part = 0, f_route = 0, f_act = 0, fwd = 0;
  size_t b_dg = 0, b_du = 0, b_act = 0, b_part = 0, b_slots = 0, bwd = 0;
  int cht = 0;           // weight-gradient chunk tiles (dw_chunk_tiles)
};

// train: the layout of a forward that saves for the backward, whose groups are
// padded to tile_pad(s) positions; an inference forward pads to whole tiles only
Layout make_layout(const FfnShape& s, bool train = true) {
  Layout L;
  const int G = s.groups();
  L.mt = max_tiles(s.tokens, s.k, G, kTileRows, train ? tile_pad(s) : kTileRows);
  L.rows = (size_t)L.mt * kTileRows;
  const size_t es = s.elem_bytes();
  const size_t act_bytes = (size_t)s.nsub() * L.rows * s.gsb() * es;
  const size_t part_bytes = (size_t)s.nsub() * L.rows * s.d_model * es;
  size_t o = 0;
  L.offsets = o;    o = align256(o + (size_t)(G + 1) * 4);
  L.tile_off = o;   o = align256(o + (size_t)(G + 1) * 4);
  L.tile_group = o; o = align256(o + (size_t)L.mt * 4);
  L.ptoken = o;     o = align256(o + L.rows * 4);
  L.pinv = o;       o = align256(o + (size_t)s.tokens * s.k * 4);
  L.hg = o;         o = align256(o + act_bytes);
  L.hu = o;         o = align256(o + act_bytes);
  L.saved = o;
  o = 0;
  L.f_bucket = o;   o = align256(o + bucket_scratch_bytes(s.tokens, G));
  L.f_part = o;     o = align256(o + part_bytes);
  L.f_route = o;    o = align256(o + L.hg);  // the routing arrays of `saved`, for saved = NULL (inference)
  L.f_act = o;      o = align256(o + fwd_split_bytes(s, L.mt));  // [hg; hu] partials of a split forward
  L.fwd = o;
  o = 0;
  L.b_dg = o;       o = align256(o + act_bytes);
  L.b_du = o;       o = align256(o + act_bytes);
  L.b_act = o;      o = align256(o + act_bytes);
  L.b_part = o;     o = align256(o + part_bytes);
  L.cht = train ? dw_chunk_tiles(s, L.mt, tile_pad(s)) : 0;
  L.b_slots = o;    o = align256(o + dw_slot_bytes(s, L.rows, L.cht));
  L.bwd = o;
  return L;
}

template <typename P>
P* at(void* base, size_t off) {
  return (P*)((char*)base + off);
}
template <typename P>
const P* at(const void* base, size_t off) {
  return (const P*)((const char*)base + off);
}

hipError_t zero_bytes(void* p, size_t bytes, hipStream_t st) {
  return launch_fill_i32((int32_t*)p, 0, bytes / 4, st);
}

}  // namespace

size_t esg::inference_fwd_scratch_bytes(const FfnShape& s) { return make_layout(s, false).fwd; }

extern "C" {

const char* esg_status_string(int status) {
  switch (status) {
    case ESG_OK: return "ok";
    case ESG_ERR_INVALID_ARG: return "invalid argument";
    case ESG_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case ESG_ERR_WORKSPACE: return "workspace too small";
    case ESG_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int esg_version(void) { return 10000; }

int esg_make_subsample_index(int d_ff, int group_size, int samples_per_group, uint64_t seed, int32_t* out) {
  if (out == nullptr) return ESG_ERR_INVALID_ARG;
  if (!pow2(group_size) || group_size < 16 || d_ff <= 0 || d_ff % group_size != 0 || d_ff / group_size < 2)
    return ESG_ERR_UNSUPPORTED;
  if (samples_per_group < 1 || samples_per_group > group_size) return ESG_ERR_UNSUPPORTED;
  subsample_index(d_ff, group_size, samples_per_group, seed, out);
  return ESG_OK;
}

int esg_grouped_topk_select_ws(const void* x, const void* w_gate, int dtype, int tokens, int d_model, int d_ff,
                               int group_size, int k, const int32_t* sub, int samples_per_group, const float* bias,
                               int32_t* idx_out, int32_t* counts_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int st = check_shape(dtype, tokens, d_model, d_ff, group_size, k);
  if (st != ESG_OK) return st;
  if ((tokens > 0 && (x == nullptr || idx_out == nullptr)) || w_gate == nullptr) return ESG_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(workspace)) return ESG_ERR_INVALID_ARG;
  int rpg = group_size;
  if (sub != nullptr) {
    if (samples_per_group < 1 || samples_per_group > group_size) return ESG_ERR_UNSUPPORTED;
    rpg = samples_per_group;
  }
  const int groups = d_ff / group_size;
  float* ews = workspace != nullptr && workspace_bytes >= select_energy_bytes(tokens, groups) ? (float*)workspace
                                                                                             : nullptr;
  return hip_status(launch_select(dtype, x, w_gate, tokens, d_model, groups, k, sub, rpg, group_size, bias,
                                  idx_out, counts_out, ews, (hipStream_t)stream));
}

int esg_grouped_topk_select(const void* x, const void* w_gate, int dtype, int tokens, int d_model, int d_ff,
                            int group_size, int k, const int32_t* sub, int samples_per_group, const float* bias,
                            int32_t* idx_out, int32_t* counts_out, void* stream) {
  return esg_grouped_topk_select_ws(x, w_gate, dtype, tokens, d_model, d_ff, group_size, k, sub, samples_per_group,
                                    bias, idx_out, counts_out, nullptr, 0, stream);
}

int esg_grouped_topk_select_workspace_size(int tokens, int d_ff, int group_size, size_t* workspace_bytes) {
  if (workspace_bytes == nullptr || tokens < 0 || d_ff <= 0 || group_size <= 0 || d_ff % group_size != 0)
    return ESG_ERR_INVALID_ARG;
  *workspace_bytes = select_energy_bytes(tokens, d_ff / group_size);
  return ESG_OK;
}

int esg_bucket_workspace_size(int tokens, int k, int groups, size_t* scratch_bytes) {
  if (scratch_bytes == nullptr || tokens < 0 || k <= 0 || groups <= 0) return ESG_ERR_INVALID_ARG;
  if (groups > kMaxGroups || k > kMaxK || (long long)tokens * k >= (1ll << 31)) return ESG_ERR_UNSUPPORTED;
  *scratch_bytes = bucket_scratch_bytes(tokens, groups);
  return ESG_OK;
}

int esg_bucket_by_group(const int32_t* idx, int tokens, int k, int groups, int32_t* offsets, int32_t* perm_token,
                        int32_t* inv, int32_t* status_dev, void* scratch, size_t scratch_bytes, void* stream) {
  size_t need = 0;
  int st = esg_bucket_workspace_size(tokens, k, groups, &need);
  if (st != ESG_OK) return st;
  if (offsets == nullptr || scratch == nullptr || (tokens > 0 && (idx == nullptr || perm_token == nullptr ||
                                                                  inv == nullptr)))
    return ESG_ERR_INVALID_ARG;
  if (scratch_bytes < need) return ESG_ERR_WORKSPACE;
  BucketOut out{offsets, perm_token, inv, nullptr, nullptr, nullptr, nullptr, status_dev};
  return hip_status(launch_bucket(idx, tokens, k, groups, kTileRows, out, scratch, (hipStream_t)stream));
}

int esg_sparse_swiglu_workspace_size(int tokens, int d_model, int d_ff, int group_size, int k, int dtype, int dense,
                                     size_t* saved_bytes, size_t* fwd_scratch_bytes, size_t* bwd_scratch_bytes) {
  int st = check_shape(dtype, tokens, d_model, d_ff, group_size, k);
  if (st != ESG_OK) return st;
  if (dense) {
    const FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
    if (k != s.groups()) return ESG_ERR_INVALID_ARG;
    if (!dense_supported(s)) return ESG_ERR_UNSUPPORTED;
    if (saved_bytes) *saved_bytes = 0;
    if (fwd_scratch_bytes) *fwd_scratch_bytes = 0;
    if (bwd_scratch_bytes) *bwd_scratch_bytes = dense_bwd_layout(tokens, d_model, d_ff).bytes;
    return ESG_OK;
  }
  if (k > kMaxK) return ESG_ERR_UNSUPPORTED;
  const Layout L = make_layout(FfnShape{dtype, tokens, d_model, d_ff, group_size, k});
  if (saved_bytes) *saved_bytes = L.saved;
  if (fwd_scratch_bytes) *fwd_scratch_bytes = L.fwd;
  if (bwd_scratch_bytes) *bwd_scratch_bytes = L.bwd;
  return ESG_OK;
}

int esg_sparse_swiglu_fwd(const void* x, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                          int tokens, int d_model, int d_ff, int group_size, int k, const int32_t* idx, void* y,
                          void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes, int32_t* status_dev,
                          void* stream) {
  int st = check_shape(dtype, tokens, d_model, d_ff, group_size, k);
  if (st != ESG_OK) return st;
  if (w_gate == nullptr || w_up == nullptr || w_down == nullptr) return ESG_ERR_INVALID_ARG;
  if (tokens == 0) return ESG_OK;  // nothing to route or compute (an empty idx may be NULL)
  if (idx == nullptr) {            // dense limit: every group active, nothing saved
    const FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
    if (k != s.groups()) return ESG_ERR_INVALID_ARG;
    if (!dense_supported(s)) return ESG_ERR_UNSUPPORTED;
    if (x == nullptr || y == nullptr) return ESG_ERR_INVALID_ARG;
    for (const void* p : {x, w_gate, w_up, w_down, (const void*)y})
      if (!aligned16(p)) return ESG_ERR_INVALID_ARG;
    return hip_status(launch_dense_fwd(s, x, w_gate, w_up, w_down, y, (hipStream_t)stream));
  }
  if (scratch == nullptr) return ESG_ERR_INVALID_ARG;
  if (k > kMaxK) return ESG_ERR_UNSUPPORTED;
  if (tokens > 0 && (x == nullptr || y == nullptr)) return ESG_ERR_INVALID_ARG;
  for (const void* p : {x, w_gate, w_up, w_down, (const void*)y, (const void*)idx, (const void*)saved,
                        (const void*)scratch})
    if (!aligned16(p)) return ESG_ERR_INVALID_ARG;
  const FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
  const bool train = saved != nullptr;  // NULL: forward only, the routing lives in the scratch
  const Layout L = make_layout(s, train);
  if ((train && saved_bytes < L.saved) || scratch_bytes < L.fwd) return ESG_ERR_WORKSPACE;
  void* route = train ? saved : at<char>(scratch, L.f_route);
  hipStream_t stream_h = (hipStream_t)stream;
  BucketOut out{at<int32_t>(route, L.offsets), nullptr, nullptr, at<int32_t>(route, L.tile_off),
                at<int32_t>(route, L.tile_group), at<int32_t>(route, L.ptoken), at<int32_t>(route, L.pinv),
                status_dev};
  const int pad = train ? tile_pad(s) : kTileRows;
  hipError_t e = launch_bucket(idx, tokens, k, s.groups(), kTileRows, out, at<char>(scratch, L.f_bucket), stream_h,
                               pad);
  if (e != hipSuccess) return ESG_ERR_HIP;
  char* hg = train ? at<char>(saved, L.hg) : nullptr;
  char* hu = train ? at<char>(saved, L.hu) : nullptr;
  e = bf16_pipelined(s, L.mt)
          ? launch_fwd2(s, x, w_gate, w_up, w_down, out.tile_group, out.ptoken, L.mt, pad, hg, hu,
                        at<char>(scratch, L.f_part), at<char>(scratch, L.f_act), stream_h)
          : launch_fwd_grouped(s, x, w_gate, w_up, w_down, out.tile_group, out.ptoken, L.mt, hg, hu,
                               at<char>(scratch, L.f_part), stream_h);
  if (e != hipSuccess) return ESG_ERR_HIP;
  e = launch_rowsum(s, at<char>(scratch, L.f_part), L.rows, out.pinv, y, stream_h);
  return hip_status(e);
}

int esg_sparse_swiglu_bwd(const void* dy, const void* x, const void* w_gate, const void* w_up, const void* w_down,
                          int dtype, int tokens, int d_model, int d_ff, int group_size, int k, const int32_t* idx,
                          const void* saved, size_t saved_bytes, void* dx, void* dw_gate, void* dw_up,
                          void* dw_down, void* scratch, size_t scratch_bytes, void* stream) {
  return esg_sparse_swiglu_bwd_overlap(dy, x, w_gate, w_up, w_down, dtype, tokens, d_model, d_ff, group_size, k, idx,
                                       saved, saved_bytes, dx, dw_gate, dw_up, dw_down, scratch, scratch_bytes, stream,
                                       nullptr);
}

int esg_sparse_swiglu_bwd_overlap(const void* dy, const void* x, const void* w_gate, const void* w_up,
                                  const void* w_down, int dtype, int tokens, int d_model, int d_ff, int group_size,
                                  int k, const int32_t* idx, const void* saved, size_t saved_bytes, void* dx,
                                  void* dw_gate, void* dw_up, void* dw_down, void* scratch, size_t scratch_bytes,
                                  void* stream, void* aux_stream) {
  int st = check_shape(dtype, tokens, d_model, d_ff, group_size, k);
  if (st != ESG_OK) return st;
  if (w_gate == nullptr || w_up == nullptr || w_down == nullptr || scratch == nullptr || dw_gate == nullptr ||
      dw_up == nullptr || dw_down == nullptr)
    return ESG_ERR_INVALID_ARG;
  if (tokens == 0) {  // no token: every weight gradient is zero (an empty idx may be NULL)
    hipStream_t stream_h = (hipStream_t)stream;
    const size_t wbytes = (size_t)d_ff * d_model * (dtype == ESG_BF16 ? 2 : 4);
    hipError_t e = zero_bytes(dw_gate, wbytes, stream_h);
    if (e == hipSuccess) e = zero_bytes(dw_up, wbytes, stream_h);
    if (e == hipSuccess) e = zero_bytes(dw_down, wbytes, stream_h);
    return hip_status(e);
  }
  if (idx == nullptr) {  // dense limit: gate/up recomputed, nothing saved
    const FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
    if (k != s.groups()) return ESG_ERR_INVALID_ARG;
    if (!dense_supported(s)) return ESG_ERR_UNSUPPORTED;
    hipStream_t stream_h = (hipStream_t)stream;
    if (x == nullptr || dy == nullptr || dx == nullptr) return ESG_ERR_INVALID_ARG;
    for (const void* p : {dy, x, w_gate, w_up, w_down, (const void*)dx, (const void*)dw_gate, (const void*)dw_up,
                          (const void*)dw_down, (const void*)scratch})
      if (!aligned16(p)) return ESG_ERR_INVALID_ARG;
    if (scratch_bytes < dense_bwd_layout(tokens, d_model, d_ff).bytes) return ESG_ERR_WORKSPACE;
    return hip_status(
        launch_dense_bwd(s, dy, x, w_gate, w_up, w_down, dx, dw_gate, dw_up, dw_down, scratch, stream_h));
  }
  if (saved == nullptr) return ESG_ERR_INVALID_ARG;
  if (k > kMaxK) return ESG_ERR_UNSUPPORTED;
  if (tokens > 0 && (x == nullptr || dy == nullptr || dx == nullptr)) return ESG_ERR_INVALID_ARG;
  for (const void* p : {dy, x, w_gate, w_up, w_down, saved, (const void*)dx, (const void*)dw_gate,
                        (const void*)dw_up, (const void*)dw_down, (const void*)scratch})
    if (!aligned16(p)) return ESG_ERR_INVALID_ARG;
  const FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
  const Layout L = make_layout(s);
  if (saved_bytes < L.saved || scratch_bytes < L.bwd) return ESG_ERR_WORKSPACE;
  hipStream_t stream_h = (hipStream_t)stream;
  const int32_t* tile_group = at<int32_t>(saved, L.tile_group);
  const int32_t* tile_off = at<int32_t>(saved, L.tile_off);
  const int32_t* ptoken = at<int32_t>(saved, L.ptoken);
  const int32_t* pinv = at<int32_t>(saved, L.pinv);
  const bool v2 = bf16_pipelined(s, L.mt);
  hipError_t e = v2 ? launch_dhdx2(s, dy, w_gate, w_up, w_down, tile_group, ptoken, L.mt, at<char>(saved, L.hg),
                                   at<char>(saved, L.hu), at<char>(scratch, L.b_dg), at<char>(scratch, L.b_du),
                                   at<char>(scratch, L.b_act), at<char>(scratch, L.b_part), stream_h)
                    : launch_bwd_dh_dx(s, dy, w_gate, w_up, w_down, tile_group, ptoken, L.mt, at<char>(saved, L.hg),
                                       at<char>(saved, L.hu), at<char>(scratch, L.b_dg), at<char>(scratch, L.b_du),
                                       at<char>(scratch, L.b_act), at<char>(scratch, L.b_part), stream_h);
  if (e != hipSuccess) return ESG_ERR_HIP;
  // The slot-order sum of dx and the weight gradients only read what dh+dx
  // wrote.  With a caller-supplied second stream the weight gradients run on
  // it beside the sum (forked after dh+dx, joined back into `stream` by two
  // events created and destroyed in this call); else one after the other.
  hipStream_t aux = (hipStream_t)aux_stream;
  hipEvent_t forked = nullptr, done = nullptr;
  if (aux != nullptr && aux != stream_h) {
    if (hipEventCreateWithFlags(&forked, hipEventDisableTiming) != hipSuccess) return ESG_ERR_HIP;
    if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess) {
      (void)hipEventDestroy(forked);
      return ESG_ERR_HIP;
    }
    e = hipEventRecord(forked, stream_h);
    if (e == hipSuccess) e = hipStreamWaitEvent(aux, forked, 0);
  } else {
    aux = stream_h;
  }
  if (e == hipSuccess)
    e = v2 ? launch_dw2(s, x, dy, tile_off, ptoken, (int)L.rows, at<char>(scratch, L.b_dg),
                        at<char>(scratch, L.b_du), at<char>(scratch, L.b_act), dw_gate, dw_up, dw_down, L.cht,
                        at<char>(scratch, L.b_slots), aux)
           : launch_bwd_dw(s, x, dy, tile_off, ptoken, (int)L.rows, at<char>(scratch, L.b_dg),
                           at<char>(scratch, L.b_du), at<char>(scratch, L.b_act), dw_gate, dw_up, dw_down, aux);
  if (e == hipSuccess) e = launch_rowsum(s, at<char>(scratch, L.b_part), L.rows, pinv, dx, stream_h);
  if (forked != nullptr) {
    if (e == hipSuccess) e = hipEventRecord(done, aux);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream_h, done, 0);
    (void)hipEventDestroy(forked);
    (void)hipEventDestroy(done);
  }
  return hip_status(e);
}

int esg_update_load_balance_bias(float* bias, float* freq_ema, const float* current_freq, float target_freq,
                                 float gamma, float bias_max, float momentum, int groups, void* stream) {
  if (bias == nullptr || freq_ema == nullptr || current_freq == nullptr || groups < 0) return ESG_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(bias, freq_ema, current_freq, nullptr, nullptr, 1, target_freq, gamma,
                                       bias_max, momentum, groups, (hipStream_t)stream));
}

int esg_update_load_balance_bias_from_counts(float* bias, float* freq_ema, const int32_t* counts, int tokens,
                                             float target_freq, float gamma, float bias_max, float momentum,
                                             int groups, void* stream) {
  if (bias == nullptr || freq_ema == nullptr || counts == nullptr || groups < 0 || tokens <= 0)
    return ESG_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(bias, freq_ema, nullptr, counts, nullptr, tokens, target_freq, gamma,
                                       bias_max, momentum, groups, (hipStream_t)stream));
}

int esg_update_load_balance_bias_from_routing(float* bias, float* freq_ema, const void* saved, size_t saved_bytes,
                                              int tokens, int d_model, int d_ff, int group_size, int k, int dtype,
                                              float target_freq, float gamma, float bias_max, float momentum,
                                              void* stream) {
  int st = check_shape(dtype, tokens, d_model, d_ff, group_size, k);
  if (st != ESG_OK) return st;
  if (bias == nullptr || freq_ema == nullptr || saved == nullptr || tokens <= 0) return ESG_ERR_INVALID_ARG;
  if (k > kMaxK) return ESG_ERR_UNSUPPORTED;
  const FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
  const Layout L = make_layout(s);
  if (saved_bytes < L.saved) return ESG_ERR_WORKSPACE;
  return hip_status(launch_bias_update(bias, freq_ema, nullptr, nullptr, at<int32_t>(saved, L.offsets), tokens,
                                       target_freq, gamma, bias_max, momentum, s.groups(), (hipStream_t)stream));
}

namespace {
int mlp_shape(int tokens, int d_model, int d_ff) {
  if (tokens < 0 || d_model <= 0 || d_ff <= 0) return ESG_ERR_INVALID_ARG;
  if (d_model % 8 || d_ff % 8) return ESG_ERR_UNSUPPORTED;
  const long long wide = d_model > d_ff ? d_model : d_ff;
  if ((long long)tokens * wide * 2 >= (1ll << 31) || (long long)d_model * d_ff * 2 >= (1ll << 31))
    return ESG_ERR_UNSUPPORTED;
  return ESG_OK;
}
}  // namespace

int esg_leaky_mlp_workspace_size(int tokens, int d_model, int d_ff, size_t* saved_bytes, size_t* scratch_bytes) {
  if (saved_bytes == nullptr || scratch_bytes == nullptr) return ESG_ERR_INVALID_ARG;
  const int e = mlp_shape(tokens, d_model, d_ff);
  if (e != ESG_OK) return e;
  const size_t tf = (size_t)tokens * d_ff * 2;
  *saved_bytes = 2 * align256(tf);
  *scratch_bytes = align256(tf) + align256(mlp_partial_bytes(tokens, d_model, d_ff));
  return ESG_OK;
}

int esg_leaky_mlp_fwd(const void* x, const void* w_up, const void* w_down, int tokens, int d_model, int d_ff,
                      void* y, void* saved, size_t saved_bytes, void* stream) {
  size_t need_saved, need_scratch;
  int e = esg_leaky_mlp_workspace_size(tokens, d_model, d_ff, &need_saved, &need_scratch);
  if (e != ESG_OK) return e;
  if (tokens == 0) return ESG_OK;
  if (x == nullptr || w_up == nullptr || w_down == nullptr || y == nullptr || saved == nullptr)
    return ESG_ERR_INVALID_ARG;
  if (saved_bytes < need_saved) return ESG_ERR_WORKSPACE;
  void* post = saved;
  void* act = (char*)saved + align256((size_t)tokens * d_ff * 2);
  return hip_status(launch_mlp_fwd(x, w_up, w_down, tokens, d_model, d_ff, y, post, act, (hipStream_t)stream));
}

int esg_leaky_mlp_bwd(const void* dy, const void* x, const void* w_up, const void* w_down, int tokens, int d_model,
                      int d_ff, const void* saved, void* dx, void* dw_up, void* dw_down, void* scratch,
                      size_t scratch_bytes, void* stream) {
  size_t need_saved, need_scratch;
  int e = esg_leaky_mlp_workspace_size(tokens, d_model, d_ff, &need_saved, &need_scratch);
  if (e != ESG_OK) return e;
  if (w_up == nullptr || w_down == nullptr || dw_up == nullptr || dw_down == nullptr) return ESG_ERR_INVALID_ARG;
  if (tokens > 0 && (dy == nullptr || x == nullptr || saved == nullptr || dx == nullptr || scratch == nullptr))
    return ESG_ERR_INVALID_ARG;
  if (tokens > 0 && scratch_bytes < need_scratch) return ESG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (tokens == 0) {  // no tokens: the weight gradients are zero
    e = hip_status(launch_fill_i32((int32_t*)dw_up, 0, (size_t)d_ff * d_model / 2, st));
    if (e != ESG_OK) return e;
    return hip_status(launch_fill_i32((int32_t*)dw_down, 0, (size_t)d_ff * d_model / 2, st));
  }
  const size_t tf = align256((size_t)tokens * d_ff * 2);
  const void* post = saved;
  const void* act = (const char*)saved + tf;
  void* dpre = scratch;
  float* part = (float*)((char*)scratch + tf);
  return hip_status(launch_mlp_bwd(dy, x, w_up, w_down, tokens, d_model, d_ff, post, act, dx, dw_up, dw_down, dpre,
                                   part, st));
}

int esg_mhffn_supported(int tokens, int heads, int d_head, int subnets, int d_sub) {
  return mhffn_supported(tokens, heads, d_head, subnets, d_sub) ? 1 : 0;
}

int esg_mhffn_fwd(const void* q, const float* r, const void* k, const void* u, const void* v, int tokens, int heads,
                  int d_head, int subnets, int d_sub, void* out, void* stream) {
  if (tokens < 0 || heads <= 0 || subnets <= 0 || d_sub <= 0) return ESG_ERR_INVALID_ARG;
  if (!mhffn_supported(tokens, heads, d_head, subnets, d_sub)) return ESG_ERR_UNSUPPORTED;
  if (tokens == 0) return ESG_OK;
  for (const void* p : {q, (const void*)r, k, u, v, (const void*)out})
    if (p == nullptr || !aligned16(p)) return ESG_ERR_INVALID_ARG;
  return hip_status(launch_mhffn_fwd(q, r, k, u, v, tokens, heads, subnets, d_sub, out, (hipStream_t)stream));
}

int esg_mhffn_bwd(const void* dout, const void* q, const float* r, const void* k, const void* u, const void* v,
                  int tokens, int heads, int d_head, int subnets, int d_sub, void* dq, float* dr, void* dk, void* du,
                  void* dv, void* stream) {
  if (tokens < 0 || heads <= 0 || subnets <= 0 || d_sub <= 0) return ESG_ERR_INVALID_ARG;
  if (!mhffn_supported(tokens, heads, d_head, subnets, d_sub)) return ESG_ERR_UNSUPPORTED;
  for (const void* p : {k, u, v, (const void*)dk, (const void*)du, (const void*)dv})
    if (p == nullptr || !aligned16(p)) return ESG_ERR_INVALID_ARG;
  if (tokens > 0)
    for (const void* p : {dout, q, (const void*)r, (const void*)dq, (const void*)dr})
      if (p == nullptr || !aligned16(p)) return ESG_ERR_INVALID_ARG;
  return hip_status(launch_mhffn_bwd(dout, q, r, k, u, v, tokens, heads, subnets, d_sub, dq, dr, dk, du, dv,
                                     (hipStream_t)stream));
}

int esg_sigmoid_topk_supported(int num_experts, int topk) { return sigmoid_topk_supported(num_experts, topk) ? 1 : 0; }

int esg_sigmoid_topk_routing(const float* logits, const float* expert_bias, int bias_stride, int tokens,
                             int num_experts, int topk, float scaling_factor, int apply_scaling, float* probs,
                             int64_t* indices, void* stream) {
  if (tokens < 0 || bias_stride < 1) return ESG_ERR_INVALID_ARG;
  if (!sigmoid_topk_supported(num_experts, topk)) return ESG_ERR_UNSUPPORTED;
  if ((size_t)tokens * topk >= (1ull << 31) || (size_t)tokens * num_experts >= (1ull << 40))
    return ESG_ERR_UNSUPPORTED;
  if (tokens == 0) return ESG_OK;
  if (logits == nullptr || expert_bias == nullptr || probs == nullptr || indices == nullptr)
    return ESG_ERR_INVALID_ARG;
  return hip_status(launch_sigmoid_topk(logits, expert_bias, bias_stride, tokens, num_experts, topk, scaling_factor,
                                        apply_scaling, probs, indices, (hipStream_t)stream));
}

int esg_mfma_rate_probe(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return ESG_ERR_INVALID_ARG;
  return hip_status(launch_mfma_probe(blocks, iters, out, (hipStream_t)stream));
}

int esg_timing_enable(int on) {
  timing_set(on != 0);
  return ESG_OK;
}

int esg_timing_reset(void) {
  timing_reset();
  return ESG_OK;
}

int esg_timing_read(const char* kernel, double* total_ms, int* launches) {
  if (kernel == nullptr || total_ms == nullptr || launches == nullptr) return ESG_ERR_INVALID_ARG;
  return timing_read(kernel, total_ms, launches) == 0 ? ESG_OK : ESG_ERR_HIP;
}

}  // extern "C"
