// C ABI of the HGA library: argument validation and kernel dispatch.
// The contract of every entry point is documented in include/hga.h.
#include "hga.h"

#include <math.h>
#include <string.h>

// (the host-only entry points -- hga_validate_shape, hga_validate_decode_shape,
// hga_status_str, hga_abi_version, hga_stage_min_groups and the workspace
// sizes -- are in hga_validate.cpp, and the workspace layouts and the staging
// checks in hga_layout.h: plain C++ that the CPU tests also build with
// sanitizers)

#include "hga_kernels.h"
#include "hga_layout.h"

namespace {

hga::Dims dims_of(const hga_shape* s) {
  hga::Dims d;
  d.B = s->batch;
  d.Hq = s->n_q_heads;
  d.Hkv = s->n_kv_heads;
  d.D = s->head_dim;
  d.Sq = s->q_len;
  d.Skv = s->kv_len;
  d.Scap = s->kv_capacity > 0 ? s->kv_capacity : s->kv_len;
  d.top_k = s->top_k;
  d.top_g = s->top_g;
  d.q0 = s->kv_len - s->q_len;
  d.nblk = s->q_len == 1 ? 1 : s->q_len / HGA_QBLOCK;
  d.scale = s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
  d.bf16 = s->dtype == HGA_DTYPE_BF16;
  return d;
}

hga_status from_hip(hipError_t e) { return e == hipSuccess ? HGA_OK : HGA_ERR_HIP; }

using hga_layout::cmask_bytes;
using hga_layout::delta_bytes;
using hga_layout::order_bytes;

int32_t* order_full(const hga_shape* s, void* ws) {
  return (int32_t*)((uint8_t*)ws + delta_bytes(s) + cmask_bytes(s));
}
int32_t* order_range(const hga_shape* s, void* ws) {
  return (int32_t*)((uint8_t*)ws + delta_bytes(s) + cmask_bytes(s) + order_bytes(s));
}

}  // namespace

extern "C" {

hga_status hga_build_summaries(const hga_shape* shape, const void* K, float* chunk_mean,
                               float* group_mean, int32_t chunk_begin, int32_t chunk_end,
                               void* stream) {
  hga_status st = shape && shape->q_len == 1 ? hga_validate_decode_shape(shape)
                                             : hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!K || !chunk_mean || !group_mean) return HGA_ERR_NULL;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > shape->kv_len / HGA_CHUNK)
    return HGA_ERR_SHAPE;
  if (chunk_end == chunk_begin) return HGA_OK;
  const hga::Dims d = dims_of(shape);
  return from_hip(hga::launch_summaries(d, K, d.Scap, 0, chunk_mean, group_mean, chunk_begin,
                                        chunk_end, (hipStream_t)stream));
}

hga_status hga_build_summaries_rows(const hga_shape* shape, const void* K_rows, int32_t row0,
                                    int32_t rows, float* chunk_mean, float* group_mean,
                                    int32_t chunk_begin, int32_t chunk_end, void* stream) {
  hga_status st = shape && shape->q_len == 1 ? hga_validate_decode_shape(shape)
                                             : hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!K_rows || !chunk_mean || !group_mean) return HGA_ERR_NULL;
  if (row0 < 0 || row0 % HGA_CHUNK != 0 || rows <= 0 || rows % HGA_CHUNK != 0 ||
      rows > shape->kv_len - row0)
    return HGA_ERR_SHAPE;
  if (chunk_begin < row0 / HGA_CHUNK || chunk_end < chunk_begin ||
      chunk_end > (row0 + rows) / HGA_CHUNK)
    return HGA_ERR_SHAPE;
  if (chunk_end == chunk_begin) return HGA_OK;
  return from_hip(hga::launch_summaries(dims_of(shape), K_rows, rows, row0, chunk_mean,
                                        group_mean, chunk_begin, chunk_end, (hipStream_t)stream));
}

hga_status hga_route(const hga_shape* shape, const void* Q, const float* chunk_mean,
                     const float* group_mean, int32_t* chunk_idx, int32_t* group_idx,
                     void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !chunk_mean) return HGA_ERR_NULL;
  if (shape->top_g > 0 && (!group_idx || !group_mean)) return HGA_ERR_NULL;
  // no budget: both index arrays have zero entries per row, nothing to write
  if (shape->top_k == 0 && shape->top_g == 0) return HGA_OK;
  return from_hip(hga::launch_route(dims_of(shape), Q, nullptr, false, chunk_mean, group_mean,
                                    shape->top_k > 0 ? chunk_idx : nullptr,
                                    shape->top_g > 0 ? group_idx : nullptr,
                                    (hipStream_t)stream));
}

hga_status hga_route_causal(const hga_shape* shape, const void* Q, const void* Q_prev,
                            const float* chunk_mean, const float* group_mean,
                            int32_t* chunk_idx, int32_t* group_idx, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !chunk_mean) return HGA_ERR_NULL;
  if (shape->top_g > 0 && (!group_idx || !group_mean)) return HGA_ERR_NULL;
  const bool routes = shape->top_k > 0 || shape->top_g > 0;
  if (routes && shape->kv_len > shape->q_len && !Q_prev) return HGA_ERR_NULL;
  // no budget: nothing to write, and Q_prev is not read
  if (!routes) return HGA_OK;
  return from_hip(hga::launch_route(dims_of(shape), Q, Q_prev, true, chunk_mean, group_mean,
                                    shape->top_k > 0 ? chunk_idx : nullptr,
                                    shape->top_g > 0 ? group_idx : nullptr,
                                    (hipStream_t)stream));
}

hga_status hga_attend_fwd(const hga_shape* shape, const void* Q, const void* K, const void* V,
                          const int32_t* group_idx, void* O, float* lse, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !O) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  return from_hip(hga::launch_attend_fwd(dims_of(shape), Q, K, V, group_idx, O, lse,
                                         (hipStream_t)stream));
}

hga_status hga_attend_bwd_dq(const hga_shape* shape, const void* Q, const void* K,
                             const void* V, const void* O, const float* lse, const void* dO,
                             const int32_t* group_idx, void* dQ, void* workspace,
                             size_t workspace_bytes, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !O || !lse || !dO || !dQ) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  // no workspace: dQ only (the caller runs hga_attend_bwd_prep for dK/dV)
  if (!workspace && workspace_bytes == 0)
    return from_hip(hga::launch_attend_bwd_dq(dims_of(shape), Q, K, V, O, lse, dO, group_idx,
                                              dQ, nullptr, nullptr, nullptr,
                                              (hipStream_t)stream));
  if (!workspace || workspace_bytes < hga_layout::bwd_workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
  return from_hip(hga::launch_attend_bwd_dq(
      dims_of(shape), Q, K, V, O, lse, dO, group_idx, dQ, (float*)workspace,
      (uint8_t*)workspace + delta_bytes(shape), order_full(shape, workspace),
      (hipStream_t)stream));
}

hga_status hga_attend_bwd_prep(const hga_shape* shape, const void* O, const void* dO,
                               const int32_t* group_idx, void* workspace,
                               size_t workspace_bytes, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!O || !dO) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  if (!workspace || workspace_bytes < hga_layout::bwd_workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
  return from_hip(hga::launch_attend_bwd_prep(
      dims_of(shape), O, dO, group_idx, (float*)workspace,
      (uint8_t*)workspace + delta_bytes(shape), order_full(shape, workspace),
      (hipStream_t)stream));
}

hga_status hga_attend_bwd_dkdv_range(const hga_shape* shape, const void* Q, const void* K,
                                     const void* V, const float* lse, const void* dO,
                                     const int32_t* group_idx, int32_t chunk_begin,
                                     int32_t chunk_end, void* dK, void* dV, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !lse || !dO || !dK || !dV) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  if (!workspace || workspace_bytes < hga_layout::bwd_workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > shape->kv_len / HGA_CHUNK)
    return HGA_ERR_SHAPE;
  if (chunk_end == chunk_begin) return HGA_OK;
  // the whole range uses the work order the dQ call wrote; a sub-range orders itself
  const bool full = chunk_begin == 0 && chunk_end == shape->kv_len / HGA_CHUNK;
  return from_hip(hga::launch_attend_bwd_dkdv(
      dims_of(shape), Q, K, V, lse, dO, group_idx, (const float*)workspace,
      (const uint8_t*)workspace + delta_bytes(shape),
      full ? order_full(shape, workspace) : order_range(shape, workspace), full, dK, dV,
      chunk_begin, chunk_end, (hipStream_t)stream));
}

hga_status hga_attend_bwd_dkdv(const hga_shape* shape, const void* Q, const void* K,
                               const void* V, const float* lse, const void* dO,
                               const int32_t* group_idx, void* dK, void* dV,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t nch = shape ? shape->kv_len / HGA_CHUNK : 0;
  return hga_attend_bwd_dkdv_range(shape, Q, K, V, lse, dO, group_idx, 0, nch, dK, dV,
                                   workspace, workspace_bytes, stream);
}

hga_status hga_attend_bwd(const hga_shape* shape, const void* Q, const void* K, const void* V,
                          const void* O, const float* lse, const void* dO,
                          const int32_t* group_idx, void* dQ, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !O || !lse || !dO || !dQ || !dK || !dV) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  if (!workspace || workspace_bytes < hga_layout::bwd_workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
  st = hga_attend_bwd_dq(shape, Q, K, V, O, lse, dO, group_idx, dQ, workspace, workspace_bytes,
                         stream);
  if (st != HGA_OK) return st;
  return hga_attend_bwd_dkdv(shape, Q, K, V, lse, dO, group_idx, dK, dV, workspace,
                             workspace_bytes, stream);
}

// Common checks and launch of the two staging calls.
static hga_status stage(const hga_shape* shape, const int32_t* group_idx, const void* K,
                        const void* V, const void* K_seg, const void* V_seg,
                        const hga_stage_prev* prev, int32_t stage_groups, int32_t stage_capacity,
                        void* K_stage, void* V_stage, int32_t* group_idx_staged, void* workspace,
                        size_t workspace_bytes, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!K || !V || !K_stage || !V_stage) return HGA_ERR_NULL;
  if ((K_seg == nullptr) != (V_seg == nullptr)) return HGA_ERR_NULL;
  if (shape->top_g > 0 && (!group_idx || !group_idx_staged)) return HGA_ERR_NULL;
  st = hga_layout::check_stage_args(shape, stage_groups, stage_capacity, prev);
  if (st != HGA_OK) return st;
  hga::StagePrevD pd{};
  if (prev) {
    pd.Ks = prev->K_stage;
    pd.Vs = prev->V_stage;
    pd.ulist = (const int32_t*)prev->workspace;
    pd.ucount = (const int32_t*)((const uint8_t*)prev->workspace +
                                 hga_layout::stage_list_bytes(shape->batch, shape->n_kv_heads,
                                                              prev->stage_groups));
    pd.sg = prev->stage_groups;
    pd.Scap = prev->stage_capacity;
    pd.q0 = prev->q0;
    pd.Sq = prev->q_len;
  }
  if (!workspace || workspace_bytes < hga_layout::stage_workspace_bytes(shape, stage_groups))
    return HGA_ERR_WORKSPACE;
  // unions, then their sizes, then the copy sources of the union slots
  const size_t lb = hga_layout::stage_list_bytes(shape->batch, shape->n_kv_heads, stage_groups);
  int32_t* ulist = (int32_t*)workspace;
  int32_t* ucount = (int32_t*)((uint8_t*)workspace + lb);
  int32_t* usrc = (int32_t*)((uint8_t*)workspace + lb +
                             hga_layout::stage_counts_bytes(shape->batch, shape->n_kv_heads));
  return from_hip(hga::launch_stage(dims_of(shape), shape->top_g > 0 ? group_idx : nullptr, K,
                                    V, K_seg, V_seg, prev ? &pd : nullptr, stage_groups,
                                    stage_capacity, K_stage, V_stage,
                                    shape->top_g > 0 ? group_idx_staged : nullptr, ulist,
                                    ucount, usrc, (hipStream_t)stream));
}

hga_status hga_stage_routed(const hga_shape* shape, const int32_t* group_idx, const void* K,
                            const void* V, int32_t stage_groups, int32_t stage_capacity,
                            void* K_stage, void* V_stage, int32_t* group_idx_staged,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return stage(shape, group_idx, K, V, nullptr, nullptr, nullptr, stage_groups, stage_capacity,
               K_stage, V_stage, group_idx_staged, workspace, workspace_bytes, stream);
}

hga_status hga_stage_routed_from(const hga_shape* shape, const int32_t* group_idx, const void* K,
                                 const void* V, const void* K_seg, const void* V_seg,
                                 const hga_stage_prev* prev, int32_t stage_groups,
                                 int32_t stage_capacity, void* K_stage, void* V_stage,
                                 int32_t* group_idx_staged, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return stage(shape, group_idx, K, V, K_seg, V_seg, prev, stage_groups, stage_capacity,
               K_stage, V_stage, group_idx_staged, workspace, workspace_bytes, stream);
}

hga_status hga_decode_route(const hga_shape* shape, const void* Q, const float* chunk_mean,
                            const float* group_mean, int32_t* chunk_idx, int32_t* group_idx,
                            void* stream) {
  hga_status st = hga_validate_decode_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  // summaries are read only when the token has candidate chunks
  const bool candidates = shape->kv_len > HGA_CHUNK && (shape->top_k > 0 || shape->top_g > 0);
  if (candidates && (!chunk_mean || (shape->top_g > 0 && !group_mean))) return HGA_ERR_NULL;
  if (shape->top_k == 0 && shape->top_g == 0) return HGA_OK;
  // launched also without candidates: it then writes the -1 padding
  return from_hip(hga::launch_route(dims_of(shape), Q, nullptr, false, chunk_mean, group_mean,
                                    shape->top_k > 0 ? chunk_idx : nullptr,
                                    shape->top_g > 0 ? group_idx : nullptr,
                                    (hipStream_t)stream));
}

hga_status hga_decode_route_causal(const hga_shape* shape, const void* Q_prev,
                                   const float* chunk_mean, const float* group_mean,
                                   int32_t* chunk_idx, int32_t* group_idx, void* stream) {
  hga_status st = hga_validate_decode_shape(shape);
  if (st != HGA_OK) return st;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  if (shape->top_k == 0 && shape->top_g == 0) return HGA_OK;
  // the token's block j = (kv_len - 1) / 64: candidates are chunks 0..j-1
  const int32_t j = (shape->kv_len - 1) / HGA_CHUNK;
  if (j > 0 && (!Q_prev || !chunk_mean || (shape->top_g > 0 && !group_mean)))
    return HGA_ERR_NULL;
  // the block route over a one-block segment ending at the block's end: its
  // only block is routed (strictly causal) with the mean of Q_prev
  hga::Dims d = dims_of(shape);
  d.Sq = HGA_QBLOCK;
  d.Skv = (j + 1) * HGA_CHUNK;
  d.q0 = j * HGA_CHUNK;
  d.nblk = 1;
  return from_hip(hga::launch_route(d, Q_prev, Q_prev, true, chunk_mean, group_mean,
                                    shape->top_k > 0 ? chunk_idx : nullptr,
                                    shape->top_g > 0 ? group_idx : nullptr,
                                    (hipStream_t)stream));
}

hga_status hga_decode_attend(const hga_shape* shape, const void* Q, const void* K, const void* V,
                             const int32_t* group_idx, void* O, float* lse, void* stream) {
  hga_status st = hga_validate_decode_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !O) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  return from_hip(hga::launch_decode_attend(dims_of(shape), Q, K, V, group_idx, O, lse,
                                            (hipStream_t)stream));
}

hga_status hga_decode(const hga_shape* shape, const void* Q, const void* K, const void* V,
                      const float* chunk_mean, const float* group_mean, int32_t* chunk_idx,
                      int32_t* group_idx, void* O, float* lse, void* stream) {
  // every argument check of both halves before anything is launched
  hga_status st = hga_validate_decode_shape(shape);
  if (st != HGA_OK) return st;
  if (!K || !V || !O) return HGA_ERR_NULL;
  st = hga_decode_route(shape, Q, chunk_mean, group_mean, chunk_idx, group_idx, stream);
  if (st != HGA_OK) return st;
  return hga_decode_attend(shape, Q, K, V, group_idx, O, lse, stream);
}

}  // extern "C"
