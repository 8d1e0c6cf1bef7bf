// Host-only layout of the caller-provided workspaces and the staging calls'
// argument checks: plain C++ arithmetic on the shape and the sizes, shared by
// the launching entry points (hga_api.hip, which also derives the workspace
// pointers from these sizes) and the host-only ones (hga_validate.cpp).  The
// CPU tests build it with the address and undefined-behaviour sanitizers and
// drive it over many argument sets.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "hga.h"

namespace hga_layout {

inline size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Backward workspace: delta (fp32 per query row), then the group-mask map
// (one byte per (routing row, chunk)), then two dK/dV work orders (one int per
// (b, kv head, chunk) each): the full range's, written by the dQ call, and a
// sub-range's, written by the range call itself (so a range call never spoils
// the other).  Valid shapes only: every factor is bounded by
// hga_validate_shape, so no product overflows.
inline size_t delta_bytes(const hga_shape* s) {
  return round256((size_t)s->batch * s->n_q_heads * s->q_len * sizeof(float));
}
inline size_t cmask_bytes(const hga_shape* s) {
  return round256((size_t)s->batch * s->n_q_heads * (s->q_len / HGA_QBLOCK) *
                  (s->kv_len / HGA_CHUNK));
}
inline size_t order_bytes(const hga_shape* s) {
  return round256((size_t)s->batch * s->n_kv_heads * (s->kv_len / HGA_CHUNK) * sizeof(int32_t));
}
inline size_t bwd_workspace_bytes(const hga_shape* s) {
  return delta_bytes(s) + cmask_bytes(s) + 2 * order_bytes(s);
}

// Staging workspace: the unions (stage_groups int32 per (b, kv head)), their
// sizes (one int32 per (b, kv head)), then the copy source of every union
// slot (stage_groups int32 per (b, kv head)).  stage_groups is bounded by the
// callers (0 .. HGA_MAX_KV_LEN / 8) before these are formed.
inline size_t stage_list_bytes(int32_t batch, int32_t kv_heads, int32_t stage_groups) {
  return round256((size_t)batch * kv_heads * (size_t)stage_groups * sizeof(int32_t));
}
inline size_t stage_counts_bytes(int32_t batch, int32_t kv_heads) {
  return round256((size_t)batch * kv_heads * sizeof(int32_t));
}
inline size_t stage_workspace_bytes(const hga_shape* s, int32_t stage_groups) {
  return 2 * stage_list_bytes(s->batch, s->n_kv_heads, stage_groups) +
         stage_counts_bytes(s->batch, s->n_kv_heads);
}

// The staging calls' checks on the buffer sizes and on the previous staging,
// for a shape hga_validate_shape accepted, in the order the calls apply them:
// the staged layout (stage_groups, stage_capacity), then the previous
// staging's pointers, geometry and workspace (its unions and their sizes are
// read).
inline hga_status check_stage_args(const hga_shape* shape, int32_t stage_groups,
                                   int32_t stage_capacity, const hga_stage_prev* prev) {
  // group counts are bounded before they are multiplied: no accepted value
  // can overflow
  if (stage_groups % 8 != 0 || stage_groups < hga_stage_min_groups(shape) ||
      stage_groups > HGA_MAX_KV_LEN / 8)
    return HGA_ERR_SHAPE;
  if (stage_capacity % HGA_CHUNK != 0 || stage_capacity < 8 * stage_groups + shape->q_len ||
      stage_capacity > HGA_MAX_KV_LEN)
    return HGA_ERR_SHAPE;
  if (!prev) return HGA_OK;
  if (!prev->K_stage || !prev->V_stage || !prev->workspace) return HGA_ERR_NULL;
  const int32_t q0 = shape->kv_len - shape->q_len;
  if (prev->stage_groups < 0 || prev->stage_groups % 8 != 0 ||
      prev->stage_groups > HGA_MAX_KV_LEN / 8 || prev->q0 < 0 || prev->q0 % HGA_CHUNK != 0 ||
      prev->q_len < HGA_CHUNK || prev->q_len % HGA_CHUNK != 0 || prev->q_len > q0 - prev->q0 ||
      prev->stage_capacity % HGA_CHUNK != 0 || prev->stage_capacity > HGA_MAX_KV_LEN ||
      prev->stage_capacity < 8 * prev->stage_groups + prev->q_len)
    return HGA_ERR_SHAPE;
  if (prev->workspace_bytes < stage_list_bytes(shape->batch, shape->n_kv_heads, prev->stage_groups) +
                                  stage_counts_bytes(shape->batch, shape->n_kv_heads))
    return HGA_ERR_WORKSPACE;
  return HGA_OK;
}

}  // namespace hga_layout
