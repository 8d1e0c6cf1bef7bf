// C ABI of the HGA library: argument validation and kernel dispatch.
// The contract of every entry point is documented in include/hga.h.
#include "hga.h"

#include <math.h>
#include <string.h>

#include "hga_kernels.h"

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

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// workspace: delta (fp32 per query row), then the group-mask map (one byte per
// (routing row, chunk)), then two dK/dV work orders (one int per (b, kv head,
// chunk) each): the full range's, written by the dQ call, and a sub-range's,
// written by the range call itself (so a range call never spoils the other)
size_t delta_bytes(const hga_shape* s) {
  return round256((size_t)s->batch * s->n_q_heads * s->q_len * sizeof(float));
}
size_t cmask_bytes(const hga_shape* s) {
  return round256((size_t)s->batch * s->n_q_heads * (s->q_len / HGA_QBLOCK) *
                  (s->kv_len / HGA_CHUNK));
}
// the dK/dV work order: one int per (b, kv head, chunk)
size_t order_bytes(const hga_shape* s) {
  return round256((size_t)s->batch * s->n_kv_heads * (s->kv_len / HGA_CHUNK) * sizeof(int32_t));
}
size_t workspace_bytes(const hga_shape* s) {
  return delta_bytes(s) + cmask_bytes(s) + 2 * order_bytes(s);
}
int32_t* order_full(const hga_shape* s, void* ws) {
  return (int32_t*)((uint8_t*)ws + delta_bytes(s) + cmask_bytes(s));
}
int32_t* order_range(const hga_shape* s, void* ws) {
  return (int32_t*)((uint8_t*)ws + delta_bytes(s) + cmask_bytes(s) + order_bytes(s));
}

// Checks shared by block and decode shapes (everything but q_len, kv_len and
// kv_capacity).
hga_status validate_common(const hga_shape* s) {
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1) return HGA_ERR_SHAPE;
  if (s->n_q_heads % s->n_kv_heads != 0) return HGA_ERR_SHAPE;
  if (s->top_k < 0 || s->top_k > HGA_MAX_TOP_K) return HGA_ERR_SHAPE;
  if (s->top_g < 0 || s->top_g > HGA_MAX_TOP_G) return HGA_ERR_SHAPE;
  // NaN or infinite scale (checked on the bit pattern: the library is built
  // with -fno-honor-nans, under which x != x may be folded away)
  uint32_t sbits;
  memcpy(&sbits, &s->softmax_scale, sizeof(sbits));
  if ((sbits & 0x7F800000u) == 0x7F800000u) return HGA_ERR_SHAPE;
  return HGA_OK;
}

}  // namespace

extern "C" {

int hga_abi_version(void) { return HGA_ABI_VERSION; }

const char* hga_status_str(hga_status s) {
  switch (s) {
    case HGA_OK: return "ok";
    case HGA_ERR_NULL: return "a required pointer is NULL";
    case HGA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case HGA_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case HGA_ERR_WORKSPACE: return "workspace missing or too small";
    case HGA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

hga_status hga_validate_shape(const hga_shape* s) {
  if (!s) return HGA_ERR_NULL;
  hga_status st = validate_common(s);
  if (st != HGA_OK) return st;
  if (s->q_len < HGA_QBLOCK || s->q_len % HGA_QBLOCK != 0) return HGA_ERR_SHAPE;
  if (s->kv_len % HGA_CHUNK != 0 || s->kv_len < s->q_len || s->kv_len > HGA_MAX_KV_LEN)
    return HGA_ERR_SHAPE;
  if (s->kv_capacity != 0 && (s->kv_capacity < s->kv_len || s->kv_capacity % HGA_CHUNK != 0 ||
                              s->kv_capacity > HGA_MAX_KV_LEN))
    return HGA_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return HGA_ERR_UNSUPPORTED;
  if (s->dtype != HGA_DTYPE_BF16 && s->dtype != HGA_DTYPE_FP32) return HGA_ERR_UNSUPPORTED;
  // launch sizes must fit a 32-bit grid
  const long long rows = (long long)s->batch * s->n_q_heads * (s->q_len / HGA_QBLOCK);
  const long long cap = s->kv_capacity > 0 ? s->kv_capacity : s->kv_len;
  const long long chunks = (long long)s->batch * s->n_kv_heads * (cap / HGA_CHUNK);
  if (rows > (1LL << 30) || chunks > (1LL << 30)) return HGA_ERR_SHAPE;
  // routing rows of one kv head must fit the 23-bit row field of the backward entry list
  if ((long long)(s->n_q_heads / s->n_kv_heads) * (s->q_len / HGA_QBLOCK) >= (1LL << 23))
    return HGA_ERR_SHAPE;
  return HGA_OK;
}

hga_status hga_validate_decode_shape(const hga_shape* s) {
  if (!s) return HGA_ERR_NULL;
  hga_status st = validate_common(s);
  if (st != HGA_OK) return st;
  if (s->q_len != 1 || s->kv_len < 1 || s->kv_len > HGA_MAX_KV_LEN) return HGA_ERR_SHAPE;
  const long long cap = s->kv_capacity > 0 ? s->kv_capacity : s->kv_len;
  if (s->kv_capacity < 0 || cap < s->kv_len || cap % HGA_CHUNK != 0 || cap > HGA_MAX_KV_LEN)
    return HGA_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return HGA_ERR_UNSUPPORTED;
  if (s->dtype != HGA_DTYPE_BF16 && s->dtype != HGA_DTYPE_FP32) return HGA_ERR_UNSUPPORTED;
  // one workgroup per (b, query head); summaries rows as for block shapes
  if ((long long)s->batch * s->n_q_heads > (1LL << 30) ||
      (long long)s->batch * s->n_kv_heads * (cap / HGA_CHUNK) > (1LL << 30))
    return HGA_ERR_SHAPE;
  return HGA_OK;
}

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
  return from_hip(hga::launch_summaries(dims_of(shape), K, chunk_mean, group_mean, chunk_begin,
                                        chunk_end, (hipStream_t)stream));
}

hga_status hga_route(const hga_shape* shape, const void* Q, const float* chunk_mean,
                     const float* group_mean, int32_t* chunk_idx, int32_t* group_idx,
                     void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !chunk_mean) return HGA_ERR_NULL;
  if (shape->top_g > 0 && (!group_idx || !group_mean)) return HGA_ERR_NULL;
  if (shape->top_k == 0 && shape->top_g == 0 && !group_idx && !chunk_idx) return HGA_OK;
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
  if (!routes && !group_idx && !chunk_idx) return HGA_OK;
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

hga_status hga_attend_bwd_workspace(const hga_shape* shape, size_t* bytes) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!bytes) return HGA_ERR_NULL;
  *bytes = workspace_bytes(shape);
  return HGA_OK;
}

hga_status hga_attend_bwd_dq(const hga_shape* shape, const void* Q, const void* K,
                             const void* V, const void* O, const float* lse, const void* dO,
                             const int32_t* group_idx, void* dQ, void* workspace,
                             size_t workspace_bytes, void* stream) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !O || !lse || !dO || !dQ) return HGA_ERR_NULL;
  if (shape->top_g > 0 && !group_idx) return HGA_ERR_NULL;
  if (!workspace || workspace_bytes < ::workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
  return from_hip(hga::launch_attend_bwd_dq(
      dims_of(shape), Q, K, V, O, lse, dO, group_idx, dQ, (float*)workspace,
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
  if (!workspace || workspace_bytes < ::workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
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
  if (!workspace || workspace_bytes < ::workspace_bytes(shape)) return HGA_ERR_WORKSPACE;
  st = hga_attend_bwd_dq(shape, Q, K, V, O, lse, dO, group_idx, dQ, workspace, workspace_bytes,
                         stream);
  if (st != HGA_OK) return st;
  return hga_attend_bwd_dkdv(shape, Q, K, V, lse, dO, group_idx, dK, dV, workspace,
                             workspace_bytes, stream);
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
