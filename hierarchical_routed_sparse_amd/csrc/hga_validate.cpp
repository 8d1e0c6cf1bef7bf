// Host-only entry points of the HGA library: shape validation, status text,
// ABI version, the staging bound and the workspace sizes.  Plain C++ (no HIP):
// it is compiled into libhga.so, and the CPU tests also build it on its own
// with the address and undefined-behaviour sanitizers and drive it over many
// shapes.
#include <string.h>

#include "hga.h"
#include "hga_layout.h"

namespace {

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

// a * b * c <= limit for non-negative factors, without overflow
bool product_at_most(long long a, long long b, long long c, long long limit) {
  if (a < 0 || b < 0 || c < 0) return false;
  if (a == 0 || b == 0 || c == 0) return true;
  if (a > limit / b) return false;
  return a * b <= limit / c;
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
  const long long cap = s->kv_capacity > 0 ? s->kv_capacity : s->kv_len;
  if (!product_at_most(s->batch, s->n_q_heads, s->q_len / HGA_QBLOCK, 1LL << 30) ||
      !product_at_most(s->batch, s->n_kv_heads, cap / HGA_CHUNK, 1LL << 30))
    return HGA_ERR_SHAPE;
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
  if (!product_at_most(s->batch, s->n_q_heads, 1, 1LL << 30) ||
      !product_at_most(s->batch, s->n_kv_heads, cap / HGA_CHUNK, 1LL << 30))
    return HGA_ERR_SHAPE;
  return HGA_OK;
}

int32_t hga_stage_min_groups(const hga_shape* shape) {
  if (hga_validate_shape(shape) != HGA_OK) return -1;
  // the union of a kv head's kept history groups is at most every history
  // group, and at most every row's top_g
  const long long hist = 8LL * ((shape->kv_len - shape->q_len) / HGA_CHUNK);
  const long long sel = (long long)(shape->n_q_heads / shape->n_kv_heads) *
                        (shape->q_len / HGA_QBLOCK) * shape->top_g;
  const long long need = hist < sel ? hist : sel;
  return (int32_t)((need + 7) / 8 * 8);
}

hga_status hga_attend_bwd_workspace(const hga_shape* shape, size_t* bytes) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!bytes) return HGA_ERR_NULL;
  *bytes = hga_layout::bwd_workspace_bytes(shape);
  return HGA_OK;
}

hga_status hga_stage_workspace(const hga_shape* shape, int32_t stage_groups, size_t* bytes) {
  hga_status st = hga_validate_shape(shape);
  if (st != HGA_OK) return st;
  if (!bytes) return HGA_ERR_NULL;
  if (stage_groups < 0 || stage_groups % 8 != 0 || stage_groups > HGA_MAX_KV_LEN / 8)
    return HGA_ERR_SHAPE;
  *bytes = hga_layout::stage_workspace_bytes(shape, stage_groups);
  return HGA_OK;
}

}  // extern "C"
