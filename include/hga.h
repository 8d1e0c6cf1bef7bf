/*
 * hga.h -- C ABI of the MI355X (gfx950) Hierarchical Global Attention library.
 *
 * Source of the method: the page "BMW's 16 GB GPU just did what needs an
 * A100" (seventnews.com, English edition), section "What HGA does
 * differently".  HGA replaces the attention module; for every block of queries
 * it routes over compact per-chunk summaries of the keys (64-token chunks),
 * keeps the best chunks, opens them at the level of 8-token groups, keeps the
 * best groups, and attends only the exact key/value tokens of those groups.
 * The router has no weights: it scores the existing projected keys, and the
 * summaries only steer selection (they are never keys or values).
 *
 * Readings fixed by this library where the page is silent:
 *   - chunk summary = mean of the chunk's 64 keys; group summary = mean of the
 *     group's 8 keys (both fp32);
 *   - a query block is 64 consecutive queries; its routing query is the mean of
 *     those 64 query vectors, and a score is the plain dot product (fp32);
 *   - routing is per query head; query head h reads kv head h / (Hq / Hkv);
 *   - the candidates of a block are the chunks strictly before the block's own
 *     chunk; the own chunk is always attended, causally;
 *   - top_g is chosen jointly over all 8 * kept-chunk groups;
 *   - ranking is (score descending, index ascending); -0.0 ranks equal to +0.0;
 *   - kept indices are written in ascending order, padded with -1;
 *   - softmax scale 1/sqrt(head_dim) unless given; lse in natural log;
 *   - the backward holds routing fixed (no gradient through the selection).
 *
 * Conventions for every call:
 *   - all tensor pointers are DEVICE pointers to contiguous row-major buffers
 *     owned by the caller, 16-byte aligned; outputs must not alias inputs; K
 *     and V may be the GPU address of pinned host memory (hipHostMalloc,
 *     hipHostGetDevicePointer): the kernels then read the rows they gather
 *     across the host link;
 *   - Q, O, dO, dQ are [B][Hq][q_len][D]; K, V, dK, dV are [B][Hkv][C][D]
 *     with C = kv_capacity (kv_len when 0): rows kv_len..C-1 of each
 *     (b, kv head) are not read, so a history that grows segment by segment
 *     can live in buffers sized once; the q_len queries are the LAST q_len
 *     positions of the kv_len-long sequence (a segment at the end of its
 *     history; q_len == kv_len is plain causal self-attention);
 *   - the summaries are [B][Hkv][C/64][D] (chunks) and [B][Hkv][C/8][D]
 *     (groups), rows past kv_len/64 (kv_len/8) unused;
 *   - element type of Q, K, V, O, dO, dQ, dK, dV is shape->dtype (bf16 or fp32);
 *     summaries, lse and the workspace are fp32; indices are int32;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); every
 *     call only enqueues work on it: no allocation, no synchronisation, no
 *     host<->device copy, no pointer kept after return;
 *   - argument errors are reported before anything is launched and leave every
 *     output untouched; a failed launch returns HGA_ERR_HIP; faults inside a
 *     kernel surface at the caller's next synchronisation;
 *   - calls are re-entrant: the library holds no mutable global state.
 */
#ifndef HGA_H_
#define HGA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HGA_ABI_VERSION 11
#define HGA_CHUNK 64      /* tokens per chunk (the page's 64-token chunks) */
#define HGA_GROUP 8       /* tokens per group (the page's 8-token groups)  */
#define HGA_QBLOCK 64     /* queries per routing block                      */
#define HGA_MAX_TOP_K 64
#define HGA_MAX_TOP_G 512
#define HGA_MAX_KV_LEN 131072

typedef enum {
  HGA_OK = 0,
  HGA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  HGA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes              */
  HGA_ERR_UNSUPPORTED = 3, /* valid but unsupported (head_dim, dtype)         */
  HGA_ERR_WORKSPACE = 4,   /* workspace missing or too small                  */
  HGA_ERR_HIP = 5          /* a HIP launch failed                             */
} hga_status;

typedef enum { HGA_DTYPE_BF16 = 0, HGA_DTYPE_FP32 = 1 } hga_dtype;

typedef struct {
  int32_t batch;        /* B  >= 1                                            */
  int32_t n_q_heads;    /* Hq >= 1, a multiple of n_kv_heads                  */
  int32_t n_kv_heads;   /* Hkv >= 1                                           */
  int32_t head_dim;     /* D in {64, 128}                                     */
  int32_t q_len;        /* multiple of 64, 64 <= q_len <= kv_len              */
  int32_t kv_len;       /* multiple of 64, <= HGA_MAX_KV_LEN                  */
  int32_t top_k;        /* chunks kept per block, 0..HGA_MAX_TOP_K            */
  int32_t top_g;        /* groups kept per block, 0..HGA_MAX_TOP_G            */
  float softmax_scale;  /* <= 0 selects 1/sqrt(head_dim)                      */
  int32_t dtype;        /* hga_dtype                                          */
  int32_t kv_capacity;  /* rows allocated per (b, kv head) in K, V, dK, dV:   */
                        /* 0 (= kv_len) or a multiple of 64 in                */
                        /* [kv_len, HGA_MAX_KV_LEN]                           */
} hga_shape;

/* ABI version (HGA_ABI_VERSION of the built library). */
int hga_abi_version(void);

/* Static text for a status code. */
const char* hga_status_str(hga_status s);

/* Host-only check of a shape against the limits above; touches no device. */
hga_status hga_validate_shape(const hga_shape* shape);

/* Host-only check of a decode shape (see hga_decode): q_len == 1,
 * 1 <= kv_len <= HGA_MAX_KV_LEN, C = kv_capacity (kv_len when 0) a multiple
 * of 64 in [kv_len, HGA_MAX_KV_LEN], the other fields as for any shape. */
hga_status hga_validate_decode_shape(const hga_shape* shape);

/* Chunk and group summaries of K (page section "What HGA does differently":
 * one compact summary vector per 64-token chunk stays resident in GPU memory;
 * the 8-token group summaries serve the second routing level).
 *   K          [B][Hkv][C][D]                dtype (C = kv_capacity or kv_len)
 *   chunk_mean [B][Hkv][C/64][D]             fp32, written for chunks in
 *                                            [chunk_begin, chunk_end) only
 *   group_mean [B][Hkv][C/8][D]              fp32, written for the groups of
 *                                            those chunks only
 * 0 <= chunk_begin <= chunk_end <= kv_len/64 (complete chunks only).  The
 * range lets a caller append the summaries of new chunks to a resident history
 * without rebuilding it.  A decode shape (q_len == 1, see hga_decode) is
 * accepted too: a decoder appends chunk c once its 64 keys are in the cache. */
hga_status hga_build_summaries(const hga_shape* shape, const void* K, float* chunk_mean,
                               float* group_mean, int32_t chunk_begin, int32_t chunk_end,
                               void* stream);

/* hga_build_summaries with the keys read from a buffer that holds a range of
 * positions only (same page passage; for the active segment in GPU memory
 * while the history lives in host RAM):
 *   K_rows     [B][Hkv][rows][D] dtype: positions row0 .. row0 + rows - 1;
 *              row0 >= 0 and rows > 0 multiples of 64, row0 + rows <= kv_len
 *   [chunk_begin, chunk_end) within [row0 / 64, (row0 + rows) / 64)
 * The summaries are written exactly as hga_build_summaries writes them from
 * a K holding the same keys at those positions. */
hga_status hga_build_summaries_rows(const hga_shape* shape, const void* K_rows, int32_t row0,
                                    int32_t rows, float* chunk_mean, float* group_mean,
                                    int32_t chunk_begin, int32_t chunk_end, void* stream);

/* Two-level routing (page section "What HGA does differently": score the
 * chunk summaries, keep the top-k chunks, open them at group level, keep the
 * best groups).  One routing row per (b, hq, block of 64 queries).
 *   Q          [B][Hq][q_len][D]                       dtype
 *   chunk_mean, group_mean                             as built above (all
 *                                                      chunks before the last
 *                                                      query block's own chunk
 *                                                      must be built)
 *   chunk_idx  [B][Hq][q_len/64][top_k]  int32, nullable when top_k == 0 or
 *                                        the caller does not want it
 *   group_idx  [B][Hq][q_len/64][top_g]  int32, nullable only when top_g == 0
 * Row (b, hq, blk) keeps min(top_k, c) chunks among the c = (kv_len-q_len)/64
 * + blk chunks before its own, then min(top_g, 8 * kept) groups of those
 * chunks; both lists ascending, -1 padded. */
hga_status hga_route(const hga_shape* shape, const void* Q, const float* chunk_mean,
                     const float* group_mean, int32_t* chunk_idx, int32_t* group_idx,
                     void* stream);

/* Strictly causal routing (page section "The one real caveat: causal leakage":
 * a block's routing mixes its query positions, so earlier tokens learn about
 * later ones; the page mentions a strictly causal variant without giving one).
 * As hga_route, except that block j is routed with the mean of the 64 queries
 * just before it: block j-1 of Q, or for the first block the 64 rows of
 * Q_prev.  No position's key set then depends on a later position.
 *   Q_prev     [B][Hq][64][D] dtype, the 64 queries before the segment
 *              (positions kv_len-q_len-64 .. kv_len-q_len-1); required when
 *              kv_len > q_len and top_k or top_g is non-zero, else not read
 * The first block of a sequence (kv_len == q_len) has no candidate chunk and
 * attends its own chunk only, as in hga_route.  Outputs as hga_route; the
 * attention and backward calls take them unchanged. */
hga_status hga_route_causal(const hga_shape* shape, const void* Q, const void* Q_prev,
                            const float* chunk_mean, const float* group_mean,
                            int32_t* chunk_idx, int32_t* group_idx, void* stream);

/* Exact-token attention forward (page section "What HGA does differently":
 * attention runs on the exact tokens of the kept groups).  The query at
 * absolute position p of block blk attends every token of the row's kept
 * groups plus its own chunk's tokens up to and including p.
 *   group_idx  [B][Hq][q_len/64][top_g]  int32, as produced by hga_route
 *              (ascending, -1 padded, every group before the own chunk).
 *              The kept groups of a row are its longest prefix of entries
 *              that lie in [0, 8 * own chunk) and each exceed the entry
 *              before them: for a row written by hga_route, exactly its
 *              non-negative entries.  Any other row is cut at its first entry
 *              that breaks this rule, so no group is read out of range or
 *              attended twice.  The backward and decode calls read rows by
 *              the same rule.
 *   O          [B][Hq][q_len][D]         dtype
 *   lse        [B][Hq][q_len]            fp32 natural-log log-sum-exp of the
 *                                        scaled logits, nullable */
hga_status hga_attend_fwd(const hga_shape* shape, const void* Q, const void* K, const void* V,
                          const int32_t* group_idx, void* O, float* lse, void* stream);

/* Workspace bytes needed by the backward calls: the fp32 row statistics
 * delta [B][Hq][q_len], then a byte map [B][Hq][q_len/64][kv_len/64] whose
 * entry (routing row, chunk c) holds the mask of the row's kept groups in
 * chunk c (bit t = group 8c + t), then two int32 work orders of the dK/dV
 * workgroups [B][Hkv][kv_len/64] (each kv head's chunks, most attended
 * first): the whole range's, written by the dQ call, and a chunk sub-range's,
 * written by hga_attend_bwd_dkdv_range itself.  Each part is rounded up to
 * 256 bytes. */
hga_status hga_attend_bwd_workspace(const hga_shape* shape, size_t* bytes);

/* Backward through the exact-token attention with the routing held fixed
 * (page section "What HGA does differently": the router has no weights and
 * gradients reach the same Q/K/V projections as dense attention).
 *   O, lse     outputs of hga_attend_fwd for the same inputs
 *   group_idx  as for hga_attend_fwd (same prefix rule)
 *   dO         [B][Hq][q_len][D]   dtype
 *   dQ         [B][Hq][q_len][D]   dtype
 *   dK, dV     [B][Hkv][C][D] dtype; every position below kv_len is written
 *              (zero where no query attends); the sum over the Hq/Hkv query heads
 *              of a kv head is formed in a fixed order, so results are
 *              bitwise reproducible
 *   workspace  device buffer of at least hga_attend_bwd_workspace() bytes */
hga_status hga_attend_bwd(const hga_shape* shape, const void* Q, const void* K, const void* V,
                          const void* O, const float* lse, const void* dO,
                          const int32_t* group_idx, void* dQ, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream);

/* hga_attend_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results, with the workspace taken from a device
 * array of HGA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on (until the process ends).  The call allocates nothing; the caller
 * still passes every input and output as for hga_attend_bwd.
 * Returns HGA_ERR_WORKSPACE when hga_attend_bwd_workspace(shape) exceeds
 * HGA_NOALLOC_SCRATCH_BYTES, and HGA_ERR_HIP when the array's device address
 * cannot be resolved.  All calls on one GPU share that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race on it and
 * must be serialised by the caller.  The array keeps the last call's contents;
 * nothing in it needs clearing between calls. */
#define HGA_NOALLOC_SCRATCH_BYTES (16u << 20)
hga_status hga_attend_bwd_noalloc(const hga_shape* shape, const void* Q, const void* K,
                                  const void* V, const void* O, const float* lse,
                                  const void* dO, const int32_t* group_idx, void* dQ, void* dK,
                                  void* dV, void* stream);

/* The two halves of hga_attend_bwd, for callers that schedule them apart.
 * hga_attend_bwd_dq computes dQ and writes the row statistics
 * delta = rowsum(dO * O), the group-mask map and the dK/dV work order of the
 * whole chunk range into the workspace; hga_attend_bwd_dkdv then reads them
 * from the same workspace and computes dK and dV.  The dkdv call must follow
 * a dq call with the same inputs, on the same stream (or after it has
 * completed), or a hga_attend_bwd_prep call (below).  A dkdv call on a
 * workspace that neither wrote gives unspecified dK/dV values but never
 * writes outside dK and dV: work-order entries outside the chunk range are
 * skipped.
 * hga_attend_bwd_dq with workspace == NULL and workspace_bytes == 0 computes
 * dQ only and touches no workspace. */
hga_status hga_attend_bwd_dq(const hga_shape* shape, const void* Q, const void* K,
                             const void* V, const void* O, const float* lse, const void* dO,
                             const int32_t* group_idx, void* dQ, void* workspace,
                             size_t workspace_bytes, void* stream);
hga_status hga_attend_bwd_dkdv(const hga_shape* shape, const void* Q, const void* K,
                               const void* V, const float* lse, const void* dO,
                               const int32_t* group_idx, void* dK, void* dV,
                               void* workspace, size_t workspace_bytes, void* stream);

/* What hga_attend_bwd_dq writes into the workspace (delta, the group-mask map,
 * the whole range's dK/dV work order), computed from O, dO and the routing
 * alone, without dQ: after it, hga_attend_bwd_dkdv and a workspace-free
 * hga_attend_bwd_dq depend on nothing but their inputs, so a caller may run
 * them side by side on two streams (page section "What HGA does differently":
 * the backward reaches Q, K and V as in dense attention; the two gradients
 * are independent given the forward's outputs).  dK/dV after it are bitwise
 * those after hga_attend_bwd_dq.
 *   O, dO      [B][Hq][q_len][D] dtype; group_idx as for hga_attend_fwd */
hga_status hga_attend_bwd_prep(const hga_shape* shape, const void* O, const void* dO,
                               const int32_t* group_idx, void* workspace,
                               size_t workspace_bytes, void* stream);

/* hga_attend_bwd_dkdv restricted to the keys of chunks [chunk_begin,
 * chunk_end): only those rows of dK and dV are written (every row in the
 * range, zero where no query attends); the other rows are left untouched and
 * cost nothing.  This is the backward of segment-wise training (page section
 * "What HGA does differently": each 2,048-token segment runs forward and
 * backward on its own and older keys/values are detached), where only the
 * segment's own keys take gradients: chunk_begin = (kv_len - q_len) / 64,
 * chunk_end = kv_len / 64.  0 <= chunk_begin <= chunk_end <= kv_len / 64.
 * Same workspace contract as hga_attend_bwd_dkdv. */
hga_status hga_attend_bwd_dkdv_range(const hga_shape* shape, const void* Q, const void* K,
                                     const void* V, const float* lse, const void* dO,
                                     const int32_t* group_idx, int32_t chunk_begin,
                                     int32_t chunk_end, void* dK, void* dV, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* The routed working set of a segment in device memory (page section "What
 * HGA does differently", memory paragraph: GPU memory holds the summaries, the
 * active segment and the routed working set, while older keys and values live
 * in host RAM).  After routing a segment (q_len queries at the end of kv_len,
 * its K and V typically pinned host memory), this call copies, per (b, kv
 * head), the distinct history groups its rows kept (their union, ascending)
 * and then the segment's own rows into a compact device buffer, and rewrites
 * every routing row against it.  The attention and backward calls then take
 * the staged shape: q_len as given, kv_len = 8 * stage_groups + q_len,
 * kv_capacity = stage_capacity, with K_stage, V_stage and group_idx_staged;
 * O, lse, dQ and the segment's dK/dV rows (chunks stage_groups / 8 onwards)
 * equal those over the full history bit for bit.
 *   group_idx         [B][Hq][q_len/64][top_g] as written by the routing
 *                     (read by the prefix rule of hga_attend_fwd)
 *   K, V              [B][Hkv][C][D] dtype, the full history (C =
 *                     kv_capacity or kv_len)
 *   stage_groups      group slots of the staged history, a multiple of 8, at
 *                     least hga_stage_min_groups(shape) (the union always
 *                     fits) and at most HGA_MAX_KV_LEN / 8; hga_stage_workspace
 *                     returns HGA_ERR_SHAPE for a negative value, one not a
 *                     multiple of 8 or one above that bound
 *   stage_capacity    rows per (b, kv head) of K_stage and V_stage, a
 *                     multiple of 64, >= 8 * stage_groups + q_len
 *   K_stage, V_stage  [B][Hkv][stage_capacity][D] dtype, device memory:
 *                     rows 8k..8k+7 = union group k; rows 8 * stage_groups ..
 *                     + q_len - 1 = the segment; slots past the union are
 *                     not written
 *   group_idx_staged  [B][Hq][q_len/64][top_g] int32: a history group g ->
 *                     its rank in the union, a group of the segment ->
 *                     g - 8 (kv_len - q_len)/64 + stage_groups, -1 padded
 *   workspace         hga_stage_workspace(shape, stage_groups) bytes: the
 *                     unions ([B][Hkv][stage_groups] int32), their sizes
 *                     ([B][Hkv] int32) and the copy sources of the union slots
 *                     ([B][Hkv][stage_groups] int32), each rounded up to 256
 *                     bytes */
int32_t hga_stage_min_groups(const hga_shape* shape);   /* -1 for an invalid shape */
hga_status hga_stage_workspace(const hga_shape* shape, int32_t stage_groups, size_t* bytes);
hga_status hga_stage_routed(const hga_shape* shape, const int32_t* group_idx, const void* K,
                            const void* V, int32_t stage_groups, int32_t stage_capacity,
                            void* K_stage, void* V_stage, int32_t* group_idx_staged,
                            void* workspace, size_t workspace_bytes, void* stream);

/* The previous staging of the same history (the segment before, routed and
 * staged by hga_stage_routed or hga_stage_routed_from), as its caller holds it. */
typedef struct {
  const void* K_stage;      /* its K_stage, V_stage (device), still unchanged       */
  const void* V_stage;
  const void* workspace;    /* its workspace (its unions and their sizes)           */
  size_t workspace_bytes;   /* that workspace's size in bytes                       */
  int32_t stage_groups;     /* its stage_groups                                     */
  int32_t stage_capacity;   /* its stage_capacity                                   */
  int32_t q0;               /* its segment's first position (its kv_len - q_len)    */
  int32_t q_len;            /* its segment's length                                 */
} hga_stage_prev;

/* hga_stage_routed with other sources for the same bytes (page "BMW's 16 GB
 * GPU just did what needs an A100", section "What HGA does differently",
 * memory paragraph: the active segment stays in GPU memory; and consecutive
 * segments share most of their routed working set).  K_stage, V_stage, group_idx_staged and the
 * workspace's unions are exactly those hga_stage_routed writes; only where
 * the rows are copied from differs:
 *   - a union group that the previous staging holds (in its union, or among
 *     its segment's rows) is copied from prev->K_stage / prev->V_stage, in
 *     device memory, instead of from K / V;
 *   - the segment's own rows come from K_seg / V_seg when they are given:
 *     [B][Hkv][q_len][D] dtype, device memory, equal to K's / V's rows
 *     kv_len - q_len .. kv_len - 1;
 *   - every other row comes from K / V as in hga_stage_routed.
 * prev may be NULL (no previous staging); K_seg and V_seg are both NULL or
 * both given.  prev must describe a staging of the same history for the same
 * batch, heads, head_dim and dtype, whose buffers have not been written
 * since: 0 <= prev->stage_groups, a multiple of 8; prev->q0 and prev->q_len
 * multiples of 64, prev->q_len >= 64, prev->q0 + prev->q_len <= kv_len -
 * q_len; prev->stage_capacity a multiple of 64 in [8 * prev->stage_groups +
 * prev->q_len, HGA_MAX_KV_LEN]; prev->workspace_bytes at least the unions and
 * sizes parts of a staging workspace for prev->stage_groups (HGA_ERR_WORKSPACE
 * otherwise).  A prev whose buffers do not hold what that staging wrote
 * gives unspecified staged values but never a read outside prev->K_stage,
 * prev->V_stage and the workspace_bytes of prev->workspace (sizes and ranks
 * are clamped to the stage_groups given).  The workspace is
 * hga_stage_workspace(shape, stage_groups) bytes, as for hga_stage_routed. */
hga_status hga_stage_routed_from(const hga_shape* shape, const int32_t* group_idx, const void* K,
                                 const void* V, const void* K_seg, const void* V_seg,
                                 const hga_stage_prev* prev, int32_t stage_groups,
                                 int32_t stage_capacity, void* K_stage, void* V_stage,
                                 int32_t* group_idx_staged, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Decode: attention of one new token per (b, query head) over a resident
 * key/value cache (page section "What HGA does differently", read for
 * generation, which the page says HGA also serves: the newest token is a
 * query block of one, routed over the resident summaries, and attends exact
 * tokens only).  Routing and attention run as two kernels on `stream`.
 *   shape      a decode shape (hga_validate_decode_shape): q_len == 1;
 *              kv_len = L counts the new token, whose position is p = L - 1
 *   Q          [B][Hq][D]          dtype, the new token's queries
 *   K, V       [B][Hkv][C][D]      dtype, rows 0..p written (row p = the new
 *                                  token's key and value); may be pinned host
 *                                  memory as for every call
 *   chunk_mean [B][Hkv][C/64][D], group_mean [B][Hkv][C/8][D]  fp32: the
 *              summaries of every chunk before the own chunk p/64 must be
 *              built (hga_build_summaries with this shape)
 *   chunk_idx  [B][Hq][top_k]      int32, nullable
 *   group_idx  [B][Hq][top_g]      int32, required when top_g > 0 (written by
 *                                  the routing, read by the attention: its
 *                                  first min(top_g, 8 * kept chunks) entries,
 *                                  cut at the first entry that is negative,
 *                                  not before the own chunk or not above the
 *                                  entry before it)
 *   O          [B][Hq][D]          dtype
 *   lse        [B][Hq]             fp32 natural-log log-sum-exp, nullable
 * Routing: the routing query is the token's query itself; the row keeps
 * min(top_k, p/64) of the chunks before its own chunk, then min(top_g,
 * 8 * kept) groups of those chunks (ascending, -1 padded, ties to the lower
 * index).  Attention: every token of the kept groups plus the own chunk's
 * positions 64 * (p/64) .. p.  No workspace. */
hga_status hga_decode(const hga_shape* shape, const void* Q, const void* K, const void* V,
                      const float* chunk_mean, const float* group_mean, int32_t* chunk_idx,
                      int32_t* group_idx, void* O, float* lse, void* stream);

/* The two halves of hga_decode, same arguments and contract, for callers that
 * schedule them apart: the routing writes group_idx (and chunk_idx), the
 * attention reads group_idx as written by it for the same shape.  Summaries
 * may be NULL when kv_len <= 64 (no candidate chunk). */
hga_status hga_decode_route(const hga_shape* shape, const void* Q, const float* chunk_mean,
                            const float* group_mean, int32_t* chunk_idx, int32_t* group_idx,
                            void* stream);
hga_status hga_decode_attend(const hga_shape* shape, const void* Q, const void* K, const void* V,
                             const int32_t* group_idx, void* O, float* lse, void* stream);

/* Decode routing under strictly causal routing (see hga_route_causal): the
 * token at position p = kv_len - 1 lies in block j = p / 64 and is routed with
 * the mean of the 64 queries of block j - 1 (positions 64(j-1) .. 64j - 1),
 * over the complete chunks before chunk j.  Neither depends on the position
 * within the block, so the result serves every token of block j: a decoder
 * calls this once when a block starts and hga_decode_attend for each token
 * (with that token's own decode shape and the same group_idx).
 *   Q_prev     [B][Hq][64][D] dtype, the 64 queries of block j - 1; not read
 *              when j == 0 (the first block has no candidate chunk)
 *   chunk_mean, group_mean   summaries of chunks 0 .. j-1 built
 *   chunk_idx  [B][Hq][top_k] int32, nullable; group_idx [B][Hq][top_g]
 * Same layouts and status codes as hga_decode_route. */
hga_status hga_decode_route_causal(const hga_shape* shape, const void* Q_prev,
                                   const float* chunk_mean, const float* group_mean,
                                   int32_t* chunk_idx, int32_t* group_idx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H_ */
