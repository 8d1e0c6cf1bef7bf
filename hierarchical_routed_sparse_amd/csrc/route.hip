// Two-level routing: block query -> top-k chunks -> top-g groups.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": a query block scores the chunk summaries, keeps the top-k
// chunks, opens those chunks at the 8-token group level and keeps the best
// groups; section "The one real caveat: causal leakage" notes that routing
// within a block depends on several query positions, which is why the block
// is routed as a whole (its routing query is the mean of its 64 queries).
//
// One wavefront owns one routing row (b, hq, block); a workgroup holds four
// rows, ordered so that the query heads of one kv head and one block sit in
// the same workgroup (they read the same summaries) and the rows of one kv
// head stay on one XCD.  Per row:
//   1. block query = mean of the 64 query rows (fp32);
//   2. lane l scores chunks l, l+64, ... (fp32 dot products, fixed order);
//   3. top-k by a wave-level radix select on order-preserving 32-bit keys:
//      32 rounds of ballot/popcount fix the k-th largest key bit by bit; ties
//      at that key are resolved toward the lower index by a ballot prefix
//      count, and kept indices are compacted in ascending order the same way;
//   4. the 8 groups of every kept chunk are scored and the top-g taken jointly
//      with the same selection.
#include "hga_device.h"
#include "hga_kernels.h"

namespace hga {
namespace {

constexpr int kMaxTopK = 64;
constexpr int kGroupSlots = 8;  // up to 512 group candidates per row

struct RouteP {
  const void* Q;
  const float* cm;
  const float* gm;
  int32_t* cidx;
  int32_t* gidx;
  int B, Hq, Hkv, Sq, Skv, q0, nblk, top_k, top_g, nrows;
};

// Order-preserving map from finite fp32 to uint32 (larger float -> larger key).
// -0.0 is mapped like +0.0 so that the two rank equal.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = s == 0.0f ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Marks the kk best of the n candidates held as key[j] by lane l for candidate
// index 64*j + l (best = larger key, then lower index).
template <int NS>
__device__ __forceinline__ void select_best(const uint32_t (&key)[NS], int n, int kk, bool (&sel)[NS]) {
  const int lane = lane_id();
  if (kk >= n) {
#pragma unroll
    for (int j = 0; j < NS; ++j) sel[j] = 64 * j + lane < n;
    return;
  }
  if (kk <= 0) {
#pragma unroll
    for (int j = 0; j < NS; ++j) sel[j] = false;
    return;
  }
  // largest threshold T with #{key >= T} >= kk, i.e. the kk-th largest key
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (64 * j < n) cnt += __popcll(__ballot(64 * j + lane < n && key[j] >= trial));
    if (cnt >= kk) T = trial;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (64 * j < n) gt += __popcll(__ballot(64 * j + lane < n && key[j] > T));
  const int need = kk - gt;  // how many of the candidates equal to T are kept
  int eq_before = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    sel[j] = false;
    if (64 * j < n) {
      const bool valid = 64 * j + lane < n;
      const bool eq = valid && key[j] == T;
      const uint64_t m = __ballot(eq);
      const int rank = eq_before + mbcnt(m);
      sel[j] = valid && (key[j] > T || (eq && rank < need));
      eq_before += __popcll(m);
    }
  }
}

template <int D>
__device__ __forceinline__ float dot_row(const float* qbar, const float* row) {
  const float4* r = reinterpret_cast<const float4*>(row);
  const float4* q = reinterpret_cast<const float4*>(qbar);
  float s = 0.f;
#pragma unroll 8
  for (int i = 0; i < D / 4; ++i) {
    const float4 a = q[i], b = r[i];
    s = fmaf(a.x, b.x, s);
    s = fmaf(a.y, b.y, s);
    s = fmaf(a.z, b.z, s);
    s = fmaf(a.w, b.w, s);
  }
  return s;
}

template <typename T, int D, int NSC>
__global__ __launch_bounds__(kThreads) void route_kernel(const RouteP p) {
  __shared__ __attribute__((aligned(16))) float s_qbar[4][D];
  __shared__ int s_chunk[4][kMaxTopK];

  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int rowid = xcd_remap(blockIdx.x, gridDim.x) * 4 + wv;
  const bool live = rowid < p.nrows;
  // row order: (b, hkv, block, query head within the kv group)
  const int r = p.Hq / p.Hkv;
  int t = live ? rowid : 0;
  const int hql = t % r;
  t /= r;
  const int blk = t % p.nblk;
  t /= p.nblk;
  const int hkv = t % p.Hkv, b = t / p.Hkv;
  const int hq = hkv * r + hql;
  const int cb = p.q0 / kChunk + blk;                 // the block's own chunk
  const long long orow = ((long long)b * p.Hq + hq) * p.nblk + blk;
  const long long nch = p.Skv / kChunk;

  // 1. block query
  if (live) {
    constexpr int E = D / 64;
    const T* Qb = reinterpret_cast<const T*>(p.Q) + (((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk) * D + lane * E;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int i = 0; i < kChunk; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += to_f32(Qb[(long long)i * D + e]);
#pragma unroll
    for (int e = 0; e < E; ++e) s_qbar[wv][lane * E + e] = acc[e] * (1.0f / 64.0f);
  }
  __syncthreads();
  const float* qbar = s_qbar[wv];

  // 2-3. chunk scores over the cb chunks before the own chunk, top-k
  const int nc = live ? cb : 0;
  const int kk = nc < p.top_k ? nc : p.top_k;
  if (live) {
    const float* cmb = p.cm + ((long long)b * p.Hkv + hkv) * nch * D;
    uint32_t key[NSC];
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      key[j] = 0;
      const int c = 64 * j + lane;
      if (64 * j < nc && c < nc) key[j] = order_key(dot_row<D>(qbar, cmb + (long long)c * D));
    }
    bool sel[NSC];
    select_best<NSC>(key, nc, kk, sel);
    int base = 0;
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      if (64 * j < nc) {
        const uint64_t m = __ballot(sel[j]);
        if (sel[j]) {
          const int pos = base + mbcnt(m);
          s_chunk[wv][pos] = 64 * j + lane;
          if (p.cidx) p.cidx[orow * p.top_k + pos] = 64 * j + lane;
        }
        base += __popcll(m);
      }
    }
    if (p.cidx)
      for (int i = kk + lane; i < p.top_k; i += 64) p.cidx[orow * p.top_k + i] = -1;
  }
  __syncthreads();

  // 4. group scores over the 8 groups of every kept chunk, joint top-g
  if (live && p.gidx) {
    const int ng = 8 * kk;
    const int gg = ng < p.top_g ? ng : p.top_g;
    const float* gmb = p.gm + ((long long)b * p.Hkv + hkv) * nch * 8 * D;
    uint32_t key[kGroupSlots];
    int gam[kGroupSlots];
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      key[j] = 0;
      gam[j] = -1;
      const int i = 64 * j + lane;
      if (64 * j < ng && i < ng) {
        gam[j] = s_chunk[wv][i >> 3] * 8 + (i & 7);
        key[j] = order_key(dot_row<D>(qbar, gmb + (long long)gam[j] * D));
      }
    }
    bool sel[kGroupSlots];
    select_best<kGroupSlots>(key, ng, gg, sel);
    int base = 0;
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      if (64 * j < ng) {
        const uint64_t m = __ballot(sel[j]);
        if (sel[j]) p.gidx[orow * p.top_g + base + mbcnt(m)] = gam[j];
        base += __popcll(m);
      }
    }
    for (int i = gg + lane; i < p.top_g; i += 64) p.gidx[orow * p.top_g + i] = -1;
  }
}

template <typename T, int D, int NSC>
hipError_t run(const Dims& d, const void* Q, const float* cm, const float* gm, int32_t* ci,
               int32_t* gi, hipStream_t s) {
  RouteP p;
  p.Q = Q; p.cm = cm; p.gm = gm; p.cidx = ci; p.gidx = gi;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_k = d.top_k; p.top_g = d.top_g;
  p.nrows = d.B * d.Hq * d.nblk;
  const int nwg = (p.nrows + 3) / 4;
  route_kernel<T, D, NSC><<<nwg, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_d(const Dims& d, const void* Q, const float* cm, const float* gm, int32_t* ci,
                 int32_t* gi, hipStream_t s) {
  const int max_cand = d.Skv / kChunk - 1;   // chunks before the last block's own chunk
  if (max_cand <= 256) return run<T, D, 4>(d, Q, cm, gm, ci, gi, s);
  if (max_cand <= 1024) return run<T, D, 16>(d, Q, cm, gm, ci, gi, s);
  return run<T, D, 32>(d, Q, cm, gm, ci, gi, s);
}

}  // namespace

hipError_t launch_route(const Dims& d, const void* Q, const float* chunk_mean,
                        const float* group_mean, int32_t* chunk_idx, int32_t* group_idx,
                        hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run_d<uint16_t, 128>(d, Q, chunk_mean, group_mean, chunk_idx, group_idx, s)
                      : run_d<uint16_t, 64>(d, Q, chunk_mean, group_mean, chunk_idx, group_idx, s);
  return d.D == 128 ? run_d<float, 128>(d, Q, chunk_mean, group_mean, chunk_idx, group_idx, s)
                    : run_d<float, 64>(d, Q, chunk_mean, group_mean, chunk_idx, group_idx, s);
}

}  // namespace hga
