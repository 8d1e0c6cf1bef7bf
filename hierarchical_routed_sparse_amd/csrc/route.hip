// Two-level routing: block query -> top-k chunks -> top-g groups.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": a query block scores the chunk summaries, keeps the top-k
// chunks, opens those chunks at the 8-token group level and keeps the best
// groups; section "The one real caveat: causal leakage" notes that routing
// within a block depends on several query positions, which is why the block
// is routed as a whole (its routing query is the mean of its 64 queries).
//
// One workgroup per (b, kv head, block, set of RW query heads of that kv head;
// RW = 2 by default, measured best against 1 and 4); those rows share the
// candidate chunks and the summaries.
//   1. each wavefront computes one row's block query (mean of its 64 query
//      rows: 16 independent 16-byte loads per lane, then a cross-lane sum);
//      in decode (a block of one query, QB = 1) the block query is the query;
//   2. chunk scores: eight lanes share one summary row (whole 128-byte lines
//      per load), each summary is loaded once for all rows of the set, and the
//      block queries stay in registers (fp32, fixed summation order); scores
//      go to LDS;
//   3. wavefront r selects row r's top-k by a wave-level radix select on
//      order-preserving 32-bit keys: the k-th largest key is fixed bit by bit
//      from the top, each round counting the keys at or above the trial
//      threshold with ballots and scalar popcounts, stopping as soon as exactly
//      k keys are at or above it; ties at the threshold go to the lower index
//      by a ballot prefix count, and kept indices are compacted in ascending
//      order the same way;
//   4. wavefront r scores the 8 groups of every kept chunk of row r (one
//      chunk's 8 consecutive group summaries per step, eight steps in flight,
//      scores to LDS), then takes row r's top-g jointly with the same
//      selection.
#include "hga_device.h"
#include "hga_kernels.h"

namespace hga {
namespace {

constexpr int kMaxTopK = 64;
#ifndef HGA_ROUTE_CHUNK_UNROLL
#define HGA_ROUTE_CHUNK_UNROLL 4
#endif
constexpr int kChunkUnroll = HGA_ROUTE_CHUNK_UNROLL;   // chunk-summary steps in flight per wavefront
constexpr int kGroupUnroll = 8;                        // group-summary steps in flight per wavefront

struct RouteP {
  const void* Q;
  const void* Qprev;   // causal: the 64 queries before the segment, [B][Hq][64][D]
  int causal;          // route block j with the mean of the 64 queries before it
  const float* cm;
  const float* gm;
  int32_t* cidx;
  int32_t* gidx;
  int B, Hq, Hkv, Sq, Skv, Scap, q0, nblk, top_k, top_g, nsets, nwork;
};

// Order-preserving map from finite fp32 to uint32 (larger float -> larger key).
// -0.0 is mapped like +0.0 so that the two rank equal.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = s == 0.0f ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Marks the kk best of the n candidates held as key[j] by lane l for candidate
// index 64*j + l (best = larger key, then lower index).  Slots and lanes past
// the n-th candidate must hold key 0: every real key is >= 0x00800000 (see
// order_key) and every trial threshold is >= 1, so they are never counted and
// the loops need no per-slot guards (no divergent branches).
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
  // largest threshold T with #{key >= T} >= kk, i.e. the kk-th largest key,
  // fixed bit by bit from the top.  The wave-wide counts are popcounts of
  // ballots (scalar unit), so T stays in a scalar register; with few slots one
  // ballot per slot, with many a per-lane count and one ballot per bit of it.
  // Once exactly kk keys are >= T the kept set is decided: every key >= T,
  // which the tie step below also yields (it keeps all keys equal to T).
  uint32_t T = 0;
  for (uint32_t bm = 0x80000000u; bm != 0; bm >>= 1) {
    // wave-uniform: kept in a scalar register (the comparisons take it as
    // their scalar operand)
    const uint32_t trial = __builtin_amdgcn_readfirstlane(T | bm);
    int tot = 0;
    if constexpr (NS <= 8) {
#pragma unroll
      for (int j = 0; j < NS; ++j) tot += __popcll(__ballot(key[j] >= trial));
    } else {
      constexpr int NB = NS < 16 ? 4 : NS < 32 ? 5 : 6;   // bits of a count <= NS
      int c = 0;
#pragma unroll
      for (int j = 0; j < NS; ++j) c += key[j] >= trial ? 1 : 0;
#pragma unroll
      for (int q = 0; q < NB; ++q) tot += __popcll(__ballot((c >> q) & 1)) << q;
    }
    if (tot >= kk) {
      T = trial;
      if (tot == kk) break;
    }
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) gt += __popcll(__ballot(key[j] > T));
  const int need = kk - gt;  // how many of the candidates equal to T are kept
  int eq_before = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bool eq = key[j] == T;
    const uint64_t m = __ballot(eq);
    const int rank = eq_before + mbcnt(m);
    sel[j] = key[j] > T || (eq && rank < need);
    eq_before += __popcll(m);
  }
}

// Partial dot product of a lane's kV float4s (elements 4(j8 + 8m) + e):
// four running sums (one per e), added as (s0 + s1) + (s2 + s3).
template <int kV>
__device__ __forceinline__ float dot4s(const float4 (&a)[kV], const float4 (&x)[kV]) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int m = 0; m < kV; ++m) {
    s0 = fmaf(a[m].x, x[m].x, s0);
    s1 = fmaf(a[m].y, x[m].y, s1);
    s2 = fmaf(a[m].z, x[m].z, s2);
    s3 = fmaf(a[m].w, x[m].w, s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// Sum over the 8 lanes 8k..8k+7 (every lane of the group gets the sum):
// neighbours, then pairs, then the other half of the group.
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

template <typename T, int D, int QB, int RW, int NSC, int NSG>
__global__ __launch_bounds__(kThreads) void route_kernel(const RouteP p) {
  constexpr int kGroupSlots = NSG;   // group candidates per row: up to 64 * NSG
  constexpr int kMaxChunks = 64 * NSC;
  constexpr int kWaves = kThreads / 64;
  constexpr int WPR = kWaves / RW;   // wavefronts scoring one row's groups
  static_assert(RW >= 1 && RW <= kWaves && kWaves % RW == 0, "rows per workgroup");
  __shared__ __attribute__((aligned(16))) float s_qbar[RW][D];
  __shared__ float s_score[RW][kMaxChunks];
  __shared__ int s_chunk[RW][kMaxTopK];
  __shared__ float s_gscore[RW][8 * kMaxTopK];

  // the wavefront index as a wave-uniform value: the per-row branches below
  // are then uniform, and the selection's threshold and bit loop stay scalar
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // work: (b, hkv, block, set of query heads); sets of one kv head run on one XCD
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int r = p.Hq / p.Hkv;
  int t = w;
  const int set = t % p.nsets;
  t /= p.nsets;
  const int blk = t % p.nblk;
  t /= p.nblk;
  const int hkv = t % p.Hkv, b = t / p.Hkv;
  const int h0 = set * RW;                               // first query head of the set (within the group)
  const int nrows = min(RW, r - h0);                     // rows of this set
  const int cb = p.q0 / kChunk + blk;                    // the block's own chunk = number of candidates
  const long long nch = p.Scap / kChunk;   // chunk rows per (b, kv head) in the summaries

  // 1. block query of row wv (head hkv*r + h0 + wv): lane (o = l%16, rg = l/16)
  //    sums rows 16rg..16rg+15 of columns 8o..8o+7
  if constexpr (QB == 1) {
    if (wv < nrows && lane < D / 8) {
      const int hq = hkv * r + h0 + wv;
      Frag<T> x;
      load_frag(x, reinterpret_cast<const T*>(p.Q) + ((long long)b * p.Hq + hq) * D + 8 * lane);
      const T* v = reinterpret_cast<const T*>(&x);
#pragma unroll
      for (int e = 0; e < 8; ++e) s_qbar[wv][8 * lane + e] = to_f32(v[e]);
    }
  } else if (wv < nrows && p.causal && cb == 0) {
    // strictly causal, first block of a sequence: no candidates, no routing query
#pragma unroll
    for (int e = 0; e < D / 64; ++e) s_qbar[wv][lane + 64 * e] = 0.f;
  } else if (wv < nrows) {
    const int hq = hkv * r + h0 + wv;
    // the block's own 64 queries; strictly causal: the 64 queries before the
    // block (the previous block, or before the segment's first block)
    const T* Qb = !p.causal ? reinterpret_cast<const T*>(p.Q) + (((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk) * D
                : blk > 0   ? reinterpret_cast<const T*>(p.Q) + (((long long)b * p.Hq + hq) * p.Sq + (long long)(blk - 1) * kChunk) * D
                            : reinterpret_cast<const T*>(p.Qprev) + ((long long)b * p.Hq + hq) * kChunk * D;
    constexpr int kOct = D / 8;                 // 8-element columns
    constexpr int kRowSets = 64 / kOct;         // lanes along the rows
    constexpr int kRowsPerLane = kChunk / kRowSets;
    const int o = lane % kOct, rg = lane / kOct;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    Frag<T> x[kRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) load_frag(x[i], Qb + (long long)(rg * kRowsPerLane + i) * D + 8 * o);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      const T* v = reinterpret_cast<const T*>(&x[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += to_f32(v[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[e];
      for (int m = kOct; m < 64; m <<= 1) v += __shfl_xor(v, m);
      acc[e] = v;
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_qbar[wv][8 * o + e] = acc[e] * (1.0f / 64.0f);
    }
  }
  __syncthreads();

  // 2. chunk scores for every row of the set.  Eight lanes share one summary
  //    row (lane j8 reads float4s j8, j8 + 8, ..., so each load instruction
  //    covers whole 128-byte lines), eight rows per wavefront step; the block
  //    queries stay in registers.  Per row: per-lane partial sums in a fixed
  //    order, then a fixed 8-lane reduction.
  constexpr int kV = D / 32;                  // float4s per lane per summary row
  const int j8 = lane & 7, rsub = lane >> 3;
  float4 qv[RW][kV];
#pragma unroll
  for (int q = 0; q < RW; ++q)
#pragma unroll
    for (int m = 0; m < kV; ++m)
      qv[q][m] = reinterpret_cast<const float4*>(&s_qbar[q][0])[j8 + 8 * m];
  {
    // kChunkUnroll steps per batch: all their loads are issued before the first use
    const float* cmb = p.cm + ((long long)b * p.Hkv + hkv) * nch * D;
    for (int c0 = 8 * wv; c0 < cb; c0 += 32 * kChunkUnroll) {
      float4 x[kChunkUnroll][kV];
#pragma unroll
      for (int u = 0; u < kChunkUnroll; ++u) {
        const int c = c0 + 32 * u + rsub;
        const float4* kr = reinterpret_cast<const float4*>(cmb + (long long)(c < cb ? c : 0) * D);
#pragma unroll
        for (int m = 0; m < kV; ++m) x[u][m] = kr[j8 + 8 * m];
      }
#pragma unroll
      for (int u = 0; u < kChunkUnroll; ++u) {
        const int c = c0 + 32 * u + rsub;
#pragma unroll
        for (int q = 0; q < RW; ++q) {
          if (q >= nrows) break;
          const float sc = sum8(dot4s<kV>(qv[q], x[u]));
          if (c < cb && j8 == 0) s_score[q][c] = sc;
        }
      }
    }
  }
  __syncthreads();

  const int nc = cb;
  const int kk = nc < p.top_k ? nc : p.top_k;    // chunks kept (same for every row)
  const int ng = 8 * kk;                          // group candidates per row
  const int gg = ng < p.top_g ? ng : p.top_g;     // groups kept

  // 3. top-k chunks of row wv
  if (wv < nrows) {
    const long long orow = ((long long)b * p.Hq + hkv * r + h0 + wv) * p.nblk + blk;
    uint32_t key[NSC];
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const int c = 64 * j + lane;
      key[j] = c < nc ? order_key(s_score[wv][c]) : 0u;
    }
    bool sel[NSC];
    select_best<NSC>(key, nc, kk, sel);
    int base = 0;
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const uint64_t m = __ballot(sel[j]);
      if (sel[j]) {
        const int pos = base + mbcnt(m);
        s_chunk[wv][pos] = 64 * j + lane;
        if (p.cidx) p.cidx[orow * p.top_k + pos] = 64 * j + lane;
      }
      base += __popcll(m);
    }
    if (p.cidx)
      for (int i = kk + lane; i < p.top_k; i += 64) p.cidx[orow * p.top_k + i] = -1;
  }
  if (!p.gidx) return;
  if constexpr (WPR == 1) {
    if (wv >= nrows) return;   // row wv is scored and selected by wavefront wv alone
    // row wv's kept chunks were written by other lanes of this wavefront
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }

  // 4a. group scores: the WPR wavefronts wv = q + RW * wr of row q score its
  //     kept chunks wr, wr + WPR, ...; one step covers the 8 groups of one
  //     kept chunk (8 consecutive summary rows), and kGroupUnroll steps are
  //     issued before the first use.  Candidate i = 8 * (rank of the kept
  //     chunk) + group in chunk.
  {
    const int q = wv % RW, wr = wv / RW;
    if (q < nrows) {
      const float* gmb = p.gm + ((long long)b * p.Hkv + hkv) * nch * 8 * D;
      float4 qw[kV];
#pragma unroll
      for (int m = 0; m < kV; ++m) qw[m] = reinterpret_cast<const float4*>(&s_qbar[q][0])[j8 + 8 * m];
      for (int i0 = wr; i0 < kk; i0 += WPR * kGroupUnroll) {
        float4 x[kGroupUnroll][kV];
#pragma unroll
        for (int u = 0; u < kGroupUnroll; ++u) {
          const int i = i0 + WPR * u;
          const int g = (i < kk ? s_chunk[q][i] : 0) * 8 + rsub;
          const float4* gr = reinterpret_cast<const float4*>(gmb + (long long)g * D);
#pragma unroll
          for (int m = 0; m < kV; ++m) x[u][m] = gr[j8 + 8 * m];
        }
#pragma unroll
        for (int u = 0; u < kGroupUnroll; ++u) {
          const int i = i0 + WPR * u;
          const float sc = sum8(dot4s<kV>(qw, x[u]));
          if (i < kk && j8 == 0) s_gscore[q][8 * i + rsub] = sc;
        }
      }
    }
  }
  if constexpr (WPR == 1) {
    // the scores of row wv were written by other lanes of this wavefront
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
    if (wv >= nrows) return;   // no barrier below
  }

  // 4b. joint top-g of row wv over its 8 * kk group candidates
  {
    const long long orow = ((long long)b * p.Hq + hkv * r + h0 + wv) * p.nblk + blk;
    uint32_t key[kGroupSlots];
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      const int i = 64 * j + lane;
      key[j] = i < ng ? order_key(s_gscore[wv][i]) : 0u;
    }
    bool sel[kGroupSlots];
    select_best<kGroupSlots>(key, ng, gg, sel);
    int base = 0;
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      const uint64_t m = __ballot(sel[j]);
      if (sel[j]) {
        const int i = 64 * j + lane;
        p.gidx[orow * p.top_g + base + mbcnt(m)] = s_chunk[wv][i >> 3] * 8 + (i & 7);
      }
      base += __popcll(m);
    }
    for (int i = gg + lane; i < p.top_g; i += 64) p.gidx[orow * p.top_g + i] = -1;
  }
}

template <typename T, int D, int QB, int RW, int NSC, int NSG>
hipError_t run(const Dims& d, const void* Q, const void* Qprev, int causal, const float* cm,
               const float* gm, int32_t* ci, int32_t* gi, hipStream_t s) {
  RouteP p;
  p.Q = Q; p.Qprev = Qprev; p.causal = causal; p.cm = cm; p.gm = gm; p.cidx = ci; p.gidx = gi;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.Scap = d.Scap; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_k = d.top_k; p.top_g = d.top_g;
  const int r = d.Hq / d.Hkv;
  p.nsets = (r + RW - 1) / RW;
  p.nwork = d.B * d.Hkv * d.nblk * p.nsets;
  route_kernel<T, D, QB, RW, NSC, NSG><<<p.nwork, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <typename T, int D, int QB, int RW, int NSC>
hipError_t run_g(const Dims& d, const void* Q, const void* Qprev, int causal, const float* cm,
                 const float* gm, int32_t* ci, int32_t* gi, hipStream_t s) {
  // 8 * top_k group candidates per row at most
  if (d.top_k <= 8) return run<T, D, QB, RW, NSC, 1>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
  if (d.top_k <= 16) return run<T, D, QB, RW, NSC, 2>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
  if (d.top_k <= 32) return run<T, D, QB, RW, NSC, 4>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
  return run<T, D, QB, RW, NSC, 8>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
}

template <typename T, int D, int QB, int RW>
hipError_t run_c(const Dims& d, const void* Q, const void* Qprev, int causal, const float* cm,
                 const float* gm, int32_t* ci, int32_t* gi, hipStream_t s) {
  const int max_cand = (d.Skv - 1) / kChunk;   // chunks before the last query's own chunk
  if (max_cand <= 256) return run_g<T, D, QB, RW, 4>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
  if (max_cand <= 1024) return run_g<T, D, QB, RW, 16>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
  return run_g<T, D, QB, RW, 32>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
}

#ifndef HGA_ROUTE_ROWS_BLOCK
#define HGA_ROUTE_ROWS_BLOCK 2
#endif
#ifndef HGA_ROUTE_ROWS_DECODE
#define HGA_ROUTE_ROWS_DECODE 2
#endif

template <typename T, int D>
hipError_t run_d(const Dims& d, const void* Q, const void* Qprev, int causal, const float* cm,
                 const float* gm, int32_t* ci, int32_t* gi, hipStream_t s) {
  return d.Sq == 1 ? run_c<T, D, 1, HGA_ROUTE_ROWS_DECODE>(d, Q, Qprev, causal, cm, gm, ci, gi, s)
                   : run_c<T, D, kChunk, HGA_ROUTE_ROWS_BLOCK>(d, Q, Qprev, causal, cm, gm, ci, gi, s);
}

}  // namespace

hipError_t launch_route(const Dims& d, const void* Q, const void* Q_prev, bool causal,
                        const float* chunk_mean, const float* group_mean, int32_t* chunk_idx,
                        int32_t* group_idx, hipStream_t s) {
  const int c = causal ? 1 : 0;
  if (d.bf16)
    return d.D == 128 ? run_d<uint16_t, 128>(d, Q, Q_prev, c, chunk_mean, group_mean, chunk_idx, group_idx, s)
                      : run_d<uint16_t, 64>(d, Q, Q_prev, c, chunk_mean, group_mean, chunk_idx, group_idx, s);
  return d.D == 128 ? run_d<float, 128>(d, Q, Q_prev, c, chunk_mean, group_mean, chunk_idx, group_idx, s)
                    : run_d<float, 64>(d, Q, Q_prev, c, chunk_mean, group_mean, chunk_idx, group_idx, s);
}

}  // namespace hga
