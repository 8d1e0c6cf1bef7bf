// Backward through the exact-token attention, routing held fixed: dK and dV.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": the router has no weights and only scores existing projected
// keys, so the gradients reach K and V exactly as in dense attention,
// restricted to the attended (query, key) pairs.  With P recomputed from the
// saved log-sum-exp and delta from the dQ pass (attend_bwd.hip):
//   dP = dO . V^T,   dS = P * (dP - delta)
//   dK = scale * dS^T . Q      dV = P^T . dO
//
// One workgroup per (b, hkv, chunk of 64 keys).  It lists, in a fixed order,
// every (query head of the kv group, query block) whose group-mask byte for
// the chunk is non-zero or whose own chunk it is (causal), and walks them
// with the rows' Q and dO tiles gathered into LDS by direct loads; wavefront
// w owns keys 16w..16w+15 and skips rows that kept neither of its two
// groups.  Each key's dK/dV is summed by one wavefront in that fixed order:
// no atomics, bitwise reproducible.  The workgroups take the chunks of a kv
// head heaviest first (the work order the dQ pass writes, or, for a chunk
// sub-range, the one dkdv_order_kernel writes).
#include "bwd_common.h"
#include "hga_device.h"
#include "hga_kernels.h"

#ifndef HGA_DKV_STAGES
#define HGA_DKV_STAGES 2
#endif

namespace hga {
namespace {

// ============================================================== dK, dV

// Work order of the dK/dV workgroups of one (b, kv head): its chunks sorted by
// the number of routing rows that attend them (the workgroup's entries),
// heaviest first.  A workgroup's time is a fixed part plus a part per entry,
// and the entries per chunk vary about threefold; started in chunk order, a
// heavy chunk dispatched late finishes long after the rest (longest-first
// scheduling bounds that tail).  The order changes no result: every
// workgroup owns its chunk's keys.  Counts above 255 share one bucket; order
// within a bucket is the order of arrival.
// 16 wavefronts per ordering workgroup: the map rows are spread over them,
// and their loads are in flight together.
constexpr int kOrderWaves = 16;
constexpr int kOrderThreads = 64 * kOrderWaves;

// Entries of chunks c0 .. c0+3 from routing rows rs, rs + 16, ... of one kv
// head (rows of the head's query-head group, head-major, so consecutive in
// the map from mrow0): rows whose own chunk it is, plus rows of later blocks
// whose group-mask byte for it is non-zero.  rs is wave-uniform, so every
// row quantity is scalar.  Batches of 8 rows: every load of a batch is issued
// before the first use (rows past the end re-read row 0 and count nothing).
// VEC: one 32-bit load per row (map rows and c0 4-byte aligned).
template <bool VEC>
__device__ __forceinline__ void count_quad(const DkvP& p, const uint8_t* mrow0, int rs, int nrows,
                                           int c0, int own0, int (&n)[4]) {
  constexpr int kBatch = 8;
  // blk = rr % nblk advances by kOrderWaves % nblk (< nblk) per row step:
  // one conditional subtraction keeps it reduced
  const int step = kOrderWaves % p.nblk;
  int blk = rs % p.nblk;
  const long long rstride = (long long)kOrderWaves * p.nchunks;
  const uint8_t* mrow = mrow0 + (long long)rs * p.nchunks;
  for (int rr0 = rs; rr0 < nrows; rr0 += kOrderWaves * kBatch) {
    uint32_t wd[kBatch];
    int ownv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bool ok = rr0 + kOrderWaves * k < nrows;
      ownv[k] = ok ? own0 + blk : -1;   // -1: below every chunk, counts nothing
      const uint8_t* m = ok ? mrow : mrow0;
      mrow += rstride;
      blk += step;
      blk -= blk >= p.nblk ? p.nblk : 0;
      if constexpr (VEC) {
        wd[k] = *reinterpret_cast<const uint32_t*>(m + c0);
      } else {
        uint32_t x = 0;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          x |= (uint32_t)m[c0 + kk < p.nchunks ? c0 + kk : c0] << (8 * kk);
        wd[k] = x;
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c = c0 + kk;
        n[kk] += ownv[k] == c ? 1 : (ownv[k] > c && ((wd[k] >> (8 * kk)) & 0xFFu) != 0) ? 1 : 0;
      }
  }
}

__global__ __launch_bounds__(kOrderThreads) void dkdv_order_kernel(const DkvP p, int32_t* order) {
  constexpr int kMaxRange = 2048;   // HGA_MAX_KV_LEN / 64
  __shared__ int s_cnt[kMaxRange];
  __shared__ int s_hist[256];
  __shared__ int s_wsum[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x, b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int r = p.Hq / p.Hkv, nrows = r * p.nblk;
  const int own0 = p.q0 / kChunk;   // own chunk of block 0
  const uint8_t* mrow0 = p.cmask + ((long long)b * p.Hq + hkv * r) * p.nblk * p.nchunks;
  for (int i = tid; i < kMaxRange; i += kOrderThreads) s_cnt[i] = 0;
  if (tid < 256) s_hist[tid] = 0;
  __syncthreads();
  // entries of every chunk of the range.  Lane q of wavefront wv counts
  // chunks 4q .. 4q+3 of a 256-chunk window over rows wv, wv + 16, ...
  const bool vec = (p.nchunks & 3) == 0 && (p.chunk0 & 3) == 0;
  for (int w0 = 0; w0 < p.nrange; w0 += 256) {
    const int i0 = w0 + 4 * lane;         // first range index of the quad
    if (i0 < p.nrange) {
      const int c0 = p.chunk0 + i0;
      int n[4] = {0, 0, 0, 0};
      if (vec)
        count_quad<true>(p, mrow0, wv, nrows, c0, own0, n);
      else
        count_quad<false>(p, mrow0, wv, nrows, c0, own0, n);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k < p.nrange && n[k] != 0) atomicAdd(&s_cnt[i0 + k], n[k]);
    }
  }
  __syncthreads();
  // counting sort on 256 buckets (bucket 255 - min(count, 255)): histogram,
  // exclusive prefix, then placement
  for (int i = tid; i < p.nrange; i += kOrderThreads) {
    const int n = s_cnt[i];
    atomicAdd(&s_hist[255 - (n < 255 ? n : 255)], 1);
  }
  __syncthreads();
  int v = 0, incl = 0;
  if (tid < 256) {
    v = s_hist[tid];
    incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if (lane >= d) incl += u;
    }
    if (lane == 63) s_wsum[wv] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    int base = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) base += k < wv ? s_wsum[k] : 0;
    s_hist[tid] = base + incl - v;   // first slot of the bucket
  }
  __syncthreads();
  for (int i = tid; i < p.nrange; i += kOrderThreads) {
    const int n = s_cnt[i];
    const int pos = atomicAdd(&s_hist[255 - (n < 255 ? n : 255)], 1);
    order[bh * p.nrange + pos] = p.chunk0 + i;
  }
}

template <typename T, int D, int S>
__global__ __launch_bounds__(kThreads) void attend_bwd_dkdv_kernel(const DkvP p) {
  using RT = RowTile<T, D>;
  constexpr int RB = RT::kUnits * 16;
  constexpr int kTileBytes = 64 * RB;                             // 64 query rows
  constexpr int kStatBytes = 4 * 128;                             // per wave: 16 lse, 16 delta
  constexpr int kStage = 2 * kTileBytes + kStatBytes;             // Q | dO | stats
  constexpr int kRPI = rows_per_issue<T, D>();
  constexpr int kIssues = 16 / kRPI;                              // per matrix per wave
  constexpr int kLoads = 2 * kIssues + 1;                         // + the stats load
  __shared__ __attribute__((aligned(1024))) char smem[S * kStage];
  __shared__ uint32_t s_ent[kRowsPerPass];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  // work items of one (b, kv head) in their work order: chunks with the most
  // entries first (written by the dQ pass for the whole range, or by
  // dkdv_order_kernel for a sub-range)
  const int bh = w / p.nrange, c = p.order[bh * p.nrange + w % p.nrange];
  // the order comes from the workspace: a chunk outside the range (a
  // workspace not written by the matching dQ or ordering pass) is skipped, so
  // no store ever leaves the range's rows of dK and dV
  if (c < p.chunk0 || c >= p.chunk0 + p.nrange) return;
  const int b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int r = p.Hq / p.Hkv;
  const int nrows = r * p.nblk;          // (query head in group, block), head-major
  const int kin = 16 * wv + l16;         // this lane's key within the chunk
  const uint32_t mygroups = 3u << (2 * wv);

  // the first entry list's mask words are read first: the list then waits on
  // those loads alone, not on the K and V loads issued after them
  EntryMasks<> em;
  load_entry_masks(p, b, hkv, c, 0, em);

  // this wavefront's 16 keys as B operands of S = Q . K^T and dP = dO . V^T
  Frag<T> kf[D / 32], vf[D / 32];
  {
    const long long off = ((long long)bh * p.Scap + (long long)c * kChunk + kin) * D + 8 * g4;
    const T* k = reinterpret_cast<const T*>(p.K) + off;
    const T* v = reinterpret_cast<const T*>(p.V) + off;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      load_frag(kf[s], k + 32 * s);
      load_frag(vf[s], v + 32 * s);
    }
  }
  f32x4 dkacc[D / 16], dvacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    dkacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = p.scale * kLog2e;

  // loop-invariant per-lane offsets (see attend_fwd.hip); query rows in
  // natural order: result item i of lane group g is query 4g + i of its
  // 16-row slice, and the transposing reads cover rows 4g .. 4g + 3 (the tile
  // swizzle keeps both read patterns conflict-free)
  RowOffsets<T, D> qro;
  qro.init();
  TrOffsets<(sizeof(T) == 2 ? D : 16)> qto;
  if constexpr (sizeof(T) == 2) qto.init();
  uint32_t ld_off[kIssues];
#pragma unroll
  for (int j = 0; j < kIssues; ++j) {
    const int rr = 16 * wv + kRPI * j + lane / RT::kUnits;
    ld_off[j] = (uint32_t)(rr * RB) + (uint32_t)(((lane % RT::kUnits) ^ RT::swz(rr)) << 4);
  }

  const uint32_t smem_lds = lds_addr(smem);
  // Q rows, dO rows (16 per wave) and this wave's 16 lse / delta values
  auto issue = [&](uint32_t ent, int slot) {
    const int rr0 = (int)(ent >> 9);
    const int hq = hkv * r + rr0 / p.nblk, blk = rr0 % p.nblk;
    const long long qrow0 = ((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk;
    const T* qb = reinterpret_cast<const T*>(p.Q) + qrow0 * D;
    const T* ob = reinterpret_cast<const T*>(p.dO) + qrow0 * D;
    const uint32_t buf = smem_lds + (uint32_t)(slot * kStage);
#pragma unroll
    for (int j = 0; j < kIssues; ++j) {
      const uint32_t dst = buf + (uint32_t)((16 * wv + kRPI * j) * RB);
      dma16_off(ld_off[j], qb, dst);
      dma16_off(ld_off[j], ob, dst + kTileBytes);
    }
    // lanes 0..3: lse of queries 16w..16w+15, lanes 4..7: delta of the same
    if (lane < 8) {
      const float* src = (lane < 4 ? p.lse : p.delta) + qrow0 + 16 * wv + 4 * (lane & 3);
      dma16(src, buf + (uint32_t)(2 * kTileBytes + 128 * wv));
    }
  };

  for (int r0 = 0; r0 < nrows; r0 += kRowsPerPass) {
    // ---- entry list for routing rows [r0, r0 + kRowsPerPass)
    if (r0 > 0) load_entry_masks(p, b, hkv, c, r0, em);
    const int nent = build_entries(p, r0, em, s_ent, s_wsum);
    if (nent == 0) continue;

    // ---- walk the entries, S - 1 of them in flight
#pragma unroll
    for (int e = 0; e < S - 1; ++e)
      if (e < nent) issue(s_ent[e], e % S);
    for (int e = 0; e < nent; ++e) {
      const int ahead = (nent - 1 - e) < (S - 2) ? (nent - 1 - e) : (S - 2);
      if (ahead >= 2) wait_vmcnt<2 * kLoads>();
      else if (ahead == 1) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (e + S - 1 < nent) issue(s_ent[e + S - 1], (e + S - 1) % S);

      const uint32_t ent = s_ent[e];
      const bool local = (ent & kLocalBit) != 0;
      if (local || (ent & mygroups)) {
        const char* qt = smem + (e % S) * kStage;
        const float* stat = reinterpret_cast<const float*>(qt + 2 * kTileBytes);

        f32x4 sacc[4], dpacc[4];
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          sacc[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
          dpacc[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // lse and delta of queries 16qs + 4g .. 16qs + 4g + 3 (wave-slot qs
        // of the stats block is [lse 16 | delta 16])
        float4 l4[4], d4[4];
        auto read_stats = [&]() {
#pragma unroll
          for (int qs = 0; qs < 4; ++qs) {
            l4[qs] = *reinterpret_cast<const float4*>(stat + 32 * qs + 4 * g4);
            d4[qs] = *reinterpret_cast<const float4*>(stat + 32 * qs + 16 + 4 * g4);
          }
        };
        // transposed operands of column blocks cc, cc + 1: fo (dO) and fq (Q),
        // fragment 2j + mm of block cc + j covers queries 32mm + 4g + t and
        // 32mm + 16 + 4g + t
        Frag<T> fo[2][4], fq[2][4];
        auto tr_addr = [&](uint32_t (&a)[8], int cc) {
          const uint32_t a0 = lds_addr(qt) + qto.o[cc], a1 = lds_addr(qt) + qto.o[cc + 1];
#pragma unroll
          for (int k = 0; k < 4; ++k) { a[k] = a0; a[4 + k] = a1; }
        };
        auto read_tr_o = [&](Frag<T> (&o)[4], int cc) {
          if constexpr (sizeof(T) == 2) {
            uint32_t a[8];
            tr_addr(a, cc);
            tr_read8_sched<kTileBytes, kTileBytes + 16 * RB, kTileBytes + 32 * RB, kTileBytes + 48 * RB,
                           kTileBytes, kTileBytes + 16 * RB, kTileBytes + 32 * RB, kTileBytes + 48 * RB>(o, a);
          }
        };
        auto read_tr_q = [&](Frag<T> (&q)[4], int cc) {
          if constexpr (sizeof(T) == 2) {
            uint32_t a[8];
            tr_addr(a, cc);
            tr_read8_sched<0, 16 * RB, 32 * RB, 48 * RB, 0, 16 * RB, 32 * RB, 48 * RB>(q, a);
          }
        };

        if constexpr (sizeof(T) == 2) {
          // S = Q . K^T and dP = dO . V^T, software-pipelined: the 8 row
          // operands of step s + 1 (or, after the last step, the stats) are
          // read while the 8 products of step s run.  The scheduling fences
          // keep the compiler from sinking the reads to their uses.
          Frag<T> ra[2][8];
          auto read_rows = [&](Frag<T> (&f)[8], int s) {
            const char* qp = qt + qro.o[s];
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
              frag_rows_at<T, D>(f[2 * qs], qp + 16 * qs * RB);
              frag_rows_at<T, D>(f[2 * qs + 1], qp + kTileBytes + 16 * qs * RB);
            }
          };
          read_rows(ra[0], 0);
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            if (s + 1 < D / 32) read_rows(ra[(s + 1) & 1], s + 1);
            else read_stats();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
              mma(sacc[qs], ra[s & 1][2 * qs], kf[s]);
              mma(dpacc[qs], ra[s & 1][2 * qs + 1], vf[s]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          // the first column pair's transposed operands load during the softmax
          read_tr_o(fo[0], 0);
          read_tr_q(fq[0], 0);
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            const char* qp = qt + qro.o[s];
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
              Frag<T> a;
              frag_rows_at<T, D>(a, qp + 16 * qs * RB);
              mma(sacc[qs], a, kf[s]);
              frag_rows_at<T, D>(a, qp + kTileBytes + 16 * qs * RB);
              mma(dpacc[qs], a, vf[s]);
            }
          }
          read_stats();
        }
        // P (zero for unattended pairs) and dS; a key outside the row's kept
        // groups gets an exponent offset of -inf, so P = exp2(-inf) = 0 (the
        // offset is added, not selected, so the stats are read unconditionally)
        const bool kvalid = local || ((ent >> (kin >> 3)) & 1u);
        const float koff = kvalid ? 0.f : -INFINITY;
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          const float lq[4] = {l4[qs].x, l4[qs].y, l4[qs].z, l4[qs].w};
          const float dq[4] = {d4[qs].x, d4[qs].y, d4[qs].z, d4[qs].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float nl = fmaf(-lq[i], kLog2e, koff);
            float pr = __builtin_amdgcn_exp2f(fmaf(sacc[qs][i], c2, nl));
            if (local && kin > 16 * qs + 4 * g4 + i) pr = 0.f;
            sacc[qs][i] = pr;
            dpacc[qs][i] = pr * (dpacc[qs][i] - dq[i]);
          }
        }
        Frag<T> pf[2], dsf[2];
        frag_from_acc(pf[0], sacc[0], sacc[1]);
        frag_from_acc(pf[1], sacc[2], sacc[3]);
        frag_from_acc(dsf[0], dpacc[0], dpacc[1]);
        frag_from_acc(dsf[1], dpacc[2], dpacc[3]);
        // dV^T += dO^T . P and dK^T += Q^T . dS
        if constexpr (sizeof(T) == 2) {
          // column pair i + 1's transposed reads are in flight while pair i's
          // products run (its dO reads go out before pair i's products, its Q
          // reads after them); per accumulator the order is mm = 0, then 1
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < D / 32; ++i) {
            const int cc = 2 * i;
            const bool more = i + 1 < D / 32;
            if (more) read_tr_o(fo[(i + 1) & 1], cc + 2);
            __builtin_amdgcn_sched_barrier(0);
            const Frag<T>(&o)[4] = fo[i & 1];
            const Frag<T>(&q)[4] = fq[i & 1];
            mma(dvacc[cc], o[0], pf[0]);
            mma(dvacc[cc + 1], o[2], pf[0]);
            mma(dvacc[cc], o[1], pf[1]);
            mma(dvacc[cc + 1], o[3], pf[1]);
            mma(dkacc[cc], q[0], dsf[0]);
            mma(dkacc[cc + 1], q[2], dsf[0]);
            mma(dkacc[cc], q[1], dsf[1]);
            mma(dkacc[cc + 1], q[3], dsf[1]);
            __builtin_amdgcn_sched_barrier(0);
            if (more) read_tr_q(fq[(i + 1) & 1], cc + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          const char* ot = qt + kTileBytes;
#pragma unroll
          for (int dd = 0; dd < D / 16; ++dd)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              Frag<T> o1, q1;
              frag_tr<T, D>(o1, ot, 32 * mm + 4 * g4, 32 * mm + 16 + 4 * g4, 16 * dd);
              frag_tr<T, D>(q1, qt, 32 * mm + 4 * g4, 32 * mm + 16 + 4 * g4, 16 * dd);
              mma(dvacc[dd], o1, pf[mm]);
              mma(dkacc[dd], q1, dsf[mm]);
            }
        }
      }
    }
    __syncthreads();   // the entry list and stage buffers are reused by the next pass
  }

  // every key of the chunk is written (zero when nothing attends it)
  const float sc = p.scale;
  if constexpr (sizeof(T) == 2) {
    // bf16: the chunk's dK and dV rows are one contiguous block each; they
    // leave as whole rows through the idle stage buffers
    static_assert(2 * 64 * D * 2 <= S * kStage, "dK/dV staging fits the stage buffers");
    char* const sk = smem;
    char* const sv = smem + 64 * 2 * D;
    __syncthreads();   // every wave is done with the stage buffers
    out_rows_put<D>(sk, dkacc, sc, kin, g4);
    out_rows_put<D>(sv, dvacc, 1.0f, kin, g4);
    __syncthreads();
    const long long crow = (long long)bh * p.Scap + (long long)c * kChunk;
    // non-temporal: the Q and dO rows that other workgroups still gather keep
    // their place in L2 (no later kernel of the step reads dK, dV)
    out_rows_flush<D, true>(sk, reinterpret_cast<char*>(p.dK) + crow * 2 * D, tid);
    out_rows_flush<D, true>(sv, reinterpret_cast<char*>(p.dV) + crow * 2 * D, tid);
  } else {
    const long long krow = (long long)bh * p.Scap + (long long)c * kChunk + kin;
    T* dk = reinterpret_cast<T*>(p.dK) + krow * D + 4 * g4;
    T* dv = reinterpret_cast<T*>(p.dV) + krow * D + 4 * g4;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      store4(dk + 16 * dd, dkacc[dd][0] * sc, dkacc[dd][1] * sc, dkacc[dd][2] * sc,
             dkacc[dd][3] * sc);
      store4(dv + 16 * dd, dvacc[dd][0], dvacc[dd][1], dvacc[dd][2], dvacc[dd][3]);
    }
  }
}

template <typename T, int D>
hipError_t run_dkdv(const Dims& d, const void* Q, const void* K, const void* V, const float* lse,
                    const void* dO, const int32_t* gi, const float* delta, const uint8_t* cmask,
                    int32_t* order, bool order_ready, void* dK, void* dV, int chunk_begin,
                    int chunk_end, hipStream_t s) {
  DkvP p;
  p.Q = Q; p.K = K; p.V = V; p.lse = lse; p.dO = dO; p.gidx = gi; p.delta = delta;
  p.cmask = cmask;
  p.dK = dK; p.dV = dV;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.Scap = d.Scap; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_g = d.top_g; p.scale = d.scale;
  p.nchunks = d.Skv / kChunk;
  p.chunk0 = chunk_begin;
  p.nrange = chunk_end - chunk_begin;
  p.nwork = d.B * d.Hkv * p.nrange;
  p.order = order;
  constexpr int kStageBytes = 2 * 64 * D * (int)sizeof(T) + 512;
  constexpr int S0 = HGA_DKV_STAGES;
  constexpr int S = S0 * kStageBytes <= 140 * 1024 ? S0 : (140 * 1024) / kStageBytes;
  static_assert(S >= 2, "at least two stages");
  // the full range's order comes with the dQ workspace; a sub-range orders its own
  if (!order_ready) dkdv_order_kernel<<<d.B * d.Hkv, kOrderThreads, 0, s>>>(p, order);
  attend_bwd_dkdv_kernel<T, D, S><<<p.nwork, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_bwd_dkdv(const Dims& d, const void* Q, const void* K, const void* V,
                                  const float* lse, const void* dO, const int32_t* group_idx,
                                  const float* delta, const uint8_t* cmask, int32_t* order,
                                  bool order_ready, void* dK, void* dV, int chunk_begin,
                                  int chunk_end, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run_dkdv<uint16_t, 128>(d, Q, K, V, lse, dO, group_idx, delta, cmask, order, order_ready, dK, dV, chunk_begin, chunk_end, s)
                      : run_dkdv<uint16_t, 64>(d, Q, K, V, lse, dO, group_idx, delta, cmask, order, order_ready, dK, dV, chunk_begin, chunk_end, s);
  return d.D == 128 ? run_dkdv<float, 128>(d, Q, K, V, lse, dO, group_idx, delta, cmask, order, order_ready, dK, dV, chunk_begin, chunk_end, s)
                    : run_dkdv<float, 64>(d, Q, K, V, lse, dO, group_idx, delta, cmask, order, order_ready, dK, dV, chunk_begin, chunk_end, s);
}

}  // namespace hga
