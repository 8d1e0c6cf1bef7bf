// Exact-token attention forward over the routed groups plus the own chunk.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": after routing, only the exact key/value tokens of the kept
// groups are loaded and attention runs on them; the summaries are never used
// as keys or values.  The query at position p of a block attends the tokens
// of the block's kept groups and its own chunk up to p (causal).
//
// One workgroup (4 wavefronts) per (b, hq, block of 64 queries); wavefront w
// owns queries 16w..16w+15.  The key/value set is walked in 64-token tiles:
// tile 0 is the own chunk (causal mask), tile i >= 1 holds kept groups
// 8(i-1)..8(i-1)+7 (a group is 8 contiguous rows: a 2 KB run of K and of V at
// head_dim 128 in bf16).  Tiles are gathered straight from global memory into
// LDS with 16-byte direct loads (no register staging), kStages tiles in
// flight, row-major with 16-byte units XOR-swizzled by row.  Per tile and
// wavefront:
//   S^T[64 keys x 16 queries] = K . Q^T      bf16 MFMA 16x16x32, fp32 acc
//   online softmax in the log2 domain (running max and sum per query)
//   O^T[D x 16 queries]      += V^T . P^T    bf16 MFMA; V^T read with the LDS
//                                            transpose read, P kept in registers
// The S^T accumulator layout (lane: one query, four keys) is directly the
// operand layout of P^T for the second product.
#include "hga_device.h"
#include "hga_kernels.h"

#ifndef HGA_FWD_TILE
#define HGA_FWD_TILE 32     // keys per tile: 32 (4 groups) or 64 (8 groups)
#endif
#ifndef HGA_FWD_STAGES
#define HGA_FWD_STAGES 2    // tiles resident in LDS (STAGES - 1 in flight)
#endif

namespace hga {
namespace {

constexpr int kMaxTopG = 512;

struct FwdP {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* gidx;
  void* O;
  float* lse;
  int B, Hq, Hkv, Sq, Skv, Scap, q0, nblk, top_g, nwork;
  float scale;
};

// The running max of a query is raised only when a tile's max exceeds it by
// more than this many powers of two; until then P = 2^(x - m) <= 2^8, exact in
// bf16 up to its usual relative rounding, and the O accumulators need no
// rescaling on most tiles.
constexpr float kRescale = 8.0f;

template <typename T, int D, int TK, int S>
__global__ __launch_bounds__(kThreads) void attend_fwd_kernel(const FwdP p) {
  using RT = RowTile<T, D>;
  constexpr int RB = RT::kUnits * 16;                             // bytes per tile row
  constexpr int kTileBytes = TK * RB;                             // one matrix, TK rows
  constexpr int kStage = 2 * kTileBytes;                          // K tile | V tile
  constexpr int kRowsPerWave = TK / 4;
  constexpr int kRPI = rows_per_issue<T, D>();
  constexpr int kIssues = kRowsPerWave / kRPI;                    // per matrix per wave
  constexpr int kLoads = 2 * kIssues;                             // per wave per tile
  constexpr int kLocalTiles = kChunk / TK;
  constexpr int kGroupsPerTile = TK / kGroup;
  constexpr int NKS = TK / 16;   // 16-key subtiles
  constexpr int NMM = TK / 32;   // 32-key slices of the P.V product
  static_assert(kRowsPerWave % kRPI == 0, "tile rows per wave");
  __shared__ __attribute__((aligned(1024))) char smem[S * kStage];
  __shared__ int s_glist[kMaxTopG];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // work item: (b, hkv)-major so that one kv head's work shares an XCD
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int r = p.Hq / p.Hkv;
  const int per_bh = r * p.nblk;
  const int bh = w / per_bh, rem = w % per_bh;
  const int blk = rem / r, hql = rem % r;
  const int b = bh / p.Hkv, hkv = bh % p.Hkv, hq = hkv * r + hql;
  const int cb = p.q0 / kChunk + blk;
  const long long row = ((long long)b * p.Hq + hq) * p.nblk + blk;

  // routing row -> LDS: its ascending prefix of groups before the own chunk
  const int nvalid = load_routing_prefix<kThreads>(p.gidx + row * p.top_g, p.top_g, cb * 8,
                                                   s_glist, s_wsum);
  const int ntiles = kLocalTiles + (nvalid + kGroupsPerTile - 1) / kGroupsPerTile;

  const T* Kbh = reinterpret_cast<const T*>(p.K) + (long long)bh * p.Scap * D;
  const T* Vbh = reinterpret_cast<const T*>(p.V) + (long long)bh * p.Scap * D;
  const long long qrow0 = ((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk;

  // this wavefront's 16 queries as B operands of S^T = K . Q^T
  Frag<T> qf[D / 32];
  {
    const T* q = reinterpret_cast<const T*>(p.Q) + (qrow0 + 16 * wv + l16) * D + 8 * g4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) load_frag(qf[s], q + 32 * s);
  }

  // loop-invariant per-lane offsets: LDS reads of the K rows, transposed reads
  // of V, and the swizzled column of each row this lane loads
  RowOffsets<T, D> kro;
  kro.init();
  TrOffsets<(sizeof(T) == 2 ? D : 16)> vto;
  if constexpr (sizeof(T) == 2) vto.init();
  int ld_row[kIssues];
  uint32_t ld_col[kIssues];
#pragma unroll
  for (int j = 0; j < kIssues; ++j) {
    ld_row[j] = kRowsPerWave * wv + kRPI * j + lane / RT::kUnits;
    ld_col[j] = (uint32_t)(((lane % RT::kUnits) ^ RT::swz(ld_row[j])) << 4);
  }

  // Tiles 0..kLocalTiles-1 cover the own chunk; later tiles hold
  // kGroupsPerTile kept groups.  A slot past the last kept group reads the own
  // chunk (any valid row works: its scores are masked, its P is exactly zero).
  const uint32_t smem_lds = lds_addr(smem);
  // kept-group list entries of the rows this lane gathers for tile ti (read
  // ahead of the issue, so the issue itself waits on no LDS read)
  auto glist_of = [&](int ti, int (&gm)[kIssues]) {
#pragma unroll
    for (int j = 0; j < kIssues; ++j) {
      const int slot = kGroupsPerTile * (ti - kLocalTiles) + (ld_row[j] >> 3);
      gm[j] = s_glist[slot < 0 ? 0 : (slot < kMaxTopG ? slot : kMaxTopG - 1)];
    }
  };
  auto issue = [&](int ti, const int (&gm)[kIssues]) {
    const uint32_t buf = smem_lds + (uint32_t)((ti % S) * kStage);
    uint32_t off[kIssues];
#pragma unroll
    for (int j = 0; j < kIssues; ++j) {
      const int rr = ld_row[j];
      uint32_t tok = (uint32_t)(cb * kChunk + (rr & (kChunk - 1)));
      if (ti < kLocalTiles) {
        tok += (uint32_t)(ti * TK);
      } else {
        const int slot = kGroupsPerTile * (ti - kLocalTiles) + (rr >> 3);
        tok = slot < nvalid ? (uint32_t)(gm[j] * kGroup + (rr & 7)) : tok;
      }
      off[j] = tok * (uint32_t)RB + ld_col[j];
    }
#pragma unroll
    for (int j = 0; j < kIssues; ++j) {
      const uint32_t dst = buf + (uint32_t)((kRowsPerWave * wv + kRPI * j) * RB);
      dma16_off(off[j], Kbh, dst);
      dma16_off(off[j], Vbh, dst + kTileBytes);
    }
  };

  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale * kLog2e;
  const int qq = 16 * wv + l16;   // this lane's query within the block

#pragma unroll
  for (int ti = 0; ti < S - 1; ++ti)
    if (ti < ntiles) {
      int gm[kIssues];
      glist_of(ti, gm);
      issue(ti, gm);
    }

  for (int ti = 0; ti < ntiles; ++ti) {
    // group-list entries of the tile issued after the barrier: their LDS
    // reads complete in the barrier's wait
    int gnext[kIssues];
    glist_of(ti + S - 1, gnext);
    // tile ti has landed once at most (tiles issued after it) x kLoads remain
    const int ahead = (ntiles - 1 - ti) < (S - 2) ? (ntiles - 1 - ti) : (S - 2);
    if (ahead >= 3) wait_vmcnt<3 * kLoads>();
    else if (ahead == 2) wait_vmcnt<2 * kLoads>();
    else if (ahead == 1) wait_vmcnt<kLoads>();
    else wait_vmcnt<0>();
    __syncthreads();   // tile ti visible to all; everyone is done with tile ti-1
    if (ti + S - 1 < ntiles) issue(ti + S - 1, gnext);

    const char* kt = smem + (ti % S) * kStage;
    const char* vt = kt + kTileBytes;

    // S^T = K . Q^T for NKS subtiles of 16 keys (raw dot products)
    f32x4 sacc[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sacc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const char* kp = kt + kro.o[s];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Frag<T> kf;
        frag_rows_at<T, D>(kf, kp + 16 * ks * RB);
        mma(sacc[ks], kf, qf[s]);
      }
    }
    // masks: causal on the own chunk, empty slots on the last group tile
    if (ti < kLocalTiles) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (TK * ti + 16 * ks + 4 * g4 + i > qq) sacc[ks][i] = -INFINITY;
    } else if (kGroupsPerTile * (ti - kLocalTiles + 1) > nvalid) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int slot = kGroupsPerTile * (ti - kLocalTiles) + 2 * ks + (g4 >> 1);
        if (slot >= nvalid) sacc[ks] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      mx = fmaxf(fmaxf(mx, fmaxf(sacc[ks][0], sacc[ks][1])), fmaxf(sacc[ks][2], sacc[ks][3]));
    const float mc = xor_max16_32(mx) * c2;
    const bool raise = mc > m_run + kRescale;
    if (__ballot(raise)) {
      const float m_new = raise ? mc : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[ks][i], c2, -m_run));
        sacc[ks][i] = e;
        psum += e;
      }
    l_run += psum;

    // O^T += V^T . P^T ; P^T items of key slice mm: keys 32mm+4g+t, 32mm+16+4g+t
    Frag<T> pf[NMM];
#pragma unroll
    for (int mm = 0; mm < NMM; ++mm) frag_from_acc(pf[mm], sacc[2 * mm], sacc[2 * mm + 1]);
    if constexpr (sizeof(T) == 2) {
      uint32_t va[D / 16];
#pragma unroll
      for (int c = 0; c < D / 16; ++c) va[c] = lds_addr(vt) + vto.o[c];
      if constexpr (NMM == 1) {
#pragma unroll
        for (int c = 0; c < D / 16; c += 4) {
          const uint32_t a[8] = {va[c], va[c], va[c + 1], va[c + 1],
                                 va[c + 2], va[c + 2], va[c + 3], va[c + 3]};
          Frag<T> vf[4];
          tr_read8_sched<0, 16 * RB, 0, 16 * RB, 0, 16 * RB, 0, 16 * RB>(vf, a);
#pragma unroll
          for (int i = 0; i < 4; ++i) mma(oacc[c + i], vf[i], pf[0]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < D / 16; c += 2) {
          const uint32_t a[8] = {va[c], va[c], va[c], va[c], va[c + 1], va[c + 1], va[c + 1], va[c + 1]};
          Frag<T> vf[4];
          tr_read8_sched<0, 16 * RB, 32 * RB, 48 * RB, 0, 16 * RB, 32 * RB, 48 * RB>(vf, a);
          mma(oacc[c], vf[0], pf[0]);
          mma(oacc[c], vf[1], pf[1]);
          mma(oacc[c + 1], vf[2], pf[0]);
          mma(oacc[c + 1], vf[3], pf[1]);
        }
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int mm = 0; mm < NMM; ++mm) {
          Frag<T> vf;
          frag_tr<T, D>(vf, vt, 32 * mm + 4 * g4, 32 * mm + 16 + 4 * g4, 16 * ds);
          mma(oacc[ds], vf, pf[mm]);
        }
    }
  }

  // epilogue: normalise, write O (4 consecutive elements per lane) and lse
  const float l_tot = xor_sum16_32(l_run);
  const float inv = 1.0f / l_tot;
  if constexpr (sizeof(T) == 2) {
    // the block's 64 output rows are contiguous: whole rows through the idle
    // stage buffers
    static_assert(64 * 2 * D <= S * kStage, "O staging fits the stage buffers");
    __syncthreads();   // every wave is done with the stage buffers
    out_rows_put<D>(smem, oacc, inv, qq, g4);
    __syncthreads();
    out_rows_flush<D>(smem, reinterpret_cast<char*>(p.O) + qrow0 * 2 * D, tid);
  } else {
    T* o = reinterpret_cast<T*>(p.O) + (qrow0 + qq) * D + 4 * g4;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      store4(o + 16 * ds, oacc[ds][0] * inv, oacc[ds][1] * inv, oacc[ds][2] * inv,
             oacc[ds][3] * inv);
  }
  if (p.lse && g4 == 0) p.lse[qrow0 + qq] = (m_run + __log2f(l_tot)) * kLn2;
}

template <typename T, int D>
hipError_t run(const Dims& d, const void* Q, const void* K, const void* V, const int32_t* gi,
               void* O, float* lse, hipStream_t s) {
  FwdP p;
  p.Q = Q; p.K = K; p.V = V; p.gidx = gi; p.O = O; p.lse = lse;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.Scap = d.Scap; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_g = d.top_g; p.scale = d.scale;
  p.nwork = d.B * d.Hq * d.nblk;
  // fp32 tiles are twice as large: cap the stages at 128 KB of LDS
  constexpr int TK = HGA_FWD_TILE;
  constexpr int kStageBytes = 2 * TK * D * (int)sizeof(T);
  constexpr int S0 = HGA_FWD_STAGES;
  constexpr int S = S0 * kStageBytes <= 128 * 1024 ? S0 : (128 * 1024) / kStageBytes;
  static_assert(S >= 2, "at least two stages");
  attend_fwd_kernel<T, D, TK, S><<<p.nwork, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_fwd(const Dims& d, const void* Q, const void* K, const void* V,
                             const int32_t* group_idx, void* O, float* lse, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run<uint16_t, 128>(d, Q, K, V, group_idx, O, lse, s)
                      : run<uint16_t, 64>(d, Q, K, V, group_idx, O, lse, s);
  return d.D == 128 ? run<float, 128>(d, Q, K, V, group_idx, O, lse, s)
                    : run<float, 64>(d, Q, K, V, group_idx, O, lse, s);
}

}  // namespace hga
