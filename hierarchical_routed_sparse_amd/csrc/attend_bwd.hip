// Backward through the exact-token attention, routing held fixed.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": the router has no weights and only scores existing projected
// keys, so the gradients reach Q, K and V exactly as in dense attention,
// restricted to the attended (query, key) pairs.  With P recomputed from the
// saved log-sum-exp:
//   delta_q = dO_q . O_q
//   dP      = dO . V^T,   dS = P * (dP - delta)
//   dQ      = scale * dS . K      dK = scale * dS^T . Q      dV = P^T . dO
//
// Two kernels; this file holds the first (the second is in attend_bwd_dkdv.hip):
//  * bwd_dq  -- one workgroup per (b, hq, block): the forward's tile walk (own
//    chunk, then the kept groups), K and V tiles gathered into LDS with direct
//    loads; writes delta and dQ.  dQ^T += K^T . dS^T reads K^T with the LDS
//    transpose read.  It also writes the row's entry of the group-mask map
//    (byte c = which of chunk c's 8 groups the row kept) for the dK/dV pass.
//  * bwd_dkdv -- one workgroup per (b, hkv, chunk of 64 keys).  It
//    lists, in a fixed order, every (query head of the kv group, query block)
//    whose mask for the chunk is non-zero or whose own chunk it is (causal),
//    and walks them with the rows' Q and dO tiles gathered into LDS by direct
//    loads; wavefront w owns keys 16w..16w+15 and skips rows that kept neither
//    of its two groups.  Each key's dK/dV is summed by one wavefront in that
//    fixed order: no atomics, bitwise reproducible.
#include <type_traits>

#include "bwd_common.h"
#include "hga_device.h"
#include "hga_kernels.h"

#ifndef HGA_DQ_TILE
#define HGA_DQ_TILE 32
#endif
#ifndef HGA_DQ_STAGES
#define HGA_DQ_STAGES 2
#endif

namespace hga {
namespace {

constexpr int kMaxTopG = 512;

// ============================================================== dQ

struct DqP {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* lse;
  const void* dO;
  const int32_t* gidx;
  void* dQ;
  float* delta;
  uint8_t* cmask;   // [routing row][chunk] kept-group masks, for the dK/dV kernel
  int32_t* order;   // [B * Hkv][nchunks]: dK/dV work order (see dq_order_block)
  int B, Hq, Hkv, Sq, Skv, Scap, q0, nblk, top_g, nwork, nchunks;
  float scale;
};

// The dK/dV work order of kv head bh = b * Hkv + hkv, computed by extra
// workgroups at the end of the dQ grid (they start as dQ workgroups finish,
// so the order costs no launch of its own): the chunks of the head sorted by
// the number of routing rows that attend them, heaviest first (see
// dkdv_order_kernel for why).  The counts come from the routing indices: a row
// attends its own chunk and the chunks of its kept groups.
template <int NT = kThreads>
__device__ __forceinline__ void dq_order_block(const DqP& p, int bh, int* s_mem) {
  constexpr int kMaxRange = 2048;   // HGA_MAX_KV_LEN / 64
  constexpr int kBatch = 16;
  int* s_cnt = s_mem;
  int* s_hist = s_mem + kMaxRange;
  int* s_wsum = s_hist + 256;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int r = p.Hq / p.Hkv, nrows = r * p.nblk;
  for (int i = tid; i < p.nchunks; i += NT) s_cnt[i] = 0;
  for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
  __syncthreads();
  for (int rr = tid; rr < nrows; rr += NT) {
    const int hq = hkv * r + rr / p.nblk, blk = rr % p.nblk;
    atomicAdd(&s_cnt[p.q0 / kChunk + blk], 1);   // the row's own chunk
    if (p.top_g == 0) continue;   // no groups kept (the indices may be absent)
    const int32_t* g = p.gidx + (((long long)b * p.Hq + hq) * p.nblk + blk) * p.top_g;
    // the row's kept groups as the attention kernels take them (see
    // load_routing_prefix): the ascending prefix of groups before the own
    // chunk; a chunk's groups are then consecutive entries
    const int limit = 8 * (p.q0 / kChunk + blk);
    int prev_g = -1, prev_c = -1;
    bool open = true;
    for (int i0 = 0; i0 < p.top_g && open; i0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) v[k] = i0 + k < p.top_g ? g[i0 + k] : -1;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        open = open && v[k] >= 0 && v[k] < limit && v[k] > prev_g;
        const int c = v[k] >> 3;
        if (open && c != prev_c) atomicAdd(&s_cnt[c], 1);
        prev_g = open ? v[k] : prev_g;
        prev_c = open ? c : prev_c;
      }
    }
  }
  __syncthreads();
  // counting sort on 256 buckets (bucket 255 - min(count, 255))
  for (int i = tid; i < p.nchunks; i += NT) {
    const int n = s_cnt[i];
    atomicAdd(&s_hist[255 - (n < 255 ? n : 255)], 1);
  }
  __syncthreads();
  static_assert(NT == 256, "one bucket per thread");
  const int v = s_hist[tid];
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) base += k < wv ? s_wsum[k] : 0;
  __syncthreads();
  s_hist[tid] = base + incl - v;   // first slot of the bucket
  __syncthreads();
  for (int i = tid; i < p.nchunks; i += NT) {
    const int n = s_cnt[i];
    const int pos = atomicAdd(&s_hist[255 - (n < 255 ? n : 255)], 1);
    p.order[(long long)bh * p.nchunks + pos] = i;
  }
}

// The routing row's entry of the group-mask map: byte c = mask of the row's
// kept groups in chunk c (bit t = group 8c + t), for every chunk of the
// history, from the row's kept groups in s_glist (nvalid of them).  Built in
// LDS as little-endian 32-bit words: group g is bit g & 31 of word g >> 5
// (byte g >> 3, bit g & 7), set with one atomic OR per kept group.  s_cm:
// nchunks bytes of 4-byte aligned LDS.  Every thread of the workgroup must
// call it.
template <typename P>
__device__ __forceinline__ void write_cmask_row(const P& p, long long row, int nvalid,
                                                const int* s_glist, uint32_t* s_cm) {
  const int tid = threadIdx.x;
  const int nch = p.Skv / kChunk;
  for (int i = tid; i < (nch + 3) / 4; i += kThreads) s_cm[i] = 0;
  __syncthreads();
  for (int i = tid; i < nvalid; i += kThreads) {
    const int g = s_glist[i];
    atomicOr(&s_cm[g >> 5], 1u << (g & 31));
  }
  __syncthreads();
  uint8_t* out = p.cmask + row * nch;
  if ((nch & 3) == 0) {
    // whole words: every row starts 4-byte aligned (the map is)
    for (int i = tid; i < nch / 4; i += kThreads) reinterpret_cast<uint32_t*>(out)[i] = s_cm[i];
  } else {
    const uint8_t* s8 = reinterpret_cast<const uint8_t*>(s_cm);
    for (int i = tid; i < nch; i += kThreads) out[i] = s8[i];
  }
}

// bf16: the register budget is held to four wavefronts per SIMD (4
// workgroups per CU, the most the LDS stages allow): the kernel is bound by
// latency more than by issue, so the extra resident wavefronts pay for the
// few values the compiler keeps in scratch
template <typename T>
constexpr int dq_waves_per_simd() { return sizeof(T) == 2 ? 4 : 2; }

template <typename T, int D, int TK, int S>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(dq_waves_per_simd<T>(), dq_waves_per_simd<T>())))
void attend_bwd_dq_kernel(const DqP p) {
  using RT = RowTile<T, D>;
  constexpr int kTileBytes = TK * RT::kUnits * 16;
  constexpr int kStage = 2 * kTileBytes;                          // K tile | V tile
  constexpr int kRowsPerWave = TK / 4;
  constexpr int kRPI = rows_per_issue<T, D>();
  constexpr int kIssues = kRowsPerWave / kRPI;
  constexpr int kLoads = 2 * kIssues;
  constexpr int kLocalTiles = kChunk / TK;
  constexpr int kGroupsPerTile = TK / kGroup;
  constexpr int NKS = TK / 16;
  constexpr int NMM = TK / 32;
  static_assert(kRowsPerWave % kRPI == 0, "tile rows per wave");
  __shared__ __attribute__((aligned(1024))) char smem[S * kStage];
  __shared__ int s_glist[kMaxTopG];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroups past the dQ work compute the dK/dV work order (launched only
  // with a workspace)
  static_assert(S * kStage >= (2048 + 256 + 4) * (int)sizeof(int), "order scratch in smem");
  if ((int)blockIdx.x >= p.nwork) {
    dq_order_block(p, (int)blockIdx.x - p.nwork, reinterpret_cast<int*>(smem));
    return;
  }
  const int w = xcd_remap(blockIdx.x, p.nwork);
  const int r = p.Hq / p.Hkv;
  const int per_bh = r * p.nblk;
  const int bh = w / per_bh, rem = w % per_bh;
  const int blk = rem / r, hql = rem % r;
  const int b = bh / p.Hkv, hkv = bh % p.Hkv, hq = hkv * r + hql;
  const int cb = p.q0 / kChunk + blk;
  const long long row = ((long long)b * p.Hq + hq) * p.nblk + blk;

  const int nvalid = load_routing_prefix<kThreads>(p.gidx + row * p.top_g, p.top_g, cb * 8,
                                                   s_glist, s_wsum);
  const int ntiles = kLocalTiles + (nvalid + kGroupsPerTile - 1) / kGroupsPerTile;

  const T* Kbh = reinterpret_cast<const T*>(p.K) + (long long)bh * p.Scap * D;
  const T* Vbh = reinterpret_cast<const T*>(p.V) + (long long)bh * p.Scap * D;
  const long long qrow0 = ((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk;
  const int qq = 16 * wv + l16;

  // Q and dO of this wavefront's 16 queries (B operands); delta = dO . O
  Frag<T> qf[D / 32], dof[D / 32];
  float delta;
  {
    const long long off = (qrow0 + qq) * D + 8 * g4;
    const T* q = reinterpret_cast<const T*>(p.Q) + off;
    const T* go = reinterpret_cast<const T*>(p.dO) + off;
    const T* o = reinterpret_cast<const T*>(p.O) + off;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      load_frag(qf[s], q + 32 * s);
      load_frag(dof[s], go + 32 * s);
      Frag<T> of;
      load_frag(of, o + 32 * s);
      part += frag_dot(dof[s], of);
    }
    delta = xor_sum16_32(part);
  }
  const float nlse2 = -p.lse[qrow0 + qq] * kLog2e;
  const float c2 = p.scale * kLog2e;

  // loop-invariant per-lane offsets (see attend_fwd.hip)
  RowOffsets<T, D> kro;
  kro.init();
  TrOffsets<(sizeof(T) == 2 ? D : 16)> kto;
  if constexpr (sizeof(T) == 2) kto.init();
  int ld_row[kIssues];
  uint32_t ld_col[kIssues];
#pragma unroll
  for (int j = 0; j < kIssues; ++j) {
    ld_row[j] = kRowsPerWave * wv + kRPI * j + lane / RT::kUnits;
    ld_col[j] = (uint32_t)(((lane % RT::kUnits) ^ RT::swz(ld_row[j])) << 4);
  }

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
      off[j] = tok * (uint32_t)(RT::kUnits * 16) + ld_col[j];
    }
#pragma unroll
    for (int j = 0; j < kIssues; ++j) {
      const uint32_t dst = buf + (uint32_t)((kRowsPerWave * wv + kRPI * j) * RT::kUnits * 16);
      dma16_off(off[j], Kbh, dst);
      dma16_off(off[j], Vbh, dst + kTileBytes);
    }
  };

  f32x4 dqacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dqacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    const int ahead = (ntiles - 1 - ti) < (S - 2) ? (ntiles - 1 - ti) : (S - 2);
    if (ahead >= 2) wait_vmcnt<2 * kLoads>();
    else if (ahead == 1) wait_vmcnt<kLoads>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (ti + S - 1 < ntiles) issue(ti + S - 1, gnext);

    const char* kt = smem + (ti % S) * kStage;
    const char* vt = kt + kTileBytes;

    constexpr int RB = RT::kUnits * 16;
    f32x4 sacc[NKS], dpacc[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      sacc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpacc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const char* kp = kt + kro.o[s];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Frag<T> a;
        frag_rows_at<T, D>(a, kp + 16 * ks * RB);
        mma(sacc[ks], a, qf[s]);
        frag_rows_at<T, D>(a, kp + kTileBytes + 16 * ks * RB);
        mma(dpacc[ks], a, dof[s]);
      }
    }
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
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[ks][i], c2, nlse2));
        sacc[ks][i] = pr * (dpacc[ks][i] - delta);   // dS
      }
    Frag<T> dsf[NMM];
#pragma unroll
    for (int mm = 0; mm < NMM; ++mm) frag_from_acc(dsf[mm], sacc[2 * mm], sacc[2 * mm + 1]);

    // dQ^T += K^T . dS^T ; K^T items of key slice mm: keys 32mm+4g+t, 32mm+16+4g+t
    if constexpr (sizeof(T) == 2) {
      uint32_t ka[D / 16];
#pragma unroll
      for (int c = 0; c < D / 16; ++c) ka[c] = lds_addr(kt) + kto.o[c];
      if constexpr (NMM == 1) {
#pragma unroll
        for (int c = 0; c < D / 16; c += 4) {
          const uint32_t a[8] = {ka[c], ka[c], ka[c + 1], ka[c + 1],
                                 ka[c + 2], ka[c + 2], ka[c + 3], ka[c + 3]};
          Frag<T> kf[4];
          tr_read8_sched<0, 16 * RB, 0, 16 * RB, 0, 16 * RB, 0, 16 * RB>(kf, a);
#pragma unroll
          for (int i = 0; i < 4; ++i) mma(dqacc[c + i], kf[i], dsf[0]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < D / 16; c += 2) {
          const uint32_t a[8] = {ka[c], ka[c], ka[c], ka[c], ka[c + 1], ka[c + 1], ka[c + 1], ka[c + 1]};
          Frag<T> kf[4];
          tr_read8_sched<0, 16 * RB, 32 * RB, 48 * RB, 0, 16 * RB, 32 * RB, 48 * RB>(kf, a);
          mma(dqacc[c], kf[0], dsf[0]);
          mma(dqacc[c], kf[1], dsf[1]);
          mma(dqacc[c + 1], kf[2], dsf[0]);
          mma(dqacc[c + 1], kf[3], dsf[1]);
        }
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int mm = 0; mm < NMM; ++mm) {
          Frag<T> kf;
          frag_tr<T, D>(kf, kt, 32 * mm + 4 * g4, 32 * mm + 16 + 4 * g4, 16 * ds);
          mma(dqacc[ds], kf, dsf[mm]);
        }
    }
  }

  // stores only after the tile pipeline: its vmcnt waits count direct loads
  // only (delta and the map are written here only when a workspace is given)
  if (p.delta && g4 == 0) p.delta[qrow0 + qq] = delta;

  // the row of the group-mask map (built in LDS, the stage buffers being free
  // once every wave is past them)
  if (p.cmask) {
    __syncthreads();
    write_cmask_row(p, row, nvalid, s_glist, reinterpret_cast<uint32_t*>(smem));
  }
  const float sc = p.scale;
  if constexpr (sizeof(T) == 2) {
    // the block's 64 dQ rows are contiguous: whole rows through the idle
    // stage buffers, past the map row's scratch at the start of smem
    constexpr int kOut = S * kStage - 64 * 2 * D;
    static_assert(kOut >= 2048, "dQ staging clear of the map row scratch");
    __syncthreads();   // every wave is done with the stage buffers
    out_rows_put<D>(smem + kOut, dqacc, sc, qq, g4);
    __syncthreads();
    out_rows_flush<D>(smem + kOut, reinterpret_cast<char*>(p.dQ) + qrow0 * 2 * D, tid);
  } else {
    T* dq = reinterpret_cast<T*>(p.dQ) + (qrow0 + qq) * D + 4 * g4;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd)
      store4(dq + 16 * dd, dqacc[dd][0] * sc, dqacc[dd][1] * sc, dqacc[dd][2] * sc,
             dqacc[dd][3] * sc);
  }
}

// The backward's preparation pass, for callers that run dQ and dK/dV side by
// side: per routing row, delta = rowsum(dO * O) and the row's entry of the
// group-mask map; per (b, kv head), the dK/dV work order (dq_order_block).
// These are what the dQ kernel otherwise writes into the workspace, computed
// the same way, so dK/dV results are bitwise the same after either.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attend_bwd_prep_kernel(const DqP p) {
  constexpr int kMaxRange = 2048;
  __shared__ __attribute__((aligned(16))) int s_mem[kMaxRange + 256 + 4];
  __shared__ int s_glist[kMaxTopG];
  __shared__ int s_wsum[4];
  if ((int)blockIdx.x >= p.nwork) {
    dq_order_block(p, (int)blockIdx.x - p.nwork, s_mem);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int w = xcd_remap(blockIdx.x, p.nwork);
  const int r = p.Hq / p.Hkv;
  const int per_bh = r * p.nblk;
  const int bh = w / per_bh, rem = w % per_bh;
  const int blk = rem / r, hql = rem % r;
  const int b = bh / p.Hkv, hkv = bh % p.Hkv, hq = hkv * r + hql;
  const int cb = p.q0 / kChunk + blk;
  const long long row = ((long long)b * p.Hq + hq) * p.nblk + blk;
  const long long qrow0 = ((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk;
  const int qq = 16 * wv + l16;
  // delta of this lane's query, summed in the dQ kernel's order
  {
    const long long off = (qrow0 + qq) * D + 8 * g4;
    const T* go = reinterpret_cast<const T*>(p.dO) + off;
    const T* o = reinterpret_cast<const T*>(p.O) + off;
    Frag<T> df[D / 32], of[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      load_frag(df[s], go + 32 * s);
      load_frag(of[s], o + 32 * s);
    }
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) part += frag_dot(df[s], of[s]);
    const float delta = xor_sum16_32(part);
    if (g4 == 0) p.delta[qrow0 + qq] = delta;
  }
  const int nvalid = load_routing_prefix<kThreads>(p.gidx + row * p.top_g, p.top_g, cb * 8,
                                                   s_glist, s_wsum);
  write_cmask_row(p, row, nvalid, s_glist, reinterpret_cast<uint32_t*>(s_mem));
}

template <typename T, int D>
DqP dq_params(const Dims& d, const void* Q, const void* K, const void* V, const void* O,
              const float* lse, const void* dO, const int32_t* gi, void* dQ, float* delta,
              uint8_t* cmask, int32_t* order) {
  DqP p;
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.lse = lse; p.dO = dO; p.gidx = gi; p.dQ = dQ;
  p.delta = delta; p.cmask = cmask; p.order = order;
  p.nchunks = d.Skv / kChunk;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.Scap = d.Scap; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_g = d.top_g; p.scale = d.scale;
  p.nwork = d.B * d.Hq * d.nblk;
  return p;
}

template <typename T, int D>
hipError_t run_dq(const Dims& d, const void* Q, const void* K, const void* V, const void* O,
                  const float* lse, const void* dO, const int32_t* gi, void* dQ, float* delta,
                  uint8_t* cmask, int32_t* order, hipStream_t s) {
  const DqP p = dq_params<T, D>(d, Q, K, V, O, lse, dO, gi, dQ, delta, cmask, order);
  constexpr int TK = HGA_DQ_TILE;
  constexpr int kStageBytes = 2 * TK * D * (int)sizeof(T);
  constexpr int S0 = HGA_DQ_STAGES;
  constexpr int S = S0 * kStageBytes <= 128 * 1024 ? S0 : (128 * 1024) / kStageBytes;
  static_assert(S >= 2, "at least two stages");
  // with a workspace: + one workgroup per (b, kv head) for the dK/dV work order
  const int extra = cmask ? d.B * d.Hkv : 0;
  attend_bwd_dq_kernel<T, D, TK, S><<<p.nwork + extra, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_prep(const Dims& d, const void* O, const void* dO, const int32_t* gi,
                    float* delta, uint8_t* cmask, int32_t* order, hipStream_t s) {
  const DqP p = dq_params<T, D>(d, nullptr, nullptr, nullptr, O, nullptr, dO, gi, nullptr,
                                delta, cmask, order);
  attend_bwd_prep_kernel<T, D><<<p.nwork + d.B * d.Hkv, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_bwd_dq(const Dims& d, const void* Q, const void* K, const void* V,
                                const void* O, const float* lse, const void* dO,
                                const int32_t* group_idx, void* dQ, float* delta,
                                uint8_t* cmask, int32_t* order, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run_dq<uint16_t, 128>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, cmask, order, s)
                      : run_dq<uint16_t, 64>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, cmask, order, s);
  return d.D == 128 ? run_dq<float, 128>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, cmask, order, s)
                    : run_dq<float, 64>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, cmask, order, s);
}

hipError_t launch_attend_bwd_prep(const Dims& d, const void* O, const void* dO,
                                  const int32_t* group_idx, float* delta, uint8_t* cmask,
                                  int32_t* order, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run_prep<uint16_t, 128>(d, O, dO, group_idx, delta, cmask, order, s)
                      : run_prep<uint16_t, 64>(d, O, dO, group_idx, delta, cmask, order, s);
  return d.D == 128 ? run_prep<float, 128>(d, O, dO, group_idx, delta, cmask, order, s)
                    : run_prep<float, 64>(d, O, dO, group_idx, delta, cmask, order, s);
}

}  // namespace hga
