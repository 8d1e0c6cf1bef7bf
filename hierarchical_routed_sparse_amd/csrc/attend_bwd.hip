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
// Two kernels:
//  * bwd_dq  -- one workgroup per (b, hq, block), the same tile walk as the
//    forward (own chunk, then 8 kept groups per tile); writes delta and dQ.
//  * bwd_dkdv -- one workgroup per (b, hkv, chunk of 64 keys).  It finds, for
//    every (query head of the kv group, query block), which of the chunk's 8
//    groups that row kept (binary search in the ascending routing row) or
//    whether the chunk is the row's own chunk (causal), compacts those rows in
//    a fixed order, and walks them: wavefront w owns keys 16w..16w+15 and skips
//    rows that kept neither of its two groups.  Each key's dK/dV is summed by
//    one wavefront in that fixed order: no atomics, bitwise reproducible.
#include "hga_device.h"
#include "hga_kernels.h"

namespace hga {
namespace {

constexpr int kMaxTopG = 512;
constexpr int kRowsPerPass = 1024;   // routing rows examined per entry-list build

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
  int B, Hq, Hkv, Sq, Skv, q0, nblk, top_g, nwork;
  float scale;
};

template <typename T, int D> struct DqCfg {
  using RT = RowTile<T, D>;
  using CT = ColTile<T, D>;
  // stage: K rows | V rows | K transposed
  static constexpr int kStage = 2 * RT::kBytes + CT::kBytes;
  static constexpr int kStages = 2 * kStage <= 140 * 1024 ? 2 : 1;
  static constexpr int kPairs = 16 * (D / 8);
  static constexpr int kJobs = 2 * kPairs;      // K pairs, then V pairs
  static constexpr int kJobsPerThread = (kJobs + kThreads - 1) / kThreads;
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attend_bwd_dq_kernel(const DqP p) {
  using Cfg = DqCfg<T, D>;
  using RT = typename Cfg::RT;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kStages * Cfg::kStage];
  __shared__ int s_glist[kMaxTopG];
  __shared__ int s_glast;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int r = p.Hq / p.Hkv;
  const int per_bh = r * p.nblk;
  const int bh = w / per_bh, rem = w % per_bh;
  const int blk = rem / r, hql = rem % r;
  const int b = bh / p.Hkv, hkv = bh % p.Hkv, hq = hkv * r + hql;
  const int cb = p.q0 / kChunk + blk;
  const long long row = ((long long)b * p.Hq + hq) * p.nblk + blk;

  if (tid == 0) s_glast = 0;
  __syncthreads();
  for (int i = tid; i < p.top_g; i += kThreads) {
    const int gm = p.gidx[row * p.top_g + i];
    const bool ok = gm >= 0 && gm < cb * 8;
    s_glist[i] = ok ? gm : -1;
    if (ok) atomicMax(&s_glast, i + 1);
  }
  __syncthreads();
  const int ntiles = 1 + (s_glast + 7) / 8;

  const T* Kbh = reinterpret_cast<const T*>(p.K) + (long long)bh * p.Skv * D;
  const T* Vbh = reinterpret_cast<const T*>(p.V) + (long long)bh * p.Skv * D;
  const long long qrow0 = ((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk;
  const int qq = 16 * wv + l16;

  // Q and dO of this wavefront's 16 queries (B operands); delta from dO . O
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
    if (g4 == 0) p.delta[qrow0 + qq] = delta;
  }
  const float lse2 = p.lse[qrow0 + qq] * kLog2e;
  const float c2 = p.scale * kLog2e;

  Pair<T> st[Cfg::kJobsPerThread];
  auto load_tile = [&](int ti) {
#pragma unroll
    for (int u = 0; u < Cfg::kJobsPerThread; ++u) {
      const int job = tid + kThreads * u;
      if (job < Cfg::kJobs) {
        const bool isv = job >= Cfg::kPairs;
        const int pr = isv ? job - Cfg::kPairs : job;
        const int q = pr / (D / 8), o = pr % (D / 8);
        long long tok = -1;
        if (ti == 0) {
          tok = (long long)cb * kChunk + 4 * q;
        } else {
          const int slot = 8 * (ti - 1) + (q >> 1);
          const int gm = slot < p.top_g ? s_glist[slot] : -1;
          if (gm >= 0) tok = (long long)gm * kGroup + 4 * (q & 1);
        }
        if (tok >= 0)
          load_pair(st[u], (isv ? Vbh : Kbh) + tok * D + 8 * o, D);
        else
          zero_pair(st[u]);
      }
    }
  };
  auto store_tile = [&](char* buf) {
#pragma unroll
    for (int u = 0; u < Cfg::kJobsPerThread; ++u) {
      const int job = tid + kThreads * u;
      if (job < Cfg::kJobs) {
        const bool isv = job >= Cfg::kPairs;
        const int pr = isv ? job - Cfg::kPairs : job;
        const int q = pr / (D / 8), o = pr % (D / 8);
        if (isv) {
          store_pair_rows<D>(buf + RT::kBytes, st[u], q, o);
        } else {
          store_pair_rows<D>(buf, st[u], q, o);
          store_pair_cols<D>(buf + 2 * RT::kBytes, st[u], q, o);
        }
      }
    }
  };

  f32x4 dqacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dqacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  store_tile(smem);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    if (ti + 1 < ntiles) load_tile(ti + 1);
    const char* buf = smem + (Cfg::kStages == 2 ? (ti & 1) : 0) * Cfg::kStage;
    const char* vs = buf + RT::kBytes;
    const char* kt = buf + 2 * RT::kBytes;

    f32x4 sacc[4], dpacc[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sacc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpacc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        Frag<T> a;
        frag_rows<T, D>(a, buf, 16 * ks + l16, s, g4);
        mma(sacc[ks], a, qf[s]);
        frag_rows<T, D>(a, vs, 16 * ks + l16, s, g4);
        mma(dpacc[ks], a, dof[s]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bool gvalid = true;
      if (ti > 0) {
        const int slot = 8 * (ti - 1) + 2 * ks + (g4 >> 1);
        gvalid = slot < p.top_g && s_glist[slot] >= 0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 16 * ks + 4 * g4 + i;
        const bool valid = ti == 0 ? kk <= qq : gvalid;
        const float pr = valid ? __builtin_amdgcn_exp2f(sacc[ks][i] * c2 - lse2) : 0.f;
        sacc[ks][i] = pr * (dpacc[ks][i] - delta);   // dS
      }
    }
    Frag<T> dsf[2];
    frag_from_acc(dsf[0], sacc[0], sacc[1]);
    frag_from_acc(dsf[1], sacc[2], sacc[3]);
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        Frag<T> a;
        frag_cols<T, D>(a, kt, 16 * dd + l16, mm, g4);
        mma(dqacc[dd], a, dsf[mm]);
      }

    if (Cfg::kStages == 1) __syncthreads();
    if (ti + 1 < ntiles) store_tile(smem + (Cfg::kStages == 2 ? ((ti + 1) & 1) : 0) * Cfg::kStage);
    __syncthreads();
  }

  T* dq = reinterpret_cast<T*>(p.dQ) + (qrow0 + qq) * D + 4 * g4;
  const float sc = p.scale;
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd)
    store4(dq + 16 * dd, dqacc[dd][0] * sc, dqacc[dd][1] * sc, dqacc[dd][2] * sc, dqacc[dd][3] * sc);
}

// ============================================================== dK, dV

struct DkvP {
  const void* Q;
  const void* K;
  const void* V;
  const float* lse;
  const void* dO;
  const int32_t* gidx;
  const float* delta;
  void* dK;
  void* dV;
  int B, Hq, Hkv, Sq, Skv, q0, nblk, top_g, nchunks, nwork;
  float scale;
};

template <typename T, int D> struct DkvCfg {
  using RT = RowTile<T, D>;
  using CT = ColTile<T, D>;
  // stage: Q rows | dO rows | Q transposed | dO transposed | lse2[64] | delta[64]
  static constexpr int kOffDo = RT::kBytes;
  static constexpr int kOffQt = 2 * RT::kBytes;
  static constexpr int kOffDot = 2 * RT::kBytes + CT::kBytes;
  static constexpr int kOffStat = 2 * RT::kBytes + 2 * CT::kBytes;
  static constexpr int kStage = kOffStat + 2 * 64 * 4;
  static constexpr int kStages = 2 * kStage <= 142 * 1024 ? 2 : 1;
  static constexpr int kPairs = 16 * (D / 8);
  static constexpr int kJobs = 2 * kPairs;      // Q pairs, then dO pairs
  static constexpr int kJobsPerThread = (kJobs + kThreads - 1) / kThreads;
};

// entry word: (row << 9) | mask, mask bits 0..7 = kept groups, bit 8 = own chunk
constexpr uint32_t kLocalBit = 1u << 8;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attend_bwd_dkdv_kernel(const DkvP p) {
  using Cfg = DkvCfg<T, D>;
  using RT = typename Cfg::RT;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kStages * Cfg::kStage];
  __shared__ uint32_t s_ent[kRowsPerPass];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / p.nchunks, c = w % p.nchunks;
  const int b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int r = p.Hq / p.Hkv;
  const int nrows = r * p.nblk;          // (query head in group, block), head-major
  const int kin = 16 * wv + l16;         // this lane's key within the chunk
  const int mygroups = 3 << (2 * wv);    // the two groups owned by this wavefront

  // this wavefront's 16 keys as B operands of S = Q . K^T and dP = dO . V^T
  Frag<T> kf[D / 32], vf[D / 32];
  {
    const long long off = ((long long)bh * p.Skv + (long long)c * kChunk + kin) * D + 8 * g4;
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
  const int blk_first = c - p.q0 / kChunk;   // rows with block >= this can touch chunk c

  Pair<T> st[Cfg::kJobsPerThread];
  float st_stat = 0.f;
  auto entry_rows = [&](uint32_t ent, int& hq, int& blk) {
    const int rr = (int)(ent >> 9);
    hq = hkv * r + rr / p.nblk;
    blk = rr % p.nblk;
  };
  auto load_entry = [&](uint32_t ent) {
    int hq, blk;
    entry_rows(ent, hq, blk);
    const long long qrow0 = ((long long)b * p.Hq + hq) * p.Sq + (long long)blk * kChunk;
#pragma unroll
    for (int u = 0; u < Cfg::kJobsPerThread; ++u) {
      const int job = tid + kThreads * u;
      if (job < Cfg::kJobs) {
        const bool isdo = job >= Cfg::kPairs;
        const int pr = isdo ? job - Cfg::kPairs : job;
        const int q = pr / (D / 8), o = pr % (D / 8);
        const T* src = reinterpret_cast<const T*>(isdo ? p.dO : p.Q) + (qrow0 + 4 * q) * D + 8 * o;
        load_pair(st[u], src, D);
      }
    }
    if (tid < 64)
      st_stat = p.lse[qrow0 + tid] * kLog2e;
    else if (tid < 128)
      st_stat = p.delta[qrow0 + tid - 64];
  };
  auto store_entry = [&](char* buf) {
#pragma unroll
    for (int u = 0; u < Cfg::kJobsPerThread; ++u) {
      const int job = tid + kThreads * u;
      if (job < Cfg::kJobs) {
        const bool isdo = job >= Cfg::kPairs;
        const int pr = isdo ? job - Cfg::kPairs : job;
        const int q = pr / (D / 8), o = pr % (D / 8);
        store_pair_rows<D>(buf + (isdo ? Cfg::kOffDo : 0), st[u], q, o);
        store_pair_cols<D>(buf + (isdo ? Cfg::kOffDot : Cfg::kOffQt), st[u], q, o);
      }
    }
    if (tid < 128) reinterpret_cast<float*>(buf + Cfg::kOffStat)[tid] = st_stat;
  };

  for (int r0 = 0; r0 < nrows; r0 += kRowsPerPass) {
    // ---- entry list for routing rows [r0, r0 + kRowsPerPass)
    int nent = 0;
    for (int base = 0; base < kRowsPerPass && r0 + base < nrows; base += kThreads) {
      const int rr = r0 + base + tid;
      uint32_t mask = 0;
      if (rr < nrows) {
        const int hq = hkv * r + rr / p.nblk, blk = rr % p.nblk;
        if (blk == blk_first) {
          mask = kLocalBit | 0xFFu;
        } else if (blk > blk_first) {
          const int32_t* g = p.gidx + (((long long)b * p.Hq + hq) * p.nblk + blk) * p.top_g;
          const int lo_g = 8 * c;
          int lo = 0, hi = p.top_g;      // first entry that is not a valid group below chunk c
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const int v = g[mid];
            if (v >= 0 && v < lo_g) lo = mid + 1; else hi = mid;
          }
          for (int i = lo; i < p.top_g && i < lo + 8; ++i) {
            const int v = g[i];
            if (v < lo_g || v >= lo_g + 8) break;
            mask |= 1u << (v - lo_g);
          }
        }
      }
      const bool f = mask != 0;
      const uint64_t bal = __ballot(f);
      if (lane == 0) s_wsum[wv] = __popcll(bal);
      __syncthreads();
      int off = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = s_wsum[i];
        off += i < wv ? v : 0;
        tot += v;
      }
      if (f) s_ent[nent + off + mbcnt(bal)] = ((uint32_t)rr << 9) | mask;
      nent += tot;
      __syncthreads();
    }
    if (nent == 0) continue;

    // ---- walk the entries
    load_entry(s_ent[0]);
    store_entry(smem);
    __syncthreads();
    for (int e = 0; e < nent; ++e) {
      if (e + 1 < nent) load_entry(s_ent[e + 1]);
      const char* buf = smem + (Cfg::kStages == 2 ? (e & 1) : 0) * Cfg::kStage;
      const uint32_t ent = s_ent[e];
      const bool local = (ent & kLocalBit) != 0;
      if (local || (ent & mygroups)) {
        const char* dos = buf + Cfg::kOffDo;
        const char* qt = buf + Cfg::kOffQt;
        const char* dot = buf + Cfg::kOffDot;
        const float* stat = reinterpret_cast<const float*>(buf + Cfg::kOffStat);
        const bool kvalid = local || ((ent >> (kin >> 3)) & 1u);

        f32x4 sacc[4], dpacc[4];
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          sacc[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
          dpacc[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            Frag<T> a;
            frag_rows<T, D>(a, buf, 16 * qs + l16, s, g4);
            mma(sacc[qs], a, kf[s]);
            frag_rows<T, D>(a, dos, 16 * qs + l16, s, g4);
            mma(dpacc[qs], a, vf[s]);
          }
        }
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          const float4 l4 = reinterpret_cast<const float4*>(stat)[4 * qs + g4];
          const float4 d4 = reinterpret_cast<const float4*>(stat + 64)[4 * qs + g4];
          const float lq[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dq[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int q = 16 * qs + 4 * g4 + i;
            const bool valid = local ? kin <= q : kvalid;
            const float pr = valid ? __builtin_amdgcn_exp2f(sacc[qs][i] * c2 - lq[i]) : 0.f;
            sacc[qs][i] = pr;
            dpacc[qs][i] = pr * (dpacc[qs][i] - dq[i]);
          }
        }
        Frag<T> pf[2], dsf[2];
        frag_from_acc(pf[0], sacc[0], sacc[1]);
        frag_from_acc(pf[1], sacc[2], sacc[3]);
        frag_from_acc(dsf[0], dpacc[0], dpacc[1]);
        frag_from_acc(dsf[1], dpacc[2], dpacc[3]);
#pragma unroll
        for (int dd = 0; dd < D / 16; ++dd)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            Frag<T> a;
            frag_cols<T, D>(a, dot, 16 * dd + l16, mm, g4);
            mma(dvacc[dd], a, pf[mm]);
            frag_cols<T, D>(a, qt, 16 * dd + l16, mm, g4);
            mma(dkacc[dd], a, dsf[mm]);
          }
      }
      if (Cfg::kStages == 1) __syncthreads();
      if (e + 1 < nent) store_entry(smem + (Cfg::kStages == 2 ? ((e + 1) & 1) : 0) * Cfg::kStage);
      __syncthreads();
    }
  }

  // every key of the chunk is written (zero when nothing attends it)
  const long long krow = (long long)bh * p.Skv + (long long)c * kChunk + kin;
  T* dk = reinterpret_cast<T*>(p.dK) + krow * D + 4 * g4;
  T* dv = reinterpret_cast<T*>(p.dV) + krow * D + 4 * g4;
  const float sc = p.scale;
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) {
    store4(dk + 16 * dd, dkacc[dd][0] * sc, dkacc[dd][1] * sc, dkacc[dd][2] * sc, dkacc[dd][3] * sc);
    store4(dv + 16 * dd, dvacc[dd][0], dvacc[dd][1], dvacc[dd][2], dvacc[dd][3]);
  }
}

template <typename T, int D>
hipError_t run_dq(const Dims& d, const void* Q, const void* K, const void* V, const void* O,
                  const float* lse, const void* dO, const int32_t* gi, void* dQ, float* delta,
                  hipStream_t s) {
  DqP p;
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.lse = lse; p.dO = dO; p.gidx = gi; p.dQ = dQ;
  p.delta = delta;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_g = d.top_g; p.scale = d.scale;
  p.nwork = d.B * d.Hq * d.nblk;
  attend_bwd_dq_kernel<T, D><<<p.nwork, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_dkdv(const Dims& d, const void* Q, const void* K, const void* V, const float* lse,
                    const void* dO, const int32_t* gi, const float* delta, void* dK, void* dV,
                    hipStream_t s) {
  DkvP p;
  p.Q = Q; p.K = K; p.V = V; p.lse = lse; p.dO = dO; p.gidx = gi; p.delta = delta;
  p.dK = dK; p.dV = dV;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_g = d.top_g; p.scale = d.scale;
  p.nchunks = d.Skv / kChunk;
  p.nwork = d.B * d.Hkv * p.nchunks;
  attend_bwd_dkdv_kernel<T, D><<<p.nwork, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_bwd_dq(const Dims& d, const void* Q, const void* K, const void* V,
                                const void* O, const float* lse, const void* dO,
                                const int32_t* group_idx, void* dQ, float* delta,
                                hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run_dq<uint16_t, 128>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, s)
                      : run_dq<uint16_t, 64>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, s);
  return d.D == 128 ? run_dq<float, 128>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, s)
                    : run_dq<float, 64>(d, Q, K, V, O, lse, dO, group_idx, dQ, delta, s);
}

hipError_t launch_attend_bwd_dkdv(const Dims& d, const void* Q, const void* K, const void* V,
                                  const float* lse, const void* dO, const int32_t* group_idx,
                                  const float* delta, void* dK, void* dV, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run_dkdv<uint16_t, 128>(d, Q, K, V, lse, dO, group_idx, delta, dK, dV, s)
                      : run_dkdv<uint16_t, 64>(d, Q, K, V, lse, dO, group_idx, delta, dK, dV, s);
  return d.D == 128 ? run_dkdv<float, 128>(d, Q, K, V, lse, dO, group_idx, delta, dK, dV, s)
                    : run_dkdv<float, 64>(d, Q, K, V, lse, dO, group_idx, delta, dK, dV, s);
}

}  // namespace hga
