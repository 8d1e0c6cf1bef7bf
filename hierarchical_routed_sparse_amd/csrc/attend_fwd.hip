// Exact-token attention forward over the routed groups plus the own chunk.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": after routing, only the exact key/value tokens of the kept
// groups are loaded and attention runs on them; the summaries are never used
// as keys or values.  The query at position p of a block attends the tokens
// of the block's kept groups and its own chunk up to p (causal).
//
// One workgroup (4 wavefronts) per (b, hq, block of 64 queries); wavefront w
// owns queries 16w..16w+15.  The key/value set is processed in 64-token tiles:
// tile 0 is the own chunk (causal mask), tile i >= 1 holds kept groups
// 8(i-1)..8(i-1)+7 (each group is 8 contiguous rows, a 2 KB run of K and of V
// at head_dim 128 in bf16).  Tiles are gathered from HBM into registers one
// tile ahead and written to LDS: K row-major (16-byte units XOR-swizzled by
// row), V transposed (so that the P.V product reads 4 consecutive keys per
// 8-byte LDS read).  Per tile and wavefront:
//   S^T[64 keys x 16 queries] = K . Q^T        (bf16 MFMA 16x16x32, fp32 acc)
//   online softmax in the log2 domain (running max and sum per query)
//   O^T[D x 16 queries]      += V^T . P^T      (bf16 MFMA, P rounded to bf16)
// The S^T accumulator layout (lane: one query, four keys) is directly the
// operand layout of P^T for the second product, so P never leaves registers.
#include "hga_device.h"
#include "hga_kernels.h"

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
  int B, Hq, Hkv, Sq, Skv, q0, nblk, top_g, nwork;
  float scale;
};

template <typename T, int D> struct FwdCfg {
  using RT = RowTile<T, D>;
  using CT = ColTile<T, D>;
  static constexpr int kStage = RT::kBytes + CT::kBytes;
  static constexpr int kStages = 2 * kStage <= 140 * 1024 ? 2 : 1;
  static constexpr int kPairs = 16 * (D / 8);   // pairs per 64-row matrix
  static constexpr int kJobs = 2 * kPairs;      // K pairs, then V pairs
  static constexpr int kJobsPerThread = (kJobs + kThreads - 1) / kThreads;
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attend_fwd_kernel(const FwdP p) {
  using Cfg = FwdCfg<T, D>;
  using RT = typename Cfg::RT;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kStages * Cfg::kStage];
  __shared__ int s_glist[kMaxTopG];
  __shared__ int s_glast;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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

  // routing row -> LDS; entries outside [0, 8*cb) are ignored
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

  // this wavefront's 16 queries as B operands of S^T = K . Q^T
  Frag<T> qf[D / 32];
  {
    const T* q = reinterpret_cast<const T*>(p.Q) + (qrow0 + 16 * wv + l16) * D + 8 * g4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) load_frag(qf[s], q + 32 * s);
  }

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
        if (isv)
          store_pair_cols<D>(buf + RT::kBytes, st[u], q, o);
        else
          store_pair_rows<D>(buf, st[u], q, o);
      }
    }
  };

  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale * kLog2e;
  const int qq = 16 * wv + l16;   // this lane's query within the block

  load_tile(0);
  store_tile(smem);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    if (ti + 1 < ntiles) load_tile(ti + 1);
    const char* buf = smem + (Cfg::kStages == 2 ? (ti & 1) : 0) * Cfg::kStage;

    // S^T = K . Q^T for 4 subtiles of 16 keys
    f32x4 sacc[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sacc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        Frag<T> kf;
        frag_rows<T, D>(kf, buf, 16 * ks + l16, s, g4);
        mma(sacc[ks], kf, qf[s]);
      }
    }
    // mask, running max
    float mt = -INFINITY;
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
        const float x = valid ? sacc[ks][i] * c2 : -INFINITY;
        sacc[ks][i] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = xor_max16_32(mt);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(sacc[ks][i] - m_new);
        sacc[ks][i] = e;
        psum += e;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;

    // O^T += V^T . P^T
    Frag<T> pf[2];
    frag_from_acc(pf[0], sacc[0], sacc[1]);
    frag_from_acc(pf[1], sacc[2], sacc[3]);
    const char* vt = buf + RT::kBytes;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        Frag<T> vf;
        frag_cols<T, D>(vf, vt, 16 * ds + l16, mm, g4);
        mma(oacc[ds], vf, pf[mm]);
      }

    if (Cfg::kStages == 1) __syncthreads();
    if (ti + 1 < ntiles) store_tile(smem + (Cfg::kStages == 2 ? ((ti + 1) & 1) : 0) * Cfg::kStage);
    __syncthreads();
  }

  // epilogue: normalise, write O (4 consecutive elements per lane) and lse
  const float l_tot = xor_sum16_32(l_run);
  const float inv = 1.0f / l_tot;
  T* o = reinterpret_cast<T*>(p.O) + (qrow0 + qq) * D + 4 * g4;
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    store4(o + 16 * ds, oacc[ds][0] * inv, oacc[ds][1] * inv, oacc[ds][2] * inv, oacc[ds][3] * inv);
  if (p.lse && g4 == 0) p.lse[qrow0 + qq] = (m_run + __log2f(l_tot)) * kLn2;
}

template <typename T, int D>
hipError_t run(const Dims& d, const void* Q, const void* K, const void* V, const int32_t* gi,
               void* O, float* lse, hipStream_t s) {
  FwdP p;
  p.Q = Q; p.K = K; p.V = V; p.gidx = gi; p.O = O; p.lse = lse;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.Sq = d.Sq; p.Skv = d.Skv; p.q0 = d.q0;
  p.nblk = d.nblk; p.top_g = d.top_g; p.scale = d.scale;
  p.nwork = d.B * d.Hq * d.nblk;
  attend_fwd_kernel<T, D><<<p.nwork, kThreads, 0, s>>>(p);
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
