// Decode: exact-token attention of one new query per (b, query head).
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently", read for generation: the newest token, routed like a query
// block that holds one query, attends the exact tokens of its kept groups and
// the tokens of its own chunk up to itself.  One query against at most
// 8 * top_g + 64 keys is a matrix-vector product: the work is bound by the
// key/value rows gathered from memory, not by arithmetic, so it runs on the
// vector ALUs (an MFMA tile would compute 15 discarded query rows for each
// useful one).
//
// One workgroup per (b, query head) with nw wavefronts (split-K).  The key
// list is the kept groups (ascending) followed by the groups of the own chunk;
// it is cut into tiles of 4 groups (32 keys), and wavefront w takes tiles
// w, w + nw, ...  Per tile:
//   - a lane loads 16 bytes of each of NI key rows and NI value rows (E
//     elements of the columns E*col..E*col+E-1; RPI rows per load instruction,
//     so every load covers whole rows), all loads issued before any use;
//   - each lane dots its key pieces with its piece of the query; a
//     reduce-scatter over the LPR lanes of a row (halve the set of partial
//     sums at each exchange) leaves the logit of key row RPI*(c/2) + rg in
//     lanes c and c^1 of the row group;
//   - online softmax across the wavefront's tiles (log2 domain), and the value
//     rows are weighted by their probabilities fetched from the lanes holding
//     them.
// The wavefronts' partial results (running max, sum and output row) are merged
// in LDS in wavefront order by wavefront 0, which writes O and lse.
#include "hga_device.h"
#include "hga_kernels.h"

namespace hga {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kTileGroups = 4;
constexpr int kTileKeys = kTileGroups * kGroup;

struct DecP {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* gidx;
  void* O;
  float* lse;
  int Hq, Hkv, Scap, top_g;
  int p;        // position of the query (kv_len - 1)
  int cp;       // its own chunk
  int ngk;      // kept groups per row (the first ngk entries of a gidx row)
  int ng;       // key-list groups: ngk + groups of the own chunk up to p
  int ntiles;   // ceil(ng / kTileGroups)
  float c2;     // softmax scale * log2(e)
};

// Element e of the 16 bytes u (bf16: element 2w in the low half of word w).
template <typename T> __device__ __forceinline__ float elem(const uint4& u, int e);
template <> __device__ __forceinline__ float elem<uint16_t>(const uint4& u, int e) {
  const uint32_t w = (&u.x)[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <> __device__ __forceinline__ float elem<float>(const uint4& u, int e) {
  return __uint_as_float((&u.x)[e]);
}

// Butterfly max / sum over the wavefront: every lane ends with the same value
// (each exchange adds the same two operands on both partners).
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Raw buffer resource over `bytes` bytes at `base` (word 3 = 0x00020000, the
// gfx9 raw-buffer format: 32-bit data, no swizzle).  A load whose offset lies
// at or past `bytes` returns zero, so masked rows need no branch, and each
// load needs one 32-bit offset register instead of a 64-bit address.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr uint32_t kMaskedOffset = 0x80000000u;   // past every resource's size

// 16 bytes of the NI key (or value) rows of a tile that this lane reads:
// load instruction i covers rows RPI*i .. RPI*i + RPI - 1 of the tile, the lane
// row RPI*i + rg, at position 8 * group + row % 8; zero for rows past the key
// list or past the query.  `col` is the lane's byte offset within a row.
template <typename T, int D, int NI, int RPI>
__device__ __forceinline__ void load_rows(uint4 (&r)[NI], __amdgpu_buffer_rsrc_t rs,
                                          const int (&g)[kTileGroups], int rg, uint32_t col,
                                          int qpos) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int gi = g[(RPI * i) / kGroup];
    const int pos = kGroup * gi + (RPI * i + rg) % kGroup;
    const uint32_t off = (gi >= 0 && pos <= qpos) ? (uint32_t)pos * (D * sizeof(T)) + col
                                                  : kMaskedOffset;
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    r[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_kernel(const DecP p) {
  constexpr int E = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int LPR = D / E;                // lanes per key row
  constexpr int RPI = 64 / LPR;             // key rows per load instruction
  constexpr int NI = kTileKeys / RPI;       // load instructions per tile (K, and V)
  static_assert(2 * NI == LPR, "the reduce-scatter assumes LPR = 2 NI");
  static_assert(kGroup % RPI == 0, "a load instruction's rows lie in one group");
  static_assert(kTileGroups == 4, "the group lookup below selects among 4");
  // value rows are fetched together with the key rows when both fit in 64
  // registers (bf16, and fp32 with D = 64); else after the logits
  constexpr bool kEarlyV = 8 * NI <= 64;
  constexpr int CPL = D / 64;               // output columns per lane in the merge
  __shared__ float s_o[kMaxWaves][D];
  __shared__ float s_m[kMaxWaves], s_l[kMaxWaves];

  // (the wavefront index is uniform: say so, so that the tile loop, the group
  // lookups and the buffer resources stay in scalar registers)
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  // work: b * Hq + hq; the query heads of one kv head run on one XCD
  const int row = xcd_remap(blockIdx.x, gridDim.x);
  const int hq = row % p.Hq, b = row / p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const int rg = lane / LPR, c = lane % LPR;

  float q[E];
  {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(p.Q) +
                                                   (long long)row * D + E * c);
#pragma unroll
    for (int e = 0; e < E; ++e) q[e] = elem<T>(u, e);
  }
  const long long kvb = ((long long)b * p.Hkv + hkv) * p.Scap * D;
  const uint32_t kvbytes = (uint32_t)p.Scap * (D * sizeof(T));
  const auto Kr = make_rsrc(reinterpret_cast<const T*>(p.K) + kvb, kvbytes);
  const auto Vr = make_rsrc(reinterpret_cast<const T*>(p.V) + kvb, kvbytes);
  const uint32_t col = E * c * sizeof(T);
  const int32_t* gl = p.gidx + (long long)row * p.top_g;

  float m_run = -INFINITY, l_run = 0.f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  // the kept groups taken from the row: its longest prefix of groups before
  // the own chunk, each above the one before it (all p.ngk entries of a row
  // written by the routing); slots past the prefix hold no key
  int nk = p.ngk;
  for (int s0 = 0; s0 < p.ngk; s0 += 64) {
    const int s = s0 + lane;
    const int v = s < p.ngk ? gl[s] : 0;
    const int prev = s > 0 && s < p.ngk ? gl[s - 1] : -1;
    const uint64_t bad = __ballot(s < p.ngk && (v < 0 || v >= kGroup * p.cp || v <= prev));
    if (bad) {
      nk = s0 + (int)__builtin_ctzll(bad);
      break;
    }
  }

  for (int t = wv; t < p.ntiles; t += nw) {
    // the tile's 4 groups (-1: no key in the slot)
    int g[kTileGroups];
#pragma unroll
    for (int j = 0; j < kTileGroups; ++j) {
      const int s = kTileGroups * t + j;
      g[j] = s < nk ? gl[s] : s < p.ngk ? -1 : (s < p.ng ? kGroup * p.cp + (s - p.ngk) : -1);
    }
    uint4 kr[NI], vr[NI];
    load_rows<T, D, NI, RPI>(kr, Kr, g, rg, col, p.p);
    if constexpr (kEarlyV) load_rows<T, D, NI, RPI>(vr, Vr, g, rg, col, p.p);
    float sd[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) a = fmaf(q[e], elem<T>(kr[i], e), a);
      sd[i] = a;
    }
    if constexpr (!kEarlyV) load_rows<T, D, NI, RPI>(vr, Vr, g, rg, col, p.p);
    // reduce-scatter over the LPR lanes of a row: at the exchange with lane
    // xor m, a lane keeps the upper half of its n partial sums when bit m of
    // its index is set, the lower half otherwise
#pragma unroll
    for (int n = NI, m = LPR / 2; n > 1; n >>= 1, m >>= 1) {
      const bool up = (c & m) != 0;
#pragma unroll
      for (int j = 0; j < n / 2; ++j) {
        const float keep = up ? sd[j + n / 2] : sd[j];
        const float send = up ? sd[j] : sd[j + n / 2];
        sd[j] = keep + __shfl_xor(send, m);
      }
    }
    const float s = sd[0] + __shfl_xor(sd[0], 1);
    // this lane's key row: RPI * (c / 2) + rg
    const int kt = RPI * (c >> 1) + rg;
    const int jt = kt / kGroup;
    const int gk = jt == 0 ? g[0] : jt == 1 ? g[1] : jt == 2 ? g[2] : g[3];
    const int pk = kGroup * gk + kt % kGroup;
    const float x = (gk >= 0 && pk <= p.p) ? s * p.c2 : -INFINITY;
    // online softmax; a tile with no key (slots cut from a malformed row)
    // leaves m at -inf, and the exponents are then taken against 0
    const float m_new = fmaxf(m_run, wave_max_f(x));
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    const float pe = __builtin_amdgcn_exp2f(x - m_ref);
    l_run = fmaf(l_run, alpha, wave_sum_f((c & 1) ? 0.f : pe));
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pi = __shfl(pe, rg * LPR + 2 * i);   // probability of row RPI*i + rg
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pi, elem<T>(vr[i], e), o[e]);
    }
  }

  // sum the row groups' partial outputs (lanes c, c + LPR, ...)
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += __shfl_xor(o[e], m);
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) s_o[wv][E * c + e] = o[e];
  }
  if (lane == 0) {
    s_m[wv] = m_run;   // -inf with l_run = 0 for a wavefront without tiles
    s_l[wv] = l_run;
  }
  __syncthreads();
  if (wv != 0) return;

  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, s_m[w]);
  float lsum = 0.f, acc[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) acc[u] = 0.f;
  for (int w = 0; w < nw; ++w) {
    const float f = __builtin_amdgcn_exp2f(s_m[w] - M);
    lsum = fmaf(f, s_l[w], lsum);
#pragma unroll
    for (int u = 0; u < CPL; ++u) acc[u] = fmaf(f, s_o[w][CPL * lane + u], acc[u]);
  }
  const float inv = 1.0f / lsum;
  T* Or = reinterpret_cast<T*>(p.O) + (long long)row * D + CPL * lane;
  if constexpr (sizeof(T) == 2 && CPL == 2) {
    *reinterpret_cast<uint32_t*>(Or) = pack_bf16(acc[0] * inv, acc[1] * inv);
  } else if constexpr (sizeof(T) == 2) {
    Or[0] = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xFFFFu);
  } else {
#pragma unroll
    for (int u = 0; u < CPL; ++u) Or[u] = acc[u] * inv;
  }
  if (p.lse && lane == 0) p.lse[row] = (M + __log2f(lsum)) * kLn2;
}

template <typename T, int D>
hipError_t run(const Dims& d, const void* Q, const void* K, const void* V, const int32_t* gi,
               void* O, float* lse, hipStream_t s) {
  DecP p;
  p.Q = Q; p.K = K; p.V = V; p.gidx = gi; p.O = O; p.lse = lse;
  p.Hq = d.Hq; p.Hkv = d.Hkv; p.Scap = d.Scap; p.top_g = d.top_g;
  p.p = d.Skv - 1;
  p.cp = p.p / kChunk;
  const int kk = d.top_k < p.cp ? d.top_k : p.cp;   // chunks kept by the routing
  p.ngk = d.top_g < kGroup * kk ? d.top_g : kGroup * kk;
  p.ng = p.ngk + (p.p - kChunk * p.cp) / kGroup + 1;
  p.ntiles = (p.ng + kTileGroups - 1) / kTileGroups;
  p.c2 = d.scale * kLog2e;
  // balance the tiles over at most kMaxWaves wavefronts
  const int rounds = (p.ntiles + kMaxWaves - 1) / kMaxWaves;
  const int nw = (p.ntiles + rounds - 1) / rounds;
  decode_kernel<T, D><<<d.B * d.Hq, 64 * nw, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attend(const Dims& d, const void* Q, const void* K, const void* V,
                                const int32_t* group_idx, void* O, float* lse, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run<uint16_t, 128>(d, Q, K, V, group_idx, O, lse, s)
                      : run<uint16_t, 64>(d, Q, K, V, group_idx, O, lse, s);
  return d.D == 128 ? run<float, 128>(d, Q, K, V, group_idx, O, lse, s)
                    : run<float, 64>(d, Q, K, V, group_idx, O, lse, s);
}

}  // namespace hga
