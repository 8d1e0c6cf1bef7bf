// The routed working set of a segment, staged into device memory.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently", memory paragraph: GPU memory holds the summaries, the active
// segment and the routed working set; older keys and values live in host
// RAM.  After a segment is routed, the distinct history groups its rows kept
// (the union over the rows of each (b, kv head)) are copied once into a
// compact device buffer, followed by the segment's own rows, and every
// routing row is rewritten against that buffer.  The attention kernels then
// run on the staged buffer as on any history: the union keeps the groups in
// ascending order, so every row's kept groups stay ascending and each tile
// holds the same rows as before, and the results equal those over the full
// history bit for bit.
//
// Staged layout per (b, kv head), `sg` group slots (a multiple of 8):
//   tokens 8k .. 8k+7        = history group union[k], k < n (n = the union's
//                              size; slots n .. sg-1 are not written)
//   tokens 8 sg .. 8 sg + q_len - 1 = the segment's own rows (positions
//                              kv_len - q_len .. kv_len - 1)
// A routing row's group g maps to its rank in the union when g lies before
// the segment, else to g - 8 (kv_len - q_len)/64 + sg.
#include "hga_kernels.h"
#include "hga_device.h"

namespace hga {
namespace {

constexpr int kUnionThreads = 1024;
constexpr int kMaxHistGroups = 16384;   // HGA_MAX_KV_LEN / 8
constexpr int kWords = kMaxHistGroups / 32;

struct StageP {
  const int32_t* gidx;   // [B][Hq][nblk][top_g]
  int32_t* gidx_out;     // [B][Hq][nblk][top_g], rewritten
  int32_t* ulist;        // [B * Hkv][sg] the union, ascending
  int32_t* ucount;       // [B * Hkv] its size
  const void* K;         // [B][Hkv][Scap][D]
  const void* V;
  void* Ks;              // [B][Hkv][Scap_s][D]
  void* Vs;
  int B, Hq, Hkv, nblk, top_g, q0, Sq, Scap, Scap_s, sg, row_bytes;
};

// Per (b, kv head): the union of the history groups its rows keep (each row
// read as its ascending prefix of groups before its own chunk, the rule of
// the attention kernels), as a bitmap in LDS, then ranks, the list, and the
// rewritten rows.
__global__ __launch_bounds__(kUnionThreads) void stage_union_kernel(const StageP p) {
  __shared__ uint32_t s_bits[kWords];
  __shared__ int s_base[kWords];
  __shared__ int s_wsum[kUnionThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NW = kUnionThreads / 64;
  const int bh = blockIdx.x, b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int r = p.Hq / p.Hkv, nrows = r * p.nblk;
  const int hist = 8 * (p.q0 / kChunk);            // history groups (before the segment)
  const int nwords = (hist + 31) / 32;
  for (int i = tid; i < kWords; i += kUnionThreads) s_bits[i] = 0;
  __syncthreads();
  // one wavefront per row: the row's prefix length, then mark its history groups
  auto row_ptr = [&](int rr) {
    const int hq = hkv * r + rr / p.nblk, blk = rr % p.nblk;
    return (((long long)b * p.Hq + hq) * p.nblk + blk) * p.top_g;
  };
  auto prefix_len = [&](const int32_t* g, int limit) {
    int n = p.top_g;
    for (int i0 = 0; i0 < p.top_g; i0 += 64) {
      const int i = i0 + lane;
      const int v = i < p.top_g ? g[i] : 0;
      const int prev = i > 0 && i < p.top_g ? g[i - 1] : -1;
      const uint64_t bad = __ballot(i < p.top_g && (v < 0 || v >= limit || v <= prev));
      if (bad) {
        n = i0 + (int)__builtin_ctzll(bad);
        break;
      }
    }
    return n;
  };
  for (int rr = wv; rr < nrows; rr += NW) {
    const int32_t* g = p.gidx + row_ptr(rr);
    const int limit = 8 * (p.q0 / kChunk + rr % p.nblk);
    const int n = prefix_len(g, limit);
    for (int i = lane; i < n; i += 64) {
      const int v = g[i];
      if (v < hist) atomicOr(&s_bits[v >> 5], 1u << (v & 31));
    }
  }
  __syncthreads();
  // exclusive prefix of the words' popcounts
  int cnt = 0;
  if (tid < kWords) cnt = tid < nwords ? __popc(s_bits[tid]) : 0;
  // kWords (512) words over the first 8 wavefronts
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int k = 0; k < wv; ++k) base += s_wsum[k];
  if (tid < kWords) s_base[tid] = base + incl - cnt;
  int total = 0;
  for (int k = 0; k < NW; ++k) total += s_wsum[k];
  __syncthreads();
  // the union, ascending
  int32_t* list = p.ulist + (long long)bh * p.sg;
  if (tid < nwords) {
    uint32_t m = s_bits[tid];
    int k = s_base[tid];
    while (m) {
      const int bit = __builtin_ctz(m);
      list[k++] = 32 * tid + bit;
      m &= m - 1;
    }
  }
  if (tid == 0) p.ucount[bh] = total;
  // every row rewritten against the staged layout
  const int seg0 = hist;   // first group of the segment
  for (int rr = wv; rr < nrows; rr += NW) {
    const long long o = row_ptr(rr);
    const int32_t* g = p.gidx + o;
    const int limit = 8 * (p.q0 / kChunk + rr % p.nblk);
    const int n = prefix_len(g, limit);
    for (int i = lane; i < p.top_g; i += 64) {
      int v = -1;
      if (i < n) {
        const int x = g[i];
        if (x < seg0) {
          const uint32_t w = s_bits[x >> 5];
          v = s_base[x >> 5] + __popc(w & ((1u << (x & 31)) - 1u));
        } else {
          v = x - seg0 + p.sg;
        }
      }
      p.gidx_out[o + i] = v;
    }
  }
}

// Copies the staged rows: workgroup j < sg / 8 takes union slots 8j .. 8j+7
// (64 token rows), the later ones 64 rows of the segment each.  The 64 rows
// are moved as one run of 64 * row_bytes destination bytes, 16 bytes per lane
// and consecutive lanes on consecutive bytes, so a wave's load covers whole
// rows (1 KB of K or V, from at most two source groups of 8 contiguous rows):
// over the host link that is a few long reads rather than many 16-byte ones.
// Every load of a thread is issued before its first store.
__global__ __launch_bounds__(256) void stage_copy_kernel(const StageP p) {
  const int per_bh = p.sg / 8 + p.Sq / kChunk;
  const int bh = blockIdx.x / per_bh, j = blockIdx.x % per_bh;
  const int tid = threadIdx.x;
  const bool uni = j < p.sg / 8;
  const int nslot = uni ? p.ucount[bh] - 8 * j : 8;   // groups of this workgroup present
  const long long kvbase = (long long)bh * p.Scap, sbase = (long long)bh * p.Scap_s;
  const int n = p.row_bytes / 64;   // 16-byte pieces per thread: 2, 4 or 8
  uint4 a[8], c[8];
  long long dst[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ok[i] = false;
    dst[i] = 0;
    if (i < n) {
      const int o = 16 * (tid + 256 * i);            // byte in the 64-row run
      const int row = o / p.row_bytes, inrow = o % p.row_bytes;
      long long src_tok, dst_tok;
      if (uni) {
        const int slot = 8 * j + row / 8;
        ok[i] = row / 8 < nslot;
        src_tok = ok[i] ? (long long)p.ulist[(long long)bh * p.sg + slot] * 8 + row % 8 : 0;
        dst_tok = (long long)slot * 8 + row % 8;
      } else {
        const int t = (j - p.sg / 8) * kChunk + row;
        ok[i] = true;
        src_tok = (long long)p.q0 + t;
        dst_tok = (long long)p.sg * 8 + t;
      }
      const long long src = (kvbase + src_tok) * p.row_bytes + inrow;
      dst[i] = (sbase + dst_tok) * p.row_bytes + inrow;
      if (ok[i]) {
        a[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.K) + src);
        c[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.V) + src);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < n && ok[i]) {
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.Ks) + dst[i]) = a[i];
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.Vs) + dst[i]) = c[i];
    }
}

}  // namespace

hipError_t launch_stage(const Dims& d, const int32_t* gidx, const void* K, const void* V,
                        int sg, int scap_s, void* Ks, void* Vs, int32_t* gidx_out,
                        int32_t* ulist, int32_t* ucount, hipStream_t s) {
  StageP p;
  p.gidx = gidx; p.gidx_out = gidx_out; p.ulist = ulist; p.ucount = ucount;
  p.K = K; p.V = V; p.Ks = Ks; p.Vs = Vs;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.nblk = d.nblk; p.top_g = d.top_g; p.q0 = d.q0;
  p.Sq = d.Sq; p.Scap = d.Scap; p.Scap_s = scap_s; p.sg = sg;
  p.row_bytes = d.D * (d.bf16 ? 2 : 4);
  stage_union_kernel<<<d.B * d.Hkv, kUnionThreads, 0, s>>>(p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_copy_kernel<<<d.B * d.Hkv * (sg / 8 + d.Sq / kChunk), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hga
