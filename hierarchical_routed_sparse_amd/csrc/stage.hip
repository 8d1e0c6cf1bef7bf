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
//
// Sources of the copies: K / V (typically pinned host memory) by default.
// Given the previous staging of the same history, a union group that it holds
// (in its union, or among its segment's rows) is copied from its staged
// buffers instead, in device memory; given the segment's rows in device
// memory, those are copied from there.  The bytes staged are the same either
// way.
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
  int32_t* usrc;         // [B * Hkv][sg] first row of each union slot in the previous
                         // staging, or -1 (copied from K / V)
  const void* K;         // [B][Hkv][Scap][D]
  const void* V;
  const void* Kseg;      // [B][Hkv][Sq][D] the segment's rows, or null
  const void* Vseg;
  void* Ks;              // [B][Hkv][Scap_s][D]
  void* Vs;
  int B, Hq, Hkv, nblk, top_g, q0, Sq, Scap, Scap_s, sg, row_bytes;
  StagePrevD prev;       // prev.Ks == null: no previous staging
};

// Per (b, kv head): the union of the history groups its rows keep (each row
// read as its ascending prefix of groups before its own chunk, the rule of
// the attention kernels), as a bitmap in LDS, then ranks, the list, and the
// rewritten rows.
__global__ __launch_bounds__(kUnionThreads) void stage_union_kernel(const StageP p) {
  __shared__ uint32_t s_bits[kWords];
  __shared__ int s_base[kWords];
  __shared__ uint32_t s_pbits[kWords];   // the previous staging's union
  __shared__ int s_pbase[kWords];
  __shared__ int s_wsum[kUnionThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NW = kUnionThreads / 64;
  const int bh = blockIdx.x, b = bh / p.Hkv, hkv = bh % p.Hkv;
  const int r = p.Hq / p.Hkv, nrows = r * p.nblk;
  const int hist = 8 * (p.q0 / kChunk);            // history groups (before the segment)
  const int nwords = (hist + 31) / 32;
  const bool has_prev = p.prev.Ks != nullptr;
  for (int i = tid; i < kWords; i += kUnionThreads) s_bits[i] = s_pbits[i] = 0;
  __syncthreads();
  // the previous staging's union, as a bitmap of groups before its segment
  // (its size clamped to its slots, its entries to its history)
  const int phist = has_prev ? p.prev.q0 / 8 : 0;
  if (has_prev) {
    int pn = p.prev.ucount[bh];
    pn = pn < 0 ? 0 : (pn > p.prev.sg ? p.prev.sg : pn);
    const int32_t* pl = p.prev.ulist + (long long)bh * p.prev.sg;
    for (int i = tid; i < pn; i += kUnionThreads) {
      const int v = pl[i];
      if (v >= 0 && v < phist) atomicOr(&s_pbits[v >> 5], 1u << (v & 31));
    }
  }
  // one wavefront per row: the row's prefix length, then mark its history groups
  auto row_ptr = [&](int rr) {
    const int hq = hkv * r + rr / p.nblk, blk = rr % p.nblk;
    return (((long long)b * p.Hq + hq) * p.nblk + blk) * p.top_g;
  };
  // prefix length of a row from entry i0s on (entries before i0s valid)
  auto prefix_from = [&](const int32_t* g, int limit, int i0s) {
    int n = p.top_g;
    for (int i0 = i0s; i0 < p.top_g; i0 += 64) {
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
  // Rows rr0, rr0 + NW, ... (kRowBatch of them, this wavefront's): the first
  // 64 entries of each are loaded together (one load per lane and row, all
  // in flight at once), with each row's prefix length; entries past the 64th
  // are read row by row where a row has them.
  constexpr int kRowBatch = 8;
  auto load_rows = [&](int rr0, int (&v)[kRowBatch], int (&n)[kRowBatch]) {
#pragma unroll
    for (int k = 0; k < kRowBatch; ++k) {
      const int rr = rr0 + NW * k;
      v[k] = rr < nrows && lane < p.top_g ? p.gidx[row_ptr(rr) + lane] : -1;
    }
#pragma unroll
    for (int k = 0; k < kRowBatch; ++k) {
      const int rr = rr0 + NW * k;
      n[k] = 0;
      if (rr < nrows) {
        const int limit = 8 * (p.q0 / kChunk + rr % p.nblk);
        const int up = __shfl_up(v[k], 1);
        const int prev = lane == 0 ? -1 : up;
        const uint64_t bad =
            __ballot(lane < p.top_g && (v[k] < 0 || v[k] >= limit || v[k] <= prev));
        n[k] = bad ? (int)__builtin_ctzll(bad)
                   : prefix_from(p.gidx + row_ptr(rr), limit, 64);
      }
    }
  };
  for (int rr0 = wv; rr0 < nrows; rr0 += NW * kRowBatch) {
    int v[kRowBatch], n[kRowBatch];
    load_rows(rr0, v, n);
#pragma unroll
    for (int k = 0; k < kRowBatch; ++k) {
      if (lane < n[k] && v[k] < hist) atomicOr(&s_bits[v[k] >> 5], 1u << (v[k] & 31));
      if (n[k] > 64) {
        const int32_t* g = p.gidx + row_ptr(rr0 + NW * k);
        for (int i = 64 + lane; i < n[k]; i += 64) {
          const int x = g[i];
          if (x < hist) atomicOr(&s_bits[x >> 5], 1u << (x & 31));
        }
      }
    }
  }
  __syncthreads();
  // exclusive prefix of the words' popcounts (kWords = 512 words over the
  // first 8 wavefronts)
  auto scan = [&](const uint32_t* bits, int nw, int* out) {
    const int cnt = tid < kWords && tid < nw ? __popc(bits[tid]) : 0;
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
    if (tid < kWords) out[tid] = base + incl - cnt;
    int total = 0;
    for (int k = 0; k < NW; ++k) total += s_wsum[k];
    __syncthreads();
    return total;
  };
  const int total = scan(s_bits, nwords, s_base);
  if (has_prev) scan(s_pbits, (phist + 31) / 32, s_pbase);
  // the union, ascending, and where each slot's rows are copied from: the
  // previous staging's segment rows or union slot, else K / V
  int32_t* list = p.ulist + (long long)bh * p.sg;
  int32_t* src = p.usrc + (long long)bh * p.sg;
  const int pseg0 = has_prev ? p.prev.q0 / 8 : 0, pseg1 = has_prev ? (p.prev.q0 + p.prev.Sq) / 8 : 0;
  if (tid < nwords) {
    uint32_t m = s_bits[tid];
    int k = s_base[tid];
    while (m) {
      const int bit = __builtin_ctz(m);
      const int g = 32 * tid + bit;
      int from = -1;
      if (has_prev) {
        if (g >= pseg0 && g < pseg1) {
          from = 8 * p.prev.sg + 8 * (g - pseg0);
        } else if (g < phist && ((s_pbits[g >> 5] >> (g & 31)) & 1u)) {
          const int rank = s_pbase[g >> 5] + __popc(s_pbits[g >> 5] & ((1u << (g & 31)) - 1u));
          from = 8 * rank;   // < 8 * prev.sg: at most prev.sg bits are set
        }
      }
      list[k] = g;
      src[k] = from;
      ++k;
      m &= m - 1;
    }
  }
  if (tid == 0) p.ucount[bh] = total;
  // every row rewritten against the staged layout
  const int seg0 = hist;   // first group of the segment
  auto staged = [&](int x) -> int {
    if (x < seg0) {
      const uint32_t w = s_bits[x >> 5];
      return s_base[x >> 5] + (int)__popc(w & ((1u << (x & 31)) - 1u));
    }
    return x - seg0 + p.sg;
  };
  for (int rr0 = wv; rr0 < nrows; rr0 += NW * kRowBatch) {
    int v[kRowBatch], n[kRowBatch];
    load_rows(rr0, v, n);
#pragma unroll
    for (int k = 0; k < kRowBatch; ++k) {
      const int rr = rr0 + NW * k;
      if (rr >= nrows) continue;
      const long long o = row_ptr(rr);
      if (lane < p.top_g) p.gidx_out[o + lane] = lane < n[k] ? staged(v[k]) : -1;
      for (int i = 64 + lane; i < p.top_g; i += 64)
        p.gidx_out[o + i] = i < n[k] ? staged(p.gidx[o + i]) : -1;
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
  const long long pbase = (long long)bh * p.prev.Scap;
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
      const char* ks;
      const char* vs;
      long long dst_tok;
      if (uni) {
        const int slot = 8 * j + row / 8;
        ok[i] = row / 8 < nslot;
        const long long si = (long long)bh * p.sg + (ok[i] ? slot : 0);
        const int from = ok[i] ? p.usrc[si] : -1;
        if (from >= 0) {   // from the previous staging, in device memory
          const long long off = (pbase + from + row % 8) * p.row_bytes + inrow;
          ks = reinterpret_cast<const char*>(p.prev.Ks) + off;
          vs = reinterpret_cast<const char*>(p.prev.Vs) + off;
        } else {
          const long long src_tok = ok[i] ? (long long)p.ulist[si] * 8 + row % 8 : 0;
          const long long off = (kvbase + src_tok) * p.row_bytes + inrow;
          ks = reinterpret_cast<const char*>(p.K) + off;
          vs = reinterpret_cast<const char*>(p.V) + off;
        }
        dst_tok = (long long)slot * 8 + row % 8;
      } else {
        const int t = (j - p.sg / 8) * kChunk + row;
        ok[i] = true;
        if (p.Kseg) {      // the segment's rows, in device memory
          const long long off = ((long long)bh * p.Sq + t) * p.row_bytes + inrow;
          ks = reinterpret_cast<const char*>(p.Kseg) + off;
          vs = reinterpret_cast<const char*>(p.Vseg) + off;
        } else {
          const long long off = (kvbase + p.q0 + t) * p.row_bytes + inrow;
          ks = reinterpret_cast<const char*>(p.K) + off;
          vs = reinterpret_cast<const char*>(p.V) + off;
        }
        dst_tok = (long long)p.sg * 8 + t;
      }
      dst[i] = (sbase + dst_tok) * p.row_bytes + inrow;
      if (ok[i]) {
        a[i] = *reinterpret_cast<const uint4*>(ks);
        c[i] = *reinterpret_cast<const uint4*>(vs);
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
                        const void* Kseg, const void* Vseg, const StagePrevD* prev, int sg,
                        int scap_s, void* Ks, void* Vs, int32_t* gidx_out, int32_t* ulist,
                        int32_t* ucount, int32_t* usrc, hipStream_t s) {
  StageP p;
  p.gidx = gidx; p.gidx_out = gidx_out; p.ulist = ulist; p.ucount = ucount; p.usrc = usrc;
  p.K = K; p.V = V; p.Kseg = Kseg; p.Vseg = Vseg; p.Ks = Ks; p.Vs = Vs;
  p.B = d.B; p.Hq = d.Hq; p.Hkv = d.Hkv; p.nblk = d.nblk; p.top_g = d.top_g; p.q0 = d.q0;
  p.Sq = d.Sq; p.Scap = d.Scap; p.Scap_s = scap_s; p.sg = sg;
  p.row_bytes = d.D * (d.bf16 ? 2 : 4);
  p.prev = prev ? *prev : StagePrevD{};
  stage_union_kernel<<<d.B * d.Hkv, kUnionThreads, 0, s>>>(p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_copy_kernel<<<d.B * d.Hkv * (sg / 8 + d.Sq / kChunk), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace hga
