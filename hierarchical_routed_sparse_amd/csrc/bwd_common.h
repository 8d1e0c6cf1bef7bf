// Shared by the two dK/dV kernels: their parameters and the inverse routing
// map (which routing rows attend a given 64-key chunk, and with which groups).
#pragma once
#include "hga_device.h"

namespace hga {

struct DkvP {
  const void* Q;
  const void* K;
  const void* V;
  const float* lse;
  const void* dO;
  const int32_t* gidx;
  const float* delta;
  const uint8_t* cmask;   // [routing row][chunk] kept-group masks (from the dQ kernel)
  void* dK;
  void* dV;
  int B, Hq, Hkv, Sq, Skv, Scap, q0, nblk, top_g, nchunks, nwork;
  int chunk0, nrange;   // the workgroups cover chunks [chunk0, chunk0 + nrange)
  const int32_t* order; // [B * Hkv][nrange]: chunk of work item i of a (b, kv head)
  float scale;
};

constexpr int kRowsPerPass = 1024;   // routing rows examined per entry-list build

// entry word: (row << 9) | mask, mask bits 0..7 = kept groups, bit 8 = own chunk
constexpr uint32_t kLocalBit = 1u << 8;

// Group-mask words of the routing rows one thread examines for chunk c in the
// pass over rows [r0, r0 + kRowsPerPass): row r0 + k * NT + tid in slot k.  A
// row whose own chunk is c gets kLocalBit | 0xFF, a row of a block that cannot
// see chunk c (or past the last row) gets 0.  Split from the list build so
// that a caller can issue these loads ahead of others and wait on them alone.
template <int NT = kThreads>
struct EntryMasks {
  uint32_t m[kRowsPerPass / NT];
};

template <int NT = kThreads>
__device__ __forceinline__ void load_entry_masks(const DkvP& p, int b, int hkv, int c, int r0,
                                                 EntryMasks<NT>& em) {
  const int tid = threadIdx.x;
  const int r = p.Hq / p.Hkv;
  const int nrows = r * p.nblk;
  const int blk_first = c - p.q0 / kChunk;   // rows with block >= this can touch chunk c
#pragma unroll
  for (int k = 0; k < kRowsPerPass / NT; ++k) {
    em.m[k] = 0;
    if (r0 + k * NT >= nrows) continue;   // uniform: no rows left
    const int rr = r0 + k * NT + tid;
    if (rr < nrows) {
      const int hq = hkv * r + rr / p.nblk, blk = rr % p.nblk;
      if (blk == blk_first) {
        em.m[k] = kLocalBit | 0xFFu;
      } else if (blk > blk_first) {
        em.m[k] = p.cmask[(((long long)b * p.Hq + hq) * p.nblk + blk) * p.nchunks + c];
      }
    }
  }
}

// Entry list of chunk c over routing rows [r0, r0 + kRowsPerPass) from the
// mask words load_entry_masks read: every (query head of kv head hkv, block)
// row that kept a group of chunk c, or whose own chunk is c, in ascending row
// order (head-major); only rows whose mask meets `want` (groups of interest |
// kLocalBit) are listed.  Returns the count.  Every thread of the NT-thread
// workgroup must call it; s_ent is valid for all of them on return (s_wsum
// holds NT / 64 ints).
template <int NT = kThreads>
__device__ __forceinline__ int build_entries(const DkvP& p, int r0, const EntryMasks<NT>& em,
                                             uint32_t* s_ent, int* s_wsum,
                                             uint32_t want = 0x1FFu) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrows = (p.Hq / p.Hkv) * p.nblk;
  int nent = 0;
#pragma unroll
  for (int k = 0; k < kRowsPerPass / NT; ++k) {
    if (r0 + k * NT >= nrows) break;   // uniform
    const int rr = r0 + k * NT + tid;
    const uint32_t mask = em.m[k];
    const bool f = (mask & want) != 0;
    const uint64_t bal = __ballot(f);
    if (lane == 0) s_wsum[wv] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int v = s_wsum[i];
      off += i < wv ? v : 0;
      tot += v;
    }
    if (f) s_ent[nent + off + mbcnt(bal)] = ((uint32_t)rr << 9) | mask;
    nent += tot;
    __syncthreads();
  }
  return nent;
}

}  // namespace hga
