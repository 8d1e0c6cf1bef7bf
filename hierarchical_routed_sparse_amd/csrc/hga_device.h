// Device-side building blocks shared by the HGA kernels (gfx950 / CDNA4).
//
// Matrix products use the 16x16 MFMA shapes:
//   bf16 : v_mfma_f32_16x16x32_bf16  (one instruction per 32-deep slice)
//   fp32 : v_mfma_f32_16x16x4_f32    (eight instructions per 32-deep slice)
// A 32-deep slice of an operand is held as a Frag: 8 elements per lane.  Lane l
// supplies row (or column) l % 16 of its 16-wide operand and "k-group"
// g = l / 16; item t of the lane stands for contraction index pi(g, t).  The
// contraction is a sum over k, so any bijection pi works as long as both
// operands of one product use the same one.  Accumulators use the fixed
// 16x16 output layout: lane l holds column l % 16, rows 4 * (l / 16) + i,
// i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hga {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;
constexpr int kGroup = 8;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------- scalars

__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kBytes = 2; };
template <> struct Elem<float> { static constexpr int kBytes = 4; };

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// ----------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// number of set bits of m below this lane
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the same column of a
// 16x16 MFMA accumulator).  v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; with both operands equal to
// v, the two results hold v and its lane-xor-32 partner in some order, so
// their max (sum) is the pairwise max (sum).  v_permlane16_swap does the same
// for lane-xor-16 partners.
__device__ __forceinline__ float xor_max16_32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xor_sum16_32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Work index for block `bid` such that consecutive work indices land on the
// same XCD.  Workgroups are dispatched round-robin over the 8 XCDs, so XCD x
// runs bids x, x+8, ...; it receives the contiguous work range
// [x*per + min(x, rem), ...) of length per + (x < rem).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// ----------------------------------------------------------------- routing rows
//
// The kept groups of a routing row, as the attention kernels read them: the
// longest prefix of the row whose entries lie in [0, limit) and each exceed
// the entry before them.  A row written by the routing (ascending, -1
// padded, every group before the own chunk) is its valid entries exactly; any
// other row is cut at its first entry that breaks the rule, so a kept group
// is never out of range and never counted twice.  The row is copied to
// s_glist (entries past the prefix are never read) and the prefix length is
// returned.  Every thread of the NT-thread workgroup must call it; s_wsum
// holds NT / 64 ints.
template <int NT>
__device__ __forceinline__ int load_routing_prefix(const int32_t* grow, int top_g, int limit,
                                                   int* s_glist, int* s_wsum) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int n = top_g;
  for (int i0 = 0; i0 < top_g; i0 += NT) {
    const int i = i0 + tid;
    const int gm = i < top_g ? grow[i] : -1;
    const int prev = i > 0 && i < top_g ? grow[i - 1] : -1;
    if (i < top_g) s_glist[i] = gm;
    const bool bad = i < top_g && (gm < 0 || gm >= limit || gm <= prev);
    const uint64_t bal = __ballot(bad);
    if (lane == 0) s_wsum[wv] = bal ? i0 + 64 * wv + (int)__builtin_ctzll(bal) : top_g;
    __syncthreads();
    int first = top_g;
#pragma unroll
    for (int k = 0; k < NW; ++k) first = min(first, s_wsum[k]);
    __syncthreads();
    if (first < top_g) {
      n = first;
      break;
    }
  }
  return n;
}

// ----------------------------------------------------------------- fragments

template <typename T> struct Frag;
template <> struct Frag<uint16_t> { uint32_t w[4]; };  // 8 bf16, item t in half t&1 of w[t>>1]
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[t], b.v[t], acc, 0, 0, 0);
}

// 8 consecutive elements (items 0..7) from global or LDS memory.
__device__ __forceinline__ void load_frag(Frag<uint16_t>& f, const uint16_t* p) {
  const uint4 x = *reinterpret_cast<const uint4*>(p);
  f.w[0] = x.x; f.w[1] = x.y; f.w[2] = x.z; f.w[3] = x.w;
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  const float4 x = reinterpret_cast<const float4*>(p)[0];
  const float4 y = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
  f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
}
// items 0..3 from p0 and items 4..7 from p1 (each 4 consecutive elements).
__device__ __forceinline__ void load_frag_split(Frag<uint16_t>& f, const uint16_t* p0, const uint16_t* p1) {
  const uint2 x = *reinterpret_cast<const uint2*>(p0);
  const uint2 y = *reinterpret_cast<const uint2*>(p1);
  f.w[0] = x.x; f.w[1] = x.y; f.w[2] = y.x; f.w[3] = y.y;
}
__device__ __forceinline__ void load_frag_split(Frag<float>& f, const float* p0, const float* p1) {
  const float4 x = *reinterpret_cast<const float4*>(p0);
  const float4 y = *reinterpret_cast<const float4*>(p1);
  f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
  f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
}
// Fragment from two accumulators: items 0..3 = a[0..3], items 4..7 = b[0..3].
__device__ __forceinline__ void frag_from_acc(Frag<uint16_t>& f, const f32x4& a, const f32x4& b) {
  f.w[0] = pack_bf16(a[0], a[1]); f.w[1] = pack_bf16(a[2], a[3]);
  f.w[2] = pack_bf16(b[0], b[1]); f.w[3] = pack_bf16(b[2], b[3]);
}
__device__ __forceinline__ void frag_from_acc(Frag<float>& f, const f32x4& a, const f32x4& b) {
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
// Partial dot product of two fragments (fp32).
__device__ __forceinline__ float frag_dot(const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(__uint_as_float(a.w[i] << 16), __uint_as_float(b.w[i] << 16), s);
    s = fmaf(__uint_as_float(a.w[i] & 0xFFFF0000u), __uint_as_float(b.w[i] & 0xFFFF0000u), s);
  }
  return s;
}
__device__ __forceinline__ float frag_dot(const Frag<float>& a, const Frag<float>& b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(a.v[i], b.v[i], s);
  return s;
}

// Stores 4 consecutive output elements (fp32 values) to memory of type T.
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  uint2 x;
  x.x = pack_bf16(a, b);
  x.y = pack_bf16(c, d);
  *reinterpret_cast<uint2*>(p) = x;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// ----------------------------------------------------------------- output rows through LDS
//
// The attention kernels end with a 64-row bf16 output block (O, dQ, dK, dV)
// that is one contiguous run in memory, held as MFMA results: lane (l16, g)
// of the wave owning rows 16w..16w+15 holds elements 16dd + 4g .. + 3 of row
// 16w + l16.  Stored directly, every instruction writes 32-byte pieces of 16
// rows.  out_rows_put packs them (bf16, nearest even, as store4 does) into an
// idle LDS area; after a barrier out_rows_flush writes the block as whole
// rows, 16 bytes per lane.  Same values as the direct stores.
//
// XOR swizzle in 16-byte units: a half-wave writes 8 bytes per lane to units
// 2dd + g/2 of 16 consecutive rows, and 16 lanes read the units of one row
// (D = 128: 256-byte rows; D = 64: two 128-byte rows per 16 lanes).  Rows 2m
// and 2m + 1 agree in the swizzle's bits 2-3 at D = 128, so the 16-lane passes
// of a ds_read_b128, which mix the units of neighbouring lane groups, stay
// conflict-free too.
template <int D>
__device__ __forceinline__ int out_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ void out_rows_put(char* lds, const f32x4 (&acc)[D / 16], float sc,
                                             int row, int g4) {
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) {
    const uint32_t off = (uint32_t)(row * 2 * D) +
                         ((uint32_t)((2 * dd + (g4 >> 1)) ^ out_swz<D>(row)) << 4) +
                         ((uint32_t)(g4 & 1) << 3);
    uint2 x;
    x.x = pack_bf16(acc[dd][0] * sc, acc[dd][1] * sc);
    x.y = pack_bf16(acc[dd][2] * sc, acc[dd][3] * sc);
    *reinterpret_cast<uint2*>(lds + off) = x;
  }
}
// NT: non-temporal stores, for outputs no later kernel of the step reads, so
// that they do not displace rows the running kernel still gathers from L2.
template <int D, bool NT = false>
__device__ __forceinline__ void out_rows_flush(const char* lds, char* out, int tid) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int OB = 2 * D;
#pragma unroll
  for (int j = 0; j < 64 * OB / (16 * kThreads); ++j) {
    const int o = 16 * (tid + kThreads * j);
    const int row = o / OB, u = (o % OB) >> 4;
    const uint32_t loff = (uint32_t)(row * OB) + ((uint32_t)(u ^ out_swz<D>(row)) << 4);
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(lds + loff);
    if constexpr (NT)
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(out + o));
    else
      *reinterpret_cast<u32x4_t*>(out + o) = x;
  }
}

// ----------------------------------------------------------------- tile staging
//
// A "pair" is a 4-row x 8-element block: rows 4q..4q+3 of a 64-row tile,
// elements 8o..8o+7.  One thread moves one pair from global memory into LDS,
// either row-major (swizzled 16-byte units) or transposed (element-major, rows
// of the tile contiguous).  Each 8-token group is 8 consecutive rows, so a
// pair never straddles two gathered groups.

template <typename T> struct Pair;
template <> struct Pair<uint16_t> { uint4 r[4]; };
template <> struct Pair<float> { float4 r[4][2]; };

__device__ __forceinline__ void zero_pair(Pair<uint16_t>& p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) p.r[i] = make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void zero_pair(Pair<float>& p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) p.r[i][0] = p.r[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
}
// row0: pointer to element 8o of the first of 4 consecutive rows, row stride ld.
__device__ __forceinline__ void load_pair(Pair<uint16_t>& p, const uint16_t* row0, long long ld) {
#pragma unroll
  for (int i = 0; i < 4; ++i) p.r[i] = *reinterpret_cast<const uint4*>(row0 + i * ld);
}
__device__ __forceinline__ void load_pair(Pair<float>& p, const float* row0, long long ld) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p.r[i][0] = reinterpret_cast<const float4*>(row0 + i * ld)[0];
    p.r[i][1] = reinterpret_cast<const float4*>(row0 + i * ld)[1];
  }
}

// Row-major tile of 64 rows x D elements in LDS, stored in 16-byte units with
// the unit index XOR-swizzled by the row.
//
// Bank rules measured on gfx950 (LDS bank-conflict counter, one probe
// dispatch per lane->address pattern): the LDS has 64 four-byte banks.  A
// ds_read_b128 is served in four passes of 16 lanes, {0-3, 12-15, 20-27} and
// {4-11, 16-19, 28-31} (and the same + 32); a pass is conflict-free when its
// 16 lanes read 16 different 16-byte units of the 256-byte bank row.  A
// ds_read_b64_tr_b16 is served per half-wave (32 lanes x 8 bytes).  The
// swizzle row ^ (row odd ? 14 : 0) (row mod 16) makes the read patterns of
// the attention kernels conflict-free under these rules: row operands (lane
// n of a 16-lane group: row n) and transposing reads of 8 consecutive rows.
// (The plain swizzle, unit ^ row, leaves the transposing reads two-way
// conflicted.)
template <typename T, int D> struct RowTile {
  static constexpr int kUnits = D * Elem<T>::kBytes / 16;   // units per row
  static constexpr int kBytes = 64 * D * Elem<T>::kBytes;
  __device__ static __forceinline__ int swz(int row) {
    static_assert(kUnits == 8 || kUnits >= 16, "tile rows of 8 or at least 16 units");
    // (8-unit rows, two per bank row: row & 6 is conflict-free for the same
    // read patterns under the same rules)
    return kUnits >= 16 ? ((row & 15) ^ ((row & 1) ? 14 : 0)) : (row & 6);
  }
  // byte offset of logical unit u of row `row`
  __device__ static __forceinline__ int off(int row, int u) {
    return row * kUnits * 16 + ((u ^ swz(row)) << 4);
  }
};

// Transposed tile: D rows (elements) x 64 columns (tile rows) + padding.
template <typename T, int D> struct ColTile {
  static constexpr int kStride = Elem<T>::kBytes == 2 ? 72 : 68;   // elements per row
  static constexpr int kBytes = D * kStride * Elem<T>::kBytes;
};

template <int D>
__device__ __forceinline__ void store_pair_rows(char* tile, const Pair<uint16_t>& p, int q, int o) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(tile + RowTile<uint16_t, D>::off(4 * q + i, o)) = p.r[i];
}
template <int D>
__device__ __forceinline__ void store_pair_rows(char* tile, const Pair<float>& p, int q, int o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<float4*>(tile + RowTile<float, D>::off(4 * q + i, 2 * o)) = p.r[i][0];
    *reinterpret_cast<float4*>(tile + RowTile<float, D>::off(4 * q + i, 2 * o + 1)) = p.r[i][1];
  }
}

template <int D>
__device__ __forceinline__ void store_pair_cols(char* tile, const Pair<uint16_t>& p, int q, int o) {
  constexpr int S = ColTile<uint16_t, D>::kStride;
  uint16_t* t = reinterpret_cast<uint16_t*>(tile);
  const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&p.r[0]);
  const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&p.r[1]);
  const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&p.r[2]);
  const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&p.r[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint2 lo, hi;   // element 2w and 2w+1, four tile rows each
    lo.x = (r0[w] & 0xFFFFu) | (r1[w] << 16);
    lo.y = (r2[w] & 0xFFFFu) | (r3[w] << 16);
    hi.x = (r0[w] >> 16) | (r1[w] & 0xFFFF0000u);
    hi.y = (r2[w] >> 16) | (r3[w] & 0xFFFF0000u);
    *reinterpret_cast<uint2*>(t + (8 * o + 2 * w) * S + 4 * q) = lo;
    *reinterpret_cast<uint2*>(t + (8 * o + 2 * w + 1) * S + 4 * q) = hi;
  }
}
template <int D>
__device__ __forceinline__ void store_pair_cols(char* tile, const Pair<float>& p, int q, int o) {
  constexpr int S = ColTile<float, D>::kStride;
  float* t = reinterpret_cast<float*>(tile);
  const float* r0 = reinterpret_cast<const float*>(&p.r[0][0]);
  const float* r1 = reinterpret_cast<const float*>(&p.r[1][0]);
  const float* r2 = reinterpret_cast<const float*>(&p.r[2][0]);
  const float* r3 = reinterpret_cast<const float*>(&p.r[3][0]);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<float4*>(t + (8 * o + e) * S + 4 * q) = make_float4(r0[e], r1[e], r2[e], r3[e]);
}

// A-or-B fragment of a row-major tile: row `row`, elements 32s + 8g .. +8.
template <typename T, int D>
__device__ __forceinline__ void frag_rows(Frag<T>& f, const char* tile, int row, int s, int g) {
  if constexpr (Elem<T>::kBytes == 2) {
    const uint4 x = *reinterpret_cast<const uint4*>(tile + RowTile<T, D>::off(row, 4 * s + g));
    f.w[0] = x.x; f.w[1] = x.y; f.w[2] = x.z; f.w[3] = x.w;
  } else {
    const float4 x = *reinterpret_cast<const float4*>(tile + RowTile<T, D>::off(row, 8 * s + 2 * g));
    const float4 y = *reinterpret_cast<const float4*>(tile + RowTile<T, D>::off(row, 8 * s + 2 * g + 1));
    f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
    f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
  }
}
// A-or-B fragment of a transposed tile: element row `e`, tile rows
// 32m + 4g + (0..3) as items 0..3 and 32m + 16 + 4g + (0..3) as items 4..7.
// This is the item order produced by frag_from_acc on the accumulators of tile
// rows 32m..32m+15 and 32m+16..32m+31.
template <typename T, int D>
__device__ __forceinline__ void frag_cols(Frag<T>& f, const char* tile, int e, int m, int g) {
  constexpr int S = ColTile<T, D>::kStride;
  const T* t = reinterpret_cast<const T*>(tile) + e * S + 32 * m + 4 * g;
  load_frag_split(f, t, t + 16);
}


// ----------------------------------------------------------------- async tile fill
//
// global_load_lds_dwordx4 (gfx950): every lane of a wavefront moves 16 bytes
// from its own global address into LDS at M0 + 16 * lane, so one instruction
// fills 1 KB of LDS.  A row-major swizzled tile is filled by choosing, for LDS
// unit (row, physical unit p), the global source (row, logical unit
// p ^ swz(row)).  Completion is tracked by vmcnt.
//
// The load is issued from inline asm: the compiler then never treats it as a
// pending LDS write, so it does not put a full vmcnt wait in front of every
// LDS read (which would serialise the tile pipeline).  The instruction has no
// register result; the kernels wait with wait_vmcnt<N>() plus a barrier
// before reading a tile.  M0 is saved and restored inside the block.

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] + vmcnt[5:4] at bits 15:14, expcnt 6:4, lgkmcnt 11:8
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Same load with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (no 64-bit address arithmetic per lane).
__device__ __forceinline__ void dma16_off(uint32_t voff, const void* sbase, uint32_t lds_base) {
  // force the base into SGPRs (it is wave-uniform by construction)
  // (readfirstlane returns int: widen through uint32_t so that the low half is
  // zero-extended, never sign-extended)
  const uint64_t b64 = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b64 >> 32));
  sbase = (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

template <typename T, int D>
__device__ constexpr int rows_per_issue() { return 64 / RowTile<T, D>::kUnits; }

// Byte offset, relative to element 0 of token 0, of the 16-byte unit this
// lane moves for tile row `row` when the row holds token `tok`.
template <typename T, int D>
__device__ __forceinline__ uint32_t dma_offset(int row, uint32_t tok) {
  constexpr int U = RowTile<T, D>::kUnits;
  const int phys = lane_id() % U;
  return tok * (uint32_t)(D * Elem<T>::kBytes) + (uint32_t)((phys ^ RowTile<T, D>::swz(row)) << 4);
}

// Issues the loads of `nrows` rows starting at row r0 (nrows a multiple of
// rows_per_issue()) of a row-major swizzled tile at LDS byte address `tile`;
// rowptr(row) returns the global address of element 0 of that row.  Every
// wavefront that calls this issues nrows / rows_per_issue() loads.
template <typename T, int D, typename RowPtr>
__device__ __forceinline__ void fill_rows_async(uint32_t tile, int r0, int nrows, RowPtr rowptr) {
  constexpr int U = RowTile<T, D>::kUnits;
  constexpr int RPI = 64 / U;
  constexpr int EPU = 16 / Elem<T>::kBytes;   // elements per 16-byte unit
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < nrows; j += RPI) {
    const int row = r0 + j + lane / U;
    const int phys = lane % U;
    const T* src = rowptr(row) + (phys ^ RowTile<T, D>::swz(row)) * EPU;
    dma16(src, __builtin_amdgcn_readfirstlane(tile + (uint32_t)((r0 + j) * U * 16)));
  }
}

// ----------------------------------------------------------------- transposed operand reads
//
// Operand fragment whose 8 items run down a column of a row-major swizzled
// tile: items 0..3 = tile[ra + t][d0 + l16], items 4..7 = tile[rb + t][d0 + l16]
// (ra, rb may differ per 16-lane group).  bf16 uses ds_read_b64_tr_b16: in a
// 16-lane group, lane j points at the 4 elements tile[r + j/4][d0 + 4(j%4) ..],
// and the hardware hands lane i the column tile[r + 0..3][d0 + i].
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <typename T, int D>
__device__ __forceinline__ void frag_tr(Frag<T>& f, const char* tile, int ra, int rb, int d0) {
  const int l16 = lane_id() & 15;
  if constexpr (Elem<T>::kBytes == 2) {
    const int col = d0 + 4 * (l16 & 3);
    const int unit = col >> 3, half = (col >> 2) & 1;
    const int r1 = ra + (l16 >> 2), r2 = rb + (l16 >> 2);
    const char* a1 = tile + RowTile<T, D>::off(r1, unit) + 8 * half;
    const char* a2 = tile + RowTile<T, D>::off(r2, unit) + 8 * half;
    const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a1);
    const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a2);
    f.w[0] = (uint32_t)(uint16_t)x[0] | ((uint32_t)(uint16_t)x[1] << 16);
    f.w[1] = (uint32_t)(uint16_t)x[2] | ((uint32_t)(uint16_t)x[3] << 16);
    f.w[2] = (uint32_t)(uint16_t)y[0] | ((uint32_t)(uint16_t)y[1] << 16);
    f.w[3] = (uint32_t)(uint16_t)y[2] | ((uint32_t)(uint16_t)y[3] << 16);
  } else {
    const int col = d0 + l16;
    const int unit = col >> 2, sub = col & 3;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f.v[t] = *reinterpret_cast<const float*>(tile + RowTile<T, D>::off(ra + t, unit) + 4 * sub);
      f.v[4 + t] = *reinterpret_cast<const float*>(tile + RowTile<T, D>::off(rb + t, unit) + 4 * sub);
    }
  }
}


// ----------------------------------------------------------------- batched transpose reads
//
// The compiler cannot tell whether an LDS transpose read aliases an LDS
// direct load still in flight and would wait for every outstanding global
// load before the first one, which serialises the tile pipeline.  These
// helpers issue eight ds_read_b64_tr_b16 and wait for them inside the same
// asm block, so no outstanding result ever leaves the block.

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void tr_read8(u32x2 (&o)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// LDS byte address of the transpose-read row pointer for tile row `row`,
// column block 0 (columns 0..15), of a bf16 row-major swizzled tile at `tile`.
// The address for column block cb (columns 16cb..16cb+15) is base ^ (32 * cb):
// lane j of a 16-lane group points at columns 4(j%4)..+3 of its row, i.e. unit
// (j%4)/2, half j%2; with units XOR-swizzled by the row, stepping the column
// block flips bit 5 of the byte offset only.
template <int D>
__device__ __forceinline__ uint32_t tr_base(uint32_t tile, int row) {
  using RT = RowTile<uint16_t, D>;
  const int j = lane_id() & 15;
  const int u0 = (j & 3) >> 1, half = j & 1;
  return tile + (uint32_t)(row * RT::kUnits * 16) + (uint32_t)(((u0 ^ RT::swz(row)) << 4) | (half << 3));
}

// Two operand fragments from 8 transpose reads: f[i] items 0..3 from a[2i],
// items 4..7 from a[2i+1], for i = 0..3.
__device__ __forceinline__ void tr_frags4(Frag<uint16_t> (&f)[4], const uint32_t (&a)[8]) {
  u32x2 o[8];
  tr_read8(o, a);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i].w[0] = o[2 * i][0]; f[i].w[1] = o[2 * i][1];
    f[i].w[2] = o[2 * i + 1][0]; f[i].w[3] = o[2 * i + 1][1];
  }
}


// ----------------------------------------------------------------- loop-invariant LDS offsets
//
// Within a row-major swizzled tile, the swizzle of a row depends on the row
// modulo 16 only, and every 16-row slice a lane reads sits at the same row
// modulo 16.  So the swizzled byte offset of everything a lane reads from a
// tile is a per-lane constant plus a multiple of 16 rows, which becomes an
// instruction immediate.

// Per-lane byte offsets of the transposed (ds_read_b64_tr_b16) reads of a bf16
// tile: o[cb] addresses column block cb (columns 16cb..16cb+15) of rows
// 4g + (l16 >> 2) (+ 16-row multiples added as immediates).
template <int D>
struct TrOffsets {
  uint32_t o[D / 16];
  __device__ __forceinline__ void init() {
    using RT = RowTile<uint16_t, D>;
    const int l = lane_id(), j = l & 15, g = l >> 4;
    const int r = 4 * g + (j >> 2);
    const int u0 = (j & 3) >> 1, half = j & 1;
    const uint32_t low = (uint32_t)(((u0 ^ RT::swz(r)) << 4) | (half << 3));
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb)
      o[cb] = (uint32_t)(r * RT::kUnits * 16) + (low ^ (uint32_t)(32 * cb));
  }
};

// Eight transposed reads at a[i] + I_i, waited for inside the block (see
// tr_read8).  Fragment i takes items 0..3 from read 2i and 4..7 from 2i+1.
template <int I0, int I1, int I2, int I3, int I4, int I5, int I6, int I7>
__device__ __forceinline__ void tr_read8_imm(Frag<uint16_t> (&f)[4], const uint32_t (&a)[8]) {
  u32x2 o[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%17\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%18\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%19\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%20\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%21\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%22\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "n"(I0), "n"(I1), "n"(I2), "n"(I3), "n"(I4), "n"(I5), "n"(I6), "n"(I7)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i].w[0] = o[2 * i][0]; f[i].w[1] = o[2 * i][1];
    f[i].w[2] = o[2 * i + 1][0]; f[i].w[3] = o[2 * i + 1][1];
  }
}


// The same eight reads through the compiler builtin: the compiler schedules
// them and waits only for the results it needs (lgkmcnt), so the reads
// overlap MFMAs.  Valid because the direct LDS loads are issued from inline
// asm that the compiler does not track (it would otherwise guard every LDS
// read with a full vmcnt wait).
template <int I0, int I1, int I2, int I3, int I4, int I5, int I6, int I7>
__device__ __forceinline__ void tr_read8_sched(Frag<uint16_t> (&f)[4], const uint32_t (&a)[8]) {
  constexpr int imm[8] = {I0, I1, I2, I3, I4, I5, I6, I7};
  v4i16 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(a[i] + imm[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4i16 x = o[2 * i], y = o[2 * i + 1];
    f[i].w[0] = (uint32_t)(uint16_t)x[0] | ((uint32_t)(uint16_t)x[1] << 16);
    f[i].w[1] = (uint32_t)(uint16_t)x[2] | ((uint32_t)(uint16_t)x[3] << 16);
    f[i].w[2] = (uint32_t)(uint16_t)y[0] | ((uint32_t)(uint16_t)y[1] << 16);
    f[i].w[3] = (uint32_t)(uint16_t)y[2] | ((uint32_t)(uint16_t)y[3] << 16);
  }
}

// Per-lane byte offsets of the row-operand (ds_read_b128) reads of a tile:
// o[s] addresses row l16 (+ 16-row multiples as immediates), elements
// 32s + 8g .. 32s + 8g + 7 (bf16: one unit; fp32: two units, the second at
// o[s] ^ 16).
template <typename T, int D>
struct RowOffsets {
  uint32_t o[D / 32];
  __device__ __forceinline__ void init() {
    using RT = RowTile<T, D>;
    const int l = lane_id(), j = l & 15, g = l >> 4;
    constexpr int upf = Elem<T>::kBytes / 2;   // units per 8 elements
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      o[s] = (uint32_t)(j * RT::kUnits * 16) + (uint32_t)((((4 * s + g) * upf) ^ RT::swz(j)) << 4);
  }
};

template <typename T, int D>
__device__ __forceinline__ void frag_rows_at(Frag<T>& f, const char* p) {
  if constexpr (Elem<T>::kBytes == 2) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    f.w[0] = x.x; f.w[1] = x.y; f.w[2] = x.z; f.w[3] = x.w;
  } else {
    // the swizzled units of logical units 2u and 2u+1 differ in their lowest bit,
    // i.e. in bit 4 of the (32-byte aligned) LDS byte address
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(reinterpret_cast<uintptr_t>(p) ^ 16u);
    f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
    f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
  }
}

}  // namespace hga
