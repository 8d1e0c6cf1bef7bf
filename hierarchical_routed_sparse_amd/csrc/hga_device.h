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

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kBytes = 2; };
template <> struct Elem<float> { static constexpr int kBytes = 4; };

// ----------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// number of set bits of m below this lane
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ float xor_max16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float xor_sum16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
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
// the unit index XOR-swizzled by the row so that 16 lanes reading the same
// logical unit of 16 consecutive rows hit distinct banks.
template <typename T, int D> struct RowTile {
  static constexpr int kUnits = D * Elem<T>::kBytes / 16;   // units per row
  static constexpr int kBytes = 64 * D * Elem<T>::kBytes;
  __device__ static __forceinline__ int swz(int row) {
    return kUnits >= 16 ? (row & 15) : ((row >> 1) & (kUnits - 1));
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

}  // namespace hga
