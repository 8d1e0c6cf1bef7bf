// Chunk and group summaries of the keys.
//
// Page "BMW's 16 GB GPU just did what needs an A100", section "What HGA does
// differently": each 64-token chunk keeps a compact summary vector in GPU
// memory, and kept chunks are opened at the level of 8-token groups.  The
// page gives no formula; the summary is the mean of the keys (of the chunk,
// or of the group), accumulated in fp32.
//
// One pass over K: each thread sums a 4-row x 8-element block with 16-byte
// loads, a lane exchange completes the 8-row group sums, and the eight group
// sums of a chunk are added in LDS.  Pure HBM streaming: K is read once and
// the summaries (1/8 + 1/64 of K's rows, fp32) are written once.
#include "hga_device.h"
#include "hga_kernels.h"

namespace hga {
namespace {

struct SumP {
  const void* K;       // [B][Hkv][Kcap][D]: positions row0 .. row0 + Kcap - 1
  float* cm;
  float* gm;
  int Scap, Kcap, row0, chunk_begin, chunk_end, nslots, nwork;   // Scap: summary capacity
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void summaries_kernel(const SumP p) {
  constexpr int kOct = D / 8;            // 8-element columns per row
  constexpr int kPpc = 16 * kOct;        // pairs per chunk
  constexpr int kCpw = kThreads / kPpc;  // chunks per workgroup
  __shared__ float s_gsum[kCpw][8][D];

  const int tid = threadIdx.x;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / p.nslots;
  const int lc = tid / kPpc;
  const int chunk = p.chunk_begin + (w % p.nslots) * kCpw + lc;
  const int pr = tid % kPpc, q = pr / kOct, o = pr % kOct;
  const bool live = chunk < p.chunk_end;
  const long long nch = p.Scap / kChunk;   // chunk rows per (b, kv head) in the summaries

  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
  if (live) {
    Pair<T> x;
    load_pair(x, reinterpret_cast<const T*>(p.K) +
                     ((long long)bh * p.Kcap + chunk * kChunk - p.row0 + 4 * q) * D + 8 * o, D);
    const T* r = reinterpret_cast<const T*>(&x);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += to_f32(r[i * 8 + e]);
  }
  // rows 4q..4q+3 plus the partner quad q^1 (lane tid ^ kOct) give one 8-row group
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] += __shfl_xor(s[e], kOct);
  if (live && (q & 1) == 0) {
    const int grp = q >> 1;
    float* g = p.gm + ((long long)bh * (nch * 8) + chunk * 8 + grp) * D + 8 * o;
    reinterpret_cast<float4*>(g)[0] = make_float4(s[0] * 0.125f, s[1] * 0.125f, s[2] * 0.125f, s[3] * 0.125f);
    reinterpret_cast<float4*>(g)[1] = make_float4(s[4] * 0.125f, s[5] * 0.125f, s[6] * 0.125f, s[7] * 0.125f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s_gsum[lc][grp][8 * o + e] = s[e];
  }
  __syncthreads();
  for (int i = tid; i < kCpw * D; i += kThreads) {
    const int c2 = i / D, d = i % D;
    const int ch = p.chunk_begin + (w % p.nslots) * kCpw + c2;
    if (ch < p.chunk_end) {
      float a = 0.f;
#pragma unroll
      for (int grp = 0; grp < 8; ++grp) a += s_gsum[c2][grp][d];
      p.cm[((long long)bh * nch + ch) * D + d] = a * (1.0f / 64.0f);
    }
  }
}

template <typename T, int D>
hipError_t run(const Dims& d, const void* K, int kcap, int row0, float* cm, float* gm, int cb,
               int ce, hipStream_t s) {
  constexpr int kCpw = kThreads / (16 * (D / 8));
  SumP p;
  p.K = K; p.cm = cm; p.gm = gm; p.Scap = d.Scap; p.Kcap = kcap; p.row0 = row0;
  p.chunk_begin = cb; p.chunk_end = ce;
  p.nslots = (ce - cb + kCpw - 1) / kCpw;
  p.nwork = d.B * d.Hkv * p.nslots;
  if (p.nwork == 0) return hipSuccess;
  summaries_kernel<T, D><<<p.nwork, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summaries(const Dims& d, const void* K, int kcap, int row0, float* chunk_mean,
                            float* group_mean, int chunk_begin, int chunk_end, hipStream_t s) {
  if (d.bf16)
    return d.D == 128 ? run<uint16_t, 128>(d, K, kcap, row0, chunk_mean, group_mean, chunk_begin, chunk_end, s)
                      : run<uint16_t, 64>(d, K, kcap, row0, chunk_mean, group_mean, chunk_begin, chunk_end, s);
  return d.D == 128 ? run<float, 128>(d, K, kcap, row0, chunk_mean, group_mean, chunk_begin, chunk_end, s)
                    : run<float, 64>(d, K, kcap, row0, chunk_mean, group_mean, chunk_begin, chunk_end, s);
}

}  // namespace hga
