// Internal launch interface between the C ABI (hga_api.hip) and the kernels.
// Shapes have been validated by the caller; every function only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hga {

struct Dims {
  int B, Hq, Hkv, D, Sq, Skv, top_k, top_g;
  int Scap;    // rows allocated per (b, kv head) in K, V, dK, dV (>= Skv)
  int q0;      // Skv - Sq: absolute position of the first query
  int nblk;    // Sq / 64 (1 for a decode shape, whose one query is a block)
  float scale; // softmax scale
  bool bf16;
};

// K holds kcap rows per (b, kv head), for positions row0 .. row0 + kcap - 1
// (the whole capacity: kcap = d.Scap, row0 = 0).
hipError_t launch_summaries(const Dims& d, const void* K, int kcap, int row0, float* chunk_mean,
                            float* group_mean, int chunk_begin, int chunk_end, hipStream_t s);

// causal: route block j with the mean of the 64 queries before it (Q_prev
// [B][Hq][64][D] = the 64 queries before the segment, for its first block).
hipError_t launch_route(const Dims& d, const void* Q, const void* Q_prev, bool causal,
                        const float* chunk_mean, const float* group_mean, int32_t* chunk_idx,
                        int32_t* group_idx, hipStream_t s);

hipError_t launch_attend_fwd(const Dims& d, const void* Q, const void* K, const void* V,
                             const int32_t* group_idx, void* O, float* lse, hipStream_t s);

hipError_t launch_attend_bwd_dq(const Dims& d, const void* Q, const void* K, const void* V,
                                const void* O, const float* lse, const void* dO,
                                const int32_t* group_idx, void* dQ, float* delta,
                                uint8_t* cmask, int32_t* order, hipStream_t s);

// delta, the group-mask map and the dK/dV work order (what the dQ kernel
// writes into the workspace when given one), without dQ.
hipError_t launch_attend_bwd_prep(const Dims& d, const void* O, const void* dO,
                                  const int32_t* group_idx, float* delta, uint8_t* cmask,
                                  int32_t* order, hipStream_t s);

hipError_t launch_attend_bwd_dkdv(const Dims& d, const void* Q, const void* K, const void* V,
                                  const float* lse, const void* dO, const int32_t* group_idx,
                                  const float* delta, const uint8_t* cmask, int32_t* order,
                                  bool order_ready, void* dK, void* dV, int chunk_begin,
                                  int chunk_end, hipStream_t s);

// The routed working set of a segment staged into a compact buffer (stage.hip).
// The previous staging of the same history, as the staging kernels read it.
struct StagePrevD {
  const void* Ks;          // its staged K, V [B][Hkv][Scap][D]; null: none
  const void* Vs;
  const int32_t* ulist;    // its unions [B * Hkv][sg]
  const int32_t* ucount;   // their sizes [B * Hkv]
  int sg, Scap, q0, Sq;    // its group slots, rows per (b, kv head), segment start and length
};

hipError_t launch_stage(const Dims& d, const int32_t* gidx, const void* K, const void* V,
                        const void* Kseg, const void* Vseg, const StagePrevD* prev, int sg,
                        int scap_s, void* Ks, void* Vs, int32_t* gidx_out, int32_t* ulist,
                        int32_t* ucount, int32_t* usrc, hipStream_t s);

// Decode attention (one query per (b, hq) at position Skv - 1; d.Sq == 1).
hipError_t launch_decode_attend(const Dims& d, const void* Q, const void* K, const void* V,
                                const int32_t* group_idx, void* O, float* lse, hipStream_t s);

}  // namespace hga
