// topk_select.h -- the wave-level top-k selection and softmax shared by the
// canonical top-k kernel and the MFMA router's candidate selection.
//
// "Every Expert Counts: ExactMoE ..." §3.1: S = TopK(z, k) and the softmax
// weights over the selected logits.  Ties go to the lower expert id.
#pragma once

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

extern "C" __device__ float __ockl_wfred_max_f32(float);
extern "C" __device__ int __ockl_wfred_min_i32(int);

// better(a, b): larger logit, or equal logit and lower expert id.  Written
// with bitwise operators so that the lane-local scans stay branch-free.
__device__ __forceinline__ bool topk_better(float va, int ea, float vb, int eb) {
  return (va > vb) | ((va == vb) & (ea < eb));
}

constexpr int kNoExpert = 0x7fffffff;

// One wave selects the k best entries (logit descending, id ascending) of the
// lane-distributed list (z[m], id[m]); unused entries carry id kNoExpert.
// Each round takes the lane-local best untaken entry, a wave max of the logit
// (DPP reduction) and, only if several lanes hold that maximum, a wave min of
// their ids.  Lane j keeps the j-th selected entry, so nothing is indexed by
// the round number.  The weights are the softmax over the selected logits
// with the first (largest) one as the max and the denominator summed in
// selection order.  Lanes < k store id and weight of the entry of rank
// `lane` in increasing id order to ids_row / w_row.
template <int PER>
__device__ __forceinline__ void topk_select_softmax(const float (&z)[PER], const int (&id)[PER],
                                                    int k, int32_t* __restrict__ ids_row,
                                                    float* __restrict__ w_row) {
  const int lane = threadIdx.x & 63;
  uint32_t taken = 0;
  int my_e = 0;            // lane j < k: id and logit of the j-th selection
  float my_z = 0.0f;
  float zmax = 0.0f;       // the first selection's logit
#pragma unroll 1
  for (int jj = 0; jj < k; ++jj) {
    float bv = -INFINITY;
    int be = kNoExpert;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const bool ok = (id[m] != kNoExpert) & (((taken >> m) & 1u) == 0u) & topk_better(z[m], id[m], bv, be);
      bv = ok ? z[m] : bv;
      be = ok ? id[m] : be;
    }
    const float wmax = __ockl_wfred_max_f32(bv);
    const bool cand = (bv == wmax) & (be != kNoExpert);
    const uint64_t mask = __ballot(cand);
    int we;
    if (__popcll(mask) == 1)
      we = __builtin_amdgcn_readlane(be, __ffsll((unsigned long long)mask) - 1);
    else
      we = __ockl_wfred_min_i32(cand ? be : kNoExpert);
    if (we == kNoExpert) we = jj;   // only reachable with NaN logits (out of domain)
#pragma unroll
    for (int m = 0; m < PER; ++m) taken |= (id[m] == we ? 1u : 0u) << m;
    if (jj == 0) zmax = wmax;
    my_e = lane == jj ? we : my_e;
    my_z = lane == jj ? wmax : my_z;
  }
  const float ex = lane < k ? expf(my_z - zmax) : 0.0f;
  float den = 0.0f;
  int rank = 0;
#pragma unroll 1
  for (int jj = 0; jj < k; ++jj) {
    den += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), jj));
    rank += __builtin_amdgcn_readlane(my_e, jj) < my_e;
  }
  if (lane < k) {
    ids_row[rank] = my_e;
    w_row[rank] = ex / den;
  }
}

}  // namespace moe
