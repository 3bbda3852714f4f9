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

// better(a, b): larger logit, or equal logit and lower expert id.
__device__ __forceinline__ bool topk_better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

constexpr int kNoExpert = 0x7fffffff;

// One wave selects the k best entries (logit descending, id ascending) of the
// lane-distributed list (z[m], id[m]); unused entries carry id kNoExpert.
// Each round takes the lane-local best untaken entry, a wave max of the logit
// (DPP reduction) and, only if several lanes hold that maximum, a wave min of
// their ids.  The weights are the softmax over the selected logits with the
// first (largest) one as the max and the denominator summed in selection
// order.  Lanes < k store id and weight of the entry of rank `lane` in
// increasing id order to ids_row / w_row.
template <int PER>
__device__ __forceinline__ void topk_select_softmax(const float (&z)[PER], const int (&id)[PER],
                                                    int k, int32_t* __restrict__ ids_row,
                                                    float* __restrict__ w_row) {
  const int lane = threadIdx.x & 63;
  uint32_t taken = 0;
  int sel_e[kMaxTopK];
  float sel_z[kMaxTopK];
#pragma unroll
  for (int jj = 0; jj < kMaxTopK; ++jj) {
    if (jj >= k) break;
    float bv = -INFINITY;
    int be = kNoExpert;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      if (id[m] != kNoExpert && !((taken >> m) & 1u) && topk_better(z[m], id[m], bv, be)) {
        bv = z[m];
        be = id[m];
      }
    }
    const float wmax = __ockl_wfred_max_f32(bv);
    const bool cand = bv == wmax && be != kNoExpert;
    const uint64_t mask = __ballot(cand);
    int we;
    if (__popcll(mask) == 1)
      we = __builtin_amdgcn_readlane(be, __ffsll((unsigned long long)mask) - 1);
    else
      we = __ockl_wfred_min_i32(cand ? be : kNoExpert);
    if (we == kNoExpert) we = jj;   // only reachable with NaN logits (out of domain)
#pragma unroll
    for (int m = 0; m < PER; ++m)
      if (id[m] == we) taken |= 1u << m;
    sel_e[jj] = we;
    sel_z[jj] = wmax;
  }
  if (lane < k) {
    int my_e = 0;
    float my_z = 0.0f, den = 0.0f;
    const float zmax = sel_z[0];
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj) {
      if (jj >= k) break;
      den += expf(sel_z[jj] - zmax);
      if (jj == lane) {
        my_e = sel_e[jj];
        my_z = sel_z[jj];
      }
    }
    int rank = 0;
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj) {
      if (jj >= k) break;
      rank += sel_e[jj] < my_e;
    }
    ids_row[rank] = my_e;
    w_row[rank] = expf(my_z - zmax) / den;
  }
}

}  // namespace moe
