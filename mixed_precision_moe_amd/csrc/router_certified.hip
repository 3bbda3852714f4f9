// router_certified.hip -- top-k routing for many tokens with the logits on
// MFMA, exact with respect to the canonical fp32 order.
//
// "Every Expert Counts: ExactMoE ..." §3.1: z = W_r h (router kept in BF16)
// and S = TopK(z, k).  The library's routing is defined by the canonical fp32
// logit order (32 chains, pairwise fold; see route.hip), which an fp32 FMA
// kernel computes at T*E*H FMAs.  For many tokens and experts these kernels
// instead
//   1. compute approximate logits v = x . w_e on bf16 MFMA (any summation
//      order, split over K), together with ||x_t||^2 and ||w_e||^2;
//   2. per token, bound |v + b_e - z_e| by eps_e for every expert: the MFMA sum
//      and the canonical sum are both sums of the same H exact products, so
//      each lies within gamma_(H-1) * sum |x_h w_h| of the exact dot product
//      for any evaluation order (gamma_n = n u / (1 - n u), u = 2^-24), and
//      sum |x_h w_h| <= ||x|| ||w_e|| (Cauchy-Schwarz).  eps doubles that
//      (an adder that truncates doubles u), adds 1% for the rounding of the
//      norms, and 4 u (|v| + |b|) for the bias addition and the comparisons;
//   3. take theta = the k-th largest v - eps.  An expert with v + eps < theta
//      has k experts whose canonical logits are strictly larger, so it is not
//      in the canonical top k; the others are the candidates (k, plus the few
//      whose margin the bound cannot resolve);
//   4. recompute the candidates' logits in the canonical order and take the
//      top k among them with the canonical selection and softmax
//      (topk_select.h).  Exactly tied logits (say, all-zero tokens) only make
//      the candidate list longer, up to all E experts.
// The result is the canonical routing, bit for bit, for every token.
#include <math.h>

#include "device_util.h"
#include "moe_internal.h"
#include "topk_select.h"

namespace moe {
namespace {

// 1. Approximate logits, one 32-token x 64-expert tile per block.  Grid
// (ceil(T/32), ceil(E/64), S): block z sums K slice [z H/S, (z+1) H/S), its
// four waves one quarter each (kw = H / (4 S), a multiple of 64).  A wave
// holds 2 x 4 tiles of v_mfma_f32_16x16x32_bf16; both operands are K-major
// rows, so a lane's 16 bytes of x or Wr are exactly its MFMA operand (lane l:
// row l % 16, k = 8 (l / 16) .. +7 of the 32-wide step).  Two steps of loads
// are in flight.  The four waves' sums meet in LDS and the block writes
// vpart[z, t, e] (no bias); blocks of the first tile column (row) also write
// the partial squared norms xpart[z, t] (wpart[z, e]).
constexpr int kRedPitch = 68;   // LDS row pitch (floats): conflict-free reads

__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E, int S,
    float* __restrict__ vpart, float* __restrict__ xpart, float* __restrict__ wpart) {
  __shared__ float red[4][32][kRedPitch];
  __shared__ float nrm[4][96];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 64, z = blockIdx.z;
  const int kw = H / (4 * S);
  const int kbeg = (z * 4 + wave) * kw;
  const int r = lane & 15, kq = lane >> 4;
  const uint16_t* ap[2];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) ap[i] = x + (size_t)min(t0 + 16 * i + r, T - 1) * H + kbeg + 8 * kq;
#pragma unroll
  for (int j = 0; j < 4; ++j) bp[j] = wr + (size_t)min(e0 + 16 * j + r, E - 1) * H + kbeg + 8 * kq;
  const bool do_xn = blockIdx.y == 0, do_wn = blockIdx.x == 0;
  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float sx[2] = {0.f, 0.f}, sw[4] = {0.f, 0.f, 0.f, 0.f};
  u32x4 a0[2], b0[4], a1[2], b1[4];
  auto load = [&](int k, u32x4 (&a)[2], u32x4 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = load_u32x4(ap[i] + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = load_u32x4(bp[j] + k);
  };
  auto sq = [](u32x4 q) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t d = (&q.x)[c];
      const float lo = bf16lo_to_f32(d), hi = bf16hi_to_f32(d);
      s = __builtin_fmaf(lo, lo, s);
      s = __builtin_fmaf(hi, hi, s);
    }
    return s;
  };
  auto consume = [&](const u32x4 (&a)[2], const u32x4 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j]);
    if (do_xn) {
#pragma unroll
      for (int i = 0; i < 2; ++i) sx[i] += sq(a[i]);
    }
    if (do_wn) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sw[j] += sq(b[j]);
    }
  };
  // kw >= 64: the loop body never loads past the slice, the tail consumes
  // the last two steps
  load(0, a0, b0);
  load(32, a1, b1);
  for (int kk = 0; kk + 64 < kw; kk += 64) {
    consume(a0, b0);
    load(kk + 64, a0, b0);
    consume(a1, b1);
    load(kk + 96, a1, b1);
  }
  consume(a0, b0);
  consume(a1, b1);
  // partial norms: the four lanes holding a row's k-slices, then the 4 waves
  if (do_xn || do_wn) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float s = sx[i];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (kq == 0) nrm[wave][16 * i + r] = s;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = sw[j];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (kq == 0) nrm[wave][32 + 16 * j + r] = s;
    }
  }
  // accumulator of lane l holds rows 4 (l / 16) + q of the tile, column l % 16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[wave][i * 16 + j * 4 + q][lane] = acc[i][j][q];
  __syncthreads();
  const int tid = threadIdx.x;
  if (do_xn && tid < 32 && t0 + tid < T)
    xpart[(size_t)z * T + t0 + tid] = nrm[0][tid] + nrm[1][tid] + nrm[2][tid] + nrm[3][tid];
  if (do_wn && tid >= 64 && tid < 128 && e0 + tid - 64 < E) {
    const int c = 32 + tid - 64;
    wpart[(size_t)z * E + e0 + tid - 64] = nrm[0][c] + nrm[1][c] + nrm[2][c] + nrm[3][c];
  }
  const int el = tid & 63, e = e0 + el;
  const int j = el >> 4, col = el & 15;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int tl = (tid >> 6) + 4 * s, t = t0 + tl;
    const int idx = (tl >> 4) * 16 + j * 4 + (tl & 3);
    const int l = 16 * ((tl & 15) >> 2) + col;
    const float sum = red[0][idx][l] + red[1][idx][l] + red[2][idx][l] + red[3][idx][l];
    if (t < T && e < E) vpart[((size_t)z * T + t) * E + e] = sum;
  }
}

// 2.-4. One block of W waves per token.  Wave 0 finds the candidates; cid /
// cb / zc (LDS) hold their ids, biases and canonical logits, numbered in
// increasing expert id.  Every half-wave of the block then recomputes its
// share of the candidates, and wave 0 selects.  With few tokens, several waves
// per token run the candidates' memory round trips side by side (Qwen3-80B
// shape, T = 1024: routing 47.9 -> 42.5 us with four); with many, one wave per
// token already fills the GPU and more only add barriers (T = 4096: 95.4 ->
// 102.8 us with four).
template <int PER, int W>
__global__ __launch_bounds__(64 * W) void router_select_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ vpart, const float* __restrict__ xpart,
    const float* __restrict__ wpart, int T, int H, int E, int S, int k, float cgam,
    int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ int cid[64 * PER];
  __shared__ float cb[64 * PER];
  __shared__ float zc[64 * PER];
  __shared__ int ncand;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  if (t >= T) return;   // block-uniform
  if (threadIdx.x < 64) {   // wave 0: the candidates
    // sums of the S partials: each split's loads for all of the lane's experts
    // are issued together
    const int per = (E + 63) / 64;
    float val[PER], eps[PER], bb[PER], w2[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      val[m] = 0.0f;
      w2[m] = 0.0f;
    }
    float xn2 = 0.0f;
    for (int z = 0; z < S; ++z) {
      xn2 += xpart[(size_t)z * T + t];
      const float* vz = vpart + ((size_t)z * T + t) * E;
      const float* wz = wpart + (size_t)z * E;
#pragma unroll
      for (int m = 0; m < PER; ++m) {   // clamped, branch-free loads
        const int e = min(lane + 64 * m, E - 1);
        val[m] += vz[e];
        w2[m] += wz[e];
      }
    }
    const float nx = sqrtf(xn2);
    float braw[PER];
    if (bias) {   // wave-uniform; clamped loads issued together
#pragma unroll
      for (int m = 0; m < PER; ++m) braw[m] = bias[min(lane + 64 * m, E - 1)];
    } else {
#pragma unroll
      for (int m = 0; m < PER; ++m) braw[m] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = lane + 64 * m;
      const bool ok = m < per && e < E;
      const float b = ok ? braw[m] : 0.0f;
      const float v = val[m] + b;
      bb[m] = b;
      val[m] = ok ? v : -INFINITY;
      eps[m] = ok ? cgam * nx * sqrtf(w2[m]) + 0x1p-22f * (fabsf(v) + fabsf(b)) + 1e-30f : 0.0f;
    }
    // theta: the k-th largest v - eps (one entry taken per round)
    uint32_t taken = 0;
    float theta = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj) {
      if (jj >= k) break;
      float bv = -INFINITY;
      int bm = -1;
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const int e = lane + 64 * m;
        const float lo = val[m] - eps[m];
        if (m < per && e < E && !((taken >> m) & 1u) && (bm < 0 || lo > bv)) {
          bv = lo;
          bm = m;
        }
      }
      const float wmax = __ockl_wfred_max_f32(bv);
      const uint64_t mask = __ballot(bm >= 0 && bv == wmax);
      // mask is 0 only with NaN logits (out of domain; then every expert
      // becomes a candidate below)
      if (lane == __ffsll((unsigned long long)mask) - 1) taken |= 1u << bm;
      if (mask) theta = wmax;
    }
    // candidates: v + eps >= theta, numbered in increasing expert id
    int c = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = lane + 64 * m;
      const bool cand = m < per && e < E && val[m] + eps[m] >= theta;
      const uint64_t mask = __ballot(cand);
      const int at = c + __popcll(mask & ((1ull << lane) - 1ull));
      if (cand) {
        cid[at] = e;
        cb[at] = bb[m];
      }
      c += __popcll(mask);
    }
    if (c < k) {   // only with NaN logits (out of domain): every expert is a candidate
      for (int i = lane; i < E; i += 64) {
        cid[i] = i;
        cb[i] = bias ? bias[i] : 0.0f;
      }
      c = E;
    }
    if (lane == 0) ncand = c;
  }   // wave 0
  __syncthreads();
  const int c = ncand;
  // canonical logits of the candidates: half-wave h (of NH) takes candidates
  // NH p + h (p = 0, 1, ...); lane j of the half is chain j.  The half
  // streams its slabs (p outer, slab inner) in batches of four, two batches
  // in flight.
  constexpr int NH = 2 * W;
  const int j = lane & 31, hw = threadIdx.x >> 5;
  const int ns = H >> 8, Q = ((c + NH - 1) / NH) * ns;
  const uint16_t* xrow = x + (size_t)t * H + 8 * j;
  int ip = 0, is = 0;   // issue cursor (round, slab)
  auto issue = [&](u32x4 (&wv)[4], u32x4 (&xv)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = cid[min(NH * ip + hw, c - 1)];
      wv[u] = load_u32x4(wr + (size_t)e * H + 256 * is + 8 * j);
      xv[u] = load_u32x4(xrow + 256 * is);
      if (++is == ns) {
        is = 0;
        ip = min(ip + 1, (c - 1) / NH);   // past the end: repeat the last round's rows
      }
    }
  };
  int cp = 0, cs = 0;   // consume cursor
  float acc = 0.0f;
  auto consume = [&](const u32x4 (&wv)[4], const u32x4 (&xv)[4], int q0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (q0 + u < Q) {                            // wave-uniform
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const uint32_t dx = (&xv[u].x)[rr >> 1], dw = (&wv[u].x)[rr >> 1];
          const float xf = (rr & 1) ? bf16hi_to_f32(dx) : bf16lo_to_f32(dx);
          const float wf = (rr & 1) ? bf16hi_to_f32(dw) : bf16lo_to_f32(dw);
          acc = __builtin_fmaf(xf, wf, acc);
        }
        if (++cs == ns) {                          // wave-uniform
#pragma unroll
          for (int sh = 16; sh >= 1; sh >>= 1) acc = acc + __shfl_down(acc, sh, 32);
          const int jc = NH * cp + hw;
          if (j == 0 && jc < c) zc[jc] = acc + cb[jc];
          acc = 0.0f;
          cs = 0;
          ++cp;
        }
      }
    }
  };
  u32x4 wa[4], xa[4], wb[4], xb[4];
  issue(wa, xa);
  issue(wb, xb);
  for (int q0 = 0; q0 < Q; q0 += 8) {
    consume(wa, xa, q0);
    issue(wa, xa);
    consume(wb, xb, q0 + 4);
    issue(wb, xb);
  }
  __syncthreads();
  if (W > 1 && threadIdx.x >= 64) return;
  // the canonical top k among the candidates
  float zz[PER];
  int id[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int i = lane + 64 * m;
    const bool ok = i < c;
    zz[m] = ok ? zc[i] : -INFINITY;
    id[m] = ok ? cid[i] : kNoExpert;
  }
  topk_select_softmax<PER>(zz, id, k, ids + (size_t)t * k, weights + (size_t)t * k);
}

}  // namespace

hipError_t launch_router_certified(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                                   int H, int E, int k, float* v, float* xn2, float* wn2,
                                   int32_t* ids, float* w, hipStream_t s) {
  const int S = router_split(T, E, H);
  const dim3 grid((T + 31) / 32, (E + 63) / 64, S);
  hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(256), 0, s, x, wr, T, H, E, S, v, xn2, wn2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // eps = 2 (2 gamma_H) ||x|| ||w_e|| (1.01) + 4 u (|v| + |b|), see the header
  const double n = (double)H, u = 0x1p-24;
  const float cgam = (float)(2.0 * 2.0 * (n * u / (1.0 - n * u)) * 1.01);
  const int per = (E + 63) / 64;
  // waves per token: about 4096 waves in all, at most four per token
  const int W = T <= 1024 ? 4 : T <= 2048 ? 2 : 1;
#define MOE_SELECT1(P, WV)                                                                  \
  hipLaunchKernelGGL((router_select_kernel<P, WV>), dim3(T), dim3(64 * WV), 0, s, x, wr, bias, \
                     v, xn2, wn2, T, H, E, S, k, cgam, ids, w)
#define MOE_SELECT(P)        \
  do {                       \
    if (W == 4)              \
      MOE_SELECT1(P, 4);     \
    else if (W == 2)         \
      MOE_SELECT1(P, 2);     \
    else                     \
      MOE_SELECT1(P, 1);     \
  } while (0)
  if (per <= 1)
    MOE_SELECT(1);
  else if (per <= 2)
    MOE_SELECT(2);
  else if (per <= 4)
    MOE_SELECT(4);
  else if (per <= 8)
    MOE_SELECT(8);
  else
    MOE_SELECT(kMaxExperts / 64);
#undef MOE_SELECT
#undef MOE_SELECT1
  return hipGetLastError();
}

}  // namespace moe
