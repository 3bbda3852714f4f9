// grouped_gemm.hip -- grouped expert GEMMs of the MoE layer on gfx950 MFMA.
//
// "Every Expert Counts: ExactMoE ..." §3.4: one fused gate/up grouped GEMM and
// one down grouped GEMM per call over the whole token matrix (no per-expert
// launches), experts found through a global expert map; §3.1: the dequantized
// weights define the operation (no fp16 expert is materialized); MxMoE
// (abstract): experts of different precisions run in the same grouped launch.
//
// One workgroup computes a BM x BN output tile of one expert.  Its M-tile comes
// from the device tile table written by the grouping kernel (rows of the
// expert's segment of the grouped route order); the expert's precision tier and
// packed weights come from the handle table, so one launch serves all tiers.
//
// Numerics.  Weights reach the MFMA as exact integers: an int4 code u = q+8 is
// turned into the bf16 value 136+q with one and-or (0x4300 | u), an int8 code
// u = q+128 into 128+q.  For every 128-wide k-group the MFMA accumulator
// starts at -OFF * R[m] (R = sum of the group's activations of row m), so after
// the group it holds sum_k a*q exactly up to fp32 rounding; it is then scaled by
// the fp16 group scale (int4) or row scale (int8) into the fp32 result.  bf16
// experts feed their weights directly.  Activations are bf16 (W4A16), all sums
// fp32.
//
// Packed layout: see quant_pack.hip.  A 16-byte load per lane of one 1 KB tile
// gives that lane's B operands for four consecutive 32-wide MFMA k-steps of
// one 16-column strip (int4), so B goes from HBM to registers with no LDS and
// no cross-lane shuffles.  A (activations) is staged through LDS per k-group.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout used here: lane l holds row
// (A) / column (B) l%16 and the 8 k-values 8*(l/16) .. +7 of the 32-wide step;
// the accumulator of lane l holds rows 4*(l/16) + i, column l%16.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

struct GemmArgs {
  const DevHandle* table;
  const TileEntry* tiles;
  const int32_t* ntiles;
  const uint16_t* a_src;     // gate/up: x [T, H]; down: act [T*k, I] in grouped order
  const int32_t* sorted;     // grouped route order (route ids t*k + j)
  const float* rsum;         // gate/up: R13 [T, H/128] by token; down: R2 [T*k, I/128] by row
  int top_k;
  int K;                     // reduction size: H (gate/up) or I (down)
  int N;                     // output columns: 2I (gate/up) or H (down)
  // gate/up epilogue
  uint16_t* act;             // [T*k, I] bf16, grouped order
  float* r2;                 // [T*k, I/128]
  int I;
  // down epilogue
  const float* topk_w;       // [T*k] routing weights by route id
  float* rows;               // [T*k, H] fp32, grouped order
};

constexpr int kLdsStride = kGroup + 8;   // bf16 per LDS row (272 B: conflict-free reads)

template <int TIER>
struct TierTraits;
template <>
struct TierTraits<MOE_TIER_INT4> {
  static constexpr int kLoads = 1, kTileBytes = 1024;
  static constexpr float kOffset = 136.0f;
};
template <>
struct TierTraits<MOE_TIER_INT8> {
  static constexpr int kLoads = 2, kTileBytes = 2048;
  static constexpr float kOffset = 128.0f;
};
template <>
struct TierTraits<MOE_TIER_BF16> {
  static constexpr int kLoads = 4, kTileBytes = 4096;
  static constexpr float kOffset = 0.0f;
};

template <int TIER>
__device__ __forceinline__ bf16x8_t b_operand(const u32x4 (&b)[TierTraits<TIER>::kLoads], int s) {
  if constexpr (TIER == MOE_TIER_INT4) {
    const uint32_t w = s == 0 ? b[0].x : s == 1 ? b[0].y : s == 2 ? b[0].z : b[0].w;
    return int4x8_to_bf16_biased(w);
  } else if constexpr (TIER == MOE_TIER_INT8) {
    const u32x4& h = b[s >> 1];
    return (s & 1) ? int8x8_to_bf16_biased(h.z, h.w) : int8x8_to_bf16_biased(h.x, h.y);
  } else {
    return as_bf16x8(b[s]);
  }
}

// Block: WN waves side by side along N; every wave covers all BM = 16*RT rows
// and NS 16-column strips.  BN = 16*NS*WN.
template <int RT, int NS, int WN>
struct Tile {
  static constexpr int BM = 16 * RT;
  static constexpr int BN = 16 * NS * WN;
  static constexpr int kThreads = 64 * WN;
  static constexpr int kChunks = BM * (kGroup / 8);          // 16-byte A chunks per group
  static constexpr int kChunksPerThread = (kChunks + kThreads - 1) / kThreads;
};

template <int TIER, int RT, int NS, int WN>
__device__ __forceinline__ void mainloop(const GemmArgs& a, const DevHandle& h, bool gate_up,
                                         int strip0, const uint16_t* const (&arow)[Tile<RT, NS, WN>::kChunksPerThread],
                                         const int (&acol)[Tile<RT, NS, WN>::kChunksPerThread],
                                         const int (&alds)[Tile<RT, NS, WN>::kChunksPerThread],
                                         const float* const (&rrow)[RT][4], uint16_t* lds,
                                         f32x4_t (&acc)[RT][NS]) {
  using TT = Tile<RT, NS, WN>;
  using TR = TierTraits<TIER>;
  const int lane = threadIdx.x & 63;
  const int K = a.K, G = K / kGroup;
  const uint8_t* blob = gate_up ? h.w13 : h.w2;
  const uint8_t* codes = blob;   // codes first, then the fp16 scales
  const uint16_t* scales16 = nullptr;
  if constexpr (TIER == MOE_TIER_INT4)
    scales16 = reinterpret_cast<const uint16_t*>(blob + (size_t)a.N * K / 2);
  else if constexpr (TIER == MOE_TIER_INT8)
    scales16 = reinterpret_cast<const uint16_t*>(blob + (size_t)a.N * K);

  float row_scale[NS];
  if constexpr (TIER == MOE_TIER_INT8) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
      row_scale[ns] = (float)__builtin_bit_cast(_Float16, scales16[16 * (strip0 + ns) + (lane & 15)]);
  }

  u32x4 b_cur[NS][TR::kLoads], b_nxt[NS][TR::kLoads];
  u32x4 a_nxt[TT::kChunksPerThread];

  auto load_b = [&](int g, u32x4 (&dst)[NS][TR::kLoads]) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const uint8_t* tp = codes + ((size_t)(strip0 + ns) * G + g) * TR::kTileBytes + 16 * lane;
#pragma unroll
      for (int q = 0; q < TR::kLoads; ++q) dst[ns][q] = load_u32x4_stream(tp + 1024 * q);
    }
  };
  auto load_a = [&](int g) {
#pragma unroll
    for (int c = 0; c < TT::kChunksPerThread; ++c)
      a_nxt[c] = arow[c] ? load_u32x4(arow[c] + kGroup * g + acol[c]) : u32x4{0, 0, 0, 0};
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int c = 0; c < TT::kChunksPerThread; ++c)
      if (alds[c] >= 0)
        *reinterpret_cast<uint4*>(lds + buf * TT::BM * kLdsStride + alds[c]) =
            make_uint4(a_nxt[c].x, a_nxt[c].y, a_nxt[c].z, a_nxt[c].w);
  };

  load_b(0, b_cur);
  load_a(0);
  store_a(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) {
      load_b(g + 1, b_nxt);
      load_a(g + 1);
    }
    f32x4_t p[RT][NS];
    if constexpr (TIER == MOE_TIER_BF16) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) p[rt][ns] = acc[rt][ns];
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4_t init;
#pragma unroll
        for (int i = 0; i < 4; ++i) init[i] = rrow[rt][i] ? -TR::kOffset * rrow[rt][i][g] : 0.0f;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) p[rt][ns] = init;
      }
    }
    const uint16_t* la = lds + buf * TT::BM * kLdsStride;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t af[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        af[rt] = as_bf16x8(load_u32x4(la + (16 * rt + (lane & 15)) * kLdsStride + 32 * s +
                                      8 * (lane >> 4)));
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const bf16x8_t bf = b_operand<TIER>(b_cur[ns], s);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) p[rt][ns] = mfma16x16x32(af[rt], bf, p[rt][ns]);
      }
    }
    if constexpr (TIER == MOE_TIER_BF16) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) acc[rt][ns] = p[rt][ns];
    } else {
      float sc[NS];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        if constexpr (TIER == MOE_TIER_INT4)
          sc[ns] = (float)__builtin_bit_cast(
              _Float16, scales16[((size_t)(strip0 + ns) * G + g) * 16 + (lane & 15)]);
        else
          sc[ns] = row_scale[ns];
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rt][ns][i] = __builtin_fmaf(sc[ns], p[rt][ns][i], acc[rt][ns][i]);
    }
    if (g + 1 < G) {
      store_a(buf ^ 1);
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int q = 0; q < TR::kLoads; ++q) b_cur[ns][q] = b_nxt[ns][q];
    }
    __syncthreads();
  }
}

template <int RT, int NS, int WN, bool GATE_UP>
__global__ __launch_bounds__(64 * WN) void grouped_gemm_kernel(GemmArgs a) {
  using TT = Tile<RT, NS, WN>;
  static_assert(!GATE_UP || (NS % 4 == 0 && TT::BN == 256), "gate/up tile covers one 128-group of I");
  const int tile_idx = blockIdx.y;
  if (tile_idx >= *a.ntiles) return;
  const TileEntry te = a.tiles[tile_idx];
  const DevHandle h = a.table[te.expert];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_block = blockIdx.x * TT::BN;
  const int strip0 = (n_block + wave * 16 * NS) / 16;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * TT::BM * kLdsStride];
  __shared__ float part[WN][TT::BM];

  // A staging role of this thread: chunk c -> (row, 16-byte column)
  const uint16_t* arow[TT::kChunksPerThread];
  int acol[TT::kChunksPerThread], alds[TT::kChunksPerThread];
  const int G = a.K / kGroup;
#pragma unroll
  for (int c = 0; c < TT::kChunksPerThread; ++c) {
    const int chunk = threadIdx.x + c * TT::kThreads;
    const int m = chunk >> 4, col = 8 * (chunk & 15);
    arow[c] = nullptr;
    acol[c] = col;
    alds[c] = -1;
    if (chunk < TT::kChunks) {
      alds[c] = m * kLdsStride + col;
      if (m < te.rows) {
        const int pos = te.row_start + m;
        if constexpr (GATE_UP)
          arow[c] = a.a_src + (size_t)(a.sorted[pos] / a.top_k) * a.K;
        else
          arow[c] = a.a_src + (size_t)pos * a.K;
      }
    }
  }
  // rows of the accumulator this lane holds, and their R rows
  const float* rrow[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * rt + 4 * (lane >> 4) + i;
      rrow[rt][i] = nullptr;
      if (m < te.rows) {
        const int pos = te.row_start + m;
        if constexpr (GATE_UP)
          rrow[rt][i] = a.rsum + (size_t)(a.sorted[pos] / a.top_k) * G;
        else
          rrow[rt][i] = a.rsum + (size_t)pos * G;
      }
    }

  f32x4_t acc[RT][NS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[rt][ns] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  switch (h.tier) {
    case MOE_TIER_INT4:
      mainloop<MOE_TIER_INT4, RT, NS, WN>(a, h, GATE_UP, strip0, arow, acol, alds, rrow, lds, acc);
      break;
    case MOE_TIER_INT8:
      mainloop<MOE_TIER_INT8, RT, NS, WN>(a, h, GATE_UP, strip0, arow, acol, alds, rrow, lds, acc);
      break;
    default:
      mainloop<MOE_TIER_BF16, RT, NS, WN>(a, h, GATE_UP, strip0, arow, acol, alds, rrow, lds, acc);
      break;
  }

  if constexpr (GATE_UP) {
    // SwiGLU: strips 4q, 4q+1 are gate, 4q+2, 4q+3 the matching up columns.
    float rs[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[rt][i] = 0.0f;
#pragma unroll
    for (int q = 0; q < NS / 4; ++q) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ns = 4 * q + half;
        const int icol = 32 * (strip0 / 4 + q) + 16 * half + (lane & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * rt + 4 * (lane >> 4) + i;
            const float gv = acc[rt][ns][i], uv = acc[rt][ns + 2][i];
            const uint32_t a16 = f32_to_bf16_rne(silu_f32(gv) * uv);
            if (m < te.rows) {
              a.act[(size_t)(te.row_start + m) * a.I + icol] = (uint16_t)a16;
              rs[rt][i] += bf16_to_f32(a16);
            }
          }
      }
    }
    // per-row sums of this block's 128 activation columns (one k-group of the
    // down GEMM), reduced in a fixed order: lanes, then waves.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = rs[rt][i];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 16);
        if ((lane & 15) == 0) part[wave][16 * rt + 4 * (lane >> 4) + i] = v;
      }
    __syncthreads();
    const int G2 = a.I / kGroup;
    for (int m = threadIdx.x; m < te.rows && m < TT::BM; m += TT::kThreads) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WN; ++w) v += part[w][m];
      a.r2[(size_t)(te.row_start + m) * G2 + blockIdx.x] = v;
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * rt + 4 * (lane >> 4) + i;
        if (m < te.rows) {
          const int pos = te.row_start + m;
          const float wgt = a.topk_w[a.sorted[pos]];
          float* out = a.rows + (size_t)pos * a.N + n_block + wave * 16 * NS + (lane & 15);
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) out[16 * ns] = wgt * acc[rt][ns][i];
        }
      }
  }
}

template <int RT, bool GATE_UP>
hipError_t launch_gg(const GemmArgs& a, int max_tiles, hipStream_t s) {
  constexpr int NS = 4, WN = 4;
  using TT = Tile<RT, NS, WN>;
  const dim3 grid(a.N / TT::BN, max_tiles);
  hipLaunchKernelGGL((grouped_gemm_kernel<RT, NS, WN, GATE_UP>), grid, dim3(TT::kThreads), 0, s, a);
  return hipGetLastError();
}

// Sum of a token's k weighted rows in ascending expert order, fp32.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ rows,
                                                      const int32_t* __restrict__ pos, int T,
                                                      int H, int k, void* __restrict__ y) {
  const int t = blockIdx.y;
  const int h4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h4 >= H) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float4 v = *reinterpret_cast<const float4*>(rows + (size_t)pos[t * k + j] * H + h4);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  if constexpr (BF16_OUT) {
    const uint32_t lo = f32_to_bf16_rne(s.x) | (f32_to_bf16_rne(s.y) << 16);
    const uint32_t hi = f32_to_bf16_rne(s.z) | (f32_to_bf16_rne(s.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * H + h4) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * H + h4) = s;
  }
}

}  // namespace

GemmPlan plan_gemm(const Layer& L, int T) {
  GemmPlan p;
  const double rows_per_expert = (double)T * L.k / L.E;
  const int bm = rows_per_expert <= 16.0 ? 16 : 64;
  p.bm13 = bm;
  p.bm2 = bm;
  p.kind = 0;
  return p;
}

hipError_t launch_gemm13(const Layer& L, const GemmPlan& gp, int T, const uint16_t* x,
                         const int32_t* sorted, const TileEntry* tiles, const int32_t* ntiles,
                         int max_tiles, const float* r13, uint16_t* act, float* r2,
                         hipStream_t s) {
  (void)T;
  GemmArgs a{};
  a.table = L.table;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.a_src = x;
  a.sorted = sorted;
  a.rsum = r13;
  a.top_k = L.k;
  a.K = L.H;
  a.N = 2 * L.I;
  a.act = act;
  a.r2 = r2;
  a.I = L.I;
  if (gp.bm13 == 16) return launch_gg<1, true>(a, max_tiles, s);
  return launch_gg<4, true>(a, max_tiles, s);
}

hipError_t launch_gemm2(const Layer& L, const GemmPlan& gp, int T, const uint16_t* act,
                        const int32_t* sorted, const float* topk_w, const TileEntry* tiles,
                        const int32_t* ntiles, int max_tiles, const float* r2, float* rows,
                        hipStream_t s) {
  (void)T;
  GemmArgs a{};
  a.table = L.table;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.a_src = act;
  a.sorted = sorted;
  a.rsum = r2;
  a.top_k = L.k;
  a.K = L.I;
  a.N = L.H;
  a.topk_w = topk_w;
  a.rows = rows;
  if (gp.bm2 == 16) return launch_gg<1, false>(a, max_tiles, s);
  return launch_gg<4, false>(a, max_tiles, s);
}

hipError_t launch_combine(const float* rows, const int32_t* pos, int T, int H, int k, void* y,
                          int y_dtype, hipStream_t s) {
  const dim3 grid((H / 4 + 255) / 256, T);
  if (y_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, rows, pos, T, H, k, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, rows, pos, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
