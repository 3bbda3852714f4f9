// grouped_gemm.hip -- grouped expert GEMMs of the MoE layer for few tokens per
// expert (decode), on gfx950 MFMA, and the routing-weighted combine.
//
// "Every Expert Counts: ExactMoE ..." §3.4: one fused gate/up grouped GEMM and
// one down grouped GEMM per call over the whole token matrix (no per-expert
// launches), experts found through a global expert map; §3.1: the dequantized
// weights define the operation (no fp16 expert is materialized); MxMoE
// (abstract): experts of different precisions run in the same grouped launch.
//
// One workgroup computes an M-tile x (WAVES*NS*16)-column tile of one expert.
// Its M-tile comes from the device tile table written by the grouping kernel
// (rows of the expert's segment of the grouped route order, plus the expert's
// precision tier and packed weights copied from the handle table), so one
// launch serves all tiers.
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
// no cross-lane shuffles.  A (activations) is staged through LDS, one K-chunk
// at a time.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout used here: lane l holds row
// (A) / column (B) l%16 and the 8 k-values 8*(l/16) .. +7 of the 32-wide step;
// the accumulator of lane l holds rows 4*(l/16) + i, column l%16.
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

struct GemmArgs {
  const TileEntry* tiles;
  const int32_t* ntiles;
  const uint16_t* a_src;     // gate/up: x [T, H]; down: act [T*k, I] in grouped order
  const int32_t* sorted;     // grouped route order (route ids t*k + j)
  const float* rsum;         // gate/up: R13 [T, H/128] by token; down: R2 partials [T*k, I/32] by row
  int top_k;
  int K;                     // reduction size: H (gate/up) or I (down)
  int N;                     // output columns: 2I (gate/up) or H (down)
  // gate/up epilogue
  uint16_t* act;             // [T*k, I] bf16, grouped order
  float* r2;                 // [T*k, I/32]: row sums of each 32-column block of act
  int I;
  // down epilogue
  const float* topk_w;       // [T*k] routing weights by route id
  float* rows;               // [T*k, H] fp32, by route id (t k + j)
  int tile_group;            // non-zero and ntiles[1] set: kDecodeTileGroup consecutive tiles of one column block share an XCD
};


template <int TIER>
struct TierTraits;
// Per tier: 16-byte loads per lane per strip and k-group, bytes of one strip's
// tile, bytes of one (quad, k-group) block, weight offset of the codes.
template <>
struct TierTraits<MOE_TIER_INT4> {
  static constexpr int kLoads = 1, kTileBytes = 1024, kBlockBytes = 4224;
  static constexpr float kOffset = 136.0f;
};
template <>
struct TierTraits<MOE_TIER_INT8> {
  static constexpr int kLoads = 2, kTileBytes = 2048, kBlockBytes = 8192;
  static constexpr float kOffset = 128.0f;
};
template <>
struct TierTraits<MOE_TIER_BF16> {
  static constexpr int kLoads = 4, kTileBytes = 4096, kBlockBytes = 16384;
  static constexpr float kOffset = 0.0f;
};

// Bytes of a packed [N, K] blob of one tier (without the 256-byte padding).
template <int TIER>
__device__ __forceinline__ uint32_t blob_payload(int N, int K) {
  if constexpr (TIER == MOE_TIER_INT4) return (uint32_t)(N / 64) * (K / kGroup) * 4224u;
  else if constexpr (TIER == MOE_TIER_INT8) return (uint32_t)N * K + 2u * N;
  else return 2u * N * K;
}

// Activation sum of k-group g of one A row.  Gate/up: R13[token][g] (one value
// per 128 inputs).  Down: the gate/up epilogue leaves one partial per 32
// activation columns, so a 128-group is the sum of four, added in a fixed order.
template <bool GATE_UP>
__device__ __forceinline__ float row_sum(const float* r, int g) {
  if (!r) return 0.0f;
  if constexpr (GATE_UP) {
    return r[g];
  } else {
    const float4 v = *reinterpret_cast<const float4*>(r + 4 * g);
    return (v.x + v.y) + (v.z + v.w);
  }
}

template <int TIER>
__device__ __forceinline__ bf16x8_t b_operand(const u32x4 (&b)[TierTraits<TIER>::kLoads], int s,
                                              Int4Consts c4) {
  if constexpr (TIER == MOE_TIER_INT4) {
    const uint32_t w = s == 0 ? b[0].x : s == 1 ? b[0].y : s == 2 ? b[0].z : b[0].w;
    return int4x8_to_bf16_biased(w, c4);
  } else if constexpr (TIER == MOE_TIER_INT8) {
    const u32x4& h = b[s >> 1];
    return (s & 1) ? int8x8_to_bf16_biased(h.z, h.w) : int8x8_to_bf16_biased(h.x, h.y);
  } else {
    return as_bf16x8(b[s]);
  }
}

// ---------------------------------------------------------------------------
// Decode kernel: few rows per expert (an M-tile of at most 16 routes), so the
// cost is streaming the expert's weights from HBM.  A block of WAVES waves
// owns one M-tile and WAVES * NS consecutive 16-column strips.  Its A rows
// (only the tile's real rows) and their group sums are staged into LDS one
// K-chunk of at most kDecodeChunkK columns at a time (one chunk for K up to
// that size), while every wave already has the chunk's first weight loads in
// flight; after the chunk's barrier each wave streams its strips over the
// chunk with the next D k-groups of weights and scales in flight, reading A
// fragments from LDS (rows beyond the tile's count feed only rows that are
// never stored).  For a gate/up matrix NS = 4 covers 32 gate and the
// matching 32 up columns.
// ---------------------------------------------------------------------------
// s_waitcnt immediate of gfx9: vmcnt(0), expcnt and lgkmcnt left unconstrained
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);
// Rows of an M-tile in the decode kernel: ROWS = 8 (MFMA rows 8..15 are
// copies), 16 (all MFMA rows), 32 or 64 (two or four MFMA row blocks per
// weight load), chosen per forward from the mean rows per expert (plan_gemm).
constexpr int kDecodeTileGroup = 8;   // tiles per column block kept on one XCD (grouped mapping)
// Group sums per k-group in LDS: one per MFMA row (16), or per tile row for
// 32-row tiles (two 16-row MFMA blocks).
__host__ __device__ constexpr int decode_rstride(int rows) { return rows > 16 ? rows : 16; }
// A columns staged per chunk (multiples of kGroup): 4096 for 8-row tiles;
// 1024 for 16-row and 512 for 32-row tiles, so that a chunk stays near 33 KB
// of LDS and four blocks fit a CU; 512 for 64-row tiles (about 67 KB: two
// blocks per CU, as their two waves per SIMD allow)
__host__ __device__ constexpr int decode_chunk_cap(int rows) {
  return rows == 8 ? 4096 : rows == 16 ? 1024 : 512;
}
__host__ __device__ constexpr int decode_chunk_k(int K, int rows) {
  return K < decode_chunk_cap(rows) ? K : decode_chunk_cap(rows);
}

template <int TIER, int NS, int WAVES, bool GATE_UP, bool KSPLIT, int ROWS>
__device__ __forceinline__ void decode_mainloop(const GemmArgs& a, const TileEntry& te,
                                                const uint8_t* blob, int strip0, uint16_t* lds_a,
                                                float* lds_r,
                                                f32x4_t (&acc)[(ROWS > 16 ? ROWS / 16 : 1) * NS]) {
  using TR = TierTraits<TIER>;
  constexpr int RB = ROWS > 16 ? ROWS / 16 : 1;   // 16-row MFMA blocks per tile
  constexpr int RS = decode_rstride(ROWS);
  const Int4Consts c4 = int4_consts();
  constexpr int D = TIER == MOE_TIER_INT4 ? 2 : 1;
  constexpr int L = TR::kLoads;
  const int lane = threadIdx.x & 63;
  const int K = a.K, G = K / kGroup;
  const int KC = decode_chunk_k(K, ROWS), GC = KC / kGroup;
  const int lda = KC + 8;                     // LDS row stride (bf16)
  const int rows = te.rows;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, blob_payload<TIER>(a.N, K));
  // The wave's NS strips are strips u0 .. u0+NS-1 of quad `quad` (NS divides 4).
  const int quad = strip0 >> 2, u0 = strip0 & 3;
  const uint32_t tile_voff = 16 * lane + u0 * TR::kTileBytes;
  const uint32_t scale_voff = 8 * (lane & 15) + 2 * u0;   // fp16 scales of row lane%16, strips u0..

  u32x4 bb[D][NS][L];
  uint2 sc[D];
  auto issue = [&](int g, int d) {
    const uint32_t block = (uint32_t)(quad * G + g) * TR::kBlockBytes;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int q = 0; q < L; ++q)
        bb[d][ns][q] = buffer_load16<true>(rsrc, tile_voff + 1024 * q + ns * TR::kTileBytes, block);
    if constexpr (TIER == MOE_TIER_INT4) {
      if constexpr (NS == 4)
        sc[d] = buffer_load8(rsrc, scale_voff, block + 4096u);
      else if constexpr (NS == 2)
        sc[d] = make_uint2(buffer_load4(rsrc, scale_voff, block + 4096u), 0u);
      else
        sc[d] = make_uint2(buffer_load_u16(rsrc, scale_voff, block + 4096u), 0u);
    }
  };

  float row_scale[NS];
  if constexpr (TIER == MOE_TIER_INT8) {
    const uint2 rs4 = buffer_load8(rsrc, 8 * (lane & 15), (uint32_t)a.N * K + 128u * quad);
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) row_scale[ns] = half_of(rs4, u0 + ns);
  }
  // A fragments: lane l reads LDS row l % ROWS (row 16 rb + l % 16 of MFMA
  // block rb for 32-row tiles).  MFMA rows ROWS..15 (and rows at or beyond
  // the tile's count) then hold copies or stale data; they only feed
  // accumulator rows that the epilogue never stores, so no lane is masked.
  const uint16_t* la = lds_a + (lane & ((ROWS > 16 ? 16 : ROWS) - 1)) * lda + 8 * (lane >> 4);

  // consume(g, d): k-group g (absolute), whose weights are in set d and whose
  // A columns and group sums sit at chunk-relative group g - c0 in LDS
  // 16-row MFMA blocks holding a real row of the tile (the others are skipped:
  // their rows are never stored)
  const int nrb = uniform((rows + 15) >> 4);
  // The tile's A rows: lane m < rows holds row m's first element in a_src
  // (every wave holds the same), for the staging DMAs below.
  int64_t row_elem = 0;
  if (lane < rows) {
    const int pos = te.row_start + lane;
    row_elem = GATE_UP ? (int64_t)(a.sorted[pos] / a.top_k) * K : (int64_t)pos * K;
  }
  int c0 = 0;
  auto consume = [&](int g, int d) {
    const int gl = g - c0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {   // tiles of 32+ rows: every MFMA block takes each weight load
      if (RB > 2 && rb >= nrb) break;
      f32x4_t p[NS];
      if constexpr (TIER == MOE_TIER_BF16) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) p[ns] = acc[rb * NS + ns];
      } else {
        const float4 r4 =
            *reinterpret_cast<const float4*>(lds_r + gl * RS + 16 * rb + 4 * (lane >> 4));
        const f32x4_t init = {-TR::kOffset * r4.x, -TR::kOffset * r4.y, -TR::kOffset * r4.z,
                              -TR::kOffset * r4.w};
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) p[ns] = init;
      }
      bf16x8_t af[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        af[s4] = as_bf16x8(load_u32x4(la + 16 * rb * lda + kGroup * gl + 32 * s4));
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) p[ns] = mfma16x16x32(af[s4], b_operand<TIER>(bb[d][ns], s4, c4), p[ns]);
      if constexpr (TIER == MOE_TIER_BF16) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) acc[rb * NS + ns] = p[ns];
      } else {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          float scf;
          if constexpr (TIER == MOE_TIER_INT4)
            scf = half_of(sc[d], ns);
          else
            scf = row_scale[ns];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[rb * NS + ns][i] = __builtin_fmaf(scf, p[ns][i], acc[rb * NS + ns][i]);
        }
      }
    }
  };

  for (; c0 < G; c0 += GC) {
    int c1 = c0 + GC < G ? c0 + GC : G;   // this chunk: groups [c0, c1)
    const int cs = c0;                    // the chunk's first group (its LDS origin)
    int w0 = c0;                          // this wave's groups of the chunk: [w0, c1)
    if constexpr (KSPLIT) {
      // K split over the block's waves inside every chunk: wave w takes the
      // chunk's groups [n w / WAVES, n (w + 1) / WAVES), n = c1 - c0, so all
      // waves work between any two of the chunk barriers
      const int w = uniform(threadIdx.x >> 6), n = c1 - cs;
      w0 = cs + n * w / WAVES;
      c1 = cs + n * (w + 1) / WAVES;
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (w0 + d < c1) issue(w0 + d, d);
    if (c0 > 0) __syncthreads();   // every wave is done with the previous chunk's A

    // stage this chunk's A columns and group sums (block-wide).  A rows go
    // from memory straight into LDS (buffer_load ... lds): one instruction
    // moves a 1 KB segment of one row (16 bytes per lane, lanes past a ragged
    // segment's end masked off), and a wave issues all of its segments back
    // to back, so the staging costs about one memory round trip.  (A loop of
    // 16-byte loads through registers waited for each load before its LDS
    // store: 16 round trips for a 64-row tile's 512 columns.)
    {
      const int ce = cs + GC < G ? cs + GC : G;
      const int kcb = (ce - cs) * kGroup * 2;             // bytes of one row in this chunk
      const int segs = (kcb + 1023) >> 10;
      typedef __attribute__((address_space(3))) uint8_t lds_b;
      lds_b* lbase = (lds_b*)lds_a;
      for (int t = uniform(threadIdx.x >> 6); t < rows * segs; t += WAVES) {   // wave-uniform
        const int m = t / segs, j = t - m * segs;
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)row_elem, m);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)row_elem >> 32), m);
        const uint16_t* rowp = a.a_src + (int64_t)(((uint64_t)hi << 32) | lo) +
                               (size_t)cs * kGroup + (size_t)j * 512;
        const int left = kcb - j * 1024;                   // >= 256
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(rowp, (uint32_t)(left < 1024 ? left : 1024));
        if (16 * lane < left)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rr, (__attribute__((address_space(3))) void*)(lbase + 2 * (m * lda + j * 512)), 16,
              16 * lane, 0, 0, 0);
      }
      if constexpr (TIER != MOE_TIER_BF16) {
        for (int i = threadIdx.x; i < (ce - cs) * RS; i += 64 * WAVES) {
          const int gl = i / RS, m = i - gl * RS;
          float r = 0.0f;
          if (m < rows) {
            const int pos = te.row_start + m;
            r = GATE_UP ? row_sum<true>(a.rsum + (size_t)(a.sorted[pos] / a.top_k) * G, cs + gl)
                        : row_sum<false>(a.rsum + (size_t)pos * (K / 32), cs + gl);
          }
          lds_r[i] = r;
        }
      }
    }
    // Drain every load before the barrier.  The staging loops above are
    // skipped by waves without work; on that path the first weight loads
    // would still be pending at the main loop, and the compiler's merged wait
    // state then drains all loads at the top of every iteration instead of
    // only the oldest group.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // Steady state: every group consumed here has a successor D groups ahead
    // in the chunk, so the body is branch-free and each register set bb[d]
    // keeps its role (no copies between loads in flight, which would force
    // early waits).
    int g0 = w0;
#pragma nounroll
    for (; g0 + 2 * D <= c1; g0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        consume(g0 + d, d);
        issue(g0 + d + D, d);
        // keep the next group's math after this reload: otherwise the
        // scheduler batches the math of all D groups ahead of every reload
        // and the wave computes with no weight loads in flight
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the chunk's last (fewer than 2D) groups
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (g0 + d < c1) {
        consume(g0 + d, d);
        if (g0 + d + D < c1) issue(g0 + d + D, d);
      }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (g0 + D + d < c1) consume(g0 + D + d, d);
  }
}

// Occupancy: three waves per SIMD for gate/up (K = H, long weight streams);
// four for down, whose short K (I) makes more, shorter waves, all of which
// then fit in one round at the decode workloads.  32-row tiles hold two
// accumulator blocks per strip: two waves per SIMD.
// KSPLIT (few tiles, so few waves for the GPU): the block's waves share its
// NS strips and split every staged K-chunk; their partial sums meet in LDS,
// added in wave order, and wave 0 runs the epilogue.
template <int NS, int WAVES, bool GATE_UP, bool KSPLIT, int ROWS>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(
    ROWS > 16 ? 2 : (GATE_UP ? 3 : 4), ROWS > 16 ? 2 : (GATE_UP ? 3 : 4))))
void gemm_decode_kernel(GemmArgs a, int blocks_per_tile) {
  static_assert(!GATE_UP || NS == 4, "a gate/up wave covers 32 gate + 32 up columns");
  static_assert(NS == 1 || NS == 2 || NS == 4, "a wave's strips lie in one quad");
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  int tile_idx, nb;
  // ntiles[0]: tile count; ntiles[1]: the grouping kernel found an expert
  // spanning three or more tiles.  One 8-byte scalar load.
  const int2 nt2 = *reinterpret_cast<const int2*>(a.ntiles);
  const int ntiles = uniform(nt2.x);
  if (a.tile_group && uniform(nt2.y) != 0) {
    // The hardware deals blocks to the 8 XCDs round robin.  The j-th block
    // an XCD receives is made logical block L = (j / Q) 8Q + xcd Q + j % Q
    // (a bijection on the grid, a multiple of 8Q blocks), and L covers
    // column block nb = (L % (bpt Q)) / Q of tile (L / (bpt Q)) Q + L % Q:
    // Q consecutive tiles with the same columns run back to back on one
    // XCD, so the sub-tiles of an expert with many routes read its weights
    // through one L2.
    constexpr int Q = kDecodeTileGroup;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int L = (j / Q) * 8 * Q + x * Q + j % Q;
    const int span = blocks_per_tile * Q, g = L / span, rem = L - g * span;
    nb = rem / Q;
    tile_idx = g * Q + (rem - nb * Q);
  } else {
    tile_idx = blockIdx.x / blocks_per_tile;
    nb = blockIdx.x - tile_idx * blocks_per_tile;
  }
  if (tile_idx >= ntiles) return;
  TileEntry te = a.tiles[tile_idx];
  te.expert = uniform(te.expert);
  te.row_start = uniform(te.row_start);
  te.rows = uniform(te.rows);
  te.tier = uniform(te.tier);
  te.w = uniform_ptr(te.w);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int chunk = KSPLIT ? nb : nb * WAVES + wave;   // this wave's group of NS strips
  const int strip0 = chunk * NS;
  uint16_t* lds_a = reinterpret_cast<uint16_t*>(dyn_lds);
  static_assert(ROWS == 8 || ROWS == 16 || ROWS == 32 || ROWS == 64,
                "an M-tile is 8, 16, 32 or 64 rows");
  constexpr int RB = ROWS > 16 ? ROWS / 16 : 1;   // 16-row MFMA blocks per tile
  float* lds_r = reinterpret_cast<float*>(dyn_lds + (size_t)ROWS * (decode_chunk_k(a.K, ROWS) + 8) * 2);

  f32x4_t acc[RB * NS];
#pragma unroll
  for (int q = 0; q < RB * NS; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* blob = te.w;
  switch (te.tier) {
    case MOE_TIER_INT4:
      decode_mainloop<MOE_TIER_INT4, NS, WAVES, GATE_UP, KSPLIT, ROWS>(a, te, blob, strip0, lds_a, lds_r, acc);
      break;
    case MOE_TIER_INT8:
      decode_mainloop<MOE_TIER_INT8, NS, WAVES, GATE_UP, KSPLIT, ROWS>(a, te, blob, strip0, lds_a, lds_r, acc);
      break;
    default:
      decode_mainloop<MOE_TIER_BF16, NS, WAVES, GATE_UP, KSPLIT, ROWS>(a, te, blob, strip0, lds_a, lds_r, acc);
      break;
  }
  if constexpr (KSPLIT) {
    static_assert(WAVES >= 2, "a split needs several waves");
    float* red = reinterpret_cast<float*>(dyn_lds);   // [WAVES - 1][RB * NS * 4][64]
    __syncthreads();                                  // every wave is done with A in LDS
    if (wave > 0) {
#pragma unroll
      for (int q = 0; q < RB * NS; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave - 1) * RB * NS * 4 + q * 4 + i) * 64 + lane] = acc[q][i];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 1; w < WAVES; ++w)
#pragma unroll
      for (int q = 0; q < RB * NS; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[q][i] += red[((w - 1) * RB * NS * 4 + q * 4 + i) * 64 + lane];
  }

  if constexpr (GATE_UP) {
    // SwiGLU on strips (0,2) and (1,3): gate and up of 32 activation columns
    const int P = a.I / 32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int icol = 32 * chunk + 16 * half + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * rb + 4 * (lane >> 4) + i;
          const uint32_t a16 =
              f32_to_bf16_rne(silu_f32(acc[rb * NS + half][i]) * acc[rb * NS + half + 2][i]);
          if (m < te.rows) {
            a.act[(size_t)(te.row_start + m) * a.I + icol] = (uint16_t)a16;
            rs[i] += bf16_to_f32(a16);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = rs[i];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 16);
        const int m = 16 * rb + 4 * (lane >> 4) + i;
        if ((lane & 15) == 0 && m < te.rows) a.r2[(size_t)(te.row_start + m) * P + chunk] = v;
      }
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * rb + 4 * (lane >> 4) + i;
        if (m < te.rows) {
          const int r = a.sorted[te.row_start + m];   // route id t k + j: rows are in route order
          const float wgt = a.topk_w[r];
          float* out = a.rows + (size_t)r * a.N + 16 * strip0 + (lane & 15);
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) out[16 * ns] = wgt * acc[rb * NS + ns][i];
        }
      }
  }
}

size_t decode_lds_bytes(int K, int rows, int NS, int WAVES, bool ksplit) {
  const int KC = decode_chunk_k(K, rows);
  const size_t stage = (size_t)rows * (KC + 8) * 2 + (size_t)(KC / kGroup) * decode_rstride(rows) * 4;
  const int rb = rows > 16 ? rows / 16 : 1;
  const size_t red = ksplit ? (size_t)(WAVES - 1) * rb * NS * 4 * 64 * 4 : 0;
  return stage > red ? stage : red;
}

// Below this many waves (one per 64 output columns of every tile, tiles
// estimated as min(E, T k)) the decode GEMMs split K over a block's waves.
constexpr int kDecodeSplitWaves = 1024;

template <int NS, bool GATE_UP>
hipError_t launch_decode(GemmArgs a, int max_tiles, int rows, bool ksplit, hipStream_t s,
                         KernelTimer kt) {
  // When an expert spans several tiles (a skewed router), group tiles by
  // XCD (8 consecutive tiles per column block).  Without such experts the
  // grouping only reshuffled the column blocks: 6.5% slower on the Mixtral
  // shape at 16 routes per expert.
  a.tile_group = 1;
  constexpr int W = 4;
  const int chunks = a.N / 16 / NS;   // groups of NS strips; N is a multiple of 256
  const size_t lds = decode_lds_bytes(a.K, rows, NS, W, ksplit);
  auto run = [&](auto split_c, auto rows_c) -> hipError_t {
    constexpr bool KS = decltype(split_c)::value;
    constexpr int RW = decltype(rows_c)::value;
    auto kern = gemm_decode_kernel<NS, W, GATE_UP, KS, RW>;
    static DeviceOnce lds_opt_in;   // one per instantiation
    const hipError_t ea = ensure_dynamic_lds(lds_opt_in, reinterpret_cast<const void*>(kern), 160 * 1024);
    if (ea != hipSuccess) return ea;
    const int bpt = KS ? chunks : chunks / W;
    unsigned blocks = (unsigned)(max_tiles * bpt);
    if (a.tile_group) {   // whole groups of Q tiles, then whole rounds of 8 groups
      const unsigned Q = (unsigned)kDecodeTileGroup;
      blocks = (unsigned)((max_tiles + Q - 1) / Q * Q * bpt);
      blocks = (blocks + 8 * Q - 1) / (8 * Q) * (8 * Q);
    }
    if (kt.start || kt.stop)
      hipExtLaunchKernelGGL(kern, dim3(blocks), dim3(64 * W), (uint32_t)lds, s, kt.start,
                            kt.stop, 0, a, bpt);
    else
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * W), lds, s, a, bpt);
    return hipGetLastError();
  };
  using R8 = std::integral_constant<int, 8>;
  using R16 = std::integral_constant<int, 16>;
  using R32 = std::integral_constant<int, 32>;
  using R64 = std::integral_constant<int, 64>;
  if (rows == 8) return ksplit ? run(std::true_type{}, R8{}) : run(std::false_type{}, R8{});
  if (rows == 16) return ksplit ? run(std::true_type{}, R16{}) : run(std::false_type{}, R16{});
  if (rows == 32) return ksplit ? run(std::true_type{}, R32{}) : run(std::false_type{}, R32{});
  // 64-row tiles serve forwards with tens of routes per expert: many tiles,
  // never split K.  (128-row tiles would need 128 accumulators per lane next
  // to the weights in flight and spill.)
  if (ksplit) return hipErrorInvalidValue;
  if (rows == 64) return run(std::false_type{}, R64{});
  return hipErrorInvalidValue;
}

// Decode tiles a forward is expected to have: one per touched expert, at
// most min(E, T k) (the launch heuristics below; the grid uses the bound).
long est_decode_tiles(const Layer& L, int T) { return std::min<long>(L.E, (long)T * L.k); }

bool decode_split_k(const Layer& L, int T, int N) {
  return est_decode_tiles(L, T) * (N / 64) < kDecodeSplitWaves;
}


// Sum of a token's k weighted rows in ascending expert order, fp32.  The down
// GEMMs write the rows by route id (t k + j), so a token's k rows are
// contiguous and slot j is expert ids[t k + j] (ids ascending).  With a slot
// map (wave mode) routes of experts mapped to the sentinel are skipped, and
// with ACC the sum is added to y (fp32 only).  KMAX >= k is the compile-time
// bound of the route loops: every row load is issued before the first add
// (loads past k repeat route k-1's row and are not added).
template <bool BF16_OUT, bool ACC, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ rows,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ slot_map, int T,
                                                      int H, int k, void* __restrict__ y) {
  const int t = blockIdx.y;
  const int h4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  uint64_t keep = ~0ull;
  if (slot_map) {   // wave mode: lane j tests route j's expert, one ballot
    const int jl = min((int)(threadIdx.x & 63), k - 1);
    keep = __ballot(slot_map[ids[t * k + jl]] >= 0);
  }
  if (h4 >= H) return;   // after the wave-wide loads above
  const float* rt = rows + (size_t)t * k * H + h4;
  float4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    v[j] = *reinterpret_cast<const float4*>(rt + (size_t)min(j, k - 1) * H);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool use = j < k && ((keep >> j) & 1ull);
    s.x = use ? s.x + v[j].x : s.x;
    s.y = use ? s.y + v[j].y : s.y;
    s.z = use ? s.z + v[j].z : s.z;
    s.w = use ? s.w + v[j].w : s.w;
  }
  if constexpr (BF16_OUT) {
    const uint32_t lo = f32_to_bf16_rne(s.x) | (f32_to_bf16_rne(s.y) << 16);
    const uint32_t hi = f32_to_bf16_rne(s.z) | (f32_to_bf16_rne(s.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * H + h4) = make_uint2(lo, hi);
  } else {
    float4* yp = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * H + h4);
    if constexpr (ACC) {
      const float4 o = *yp;
      s = make_float4(o.x + s.x, o.y + s.y, o.z + s.z, o.w + s.w);
    }
    *yp = s;
  }
}

}  // namespace

constexpr double kDecodeRows8Max = 4.0;    // mean routes per expert up to which tiles are 8 rows
constexpr double kDecodeRows16Max = 12.0;  // ... 16 rows
// Layers whose decode launches have at least kManyDecodeWaves waves (one per
// 64 output columns of one tile per touched expert, the narrower GEMM): 64-row
// tiles up to kDecodeRows64Max, then (I <= 512) the mixed plan up to
// kMixedRowsMax, then the large-batch kernel for both GEMMs.  Layers with
// fewer (few experts, as the Mixtral shape): 32-row tiles up to
// kFewWavesRows32Max, then the large-batch kernel.
constexpr long kManyDecodeWaves = 2048;
constexpr double kDecodeRows64Max = 60.0;
constexpr double kMixedRowsMax = 128.0;
constexpr double kFewWavesRows32Max = 28.0;

GemmPlan plan_gemm(const Layer& L, int T) {
  GemmPlan p;
  const double rows = (double)T * L.k / L.E;
  // The boundaries come from per-GEMM sweeps on one MI355X (gate/up + down
  // kernel times in us at the mean routes per expert given):
  //   * 8- and 16-row tiles for few routes: the Qwen3-30B shape at 2 routes
  //     53.6 (8 rows) against 70.2 (64 rows), the Qwen3-80B shape at 5 and
  //     10 routes 171 and 189 (16 rows) against 206 and 218 (64 rows);
  //   * 64-row decode tiles (row-skipping, so an expert of up to 64 routes
  //     streams its weights once) from 12 routes on layers with many waves:
  //     Qwen3-80B at 15, 40, 50 routes 222, 322, 376 against 235 (16 rows),
  //     490 and 514 (large batch); OLMoE at 24 and 48 62 and 86 against 71
  //     (16 rows) and 98 (large batch);
  //   * past 60 routes the large-batch gate/up GEMM wins there while the
  //     decode down GEMM keeps winning on short I: Qwen3-80B (I = 512) at 70
  //     and 80 routes 514 and 546 (mixed) against 568 and 622 (64 rows) and
  //     609 and 647 (large batch); OLMoE (I = 1024) at 64 routes 110 either
  //     way, 122 with 64-row tiles;
  //   * with few waves (Mixtral shape: 8 experts, 64 down-GEMM column strips
  //     each) 64-row tiles leave the GPU mostly idle: 32-row tiles up to 28
  //     routes (24 and 28 routes: 196 and 198 against 253 and 249 large
  //     batch), the large-batch kernel above (32 and 40 routes: 269 and 285
  //     against 298 and 383).
  const long tiles = est_decode_tiles(L, T);
  const bool many_waves = tiles * (std::min(2 * L.I, L.H) / 64) >= kManyDecodeWaves;
  int bm13 = 256, bm2 = 256;
  bool dec13 = false, dec2 = false;
  if (rows <= kDecodeRows8Max) {
    bm13 = bm2 = 8;
    dec13 = dec2 = true;
  } else if (rows <= kDecodeRows16Max) {
    bm13 = bm2 = 16;
    dec13 = dec2 = true;
  } else if (many_waves) {
    if (rows <= kDecodeRows64Max) {
      bm13 = bm2 = 64;
      dec13 = dec2 = true;
    } else if (L.I <= 512 && rows <= kMixedRowsMax) {
      bm2 = 64;
      dec2 = true;
    }
  } else if (rows <= kFewWavesRows32Max) {
    // not with the few tiles of a split-K launch (the tiny layer: 12% slower)
    bm13 = bm2 = decode_split_k(L, T, 2 * L.I) ? 16 : 32;
    dec13 = dec2 = true;
  }
  p.bm13 = bm13;
  p.bm2 = bm2;
  p.kind = dec13 ? kGemmDecode : kGemmPrefill;
  p.kind2 = dec2 ? kGemmDecode : kGemmPrefill;
  return p;
}

hipError_t launch_gemm13(const Layer& L, const GemmPlan& gp, int T, const uint16_t* x,
                         const int32_t* sorted, const TileEntry* tiles, const int32_t* ntiles,
                         int max_tiles, const float* r13, uint16_t* act, float* r2,
                         hipStream_t s, KernelTimer kt) {
  GemmArgs a{};
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
  if (gp.kind != kGemmDecode) return hipErrorInvalidValue;
  return launch_decode<4, true>(a, max_tiles, gp.bm13, gp.bm13 < 64 && decode_split_k(L, T, a.N), s,
                                kt);
}

hipError_t launch_gemm2(const Layer& L, const GemmPlan& gp, int T, const uint16_t* act,
                        const int32_t* sorted, const float* topk_w, const TileEntry* tiles,
                        const int32_t* ntiles, int max_tiles, const float* r2, float* rows,
                        hipStream_t s) {
  GemmArgs a{};
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
  if (gp.kind2 != kGemmDecode) return hipErrorInvalidValue;
  const bool ks = gp.bm2 < 64 && decode_split_k(L, T, a.N);
  // Very few column blocks even with split K (a wide-K, narrow-N down GEMM
  // over one or two tiles, e.g. the Mixtral shape at one token): two strips
  // per wave double the blocks.  Mixtral T = 1: 64.9 -> 61.3 us per layer;
  // at 1280 or more waves it gained nothing, and at T = 4 it lost 7%.
  if (ks && est_decode_tiles(L, T) * (a.N / 64) * 4 < kDecodeSplitWaves)
    return launch_decode<2, false>(a, max_tiles, gp.bm2, ks, s, KernelTimer{nullptr, nullptr});
  return launch_decode<4, false>(a, max_tiles, gp.bm2, ks, s, KernelTimer{nullptr, nullptr});
}

hipError_t launch_combine(const float* rows, const int32_t* ids, const int32_t* slot_map, int T,
                          int H, int k, void* y, int y_dtype, bool accumulate, hipStream_t s) {
  const dim3 grid((H / 4 + 255) / 256, T);
  auto run = [&](auto kmax) {
    constexpr int KM = decltype(kmax)::value;
    if (y_dtype == MOE_DTYPE_BF16)
      hipLaunchKernelGGL((combine_kernel<true, false, KM>), grid, dim3(256), 0, s, rows, ids,
                         slot_map, T, H, k, y);
    else if (accumulate)
      hipLaunchKernelGGL((combine_kernel<false, true, KM>), grid, dim3(256), 0, s, rows, ids,
                         slot_map, T, H, k, y);
    else
      hipLaunchKernelGGL((combine_kernel<false, false, KM>), grid, dim3(256), 0, s, rows, ids,
                         slot_map, T, H, k, y);
    return hipGetLastError();
  };
  static_assert(kMaxTopK <= 16, "combine buckets");
  if (k <= 2) return run(std::integral_constant<int, 2>{});
  if (k <= 4) return run(std::integral_constant<int, 4>{});
  if (k <= 8) return run(std::integral_constant<int, 8>{});
  return run(std::integral_constant<int, 16>{});
}

}  // namespace moe
