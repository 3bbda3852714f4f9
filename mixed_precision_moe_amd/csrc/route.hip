// route.hip -- router logits, top-k + softmax weights, and grouping by expert.
//
// "Every Expert Counts: ExactMoE ..." §3.1: z = W_r h, S = TopK(z, k), the
// router kept in BF16 and unchanged; §3.4 and Fig. 1: tokens are grouped by
// selected expert before the grouped GEMMs.
//
// Logits are fp32 in one fixed order so that the top-k choice is reproducible
// bit for bit: 32 chains per dot product, chain j summing x[h]*w[h] for
// h = 256i + 8j + r (slab i outer, r = 0..7 inner) from +0, then the chains
// folded pairwise (chain j += chain j+s for s = 16, 8, 4, 2, 1), then + bias.
// Every bf16 x bf16 product is exact in fp32, so fma and mul-then-add agree.
// On the GPU one chain is one lane of a half-wave: lane j reads the 16-byte
// chunk at 256i + 8j, so a half-wave reads each 512-byte slab coalesced, and the
// fold is a shuffle tree.
#include "device_util.h"
#include "moe_internal.h"
#include "topk_select.h"

namespace moe {
namespace {

// Sum of the 128 activations of one k-group: each of 16 lanes adds its 8
// values pairwise, then a shuffle tree over the 16 lanes.  Every routing path
// uses this one order, so the group sums agree bit for bit between them.
__device__ __forceinline__ float group_sum_16lanes(const u32x4 q) {
  float v = (bf16lo_to_f32(q.x) + bf16hi_to_f32(q.x)) + (bf16lo_to_f32(q.y) + bf16hi_to_f32(q.y)) +
            (bf16lo_to_f32(q.z) + bf16hi_to_f32(q.z)) + (bf16lo_to_f32(q.w) + bf16hi_to_f32(q.w));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 16);
  return v;
}

// Block: 8 half-waves (256 threads) arranged 2 (token groups) x 4 (expert
// groups).  Each half-wave owns TT tokens x TE experts; block tile is
// (2*TT) tokens x (4*TE) experts.  The slab loop takes SG slabs per step.
template <int TT, int TE, int SG>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            int T, int H, int E,
                                                            float* __restrict__ logits,
                                                            float* __restrict__ r13) {
  const int j = threadIdx.x & 31;           // chain index
  const int hw = threadIdx.x >> 5;          // half-wave 0..7
  const int t0 = blockIdx.x * (2 * TT) + (hw >> 2) * TT;
  const int e0 = blockIdx.y * (4 * TE) + (hw & 3) * TE;
  const uint16_t* xp[TT];
  const uint16_t* wp[TE];
#pragma unroll
  for (int a = 0; a < TT; ++a) xp[a] = x + (size_t)min(t0 + a, T - 1) * H + 8 * j;
#pragma unroll
  for (int b = 0; b < TE; ++b) wp[b] = wr + (size_t)min(e0 + b, E - 1) * H + 8 * j;
  float acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[a][b] = 0.0f;

  // Half-waves of expert group 0 also produce R13[t][g] = sum of the 128
  // activations of group g (used by the GEMMs to remove their weight offset).
  const bool do_r13 = r13 != nullptr && blockIdx.y == 0 && (hw & 3) == 0;
  const int G = H / kGroup;
  // SG slabs per step, all their loads issued before the step's FMAs
  for (int base0 = 0; base0 < H; base0 += 256 * SG) {
    u32x4 xv[SG][TT], wv[SG][TE];
#pragma unroll
    for (int sg = 0; sg < SG; ++sg) {
      const int base = base0 + 256 * sg;
#pragma unroll
      for (int a = 0; a < TT; ++a) xv[sg][a] = base < H ? load_u32x4(xp[a] + base) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < TE; ++b) wv[sg][b] = base < H ? load_u32x4(wp[b] + base) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int sg = 0; sg < SG; ++sg) {
      const int base = base0 + 256 * sg;
      if (base >= H) break;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float xf[TT], wf[TE];
#pragma unroll
        for (int a = 0; a < TT; ++a) {
          const uint32_t d = (&xv[sg][a].x)[r >> 1];
          xf[a] = (r & 1) ? bf16hi_to_f32(d) : bf16lo_to_f32(d);
        }
#pragma unroll
        for (int b = 0; b < TE; ++b) {
          const uint32_t d = (&wv[sg][b].x)[r >> 1];
          wf[b] = (r & 1) ? bf16hi_to_f32(d) : bf16lo_to_f32(d);
        }
#pragma unroll
        for (int a = 0; a < TT; ++a)
#pragma unroll
          for (int b = 0; b < TE; ++b) acc[a][b] = __builtin_fmaf(xf[a], wf[b], acc[a][b]);
      }
      if (do_r13) {
#pragma unroll
        for (int a = 0; a < TT; ++a) {
          const float v = group_sum_16lanes(xv[sg][a]);
          const int t = t0 + a;
          if ((j & 15) == 0 && t < T) r13[(size_t)t * G + base / kGroup + (j >> 4)] = v;
        }
      }
    }
  }
  // fold the 32 chains: chain j += chain j+s, s = 16 .. 1
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) {
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b) {
        const float other = __shfl_down(acc[a][b], s, 32);
        acc[a][b] = acc[a][b] + other;
      }
  }
  if (j == 0) {
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b) {
        const int t = t0 + a, e = e0 + b;
        if (t < T && e < E) {
          const float bb = bias ? bias[e] : 0.0f;
          logits[(size_t)t * E + e] = acc[a][b] + bb;
        }
      }
  }
}

// One wave per token: the k largest logits (ties -> lower id) and their
// softmax weights, stored with ids ascending (topk_select.h).  Lane l holds
// experts l, l+64, ...
constexpr int kMaxPerLane = kMaxExperts / 64;

// PER (a power of two, PER * 64 >= E) is the compile-time bound of the
// lane-local loops, so small E does not pay for the largest.
template <int PER>
__global__ __launch_bounds__(64) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                  int k, int32_t* __restrict__ ids,
                                                  float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  if (t >= T) return;
  const float* z = logits + (size_t)t * E;
  float v[PER];
  int id[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {   // clamped loads: all issued back to back, no branches
    const int e = lane + 64 * m;
    const bool ok = e < E;
    const float ze = z[ok ? e : E - 1];
    v[m] = ok ? ze : -INFINITY;
    id[m] = ok ? e : kNoExpert;
  }
  topk_select_softmax<PER>(v, id, k, ids + (size_t)t * k, weights + (size_t)t * k);
}

// Few tokens: one block per token computes the token's E logits in the
// canonical order (the chains and fold of router_logits_kernel), keeps them in
// LDS, and its first wave selects the top k as topk_kernel does.  One launch
// and no logits round trip through memory.  The token's activation row is
// staged in LDS once; half-wave hw (of 32) owns experts hw + 32 b, b < TE,
// with SG slabs of weight loads issued per step.
constexpr int kSmallRouteMaxH = 8192;
template <int PER, int TE, int SG>
__global__ __launch_bounds__(1024) void router_topk_small_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    int H, int E, int k, float* __restrict__ r13, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kSmallRouteMaxH];
  __shared__ float zs[64 * PER];
  const int t = blockIdx.x;
  const int j = threadIdx.x & 31, hw = threadIdx.x >> 5;
  const uint16_t* xrow = x + (size_t)t * H;
  for (int c = threadIdx.x; c < H / 8; c += 1024)
    *reinterpret_cast<u32x4*>(xs + 8 * c) = load_u32x4(xrow + 8 * c);
  __syncthreads();

  if (hw < E) {   // half-waves with no expert skip the dot products
    const uint16_t* wp[TE];
#pragma unroll
    for (int b = 0; b < TE; ++b) wp[b] = wr + (size_t)min(hw + 32 * b, E - 1) * H + 8 * j;
    float acc[TE];
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[b] = 0.0f;
    const bool do_r13 = r13 != nullptr && hw == 0;
    const int G = H / kGroup;
    for (int base0 = 0; base0 < H; base0 += 256 * SG) {
      u32x4 xv[SG], wv[SG][TE];
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const int base = base0 + 256 * sg;
#pragma unroll
        for (int b = 0; b < TE; ++b) wv[sg][b] = base < H ? load_u32x4(wp[b] + base) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const int base = base0 + 256 * sg;
        xv[sg] = base < H ? *reinterpret_cast<const u32x4*>(xs + base + 8 * j) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const int base = base0 + 256 * sg;
        if (base >= H) break;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint32_t dx = (&xv[sg].x)[r >> 1];
          const float xf = (r & 1) ? bf16hi_to_f32(dx) : bf16lo_to_f32(dx);
#pragma unroll
          for (int b = 0; b < TE; ++b) {
            const uint32_t d = (&wv[sg][b].x)[r >> 1];
            const float wf = (r & 1) ? bf16hi_to_f32(d) : bf16lo_to_f32(d);
            acc[b] = __builtin_fmaf(xf, wf, acc[b]);
          }
        }
        if (do_r13) {
          const float v = group_sum_16lanes(xv[sg]);
          if ((j & 15) == 0) r13[(size_t)t * G + base / kGroup + (j >> 4)] = v;
        }
      }
    }
#pragma unroll
    for (int sh = 16; sh >= 1; sh >>= 1)
#pragma unroll
      for (int b = 0; b < TE; ++b) acc[b] = acc[b] + __shfl_down(acc[b], sh, 32);
    if (j == 0) {
#pragma unroll
      for (int b = 0; b < TE; ++b) {
        const int e = hw + 32 * b;
        if (e < E) zs[e] = acc[b] + (bias ? bias[e] : 0.0f);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float v[PER];
    int id[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = lane + 64 * m;
      v[m] = e < E ? zs[e] : -INFINITY;
      id[m] = e < E ? e : kNoExpert;
    }
    topk_select_softmax<PER>(v, id, k, ids + (size_t)t * k, weights + (size_t)t * k);
  }
}

// The decode GEMMs' group sums R13 [T, H/128] alone, for forwards whose
// routing runs on the MFMA router: 16 consecutive threads hold one group,
// summed in the same order as router_logits_kernel (bit-identical sums).
// n8 is a multiple of 16, so the threads past the end leave in whole groups.
__global__ __launch_bounds__(256) void group_sums_kernel(const uint16_t* __restrict__ x,
                                                         float* __restrict__ r13, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float g = group_sum_16lanes(load_u32x4(x + 8 * i));
  if ((i & 15) == 0) r13[i / 16] = g;
}

// Exclusive prefix sum over the 1024 threads of a block; also returns the total.
// Wave-level inclusive scan with shuffles, then one pass over the 16 wave totals.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();   // wave_tot may be reused by the caller's next scan
  total = tot;
  return base + inc - v;
}

// M-tile tables (1024 threads, expert e = thread e; off[] in LDS): expert e
// with c_e routes gets ceil(c_e / bm) tiles of each grouped GEMM, each entry
// carrying the expert's tier and packed weights from the handle table (or, in
// wave mode, from its resident slot).
// The handle of expert e = thread e (and whether wave mode gives it a slot):
// independent of the grouping, so callers load it first and its latency
// overlaps the counting.
struct TileSource {
  DevHandle h;
  bool active;
};
__device__ __forceinline__ TileSource tile_source(const DevHandle* table, WaveMap wave, int E) {
  const int e = min((int)threadIdx.x, E - 1);
  // wave mode: only experts mapped to a resident slot get tiles, with the
  // slot's weights (ExactMoE 3.4: the other experts map to the sentinel)
  const int slot = wave.slot_map ? wave.slot_map[e] : 0;
  const bool active = !wave.slot_map || (slot >= 0 && slot < E);
  return TileSource{wave.slot_map ? wave.slots[active ? slot : 0] : table[e], active};
}

// Tile tables of bm >= kSortTilesMinBm rows are ordered by cost, since the
// GEMMs process tiles in table order and the cheapest should fill the GPU's
// last round.  Large-batch tables (256 rows) list every expert's full tiles
// first (expert order), then the partial tiles by row count, descending
// (row-aware partial tiles are cheaper); 64-row decode tables put the bf16
// tiles before the others, each part in that same order (see place_tiles).
// The orders come from counting sorts (LDS histogram, block scan, atomic
// placement); tiles with equal keys may land in either order, which changes
// no result (every tile writes only its own rows).  hist[] is LDS scratch of
// kMaxTileRows ints.
constexpr int kSortTilesMinBm = 64;
constexpr int kMaxTileRows = 256;

// The M-tiles of bm rows of every expert, written to tiles13 (with the
// gate/up weights) and/or tiles2 (with the down weights), whichever is
// non-null: both when the two GEMMs share one M-tiling.
__device__ __forceinline__ void place_tiles(const TileSource& src, const int* off, int E,
                                            TileEntry* tiles13, int32_t* ntiles13,
                                            TileEntry* tiles2, int32_t* ntiles2, int bm,
                                            int* scan, int* hist) {
  const int tid = threadIdx.x;
  const DevHandle& h = src.h;
  const bool active = src.active;
  const int ce = tid < E && active ? off[tid + 1] - off[tid] : 0;
  auto put = [&](int at, int i, int rows) {
    TileEntry te2;
    te2.expert = tid;
    te2.row_start = off[tid] + i * bm;
    te2.rows = rows;
    te2.tier = h.tier;
    te2.pad = 0;
    if (tiles13) {
      te2.w = h.w13;
      tiles13[at] = te2;
    }
    if (tiles2) {
      te2.w = h.w2;
      tiles2[at] = te2;
    }
  };
  int count = 0, many = 0;
  if (bm < kSortTilesMinBm || bm > kMaxTileRows) {   // block-uniform
    const int nt = (ce + bm - 1) / bm;
    // one scan gives each expert's first tile (low 20 bits; a decode table
    // holds far fewer than 2^20 tiles) and the number of experts spanning
    // three or more tiles (high bits)
    int tot = 0;
    const int first = block_exclusive_scan(nt | (nt >= 3 ? 1 << 20 : 0), scan, tot) & 0xfffff;
    for (int i = 0; i < nt; ++i) put(first + i, i, min(bm, ce - i * bm));
    count = tot & 0xfffff;
    many = (tot >> 20) > 0 ? 1 : 0;
  } else if (2 * bm <= kMaxTileRows) {
    // 64-row decode tiles: a bf16 tile streams four times the weight bytes of
    // an int4 one whatever its rows, so bf16 tiles come first (full, then
    // partial by rows descending), then the other tiers' tiles in the same
    // order: the costliest tiles start in the first round (Zipf-biased
    // mixed-tier layer, T = 256: 146.5 -> 135.1 us per layer; putting int8
    // before int4 as well cost the Qwen3-80B T = 4096 down GEMM 4%).  A
    // counting sort over 2 bm keys; an expert's full tiles stay consecutive,
    // and tiles with equal keys may land in either order (every tile writes
    // only its own rows).
    const int nfull = ce / bm, rem = ce - nfull * bm;
    const int cls = h.tier == MOE_TIER_BF16 ? 0 : 1;
    const int kfull = cls * bm, kpart = cls * bm + bm - rem;   // rem in 1..bm-1
    const int nk = 2 * bm;
    for (int i = tid; i < nk; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    if (nfull > 0) atomicAdd(&hist[kfull], nfull);
    if (rem > 0) atomicAdd(&hist[kpart], 1);
    __syncthreads();
    const int cnt = tid < nk ? hist[tid] : 0;
    int tot = 0;
    const int base = block_exclusive_scan(cnt, scan, tot);   // its barriers order the read above
    if (tid < nk) hist[tid] = base;
    __syncthreads();
    if (nfull > 0) {
      const int at = atomicAdd(&hist[kfull], nfull);
      for (int i = 0; i < nfull; ++i) put(at + i, i, bm);
    }
    if (rem > 0) put(atomicAdd(&hist[kpart], 1), nfull, rem);
    count = tot;
    // an expert spanning six or more 64-row tiles (most of a group of
    // kDecodeTileGroup = 8) turns on the decode GEMMs' XCD grouping of
    // consecutive tiles; an expert's full tiles are consecutive here
    many = __syncthreads_or(nfull + (rem > 0 ? 1 : 0) >= 6) ? 1 : 0;
  } else {
    const int nfull = ce / bm, rem = ce - nfull * bm;
    int nf = 0;
    const int first = block_exclusive_scan(nfull, scan, nf);
    for (int i = 0; i < nfull; ++i) put(first + i, i, bm);
    const int key = bm - 1 - rem;                       // more rows first
    if (tid < bm) hist[tid] = 0;
    __syncthreads();
    if (rem > 0) atomicAdd(&hist[key], 1);
    __syncthreads();
    const int cnt = tid < bm ? hist[tid] : 0;
    int np = 0;
    const int base = block_exclusive_scan(cnt, scan, np);   // its barriers order the read above
    if (tid < bm) hist[tid] = base;
    __syncthreads();
    if (rem > 0) put(nf + atomicAdd(&hist[key], 1), nfull, rem);
    count = nf + np;
  }
  // ntiles[1]: some expert spans three or more decode tiles (the decode
  // GEMMs then keep an expert's sub-tiles on one XCD)
  if (tid == 0) {
    if (ntiles13) {
      ntiles13[0] = count;
      ntiles13[1] = many;
    }
    if (ntiles2) {
      ntiles2[0] = count;
      ntiles2[1] = many;
    }
  }
}

__device__ __forceinline__ void write_tile_tables(const TileSource& src, Hotness hotness,
                                                  const int* off, int E,
                                                  TileEntry* tiles13, int32_t* ntiles13, int bm13,
                                                  TileEntry* tiles2, int32_t* ntiles2, int bm2,
                                                  int* scan, int* hist) {
  const int tid = threadIdx.x;
  // DynaExq hotness from the router trace: decayed count of routes per expert
  if (hotness.hot && tid < E)
    hotness.hot[tid] = hotness.decay * hotness.hot[tid] + (float)(off[tid + 1] - off[tid]);
  if (bm13 == bm2) {   // one pass places every tile in both tables
    place_tiles(src, off, E, tiles13, ntiles13, tiles2, ntiles2, bm13, scan, hist);
  } else {
    place_tiles(src, off, E, tiles13, ntiles13, nullptr, nullptr, bm13, scan, hist);
    __syncthreads();   // scan and hist serve the second table
    place_tiles(src, off, E, nullptr, nullptr, tiles2, ntiles2, bm2, scan, hist);
  }
}

// Grouping by expert in one workgroup of 1024 threads (16 waves), for small T.
// Tokens are split into 16 contiguous chunks, one per wave.  Per-chunk expert
// histograms (LDS integer atomics, so the counts are exact) give every wave
// the base position of its routes inside each expert's segment; a wave then
// walks its tokens in order, placing the token's k routes (distinct experts)
// in one step.  The result is the stable order by (expert, token).
// Finally the M-tile tables of both grouped GEMMs are written, each entry
// carrying the expert's tier and packed weights from the handle table.
__global__ __launch_bounds__(1024) void permute_kernel(
    const DevHandle* __restrict__ table, WaveMap wmap, Hotness hotness, const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos, TileEntry* __restrict__ tiles13,
    int32_t* __restrict__ ntiles13, int bm13, TileEntry* __restrict__ tiles2,
    int32_t* __restrict__ ntiles2, int bm2) {
  extern __shared__ int lds[];
  int* cnt = lds;                 // [16][E]
  int* off = cnt + 16 * E;        // [E+1] exclusive scan of totals
  int* scan = off + E + 1;        // [1024] scan scratch
  int* hist = off + E + 1 + 1024;  // [kMaxTileRows] tile-ordering histogram
  int* eid = hist + kMaxTileRows;  // [T k] the routes' experts (clamped)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int chunk = (T + 15) / 16;
  const int tb = min(T, wave * chunk), te = min(T, tb + chunk);
  const TileSource src = tile_source(table, wmap, E);

  // every route's expert into LDS with one coalesced pass, so the walks
  // below (one token after another) read LDS instead of memory
  for (int r = tid; r < T * k; r += 1024) eid[r] = min(max(ids[r], 0), E - 1);
  for (int i = tid; i < 16 * E; i += 1024) cnt[i] = 0;
  __syncthreads();
  for (int r = tb * k + lane; r < te * k; r += 64) atomicAdd(&cnt[wave * E + eid[r]], 1);
  __syncthreads();

  // per expert: prefix over the 16 chunks; total -> off[e]
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
    off[e] = run;
  }
  __syncthreads();

  // exclusive scan of totals over experts (E <= 1024: one value per thread)
  int total = 0;
  const int excl = block_exclusive_scan(tid < E ? off[tid] : 0, scan, total);
  if (tid < E) off[tid] = excl;
  if (tid == 0) off[E] = total;
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];

  // stable scatter: each wave walks its tokens in order
  for (int t = tb; t < te; ++t) {
    if (lane < k) {
      const int r = t * k + lane;
      const int e = eid[r];
      const int p = off[e] + cnt[wave * E + e];
      cnt[wave * E + e] += 1;
      sorted[p] = r;
      pos[r] = p;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  write_tile_tables(src, hotness, off, E, tiles13, ntiles13, bm13, tiles2, ntiles2, bm2, scan, hist);
}

// Rank pass of the multi-block grouping (large T).  Block c owns the 256
// tokens [256c, 256c + 256); each of its 4 waves walks 64 of them in order and
// numbers the routes of every expert within the wave (a token's k routes go
// to distinct experts, so one step places all of them); the waves' counts
// then give every route its stable rank among the block's routes of its
// expert.  Writes rank[r] and the block's per-expert counts.
__global__ __launch_bounds__(256) void permute_rank_kernel(const int32_t* __restrict__ ids, int T,
                                                           int k, int E, int32_t* __restrict__ rank,
                                                           int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[4][kMaxExperts];
  __shared__ int rk[kPermChunk * kMaxTopK];
  __shared__ int eid[kPermChunk * kMaxTopK];   // the block's routes' experts (clamped)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kPermChunk;
  const int nr = (min(T, t0 + kPermChunk) - t0) * k;   // routes of this block
  // one coalesced pass brings the block's experts into LDS: the walk below
  // (one token after another) then reads LDS instead of memory
  for (int i = tid; i < nr; i += 256) eid[i] = min(max(ids[(size_t)t0 * k + i], 0), E - 1);
  for (int e = tid; e < 4 * kMaxExperts; e += 256) (&cnt[0][0])[e] = 0;
  __syncthreads();
  const int tb = min(T, t0 + 64 * wave), te = min(T, tb + 64);
  for (int t = tb; t < te; ++t) {
    if (lane < k) {
      const int e = eid[(t - t0) * k + lane];
      rk[(t - t0) * k + lane] = cnt[wave][e];
      cnt[wave][e] += 1;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int i = lane; i < (te - tb) * k; i += 64) {
    const int r = tb * k + i;
    const int e = eid[r - t0 * k];
    int before = 0;
    for (int w = 0; w < wave; ++w) before += cnt[w][e];
    rank[r] = rk[r - t0 * k] + before;
  }
  for (int e = tid; e < E; e += 256)
    chunk_counts[(size_t)blockIdx.x * E + e] = cnt[0][e] + cnt[1][e] + cnt[2][e] + cnt[3][e];
}

// Scan pass of the multi-block grouping: per expert e (one thread each),
// chunk_counts[c][e] becomes the number of routes to e in token blocks before
// c (exclusive prefix over c, in place) and chunk_tot[e] the total.  Every
// count is read once, so the pass costs O(nchunks * E) for any T; the loads of
// eight blocks are issued before their adds.
__global__ __launch_bounds__(256) void permute_scan_kernel(int32_t* __restrict__ chunk_counts,
                                                           int32_t* __restrict__ chunk_tot,
                                                           int nchunks, int E) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  int32_t* col = chunk_counts + e;
  int run = 0;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = col[(size_t)(c + i) * E];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      col[(size_t)(c + i) * E] = run;
      run += v[i];
    }
  }
  for (; c < nchunks; ++c) {
    const int v = col[(size_t)c * E];
    col[(size_t)c * E] = run;
    run += v;
  }
  chunk_tot[e] = run;
}

// Scatter pass of the multi-block grouping.  Block c reads its bases (routes
// of each expert in blocks before c) and the totals from the scan pass, scans
// the totals into the expert offsets, and places its routes at offset + base +
// rank: the stable order by (expert, token).  Block 0 also writes the offsets
// and the M-tile tables.
__global__ __launch_bounds__(1024) void permute_scatter_kernel(
    const DevHandle* __restrict__ table, WaveMap wmap, Hotness hotness, const int32_t* __restrict__ ids, int T, int k, int E,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ chunk_tot, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos, TileEntry* __restrict__ tiles13,
    int32_t* __restrict__ ntiles13, int bm13, TileEntry* __restrict__ tiles2,
    int32_t* __restrict__ ntiles2, int bm2) {
  __shared__ int base[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int scan[16];
  __shared__ int hist[kMaxTileRows];
  const int tid = threadIdx.x, c = blockIdx.x;
  TileSource src{};
  if (c == 0) src = tile_source(table, wmap, E);   // block 0 writes the tile tables
  int total = 0;
  if (tid < E) {
    base[tid] = chunk_base[(size_t)c * E + tid];
    total = chunk_tot[tid];
  }
  int all = 0;
  const int excl = block_exclusive_scan(total, scan, all);
  if (tid < E) off[tid] = excl;
  if (tid == 0) off[E] = all;
  __syncthreads();
  const int r0 = c * kPermChunk * k, r1 = min(T, (c + 1) * kPermChunk) * k;
  for (int r = r0 + tid; r < r1; r += 1024) {
    const int e = min(max(ids[r], 0), E - 1);
    const int p = off[e] + base[e] + rank[r];
    sorted[p] = r;
    pos[r] = p;
  }
  if (c != 0) return;
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];
  write_tile_tables(src, hotness, off, E, tiles13, ntiles13, bm13, tiles2, ntiles2, bm2, scan, hist);
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                                int H, int E, float* logits, float* r13, hipStream_t s) {
  if (T <= 64) {   // few tokens: many small blocks, 8 slabs of loads in flight per step
    constexpr int TT = 1, TE = 2;
    const dim3 grid((T + 2 * TT - 1) / (2 * TT), (E + 4 * TE - 1) / (4 * TE));
    hipLaunchKernelGGL((router_logits_kernel<TT, TE, 8>), grid, dim3(256), 0, s, x, wr, bias, T, H,
                       E, logits, r13);
  } else {
    constexpr int TT = 4, TE = 4;
    const dim3 grid((T + 2 * TT - 1) / (2 * TT), (E + 4 * TE - 1) / (4 * TE));
    hipLaunchKernelGGL((router_logits_kernel<TT, TE, 1>), grid, dim3(256), 0, s, x, wr, bias, T, H,
                       E, logits, r13);
  }
  return hipGetLastError();
}

bool use_small_router(int T, int E, int H) {
  return T <= kSmallRouteMaxT && E <= kSmallRouteMaxE && H <= kSmallRouteMaxH &&
         (size_t)E * H * 2 <= kSmallRouteMaxBytes;
}

hipError_t launch_router_topk_small(const uint16_t* x, const uint16_t* wr, const float* bias,
                                    int T, int H, int E, int k, float* r13, int32_t* ids,
                                    float* w, hipStream_t s) {
  if (!use_small_router(T, E, H)) return hipErrorInvalidValue;
  if (E <= 32)
    hipLaunchKernelGGL((router_topk_small_kernel<1, 1, 8>), dim3(T), dim3(1024), 0, s, x, wr, bias,
                       H, E, k, r13, ids, w);
  else if (E <= 64)
    hipLaunchKernelGGL((router_topk_small_kernel<1, 2, 8>), dim3(T), dim3(1024), 0, s, x, wr, bias,
                       H, E, k, r13, ids, w);
  else
    hipLaunchKernelGGL((router_topk_small_kernel<2, 4, 4>), dim3(T), dim3(1024), 0, s, x, wr, bias,
                       H, E, k, r13, ids, w);
  return hipGetLastError();
}

hipError_t launch_group_sums(const uint16_t* x, int T, int H, float* r13, hipStream_t s) {
  const size_t n8 = (size_t)T * H / 8;   // a multiple of 16: H % 256 == 0
  hipLaunchKernelGGL(group_sums_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x,
                     r13, n8);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t s) {
  const int per = (E + 63) / 64;
  if (per <= 1)
    hipLaunchKernelGGL(topk_kernel<1>, dim3(T), dim3(64), 0, s, logits, T, E, k, ids, w);
  else if (per <= 2)
    hipLaunchKernelGGL(topk_kernel<2>, dim3(T), dim3(64), 0, s, logits, T, E, k, ids, w);
  else if (per <= 4)
    hipLaunchKernelGGL(topk_kernel<4>, dim3(T), dim3(64), 0, s, logits, T, E, k, ids, w);
  else if (per <= 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3(T), dim3(64), 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(topk_kernel<kMaxPerLane>, dim3(T), dim3(64), 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_permute(const DevHandle* table, WaveMap wave, Hotness hotness, const int32_t* ids, int T, int k,
                          int E, int32_t* offsets, int32_t* sorted, int32_t* pos,
                          TileEntry* tiles13, int32_t* ntiles13, int bm13, TileEntry* tiles2,
                          int32_t* ntiles2, int bm2, int32_t* rank, int32_t* chunk_counts,
                          int32_t* chunk_tot, hipStream_t s) {
  if (T > kPermSmallT) {
    const int nchunks = (T + kPermChunk - 1) / kPermChunk;
    hipLaunchKernelGGL(permute_rank_kernel, dim3(nchunks), dim3(256), 0, s, ids, T, k, E, rank,
                       chunk_counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_scan_kernel, dim3((E + 255) / 256), dim3(256), 0, s, chunk_counts,
                       chunk_tot, nchunks, E);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(1024), 0, s, table, wave, hotness, ids, T, k, E,
                       rank, chunk_counts, chunk_tot, offsets, sorted, pos, tiles13, ntiles13, bm13,
                       tiles2, ntiles2, bm2);
    return hipGetLastError();
  }
  const size_t lds = sizeof(int) * (17 * (size_t)E + 1025 + kMaxTileRows + (size_t)T * k);
  // > 64 KB of LDS needs an opt-in (gfx950 has 160 KB; the largest case,
  // 1024 experts and 1024 tokens at top-16, takes 137 KB)
  static DeviceOnce lds_opt_in;
  const hipError_t ea = ensure_dynamic_lds(
      lds_opt_in, reinterpret_cast<const void*>(permute_kernel),
      (int)(sizeof(int) * (17 * kMaxExperts + 1025 + kMaxTileRows + kPermSmallT * kMaxTopK)));
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), lds, s, table, wave, hotness, ids, T, k, E, offsets, sorted,
                     pos, tiles13, ntiles13, bm13, tiles2, ntiles2, bm2);
  return hipGetLastError();
}

}  // namespace moe
