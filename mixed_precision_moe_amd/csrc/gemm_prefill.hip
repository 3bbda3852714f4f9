// gemm_prefill.hip -- large-batch grouped expert GEMMs (MFMA-bound regime).
//
// "Every Expert Counts: ExactMoE ..." §3.4: one fused gate/up grouped GEMM and
// one down grouped GEMM over the whole token matrix; §5.4 (Table 4): more
// routes coalesced per expert turn the grouped kernel from weight streaming
// into arithmetic.  Weights are dequantized in registers, never materialized
// as a full fp16 matrix (§3.1, §3.3); as in the MARLIN kernel the pages use,
// the dequantized weight q*s is rounded once to fp16 (relative error at most
// 2^-11, fp16's unit roundoff, for scales in fp16's normal range) and the
// product runs on fp16 MFMA with fp32 accumulation.
// Activations enter as fp16 re-encodings of their bf16 values (exact for
// magnitudes in [2^-14, 65504]; larger magnitudes saturate to +-65504).
//
// Block: 512 threads (8 waves, two per SIMD so that one wave's MFMAs cover
// the other's waits), tile 256 rows x 256 columns of one expert; wave (wm, wn)
// of the 2 x 4 grid owns 128 rows x 64 columns (one quad of the packed layout;
// 8 x 4 MFMA tiles, 128 fp32 accumulators).  K runs in chunks of 64 with the
// activation panel double-buffered in LDS: rows (gathered through the grouped
// route order) go from memory straight into LDS with buffer_load ... lds, one
// instruction filling 8 rows x 128 bytes (whole cache lines), 16-byte slots
// permuted within a row by an XOR of the row index so that the MFMA operand
// reads hit 16 distinct bank groups.  Weights: an int4 lane word of the packed
// tile is exactly that lane's B operand of one 32-wide k-step, so int4 codes
// go from memory into registers two chunks ahead and are dequantized there;
// int8 and bf16 weights (two and four times the bytes) are loaded once per
// block, dequantized by one thread per column and k-step and staged through
// LDS in fragment-major order (a 1 KB fragment holds one 16 x 32 operand with
// lane l's 16 bytes at 16*l).  Each chunk: 2 x 8 x 4 v_mfma_f32_16x16x32_f16
// per wave.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
// LDS pointers with their address space spelled out, so every access is a
// ds_read / ds_write (a generic pointer would become a flat access).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) v4u32 lds_u4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) float lds_f32;
typedef short f16x8_t __attribute__((__vector_size__(8 * sizeof(short))));

constexpr int PBM = 256, PBN = 256, PBK = 64;
constexpr int kPrefillThreads = 512;
constexpr int kFragBytes = 1024;                         // one 16 x 32 fp16 operand
constexpr int kPanelBytes = 2 * (PBM / 16) * kFragBytes; // A or B of one chunk: 32 fragments
// The int4 path double-buffers its activations in steps of two 64-wide
// chunks (two panels per buffer).  Deeper prefetch (a third buffer) measured
// slower on every large-batch workload: the workgroup fence of
// __syncthreads() waits for every LDS DMA in flight, and a bare s_barrier with
// explicit waits cost more than the deeper prefetch saved.
// 2 buffers x (activations + staged weights) = 128 KB; the int4 path uses the
// activation half only
constexpr size_t kPrefillLds = (size_t)2 * 2 * kPanelBytes;
static_assert(4 * kPanelBytes <= (int)kPrefillLds, "int4 activation buffers fit the block's LDS");

struct PrefillArgs {
  const TileEntry* tiles;
  const int32_t* ntiles;
  int max_tiles;
  const uint16_t* a16;       // fp16 activations: gate/up x16 [T, H]; down act16 [T*k, I]
  uint32_t a16_bytes;        // size of that array
  const int32_t* sorted;
  int top_k;
  int K, N;
  uint16_t* act16;           // gate/up output [T*k, I]: fp16 re-encodings of bf16-rounded
                             // values, or the bf16 values themselves (BF16_OUT)
  float* r2;                 // BF16_OUT: each row's sum of every 32 activation columns [T*k, I/32]
  int I;
  const float* topk_w;       // down epilogue
  float* rows;               // [T*k, H] fp32, by route id
  int xcd_group;             // > 0: launch-order groups of this many blocks stay on one XCD
};

__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// fp16 magic: 0x6400 | u is the fp16 value 1024 + u for u < 1024.  The mask
// and magic come from fp16_int4_consts() (an SGPR and a VGPR the compiler
// cannot see through), so each element pair is one v_and_or_b32 (after a
// shift for pairs 1..3) instead of an and and an or with literals.
__device__ __forceinline__ Int4Consts fp16_int4_consts() {
  return Int4Consts{opaque_sgpr(0x000f000fu), opaque_vgpr(0x64006400u)};
}

__device__ __forceinline__ void dequant_int4_word(uint32_t w, half2_t s2, uint32_t out[4],
                                                  Int4Consts c) {
  const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = ((w >> (4 * j)) & c.mask) | c.magic;  // elements 2j, 2j+1
    const half2_t q = as_h2(t) + bias;                       // exact: q in [-8, 7]
    out[j] = as_u32(q * s2);                                 // fp16(q * s)
  }
}

__device__ __forceinline__ void dequant_int8_word(uint32_t w, half2_t s2, uint32_t& lo, uint32_t& hi) {
  const uint32_t mask = 0x00ff00ffu, magic = 0x64006400u;
  const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const uint32_t t02 = as_u32((as_h2((w & mask) | magic) + bias) * s2);          // e0, e2
  const uint32_t t13 = as_u32((as_h2(((w >> 8) & mask) | magic) + bias) * s2);   // e1, e3
  lo = __builtin_amdgcn_perm(t13, t02, 0x05040100u);   // (e0, e1)
  hi = __builtin_amdgcn_perm(t13, t02, 0x07060302u);   // (e2, e3)
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fminf(fmaxf(lo, -65504.f), 65504.f),
                                                                fminf(fmaxf(hi, -65504.f), 65504.f)));
}

template <int TIER>
struct PTier;
template <>
struct PTier<MOE_TIER_INT4> { static constexpr int kBlock = 4224; };
template <>
struct PTier<MOE_TIER_INT8> { static constexpr int kBlock = 8192; };
template <>
struct PTier<MOE_TIER_BF16> { static constexpr int kBlock = 16384; };

template <int TIER>
__device__ __forceinline__ uint32_t payload_bytes(int N, int K) {
  if constexpr (TIER == MOE_TIER_INT4) return (uint32_t)(N / 64) * (K / kGroup) * 4224u;
  else if constexpr (TIER == MOE_TIER_INT8) return (uint32_t)N * K + 2u * N;
  else return 2u * N * K;
}

// Staged weights (int8 and bf16 tiers): staging role of one thread: column r
// of strip cb (16 strips of the block), k-step ks (32 k) of the chunk.  Raw registers: int4 4 words (c =
// 0..3, 8 codes each) + the group scale, int8 4 x 8 B, bf16 4 x 16 B.
template <int TIER>
struct BStage;
template <>
struct BStage<MOE_TIER_INT4> { uint32_t w[4]; uint32_t scale; };
template <>
struct BStage<MOE_TIER_INT8> { uint2 w[4]; };
template <>
struct BStage<MOE_TIER_BF16> { u32x4 w[4]; };

// voff: this thread's byte offset inside the block's first quad row of blocks
// (its quad within the block times G blocks, plus the strip and column
// position); soff: the block-uniform offset of k-group g of the block's first
// quad; h: which half of the group the chunk is.  In every tier's packed tile,
// lane slot 16 c + r holds column r's k = 32 s + 8 c + 0..7 for the group's
// four 32-wide steps s; the chunk's k-step ks is step s = 2 h + ks.
template <int TIER>
__device__ __forceinline__ void load_b_chunk(BStage<TIER>& raw, __amdgpu_buffer_rsrc_t rsrc,
                                             uint32_t voff, uint32_t soff, int h, int ks) {
  if constexpr (TIER == MOE_TIER_INT4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) raw.w[c] = buffer_load4(rsrc, voff + 256 * c + 4 * (2 * h + ks), soff);
  } else if constexpr (TIER == MOE_TIER_INT8) {
#pragma unroll
    for (int c = 0; c < 4; ++c) raw.w[c] = buffer_load8(rsrc, voff + 1024 * h + 256 * c + 8 * ks, soff);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      raw.w[c] = buffer_load16<true>(rsrc, voff + 1024 * (2 * h + ks) + 256 * c, soff);
  }
}

// Dequantize the thread's raw k-step and write it into B fragment (cb, ks):
// the 8 values k = 32 ks + 8 c + 0..7 go to lane slot r + 16 c.  `bfrag`
// points at slot r of that fragment.
template <int TIER>
__device__ __forceinline__ void store_b_chunk(const BStage<TIER>& raw, float row_scale, lds_u8* bfrag) {
  auto put = [&](int c, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
    *reinterpret_cast<lds_u4*>(bfrag + 256 * c) = v4u32{x0, x1, x2, x3};
  };
  if constexpr (TIER == MOE_TIER_INT4) {
    const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)raw.scale);
    const half2_t s2 = {sh, sh};
    const Int4Consts k4 = fp16_int4_consts();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t o[4];
      dequant_int4_word(raw.w[c], s2, o, k4);
      put(c, o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (TIER == MOE_TIER_INT8) {
    const _Float16 sh = (_Float16)row_scale;
    const half2_t s2 = {sh, sh};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t a0, a1, b0, b1;
      dequant_int8_word(raw.w[c].x, s2, a0, a1);   // elements 0..3
      dequant_int8_word(raw.w[c].y, s2, b0, b1);   // elements 4..7
      put(c, a0, a1, b0, b1);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = raw.w[c];
      put(c, bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
    }
  }
}

// int4 weights of one wave and chunk, straight from the packed layout into
// registers.  The wave's 64 columns are one quad (strips j = 0..3).  In the
// int4 tile, lane slot l holds column l % 16's codes k = 32 s + 8 (l / 16) +
// 0..7 for the group's four 32-wide steps s (word s), which is exactly lane
// l's v_mfma 16x16x32 B operand of step s; the chunk's k-steps are s = 2h,
// 2h+1.  Per lane: 8 bytes per strip plus the 4 strips' group scales.
struct BDirect { uint2 w[4]; uint2 scale; };

typedef _Float16 f16x8v_t __attribute__((__vector_size__(8 * sizeof(_Float16))));

__device__ __forceinline__ f32x4_t mfma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8v_t, a),
                                                __builtin_bit_cast(f16x8v_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f16x8_t pack_f16x8(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  return __builtin_bit_cast(f16x8_t, v4u32{x0, x1, x2, x3});
}

// Dequantize the chunk's int4 codes into the B operands of both k-steps.
__device__ __forceinline__ void dequant_b(const BDirect& raw, f16x8_t (&fb)[2][4], Int4Consts k4) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 sh = (_Float16)half_of(raw.scale, j);
    const half2_t s2 = {sh, sh};
    uint32_t o[4];
    dequant_int4_word(raw.w[j].x, s2, o, k4);
    fb[0][j] = pack_f16x8(o[0], o[1], o[2], o[3]);
    dequant_int4_word(raw.w[j].y, s2, o, k4);
    fb[1][j] = pack_f16x8(o[0], o[1], o[2], o[3]);
  }
}

// s_waitcnt immediate of gfx9 for vmcnt(n), n < 16, with expcnt and lgkmcnt
// left unconstrained
constexpr int wait_vmcnt(int n) { return n | (0x7 << 4) | (0xF << 8); }

// Row-aware work of a tile with fewer than 256 rows (FULL = false; all
// conditions wave-uniform): a wave issues the activation DMA only for its
// 32-row slice of the panel if that holds a real row, and MFMAs (and operand
// reads) only for its 64-row halves that hold one; a wave whose 128 rows are
// all past the tile's count loads no weights.  The others' results are never
// stored, so the skipped work changes no output.
struct RowWork {
  int rows;                       // real rows of the tile (1 .. 256)
  __device__ bool dma(int wave) const { return 32 * wave < rows; }
  __device__ bool blk(int wm, int i) const { return 128 * wm + 16 * i < rows; }
  __device__ bool any(int wm) const { return 128 * wm < rows; }
};

// Tiles of at most 128 rows (KSPLIT): the two wave rows split K instead of M.
// Wave (h, wn) takes the 64-wide chunks 2j + h of K for all of the tile's rows,
// so every wave of the block loads weights and runs MFMAs and the block needs
// half the K steps; a step's LDS buffer holds chunk 2j in 16-row blocks 0..7
// and chunk 2j + 1 in blocks 8..15.  The two halves' sums meet in LDS after the
// loop (even chunks + odd chunks, a fixed order).
constexpr int kSplitKMaxRows = 128;

// int4 tier: weights straight from memory into MFMA operands.
template <bool GATE_UP, bool FULL, bool KSPLIT>
__device__ __forceinline__ void prefill_mainloop_direct(const PrefillArgs& a, const uint8_t* blob,
                                                        const int (&arow)[4], int n_block,
                                                        lds_u8* lds, f32x4_t (&acc)[8][4],
                                                        RowWork rw) {
  static_assert(!(FULL && KSPLIT), "split K serves partial tiles");
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int rm = KSPLIT ? 0 : wm;                       // the wave's row half of the tile
  const bool wave_b = FULL || rw.any(rm);               // this wave needs weights
  const int K = a.K, G = K / kGroup, KC = K / PBK;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, payload_bytes<MOE_TIER_INT4>(a.N, K));
  const int quad = n_block / 64 + wn;                   // this wave's quad (wave-uniform)
  constexpr int kBlk = PTier<MOE_TIER_INT4>::kBlock;
  // Activation panel: 16-row blocks of 2 KB; row rr of a block holds its 64
  // chunk values (128 B) with the 8-value slice kb in 16-byte slot kb ^ (rr/2).
  // Staging role: wave w fills tile rows 32w .. 32w+31 with 4 DMAs; lane l of
  // DMA i loads tile row 32w + 8i + l/8 into slot l%8.
  // KSPLIT: waves 4..7 stage the odd chunk of each pair, 128 bytes further on
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a.a16, a.a16_bytes);
  uint32_t avoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 8 * (i & 1) + (lane >> 3);              // row within the 16-row block
    avoff[i] = (uint32_t)arow[i] * K * 2u + 16u * ((lane & 7) ^ (rr >> 1)) +
               (KSPLIT ? 2u * PBK * (uint32_t)wm : 0u);
  }
  // operand read offsets within a 16-row block, k-steps 0 and 1
  uint32_t aread[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rr = lane & 15, kb = 4 * ks + (lane >> 4);
    aread[ks] = 128u * rr + 16u * (kb ^ (rr >> 1));
  }
  // A step of the loop covers kStep 64-wide chunks per wave (half c of the
  // step), each with its own 32 KB panel; the activations are double-buffered
  // by step.  Full tiles take one chunk per step; partial tiles (latency-bound
  // over K: few rows, or KSPLIT) two, so one barrier and one DMA wait cover
  // 128 k per wave (Mixtral-shaped full tiles measured 3% slower with two,
  // OLMoE T = 512 7% and Mixtral T = 256 8% faster).
  constexpr int kStep = FULL ? 1 : 2;
  auto As = [&](int buf, int c) { return lds + (kStep * buf + c) * kPanelBytes; };
  const Int4Consts k4 = fp16_int4_consts();
  // K chunk of this wave in half c of step j (KSPLIT: wave row h takes chunks
  // 2 kStep j + 2c + h), clamped into K: a clamped chunk only feeds a skipped
  // half or a prefetch that is never used
  auto chunk_of = [&](int j, int c) {
    return min(KSPLIT ? 2 * kStep * j + 2 * c + wm : kStep * j + c, KC - 1);
  };
  const int NJ = KSPLIT ? (KC + 2 * kStep - 1) / (2 * kStep) : KC / kStep;   // KC is even

  BDirect braw0, braw1;
  auto load_b = [&](int kc, BDirect& raw) {
    if (!wave_b) return;
    const uint32_t block = (uint32_t)(quad * G + (kc >> 1)) * kBlk;
#pragma unroll
    for (int j = 0; j < 4; ++j) raw.w[j] = buffer_load8(rsrc, 16 * lane + 1024 * j, block + 8 * (kc & 1));
    raw.scale = buffer_load8(rsrc, 8 * (lane & 15), block + 4096u);
  };
  // activations of step j: half c holds chunk kStep j + c (KSPLIT: chunks
  // 2 kStep j + 2c and the one after, by wave rows 0 and 1)
  auto dma_a = [&](int j, int buf) {
    if (!FULL && !rw.dma(KSPLIT ? (wave & 3) : wave)) return;
#pragma unroll
    for (int c = 0; c < kStep; ++c) {
      const int cc = KSPLIT ? min(2 * kStep * j + 2 * c, KC - 2) : kStep * j + c;
      lds_u8* dst = As(buf, c) + 4 * wave * 1024;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void*)(dst + i * 1024), 16, avoff[i],
                                                 2u * PBK * cc, 0, 0);
    }
  };

  f16x8_t fa[2][8], fb[2][4];
  auto read_frags = [&](int buf, int c, int ks) {
    const lds_u8* Aw = As(buf, c) + 8 * wm * 2048 + aread[ks];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (FULL || rw.blk(rm, 2 * h)) {
#pragma unroll
        for (int i = 2 * h; i < 2 * h + 2; ++i)
          fa[ks][i] = __builtin_bit_cast(f16x8_t, (v4u32)*reinterpret_cast<const lds_u4*>(Aw + i * 2048));
      }
  };
  auto mfma_block = [&](int ks) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (FULL || rw.blk(rm, 2 * h)) {
#pragma unroll
        for (int i = 2 * h; i < 2 * h + 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f16(fa[ks][i], fb[ks][j], acc[i][j]);
      }
  };
  // one chunk of a step: dequantize its weights (loaded two chunks ago),
  // refill their register slot with chunk `ahead`, then the 2 x 8 x 4 MFMAs
  auto chunk = [&](int buf, int c, int ahead, BDirect& raw) {
    if (wave_b) dequant_b(raw, fb, k4);
    load_b(ahead, raw);
    read_frags(buf, c, 0);
    read_frags(buf, c, 1);
    mfma_block(0);
    mfma_block(1);
  };

  // Each step first streams the next step's activations into the other
  // buffer by DMA (4 loads per chunk and lane).  Prefetch indices are clamped
  // at the end of K (repeated loads, never used), so the body has no branches
  // and the compiler's load waits stay exact.  Before the barrier each wave
  // waits for its DMA of the next step; the weight loads it issued after that
  // DMA (5 per chunk: two chunks ahead) stay in flight.
  constexpr int kWaitNext = wait_vmcnt(5 * kStep);
  if constexpr (kStep == 1) {
    // slots alternate by chunk parity (unrolled by two, KC even)
    load_b(chunk_of(0, 0), braw0);
    load_b(chunk_of(min(1, NJ - 1), 0), braw1);
    dma_a(0, 0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __syncthreads();
    auto step = [&](int j, BDirect& raw) {
      const int buf = j & 1;
      dma_a(min(j + 1, NJ - 1), buf ^ 1);
      chunk(buf, 0, chunk_of(min(j + 2, NJ - 1), 0), raw);
      __builtin_amdgcn_s_waitcnt(kWaitNext);
      __syncthreads();
    };
    for (int j = 0; j < NJ; j += 2) {
      step(j, braw0);
      step(j + 1, braw1);
    }
  } else {
    // slot c holds half c, one step ahead
    load_b(chunk_of(0, 0), braw0);
    load_b(chunk_of(0, 1), braw1);
    dma_a(0, 0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __syncthreads();
    for (int j = 0; j < NJ; ++j) {
      const int buf = j & 1;
      const int jn = min(j + 1, NJ - 1);
      dma_a(jn, buf ^ 1);
      chunk(buf, 0, chunk_of(jn, 0), braw0);
      // KSPLIT with K / 128 odd: the last step has one chunk per wave row
      if (!KSPLIT || 4 * j + 2 < KC) chunk(buf, 1, chunk_of(jn, 1), braw1);
      __builtin_amdgcn_s_waitcnt(kWaitNext);
      __syncthreads();
    }
  }
  if constexpr (KSPLIT) {
    // the odd chunks' sums (wave row 1) join the even chunks' (wave row 0) in
    // LDS, which the loop's last barrier has freed; only 16-row blocks with a
    // real row travel
    lds_f32* red = reinterpret_cast<lds_f32*>(lds) + wn * 8 * 4 * 4 * 64;
    if (wm == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (rw.blk(0, i)) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((i * 4 + jj) * 4 + e) * 64 + lane] = acc[i][jj][e];
        }
    }
    __syncthreads();
    if (wm == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (rw.blk(0, i)) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][jj][e] += red[((i * 4 + jj) * 4 + e) * 64 + lane];
        }
    }
  }
}

// global loads of one chunk's staged weights per thread
template <int TIER>
constexpr int staged_loads() { return TIER == MOE_TIER_INT4 ? 5 : 4; }

// int8 and bf16 tiers: the weights, two to four times the int4 bytes, are
// staged once per block through LDS (dequantized by one thread per column and
// k-step) instead of being fetched by both waves that share a column range.
template <int TIER, bool GATE_UP, bool FULL>
__device__ __forceinline__ void prefill_mainloop_staged(const PrefillArgs& a, const uint8_t* blob,
                                                 const int (&arow)[4], int n_block,
                                                 lds_u8* lds, f32x4_t (&acc)[8][4], RowWork rw) {
  (void)rw;   // used only when FULL is false
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // FULL false (a tile of at most 128 rows): wave row 1 holds no real row, so
  // it runs a loop of its own that only stages (its share of the weights and
  // of the activation DMA, whose rows past the tile repeat real ones) and
  // skips the operand reads and MFMAs.  The skip is per wave and loop: a
  // per-64-row-half variant, and one that also skipped the DMA of empty rows,
  // spilled 60-158 VGPRs.
  const bool active = FULL || rw.any(wm);               // wave-uniform
  const int K = a.K, G = K / kGroup, KC = K / PBK;
  constexpr int kWaitVmcntB = wait_vmcnt(staged_loads<TIER>());
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(blob, payload_bytes<TIER>(a.N, K));
  // weight staging role: column r of strip cb = 4 qloc + u, k-step ks
  const int ks_own = tid >> 8, qloc = (tid >> 6) & 3, u = (tid >> 4) & 3, r = tid & 15;
  const int quad0 = n_block / 64;                       // block-uniform
  constexpr int kBlk = PTier<TIER>::kBlock;
  uint32_t bvoff;
  if constexpr (TIER == MOE_TIER_INT4)
    bvoff = (uint32_t)qloc * G * kBlk + 1024u * u + 16u * r;
  else if constexpr (TIER == MOE_TIER_INT8)
    bvoff = (uint32_t)qloc * G * kBlk + 2048u * u + 16u * r;
  else
    bvoff = (uint32_t)qloc * G * kBlk + 4096u * u + 16u * r;
  // int4 scale of (column r, strip u) within the block's scale area
  const uint32_t svoff = (uint32_t)qloc * G * kBlk + 2u * (4 * r + u);
  float row_scale = 0.0f;
  if constexpr (TIER == MOE_TIER_INT8)
    row_scale = (float)__builtin_bit_cast(
        _Float16, buffer_load_u16(rsrc, 2 * (64 * qloc + 4 * r + u), (uint32_t)a.N * K + 128u * quad0));
  // Activation panel: 16-row blocks of 2 KB; row rr of a block holds its 64
  // chunk values (128 B) with the 8-value slice kb in 16-byte slot kb ^ (rr/2).
  // Staging role: wave w fills tile rows 32w .. 32w+31 with 4 DMAs; lane l of
  // DMA i loads tile row 32w + 8i + l/8 into slot l%8.
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a.a16, a.a16_bytes);
  uint32_t avoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 8 * (i & 1) + (lane >> 3);              // row within the 16-row block
    avoff[i] = (uint32_t)arow[i] * K * 2u + 16u * ((lane & 7) ^ (rr >> 1));
  }
  // operand read offsets within a 16-row block, k-steps 0 and 1
  uint32_t aread[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rr = lane & 15, kb = 4 * ks + (lane >> 4);
    aread[ks] = 128u * rr + 16u * (kb ^ (rr >> 1));
  }

  // LDS: buffer b holds the A panel at b * 2P and the B panel at b * 2P + P
  auto As = [&](int buf) { return lds + buf * 2 * kPanelBytes; };
  auto Bs = [&](int buf) { return lds + buf * 2 * kPanelBytes + kPanelBytes; };

  // weights of chunk c travel in register slot c % 2, two chunks ahead
  BStage<TIER> braw0, braw1;
  auto load_b = [&](int kc, BStage<TIER>& raw) {
    const uint32_t soff = (uint32_t)(quad0 * G + (kc >> 1)) * kBlk;
    load_b_chunk<TIER>(raw, rsrc, bvoff, soff, kc & 1, ks_own);
    if constexpr (TIER == MOE_TIER_INT4) raw.scale = buffer_load_u16(rsrc, svoff, soff + 4096u);
  };
  auto dma_a = [&](int kc, int buf) {   // every wave (a conditional DMA here spills)
    lds_u8* dst = As(buf) + 4 * wave * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void*)(dst + i * 1024), 16, avoff[i],
                                               2u * PBK * kc, 0, 0);
  };
  auto store_b = [&](int buf, const BStage<TIER>& raw) {
    store_b_chunk<TIER>(raw, row_scale, Bs(buf) + (2 * (4 * qloc + u) + ks_own) * kFragBytes + 16 * r);
  };

  f16x8_t fa[2][8], fb[2][4];
  auto read_frags = [&](int buf, int ks) {
    const lds_u8* Aw = As(buf) + 8 * wm * 2048 + aread[ks];
    const lds_u8* Bw = Bs(buf) + (2 * 4 * wn + ks) * kFragBytes + 16 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      fa[ks][i] = __builtin_bit_cast(f16x8_t, (v4u32)*reinterpret_cast<const lds_u4*>(Aw + i * 2048));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[ks][j] = __builtin_bit_cast(f16x8_t, (v4u32)*reinterpret_cast<const lds_u4*>(Bw + 2 * j * kFragBytes));
  };
  auto mfma_block = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f16(fa[ks][i], fb[ks][j], acc[i][j]);
  };

  // One chunk: its successor's activations stream into the other buffer by
  // DMA and the weights two chunks ahead into a register slot; the
  // successor's weights (loaded a chunk earlier, so already in registers) are
  // dequantized into the other buffer ahead of this chunk's MFMAs, with which
  // the scheduler can interleave them.  Prefetch indices are clamped at the
  // end of K (a repeated load of the last chunk, never used), so the body has
  // no branches and the compiler's load waits stay exact.  KC is even (K is a
  // multiple of 128): unrolled by two, each register slot keeps its role.
  auto step = [&](int kc, BStage<TIER>& next_raw, BStage<TIER>& ahead_raw) {
    const int buf = kc & 1;
    dma_a(min(kc + 1, KC - 1), buf ^ 1);
    load_b(min(kc + 2, KC - 1), ahead_raw);
    read_frags(buf, 0);
    read_frags(buf, 1);
    store_b(buf ^ 1, next_raw);
    mfma_block(0);
    mfma_block(1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcntB);   // the successor's DMA is done; the weights ahead may fly
    __syncthreads();
  };
  // the same step for a wave row without real rows: its share of the
  // activation DMA (none past the rows) and of the weight staging, and the
  // same barriers
  auto step_stage_only = [&](int kc, BStage<TIER>& next_raw, BStage<TIER>& ahead_raw) {
    const int buf = kc & 1;
    dma_a(min(kc + 1, KC - 1), buf ^ 1);
    load_b(min(kc + 2, KC - 1), ahead_raw);
    store_b(buf ^ 1, next_raw);
    __builtin_amdgcn_s_waitcnt(kWaitVmcntB);
    __syncthreads();
  };
  load_b(0, braw0);
  dma_a(0, 0);
  load_b(1, braw1);
  store_b(0, braw0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcntB);
  __syncthreads();
  if (FULL || active) {
    for (int kc = 0; kc < KC; kc += 2) {
      step(kc, braw1, braw0);
      step(kc + 1, braw0, braw1);
    }
  } else {
    for (int kc = 0; kc < KC; kc += 2) {
      step_stage_only(kc, braw1, braw0);
      step_stage_only(kc + 1, braw0, braw1);
    }
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_as_f16(float v) {
  // round to bf16 (the activation precision of the layer), then re-encode as fp16
  const float b = __uint_as_float(f32_to_bf16_rne(v) << 16);
  const float c = fminf(fmaxf(b, -65504.f), 65504.f);
  return __builtin_bit_cast(uint16_t, (_Float16)c);
}

// One tile of one tier: accumulate, then the epilogue (SwiGLU -> fp16
// activations for gate/up, or for the decode down GEMM (BF16_OUT) bf16 ones
// and their 32-column row sums; routing weight -> fp32 rows for down).
// BF16_OUT is a template argument, so each kernel carries one epilogue.  The
// row sums go through a per-wave LDS scratch, not cross-lane shuffles: with
// shuffles the compiler copied the epilogue and main loops per tier and tile
// kind, and the kernel, 2.5 times the code, ran 20% slower.
template <int TIER, bool GATE_UP, bool BF16_OUT>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, const TileEntry& te,
                                             const uint8_t* blob, const int (&arow)[4],
                                             int n_block, lds_u8* plds) {
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // row-aware main loop for partial int4 tiles, skipping 32-row pairs of
  // 16-row blocks past the tile's rows; the staged tiers skip only a whole
  // empty wave row (tiles of at most 128 rows)
  const RowWork rw{te.rows};
  const bool full = te.rows >= PBM;          // tile-uniform
  if constexpr (TIER == MOE_TIER_INT4) {
    if (full) {
      prefill_mainloop_direct<GATE_UP, true, false>(a, blob, arow, n_block, plds, acc, rw);
    } else if (te.rows <= kSplitKMaxRows) {
      prefill_mainloop_direct<GATE_UP, false, true>(a, blob, arow, n_block, plds, acc, rw);
      if (wm == 1) return;                   // its sums went to wave row 0
    } else {
      prefill_mainloop_direct<GATE_UP, false, false>(a, blob, arow, n_block, plds, acc, rw);
    }
  } else if (full || te.rows > kSplitKMaxRows) {
    prefill_mainloop_staged<TIER, GATE_UP, true>(a, blob, arow, n_block, plds, acc, rw);
  } else {
    prefill_mainloop_staged<TIER, GATE_UP, false>(a, blob, arow, n_block, plds, acc, rw);
  }
  const int col0 = n_block + 64 * wn;      // first packed column of this wave (one quad)
  if constexpr (GATE_UP) {
    // strips 0, 1 of the quad are gate, 2, 3 the matching up columns: the
    // wave's quad is activation columns 32 c .. 32 c + 31, c = col0 / 64
    const int c = col0 / 64;
    if constexpr (BF16_OUT) {
      // Every main loop ends at a block barrier past its last LDS read, so
      // the wave owns 16 KB of LDS here: for the split-K tiles, the part its
      // own reduction has just read (wave row 1 has left).  Lane (r, col)
      // leaves its pair of bf16 values' sum for tile row r of the wave's 128;
      // each lane then adds the 16 of two rows in column order.
      lds_f32* sc = reinterpret_cast<lds_f32*>(plds + wn * 32768 + wm * 16384);
      constexpr int kStride = 17;   // floats per row: the column writes spread over the banks
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ml = 16 * i + 4 * (lane >> 4) + e, m = 128 * wm + ml;
          float rs = 0.0f;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t b16 = f32_to_bf16_rne(silu_f32(acc[i][half][e]) * acc[i][half + 2][e]);
            if (m < te.rows)
              a.act16[(size_t)(te.row_start + m) * a.I + 32 * c + 16 * half + (lane & 15)] = (uint16_t)b16;
            rs += bf16_to_f32(b16);
          }
          sc[ml * kStride + (lane & 15)] = rs;
        }
      // one wave's LDS operations complete in order; this keeps the compiler
      // from moving the reads above the writes
      __asm__ volatile("" ::: "memory");
      const int P = a.I / 32;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ml = lane + 64 * h, m = 128 * wm + ml;
        float r = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) r += sc[ml * kStride + j];
        if (m < te.rows) a.r2[(size_t)(te.row_start + m) * P + c] = r;
      }
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int icol = 32 * c + 16 * half + (lane & 15);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 128 * wm + 16 * i + 4 * (lane >> 4) + e;
            if (m < te.rows) {
              const float g = acc[i][half][e], up = acc[i][half + 2][e];
              a.act16[(size_t)(te.row_start + m) * a.I + icol] = f32_to_bf16_as_f16(silu_f32(g) * up);
            }
          }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 128 * wm + 16 * i + 4 * (lane >> 4) + e;
        if (m < te.rows) {
          const int r = a.sorted[te.row_start + m];   // route id t k + j: rows are in route order
          const float wgt = a.topk_w[r];
          float* out = a.rows + (size_t)r * a.N + col0 + (lane & 15);
#pragma unroll
          for (int j = 0; j < 4; ++j) out[16 * j] = wgt * acc[i][j][e];
        }
      }
  }
}

constexpr int kXcdGroupMinK = 4096;

template <bool GATE_UP, bool BF16_OUT>
__global__ __launch_bounds__(kPrefillThreads, 1) void gemm_prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t plds[];
  // Column blocks of one M-tile are adjacent in launch order, so the blocks
  // sharing an activation tile run together (it is read from HBM about once),
  // and consecutive M-tiles of an expert reuse its weights from the last-level
  // cache.  The hardware deals blocks to the 8 XCDs round robin; with
  // xcd_group = C, the j-th block an XCD receives is made logical block
  // (j / C) 8C + xcd C + j % C, so each run of C logical blocks stays on one
  // XCD (a bijection on the grid, which is padded to a multiple of 8C).
  const int n_blocks = a.N / PBN;
  int lb = blockIdx.x;
  if (a.xcd_group > 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3, C = a.xcd_group;
    lb = (j / C) * 8 * C + x * C + (j % C);
  }
  const int tile_idx = lb / n_blocks;
  const int nb = lb - tile_idx * n_blocks;
  if (tile_idx >= uniform(*a.ntiles)) return;
  TileEntry te = a.tiles[tile_idx];
  te.expert = uniform(te.expert);
  te.row_start = uniform(te.row_start);
  te.rows = uniform(te.rows);
  te.tier = uniform(te.tier);
  te.w = uniform_ptr(te.w);
  const int tid = threadIdx.x;
  const int n_block = nb * PBN;

  // activation rows this thread's lane loads: row 32 wave + 8 i + lane / 8
  // (int4 tiles of at most 128 rows, whose wave rows split K: row
  // 32 (wave % 4) + 8 i + lane / 8); rows past the tile's count read the
  // tile's last row (their results are never stored)
  const bool ksplit = te.tier == MOE_TIER_INT4 && te.rows <= kSplitKMaxRows;   // tile-uniform
  const int wrow = ksplit ? (tid >> 6) & 3 : tid >> 6;
  int arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = min(32 * wrow + 8 * j + ((tid & 63) >> 3), te.rows - 1);
    const int pos = te.row_start + m;
    arow[j] = GATE_UP ? a.sorted[pos] / a.top_k : pos;
  }

  const uint8_t* blob = te.w;
  lds_u8* lds = (lds_u8*)plds;
  switch (te.tier) {
    case MOE_TIER_INT4: prefill_body<MOE_TIER_INT4, GATE_UP, BF16_OUT>(a, te, blob, arow, n_block, lds); break;
    case MOE_TIER_INT8: prefill_body<MOE_TIER_INT8, GATE_UP, BF16_OUT>(a, te, blob, arow, n_block, lds); break;
    default: prefill_body<MOE_TIER_BF16, GATE_UP, BF16_OUT>(a, te, blob, arow, n_block, lds); break;
  }
}

// x (bf16) -> fp16 re-encoding for the large-batch path (exact in fp16's
// normal range, saturating beyond it).  8 elements per thread.
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ x16, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(x)[i];
  reinterpret_cast<uint4*>(x16)[i] =
      make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
}

}  // namespace

size_t prefill_lds_bytes() { return kPrefillLds; }

hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* x16, size_t n, hipStream_t s) {
  const size_t n8 = n / 8;
  hipLaunchKernelGGL(x_to_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, x16, n8);
  return hipGetLastError();
}

hipError_t launch_prefill(bool gate_up, const Layer& L, int T, const uint16_t* a16, const int32_t* sorted,
                          const TileEntry* tiles, const int32_t* ntiles, int max_tiles,
                          uint16_t* act16, float* r2, const float* topk_w, float* rows,
                          hipStream_t s, KernelTimer kt) {
  PrefillArgs a{};
  a.r2 = gate_up ? r2 : nullptr;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.max_tiles = max_tiles;
  a.a16 = a16;
  a.a16_bytes = (uint32_t)((gate_up ? (size_t)T * L.H : (size_t)T * L.k * L.I) * 2);
  a.sorted = sorted;
  a.top_k = L.k;
  a.K = gate_up ? L.H : L.I;
  a.N = gate_up ? 2 * L.I : L.H;
  a.act16 = act16;
  a.I = L.I;
  a.topk_w = topk_w;
  a.rows = rows;
  static DeviceOnce lds_opt_in[3];
  const int variant = !gate_up ? 0 : a.r2 ? 2 : 1;
  const void* kern = variant == 0 ? reinterpret_cast<const void*>(gemm_prefill_kernel<false, false>)
                     : variant == 1 ? reinterpret_cast<const void*>(gemm_prefill_kernel<true, false>)
                                    : reinterpret_cast<const void*>(gemm_prefill_kernel<true, true>);
  const hipError_t ea = ensure_dynamic_lds(lds_opt_in[variant], kern, (int)kPrefillLds);
  if (ea != hipSuccess) return ea;
  // Down GEMM with a long K (= I): an M-tile's column blocks share one XCD,
  // whose L2 then takes the tile's activation rows (256 x I fp16) once
  // instead of in every XCD: 3.5% faster on the Mixtral shape (I 14336).
  // With I 512 (Qwen3-80B shape) it was 3% slower, and gate/up (K = H)
  // gained nothing.
  a.xcd_group = !gate_up && a.K >= kXcdGroupMinK ? a.N / PBN : 0;
  unsigned blocks = (unsigned)((a.N / PBN) * max_tiles);
  if (a.xcd_group > 0) {
    const unsigned span = 8u * (unsigned)a.xcd_group;
    blocks = (blocks + span - 1) / span * span;   // padding blocks find no tile and exit
  }
  const dim3 grid(blocks);
  auto run = [&](auto kern) {
    if (gate_up && (kt.start || kt.stop))
      hipExtLaunchKernelGGL(kern, grid, dim3(kPrefillThreads), (uint32_t)kPrefillLds, s, kt.start,
                            kt.stop, 0, a);
    else
      hipLaunchKernelGGL(kern, grid, dim3(kPrefillThreads), kPrefillLds, s, a);
    return hipGetLastError();
  };
  if (variant == 0) return run(gemm_prefill_kernel<false, false>);
  if (variant == 1) return run(gemm_prefill_kernel<true, false>);
  return run(gemm_prefill_kernel<true, true>);
}

}  // namespace moe
