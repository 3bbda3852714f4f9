// quant_pack.hip -- quantize a bf16 weight matrix and write the packed layout.
//
// Quantizer: "Every Expert Counts: ExactMoE ..." §3.2 (symmetric, s = max|W|/7,
// q = clip(round(W/s), -8, 7), groups of 128 inputs per output row, FP16 scales
// as stored in §3.3).  The int8 tier applies the same rule per output row with
// range +-127.  Round-half-to-even of the fp32 quotient; the scale is the fp32
// quotient max/7 (or /127) rounded to fp16, and codes are taken against that
// stored scale.
//
// Packed layout v2 (the kernels' operand order on gfx950): 16-row strips t,
// grouped in quads Q = t/4 (u = t%4), x 128-column groups g.  Inside a tile
// lane l = 16c + r owns row r and, for each of the four 32-wide MFMA k-steps s,
// the 8 columns 32s + 8c .. +7.  Per (Q, g) one contiguous block:
//   int4: 4224 B = tiles u at 1024u (lane bytes 16l..16l+15, step s = 32-bit
//         word s, element i in nibble (i/2) + 4(i%2), nibble value q+8), then
//         the 64 fp16 group scales at 4096 + 2(4r + u);
//   int8: 8192 B = tiles u at 2048u, step s in half s/2 at 1024(s/2) + 16l +
//         8(s%2) + i, byte value q+128; fp16 row scales after all codes at
//         element 64Q + 4r + u;
//   bf16: 16384 B = tiles u at 4096u, step s at 1024s + 16l + 2i.
// Gate/up matrices ([2I, H], gate rows first) are stored with gate and up rows
// interleaved in blocks of 32 so one 64-row quad holds gate and up of the same
// 32 intermediate channels.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int src_row(int p, int n, int layout) {
  if (layout == MOE_LAYOUT_PLAIN) return p;
  const int b = p >> 6, w = p & 63;
  return w < 32 ? 32 * b + w : (n >> 1) + 32 * b + (w - 32);
}

__device__ __forceinline__ bool bf16_nonfinite(uint32_t h) { return (h & 0x7f80u) == 0x7f80u; }

// Load the 32 elements lane (r, c) owns in group g: steps s = 0..3, i = 0..7.
__device__ __forceinline__ void load_lane_group(const uint16_t* row, int g, int c, float v[32],
                                                bool& bad) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 q = load_u32x4(row + kGroup * g + 32 * s + 8 * c);
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bad = bad || bf16_nonfinite(d[j] & 0xffffu) || bf16_nonfinite(d[j] >> 16);
      v[8 * s + 2 * j] = bf16lo_to_f32(d[j]);
      v[8 * s + 2 * j + 1] = bf16hi_to_f32(d[j]);
    }
  }
}

__device__ __forceinline__ float max4_lanes(float m) {
  // lanes r, r+16, r+32, r+48 share a row
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  return m;
}

__device__ __forceinline__ int quant_code(float w, float s, int lo, int hi) {
  if (s == 0.0f) return 0;
  float r = __builtin_rintf(w / s);   // IEEE division, round half to even
  r = fminf(fmaxf(r, (float)lo), (float)hi);
  return (int)r;
}

// One wave per 16-row strip.  blockDim = 256 (4 strips per block).
__global__ __launch_bounds__(256) void quant_pack_int4(const uint16_t* __restrict__ w, int n,
                                                       int k, int layout,
                                                       uint8_t* __restrict__ dst,
                                                       int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int strip = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (strip * 16 >= n) return;
  const int r = lane & 15, c = lane >> 4;
  const int p = strip * 16 + r;
  const uint16_t* row = w + (size_t)src_row(p, n, layout) * k;
  const int G = k / kGroup;
  const int Q = strip >> 2, u = strip & 3;
  bool bad = false;
  for (int g = 0; g < G; ++g) {
    float v[32];
    load_lane_group(row, g, c, v, bad);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    m = max4_lanes(m);
    const _Float16 s16 = (_Float16)(m / 7.0f);
    const float sf = (float)s16;
    bad |= !__builtin_isfinite(sf);
    uint32_t word[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t acc = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u = (uint32_t)(quant_code(v[8 * s + i], sf, -8, 7) + 8);
        acc |= u << (4 * ((i >> 1) + 4 * (i & 1)));
      }
      word[s] = acc;
    }
    uint8_t* block = dst + ((size_t)Q * G + g) * 4224;
    *reinterpret_cast<uint4*>(block + 1024 * u + 16 * lane) =
        make_uint4(word[0], word[1], word[2], word[3]);
    if (c == 0)
      *reinterpret_cast<uint16_t*>(block + 4096 + 2 * (4 * r + u)) = __builtin_bit_cast(uint16_t, s16);
  }
  if (bad) atomicOr(err, 1);
}

__global__ __launch_bounds__(256) void quant_pack_int8(const uint16_t* __restrict__ w, int n,
                                                       int k, int layout,
                                                       uint8_t* __restrict__ dst,
                                                       int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int strip = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (strip * 16 >= n) return;
  const int r = lane & 15, c = lane >> 4;
  const int p = strip * 16 + r;
  const uint16_t* row = w + (size_t)src_row(p, n, layout) * k;
  const int G = k / kGroup;
  const int Q = strip >> 2, u = strip & 3;
  bool bad = false;
  float m = 0.0f;
  for (int g = 0; g < G; ++g) {
    float v[32];
    load_lane_group(row, g, c, v, bad);
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = max4_lanes(m);
  const _Float16 s16 = (_Float16)(m / 127.0f);
  const float sf = (float)s16;
  bad |= !__builtin_isfinite(sf);
  for (int g = 0; g < G; ++g) {
    float v[32];
    load_lane_group(row, g, c, v, bad);
    uint8_t* tile = dst + ((size_t)Q * G + g) * 8192 + 2048 * u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t word[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {       // 4 words = steps 2h, 2h+1 x 8 bytes
        uint32_t acc = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int e = 16 * h + 4 * j + b;   // element index into v[]: 8*s + i
          acc |= (uint32_t)(quant_code(v[e], sf, -128, 127) + 128) << (8 * b);
        }
        word[j] = acc;
      }
      *reinterpret_cast<uint4*>(tile + 1024 * h + 16 * lane) =
          make_uint4(word[0], word[1], word[2], word[3]);
    }
  }
  if (c == 0)
    reinterpret_cast<uint16_t*>(dst + (size_t)n * k)[64 * Q + 4 * r + u] = __builtin_bit_cast(uint16_t, s16);
  if (bad) atomicOr(err, 1);
}

__global__ __launch_bounds__(256) void pack_bf16(const uint16_t* __restrict__ w, int n, int k,
                                                 int layout, uint8_t* __restrict__ dst,
                                                 int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int strip = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (strip * 16 >= n) return;
  const int r = lane & 15, c = lane >> 4;
  const int p = strip * 16 + r;
  const uint16_t* row = w + (size_t)src_row(p, n, layout) * k;
  const int G = k / kGroup;
  const int Q = strip >> 2, u = strip & 3;
  bool bad = false;
  for (int g = 0; g < G; ++g) {
    uint8_t* tile = dst + ((size_t)Q * G + g) * 16384 + 4096 * u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 q = load_u32x4(row + kGroup * g + 32 * s + 8 * c);
      const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bad = bad || bf16_nonfinite(d[j] & 0xffffu) || bf16_nonfinite(d[j] >> 16);
      *reinterpret_cast<uint4*>(tile + 1024 * s + 16 * lane) = make_uint4(q.x, q.y, q.z, q.w);
    }
  }
  if (bad) atomicOr(err, 1);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_words; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const size_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     s, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(int tier, int layout, const uint16_t* w, int64_t n, int64_t k,
                                uint8_t* dst, int* err_flag, hipStream_t s) {
  const int strips = (int)(n / 16);
  const dim3 grid((strips + 3) / 4), block(256);
  if (tier == MOE_TIER_INT4)
    hipLaunchKernelGGL(quant_pack_int4, grid, block, 0, s, w, (int)n, (int)k, layout, dst, err_flag);
  else if (tier == MOE_TIER_INT8)
    hipLaunchKernelGGL(quant_pack_int8, grid, block, 0, s, w, (int)n, (int)k, layout, dst, err_flag);
  else
    hipLaunchKernelGGL(pack_bf16, grid, block, 0, s, w, (int)n, (int)k, layout, dst, err_flag);
  return hipGetLastError();
}

}  // namespace moe
