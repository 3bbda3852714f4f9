// unpack.hip -- host-side reader of the packed expert layout (no GPU work).
//
// "Every Expert Counts: ExactMoE ..." §3.3: the routed experts are stored once
// in the kernel's own format, packed gate/up codes, packed down codes and FP16
// scales.  moe_unpack_codes reads one packed matrix back into plain row-major
// codes and scales, so a caller (or a test) can check a blob against the
// quantizer of §3.2 without a GPU.  It is the inverse of the layout the
// quantize-pack kernel writes:
//   packed row p holds source row p (plain) or, for the fused gate/up matrix,
//   gate row 32 (p/64) + p%64 when p%64 < 32, else up row 32 (p/64) + p%64 - 32;
//   p = 64 Q + 16 u + r (quad Q, strip u, row r), column k = 128 g + 32 s + 8 c + i
//   (group g, step s, chunk c, element i), lane l = 16 c + r;
//   int4: block (Q, g) at 4224 (Q G + g); code nibble (i/2) + 4 (i%2) of the
//         32-bit word at 1024 u + 16 l + 4 s, value q + 8; scale at
//         4096 + 2 (4 r + u) of the block;
//   int8: block (Q, g) at 8192 (Q G + g); byte 2048 u + 1024 (s/2) + 16 l +
//         8 (s%2) + i, value q + 128; row scales after all codes at element
//         64 Q + 4 r + u;
//   bf16: block (Q, g) at 16384 (Q G + g); element at 4096 u + 1024 s + 16 l + 2 i.
#include <string.h>

#include "moe_internal.h"

namespace moe {
namespace {

int64_t source_row(int64_t p, int64_t n, int layout) {
  if (layout == MOE_LAYOUT_PLAIN) return p;
  const int64_t b = p / 64, w = p % 64;
  return w < 32 ? 32 * b + w : n / 2 + 32 * b + (w - 32);
}

uint32_t load_le32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

uint16_t load_le16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_unpack_codes(int tier, int layout, const void* src, size_t src_bytes,
                                int64_t n_out, int64_t k_in, int8_t* q, uint16_t* aux) {
  clear_error();
  if (tier < MOE_TIER_BF16 || tier > MOE_TIER_INT4)
    return set_error(MOE_EINVAL, "bad tier %d", tier);
  if (layout != MOE_LAYOUT_PLAIN && layout != MOE_LAYOUT_GATE_UP)
    return set_error(MOE_EINVAL, "bad layout %d", layout);
  if (!src || !aux || (tier != MOE_TIER_BF16 && !q)) return set_error(MOE_EINVAL, "null pointer");
  if (n_out <= 0 || k_in <= 0 || k_in % kGroup || n_out % 64 || n_out > (1 << 30) ||
      k_in > (1 << 30))
    return set_error(MOE_ESHAPE, "need k_in %% 128 == 0 and n_out %% 64 == 0 (got %lld x %lld)",
                     (long long)n_out, (long long)k_in);
  const int64_t N = n_out, K = k_in, G = K / kGroup;
  size_t payload;
  switch (tier) {
    case MOE_TIER_INT4: payload = (size_t)N * K / 2 + (size_t)N * G * 2; break;
    case MOE_TIER_INT8: payload = (size_t)N * K + 2 * (size_t)N; break;
    default: payload = 2 * (size_t)N * K; break;
  }
  if (src_bytes < payload)
    return set_error(MOE_ENOSPC, "src has %zu bytes, a packed %lld x %lld matrix needs %zu",
                     src_bytes, (long long)N, (long long)K, payload);
  const uint8_t* b = static_cast<const uint8_t*>(src);
  for (int64_t p = 0; p < N; ++p) {
    const int64_t row = source_row(p, N, layout);
    const int64_t Q = p / 64, u = (p / 16) % 4, r = p % 16;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t g = k / kGroup, kk = k % kGroup;
      const int64_t s = kk / 32, c = (kk % 32) / 8, i = kk % 8;
      const int64_t lane = 16 * c + r;
      switch (tier) {
        case MOE_TIER_INT4: {
          const uint8_t* blk = b + (size_t)(Q * G + g) * 4224;
          const uint32_t word = load_le32(blk + 1024 * u + 16 * lane + 4 * s);
          const int nib = (int)(i / 2 + 4 * (i % 2));
          q[row * K + k] = (int8_t)((int)((word >> (4 * nib)) & 0xfu) - 8);
          if (kk == 0) aux[row * G + g] = load_le16(blk + 4096 + 2 * (4 * r + u));
          break;
        }
        case MOE_TIER_INT8: {
          const uint8_t* blk = b + (size_t)(Q * G + g) * 8192;
          q[row * K + k] = (int8_t)((int)blk[2048 * u + 1024 * (s / 2) + 16 * lane + 8 * (s % 2) + i] - 128);
          if (k == 0) aux[row] = load_le16(b + (size_t)N * K + 2 * (64 * Q + 4 * r + u));
          break;
        }
        default: {
          const uint8_t* blk = b + (size_t)(Q * G + g) * 16384;
          aux[row * K + k] = load_le16(blk + 4096 * u + 1024 * s + 16 * lane + 2 * i);
          break;
        }
      }
    }
  }
  return MOE_OK;
}
