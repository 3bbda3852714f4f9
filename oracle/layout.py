"""Independent writer of the packed expert-weight byte layout (oracle side).

The pages require the routed experts to be quantized once, offline, into the
exact packed form the GPU kernel consumes, with FP16 scales stored beside the
codes ([ExactMoE] "Every Expert Counts ..." §3.3 and §6, "kernel-native
storage").  The byte layout itself is this project's own design for gfx950;
it is specified here, in words, and the HIP quantize-pack kernel writes the
same bytes from its own code.  Tests compare the two byte for byte.

Layout v2 of a weight W [N, K] (N output rows, K inputs; K % 128 == 0,
N % 64 == 0; the gate/up form needs N = 2I with I % 32 == 0):

  row order     PLAIN: packed row p is source row p.
                GATE_UP (fused gate/up matrix [2I, H], gate rows first):
                packed rows come in blocks of 64; inside block b, rows 0..31 are
                gate rows 32b..32b+31 and rows 32..63 are up rows 32b..32b+31.
  strips, quads packed rows are cut into 16-row strips t = p // 16, r = p % 16,
                and strips into quads Q = t // 4, u = t % 4 (64 rows per quad);
                K is cut into groups g = k // 128 (G = K/128 groups).
  inside a tile (one strip x one group) the 128 columns split as
                k%128 = 32*s + 8*c + i (step s 0..3, chunk c 0..3, element i
                0..7) and lane l = 16*c + r (0..63) owns elements (r, s, c, i).
  int4          block (Q, g) of 4224 bytes at (Q*G + g)*4224: the four tiles
                u = 0..3 at 1024*u (nibble value q+8; lane l's 16 bytes at
                16*l; step s is the little-endian 32-bit word at 16*l + 4*s;
                element i in nibble (i // 2) + 4*(i % 2)), then the 64 fp16
                group scales at 4096 + 2*(4*r + u).
  int8          block (Q, g) of 8192 bytes at (Q*G + g)*8192: tile u at
                2048*u; byte value q+128; step s in half s // 2 (1024 B each);
                lane l's 16 bytes of that half at 16*l; step s uses bytes
                8*(s % 2) .. +7, element i at byte i.  The fp16 row scales
                follow all codes (at N*K): scale of strip t, row r at element
                index 64*Q + 4*r + u.
  bf16          block (Q, g) of 16384 bytes at (Q*G + g)*16384: tile u at
                4096*u, step s at 1024*s within it, lane l's 16 bytes at 16*l,
                element i the uint16 at 2*i.
  size          int4 N*K/2 + N*(K/128)*2 (exactly the [ExactMoE] §3.2 memory
                equation: 4 bits per weight plus 16 bits per 128 weights);
                int8 N*K + 2*N; bf16 2*N*K.  Blobs are padded with zero bytes to
                a multiple of 256.
A wave that owns one quad reads, per k-group, one contiguous block: its four
strips' operands and (int4) their scales.
"""

from __future__ import annotations

import numpy as np

TIER_BF16, TIER_INT8, TIER_INT4 = 0, 1, 2
LAYOUT_PLAIN, LAYOUT_GATE_UP = 0, 1
GROUP = 128
BLOB_ALIGN = 256


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def payload_size(tier: int, n: int, k: int) -> int:
    if tier == TIER_INT4:
        return n * k // 2 + n * (k // GROUP) * 2
    if tier == TIER_INT8:
        return n * k + 2 * n
    if tier == TIER_BF16:
        return 2 * n * k
    raise ValueError(f"bad tier {tier}")


def packed_size(tier: int, n: int, k: int) -> int:
    return _round_up(payload_size(tier, n, k), BLOB_ALIGN)


def packed_row_source(n: int, layout: int) -> np.ndarray:
    """src[p] = source row stored at packed row p."""
    p = np.arange(n)
    if layout == LAYOUT_PLAIN:
        return p
    if layout == LAYOUT_GATE_UP:
        half = n // 2
        b, w = p // 64, p % 64
        return np.where(w < 32, 32 * b + w, half + 32 * b + (w - 32))
    raise ValueError(f"bad layout {layout}")


def _check(n: int, k: int, layout: int):
    if k % GROUP or n % 64:
        raise ValueError("layout needs K % 128 == 0 and N % 64 == 0")
    if layout == LAYOUT_GATE_UP and (n % 64):
        raise ValueError("gate/up layout needs N = 2I with I % 32 == 0")


def _tile_elements(n: int, k: int):
    """For every (quad, group, strip-in-quad, lane, step, element) give the
    (packed row, column).  Arrays shaped [Q, G, 4, 64 lanes, 4 steps, 8 elements]."""
    Q, G = n // 64, k // GROUP
    q = np.arange(Q)[:, None, None, None, None, None]
    g = np.arange(G)[None, :, None, None, None, None]
    u = np.arange(4)[None, None, :, None, None, None]
    lane = np.arange(64)[None, None, None, :, None, None]
    s = np.arange(4)[None, None, None, None, :, None]
    i = np.arange(8)[None, None, None, None, None, :]
    r, c = lane % 16, lane // 16
    row = 64 * q + 16 * u + r
    col = GROUP * g + 32 * s + 8 * c + i
    return np.broadcast_arrays(row, col)


def pack_matrix(tier: int, layout: int, q=None, s=None, w_bf16=None) -> np.ndarray:
    """Packed blob (uint8) of one matrix from its codes and scales.

    int4: q int8 [N, K], s float16 [N, K/128];  int8: q int8 [N, K], s float16 [N];
    bf16: w_bf16 uint16 [N, K].
    """
    src_mat = w_bf16 if tier == TIER_BF16 else q
    n, k = src_mat.shape
    _check(n, k, layout)
    src = packed_row_source(n, layout)
    row, col = _tile_elements(n, k)            # packed coordinates
    srow = src[row]                            # source row of each element
    blob = np.zeros(packed_size(tier, n, k), dtype=np.uint8)
    Q, G = n // 64, k // GROUP

    if tier == TIER_INT4:
        u = (q[srow, col].astype(np.int16) + 8).astype(np.uint32)   # [Q,G,4,64,4,8]
        nib_pos = (np.arange(8) // 2) + 4 * (np.arange(8) % 2)
        words = np.zeros(u.shape[:-1], dtype=np.uint32)
        for i in range(8):
            words |= u[..., i] << np.uint32(4 * nib_pos[i])
        codes = words.reshape(Q, G, 4096 // 4).astype("<u4").view(np.uint8)   # [Q,G,4096]
        # scales of block (Q, g): element 4*r + u -> s[src row of 64Q + 16u + r, g]
        qq = np.arange(Q)[:, None, None, None]
        gg = np.arange(G)[None, :, None, None]
        rr = np.arange(16)[None, None, :, None]
        uu = np.arange(4)[None, None, None, :]
        sc = np.asarray(s, dtype=np.float16)[src[64 * qq + 16 * uu + rr], gg]   # [Q,G,16,4]
        scb = sc.reshape(Q, G, 64).astype("<f2").view(np.uint8)                 # [Q,G,128]
        blocks = np.concatenate([codes, scb], axis=2)                           # [Q,G,4224]
        blob[: blocks.size] = blocks.reshape(-1)
        return blob

    if tier == TIER_INT8:
        v = (q[srow, col].astype(np.int16) + 128).astype(np.uint8)  # [Q,G,4,64,4,8]
        v = v.reshape(Q, G, 4, 64, 2, 2, 8)        # s -> (h, s%2)
        v = v.transpose(0, 1, 2, 4, 3, 5, 6)       # Q, G, u, h, lane, s%2, i
        blob[: n * k] = v.reshape(-1)
        qq = np.arange(Q)[:, None, None]
        rr = np.arange(16)[None, :, None]
        uu = np.arange(4)[None, None, :]
        sc = np.asarray(s, dtype=np.float16)[src[64 * qq + 16 * uu + rr]]      # [Q,16,4]
        blob[n * k: n * k + 2 * n] = sc.reshape(-1).astype("<f2").view(np.uint8)
        return blob

    if tier == TIER_BF16:
        v = np.asarray(w_bf16, dtype=np.uint16)[srow, col]          # [Q,G,4,64,4,8]
        v = v.transpose(0, 1, 2, 4, 3, 5)          # Q, G, u, s, lane, i
        blob[: 2 * n * k] = v.reshape(-1).astype("<u2").view(np.uint8)
        return blob

    raise ValueError(f"bad tier {tier}")
