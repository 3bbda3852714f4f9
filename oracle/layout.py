"""Independent writer of the packed expert-weight byte layout (oracle side).

The pages require the routed experts to be quantized once, offline, into the
exact packed form the GPU kernel consumes, with FP16 scales stored beside the
codes ([ExactMoE] "Every Expert Counts ..." §3.3 and §6, "kernel-native
storage").  The byte layout itself is this project's own design for gfx950;
it is specified here, in words, and the HIP quantize-pack kernel writes the
same bytes from its own code.  Tests compare the two byte for byte.

Layout v1 of a weight W [N, K] (N output rows, K inputs; K % 128 == 0,
N % 16 == 0; the gate/up form needs N = 2I with I % 32 == 0):

  row order     PLAIN: packed row p is source row p.
                GATE_UP (fused gate/up matrix [2I, H], gate rows first):
                packed rows come in blocks of 64; inside block b, rows 0..31 are
                gate rows 32b..32b+31 and rows 32..63 are up rows 32b..32b+31.
  tiles         packed rows are cut into 16-row strips t = p // 16, r = p % 16;
                K is cut into groups g = k // 128 (G = K/128 groups).  Tile
                (t, g) is stored at index t*G + g.
  inside a tile the 128 columns of the group split as k%128 = 32*s + 8*c + i
                (step s 0..3, chunk c 0..3, element i 0..7) and lane
                l = 16*c + r (0..63) owns elements (r, s, c, i) for all s, i.
  int4 codes    nibble value q+8.  Tile = 1024 B; lane l's 16 bytes start at
                16*l; step s is the little-endian 32-bit word at 16*l + 4*s;
                element i sits in nibble (i // 2) + 4*(i % 2) of that word.
  int4 scales   after all codes (at byte N*K/2): fp16 scale of (packed row p,
                group g) at element index (t*G + g)*16 + r.
  int8 codes    byte value q+128.  Tile = 2048 B; step s lives in half
                s // 2 (1024 B each); lane l's 16 bytes of that half start at
                16*l; step s uses bytes 8*(s % 2) .. +7 of them, element i at
                byte i.
  int8 scales   after all codes (at byte N*K): fp16 scale of packed row p at
                element index p.
  bf16 values   Tile = 4096 B; step s lives in quarter s (1024 B); lane l's
                16 bytes start at 16*l; element i is the uint16 at byte 2*i.
  size          int4 N*K/2 + N*(K/128)*2 (exactly the [ExactMoE] §3.2 memory
                equation: 4 bits per weight plus 16 bits per 128 weights);
                int8 N*K + 2*N; bf16 2*N*K.  Blobs are padded with zero bytes to
                a multiple of 256.
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
    if k % GROUP or n % 16:
        raise ValueError("layout needs K % 128 == 0 and N % 16 == 0")
    if layout == LAYOUT_GATE_UP and (n % 64):
        raise ValueError("gate/up layout needs N = 2I with I % 32 == 0")


def _tile_elements(n: int, k: int):
    """For every (tile, lane, step, element) give the (packed row, column).

    Returns arrays shaped [T, G, 64 lanes, 4 steps, 8 elements].
    """
    T, G = n // 16, k // GROUP
    t = np.arange(T)[:, None, None, None, None]
    g = np.arange(G)[None, :, None, None, None]
    lane = np.arange(64)[None, None, :, None, None]
    s = np.arange(4)[None, None, None, :, None]
    i = np.arange(8)[None, None, None, None, :]
    r, c = lane % 16, lane // 16
    row = 16 * t + r
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
    T, G = n // 16, k // GROUP

    if tier == TIER_INT4:
        u = (q[srow, col].astype(np.int16) + 8).astype(np.uint32)   # [T,G,64,4,8]
        nib_pos = (np.arange(8) // 2) + 4 * (np.arange(8) % 2)
        words = np.zeros(u.shape[:-1], dtype=np.uint32)
        for i in range(8):
            words |= u[..., i] << np.uint32(4 * nib_pos[i])
        codes = words.reshape(-1).astype("<u4").view(np.uint8)      # order t,g,lane,s
        blob[: n * k // 2] = codes
        # scales: [t, g, r] -> s[src row of 16t+r, g]
        tt = np.arange(T)[:, None, None]
        gg = np.arange(G)[None, :, None]
        rr = np.arange(16)[None, None, :]
        sc = np.asarray(s, dtype=np.float16)[src[16 * tt + rr], gg]
        blob[n * k // 2: n * k // 2 + sc.size * 2] = sc.reshape(-1).astype("<f2").view(np.uint8)
        return blob

    if tier == TIER_INT8:
        u = (q[srow, col].astype(np.int16) + 128).astype(np.uint8)  # [T,G,64,4,8]
        # tile bytes: half h = s//2, lane, 8*(s%2) + i
        u = u.reshape(T, G, 64, 2, 2, 8)          # s -> (h, s%2)
        u = u.transpose(0, 1, 3, 2, 4, 5)          # T, G, h, lane, s%2, i
        blob[: n * k] = u.reshape(-1)
        sc = np.asarray(s, dtype=np.float16)[src]
        blob[n * k: n * k + 2 * n] = sc.astype("<f2").view(np.uint8)
        return blob

    if tier == TIER_BF16:
        v = np.asarray(w_bf16, dtype=np.uint16)[srow, col]          # [T,G,64,4,8]
        v = v.transpose(0, 1, 3, 2, 4)             # T, G, s, lane, i
        blob[: 2 * n * k] = v.reshape(-1).astype("<u2").view(np.uint8)
        return blob

    raise ValueError(f"bad tier {tier}")
