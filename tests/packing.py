"""Test-side packers and decoders, written independently of both the oracle and the HIP path.

* pack_codes / unpack_codes: the logical GPTQ-style layout (8 four-bit codes per int32 word along
  the reduction dimension, element 8*i + t in bits 4t..4t+3 of word i, code = value + 8).
* decode_packed: reads the HIP library's prepacked buffer back into logical codes and scales,
  following the layout as the library's header documents it (block (expert, column superblock of
  64, group quad) = 4 KiB of codes + 512 B of scales).
"""
import numpy as np


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Signed values q [R, C] in [-8, 7] (R % 8 == 0) -> int32 words [R/8, C]."""
    q = np.asarray(q, dtype=np.int64)
    R, Cc = q.shape
    u = (q + 8).astype(np.uint64).reshape(R // 8, 8, Cc)
    word = np.zeros((R // 8, Cc), dtype=np.uint64)
    for t in range(8):
        word |= u[:, t, :] << np.uint64(4 * t)
    return word.astype(np.uint32).view(np.int32)


def unpack_codes(words: np.ndarray) -> np.ndarray:
    """int32 words [R/8, C] -> signed values [R, C] via a byte view (two codes per byte)."""
    w = np.ascontiguousarray(words, dtype=np.int32)
    R8, Cc = w.shape
    b = w.view(np.uint8).reshape(R8, Cc, 4)           # little-endian bytes of each word
    lo = (b & 0x0F).astype(np.int64) - 8               # element 2*byte
    hi = (b >> 4).astype(np.int64) - 8                 # element 2*byte + 1
    vals = np.stack([lo, hi], axis=-1).reshape(R8, Cc, 8)   # [word row, col, t]
    return vals.transpose(0, 2, 1).reshape(R8 * 8, Cc)


def bf16_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant(words, scales, group=32):
    """Dense fp64 weights [R, C] = value * scale (test-side, numpy)."""
    q = unpack_codes(words).astype(np.float64)
    s = bf16_f64(scales)
    return q * np.repeat(s, group, axis=0)


# ---- the HIP library's prepacked layout (decoder written from the header's description) ----
NIBBLE_POS = (0, 16, 4, 20, 8, 24, 12, 28)   # bit position of element t of an 8-row slice


def _column_of(kind, csb, j, m, N):
    if kind == "w1":
        return (32 * csb + 16 * j + m) if j < 2 else (N + 32 * csb + 16 * (j - 2) + m)
    return 64 * csb + 16 * j + m


def decode_packed(buf: np.ndarray, kind: str, E: int, R: int, Ccols: int, N: int):
    """Decode a prepacked buffer (bytes) of one matrix kind ('w1' or 'w2') into logical
    (codes int8 [E, R, C], scales uint16 [E, R/32, C])."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    ncsb, GQ = Ccols // 64, R // 128
    blocks = buf.reshape(E, ncsb, GQ, 4608)
    codes = np.zeros((E, R, Ccols), dtype=np.int8)
    scales = np.zeros((E, R // 32, Ccols), dtype=np.uint16)
    words = blocks[..., :4096].copy().view(np.uint32).reshape(E, ncsb, GQ, 4, 64, 4)  # [.., gsub, lane, j]
    sc = blocks[..., 4096:].copy().view(np.uint16).reshape(E, ncsb, GQ, 16, 4, 4)     # [.., m, gsub, j]
    for csb in range(ncsb):
        for j in range(4):
            for m in range(16):
                col = _column_of(kind, csb, j, m, N)
                for gsub in range(4):
                    # scales of groups g = 4*gq + gsub
                    scales[:, gsub::4, col] = sc[:, csb, :, m, gsub, j]
                    for kk in range(4):
                        lane = 16 * kk + m
                        wd = words[:, csb, :, gsub, lane, j]             # [E, GQ]
                        for t in range(8):
                            u = (wd >> np.uint32(NIBBLE_POS[t])) & np.uint32(0xF)
                            rows = np.arange(GQ) * 128 + gsub * 32 + kk * 8 + t
                            codes[:, rows, col] = u.astype(np.int8) - 8
    return codes, scales
