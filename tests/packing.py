"""Test-side packers and decoders, written independently of both the oracle and the HIP path.

* pack_codes / unpack_codes: the logical GPTQ-style layout (8 four-bit codes per int32 word along
  the reduction dimension, element 8*i + t in bits 4t..4t+3 of word i, code = value + 8);
  pack_codes8 / unpack_codes8 the 8-bit one (4 codes per word, bits 8t..8t+7, code = value + 128).
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


def pack_codes8(q: np.ndarray) -> np.ndarray:
    """Signed values q [R, C] in [-128, 127] (R % 4 == 0) -> int32 words [R/4, C], element 4*i + t
    in bits 8t..8t+7 of word i, code = value + 128."""
    q = np.asarray(q, dtype=np.int64)
    R, Cc = q.shape
    u = (q + 128).astype(np.uint64).reshape(R // 4, 4, Cc)
    word = np.zeros((R // 4, Cc), dtype=np.uint64)
    for t in range(4):
        word |= u[:, t, :] << np.uint64(8 * t)
    return word.astype(np.uint32).view(np.int32)


def unpack_codes8(words: np.ndarray) -> np.ndarray:
    """int32 words [R/4, C] -> signed values [R, C] via a byte view (one code per byte)."""
    w = np.ascontiguousarray(words, dtype=np.int32)
    R4, Cc = w.shape
    b = w.view(np.uint8).reshape(R4, Cc, 4).astype(np.int64) - 128
    return b.transpose(0, 2, 1).reshape(R4 * 4, Cc)


def bf16_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant(words, scales, group=32, bits=4):
    """Dense fp64 weights [R, C] = value * scale (test-side, numpy)."""
    q = (unpack_codes(words) if bits == 4 else unpack_codes8(words)).astype(np.float64)
    s = bf16_f64(scales)
    return q * np.repeat(s, group, axis=0)


# ---- the HIP library's prepacked layout (decoder written from the header's description) ----
NIBBLE_POS = (0, 16, 4, 20, 8, 24, 12, 28)   # bit position of element t of an 8-row slice


def decode_packed(buf: np.ndarray, kind: str, E: int, R: int, Ccols: int, N: int, bits: int = 4):
    """Decode a prepacked buffer (bytes) of one matrix kind ('w1' or 'w2') into logical
    (codes int [E, R, C], scales uint16 [E, R/32, C]). 8-bit blocks hold a low- and a high-nibble
    plane of the codes (value + 128) before the scales."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    planes = bits // 4
    blk = 4096 * planes + 512
    ncsb, GQ = Ccols // 64, R // 128
    blocks = buf.reshape(E, ncsb, GQ, blk)
    sc = np.ascontiguousarray(blocks[..., 4096 * planes:]).view(np.uint16).reshape(E, ncsb, GQ, 16, 4, 4)  # m, gsub, j
    cs = np.arange(ncsb)[:, None, None, None, None]
    gq = np.arange(GQ)[None, :, None, None, None]
    gsub = np.arange(4)[None, None, :, None, None]
    lane = np.arange(64)[None, None, None, :, None]
    j = np.arange(4)[None, None, None, None, :]
    col = _column_of_vec(kind, cs, j, lane % 16, N)
    nib = np.zeros((planes, E, R, Ccols), dtype=np.int16)
    for p in range(planes):
        words = np.ascontiguousarray(blocks[..., 4096 * p:4096 * (p + 1)]).view(np.uint32).reshape(E, ncsb, GQ, 4, 64, 4)
        for t in range(8):
            row = gq * 128 + gsub * 32 + (lane // 16) * 8 + t
            r_b, c_b = np.broadcast_arrays(row, col)
            nib[p][:, r_b, c_b] = ((words >> np.uint32(NIBBLE_POS[t])) & np.uint32(0xF)).astype(np.int16)
    codes = nib[0] - 8 if bits == 4 else nib[0] + 16 * nib[1] - 128
    m = np.arange(16)[None, None, :, None, None]
    gsub_s = np.arange(4)[None, None, None, :, None]
    cs_s = np.arange(ncsb)[:, None, None, None, None]
    gq_s = np.arange(GQ)[None, :, None, None, None]
    col_s = _column_of_vec(kind, cs_s, j, m, N)
    g_b, c_b = np.broadcast_arrays(gq_s * 4 + gsub_s, col_s)
    scales = np.zeros((E, R // 32, Ccols), dtype=np.uint16)
    scales[:, g_b, c_b] = sc
    return codes, scales


def _column_of_vec(kind, cs, j, m, N):
    if kind == "w1":
        return np.where(j < 2, 32 * cs + 16 * j + m, N + 32 * cs + 16 * (j - 2) + m)
    return 64 * cs + 16 * j + m
