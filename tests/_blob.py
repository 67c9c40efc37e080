"""Hand-built expert blobs for closed-form tests.

Packs codes and scale/min words straight from the format's description, so
tests can build experts whose decoded weights are known exactly:

* a [R x K] matrix is split in blocks of 32 along K, each with an fp16 scale s
  and fp16 min m; the weight is s*q + m for a b-bit code q;
* code plane: per row K*b/32 little-endian uint32 words.  b = 2, 4: word w
  holds columns w*(32/b) ..; column c of the word sits at bit
  16*(c % 2) + b*(c // 2).  b = 3: three words per 32-column block, the low two
  bits of each code in words 0-1 as for b = 2, the high bit in word 2 at bit
  16*(j % 2) + j // 2 for block column j;
* s/m plane: per row K/32 uint32 words, scale in the low half, min in the high;
* blob: Wg codes, Wg s/m, Wu codes, Wu s/m, Wd codes, Wd s/m, each plane on a
  256-byte boundary; Wg, Wu are [I x H], Wd is [H x I].
"""
import numpy as np


def _up256(v):
    return (v + 255) // 256 * 256


def layout(H, I, bits):
    pos, off = 0, []
    for R, K in ((I, H), (I, H), (H, I)):
        off.append(pos)
        pos = _up256(pos + R * K * bits // 8)
        off.append(pos)
        pos = _up256(pos + R * (K // 32) * 4)
    off.append(pos)
    return off


def f16_bits(x: float) -> int:
    return int(np.array([x], np.float16).view(np.uint16)[0])


def pack_matrix(q: np.ndarray, scale: np.ndarray, mn: np.ndarray, bits: int):
    """q: int [R,K] codes; scale, mn: float [R,K/32] (must be exact fp16 values)."""
    R, K = q.shape
    codes = np.zeros((R, K * bits // 32), np.uint32)
    for r in range(R):
        for col in range(K):
            v = int(q[r, col])
            if bits == 3:
                blk, j = divmod(col, 32)
                half, c = divmod(j, 16)
                codes[r, 3 * blk + half] |= np.uint32((v & 3) << (16 * (c % 2) + 2 * (c // 2)))
                codes[r, 3 * blk + 2] |= np.uint32((v >> 2) << (16 * (j % 2) + j // 2))
            else:
                w, c = divmod(col, 32 // bits)
                codes[r, w] |= np.uint32(v << (16 * (c % 2) + bits * (c // 2)))
    sm = np.zeros((R, K // 32), np.uint32)
    for r in range(R):
        for b in range(K // 32):
            s16, m16 = f16_bits(float(scale[r, b])), f16_bits(float(mn[r, b]))
            assert float(np.float16(scale[r, b])) == float(scale[r, b]), "scale must be an exact fp16 value"
            assert float(np.float16(mn[r, b])) == float(mn[r, b]), "min must be an exact fp16 value"
            sm[r, b] = s16 | (m16 << 16)
    return codes, sm


def build_blob(H, I, bits, mats):
    """mats: three (q, scale, min) triples for Wg [I,H], Wu [I,H], Wd [H,I]."""
    off = layout(H, I, bits)
    blob = np.zeros(off[6], np.uint8)
    for m, (q, s, mn) in enumerate(mats):
        codes, sm = pack_matrix(q, s, mn, bits)
        cb = codes.astype("<u4").tobytes()
        sb = sm.astype("<u4").tobytes()
        blob[off[2 * m]:off[2 * m] + len(cb)] = np.frombuffer(cb, np.uint8)
        blob[off[2 * m + 1]:off[2 * m + 1] + len(sb)] = np.frombuffer(sb, np.uint8)
    return blob


def constant_matrix(R, K, q, s, m):
    return (np.full((R, K), q, np.int64), np.full((R, K // 32), s), np.full((R, K // 32), m))


def one_hot_matrix(cols, K, value, bits, with_min=False):
    """Row r has `value` at column cols[r] and 0 elsewhere.

    Without a min: s = value, m = 0, q = 1 at the column, 0 elsewhere.
    With a min:    s = value, m = -value, q = 2 at the column, 1 elsewhere.
    """
    R = len(cols)
    if with_min:
        q = np.ones((R, K), np.int64)
        for r, c in enumerate(cols):
            q[r, c] = 2
        return q, np.full((R, K // 32), value), np.full((R, K // 32), -value)
    q = np.zeros((R, K), np.int64)
    for r, c in enumerate(cols):
        q[r, c] = 1
    return q, np.full((R, K // 32), value), np.zeros((R, K // 32))
