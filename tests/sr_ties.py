"""Inputs for E2M1 stochastic rounding where the discarded fraction agrees
with the element's SR word in its top 22 bits, so that the word's low 10 bits
alone decide the rounding (round up iff r < F, F the top 32 bits of
the discarded fraction).  The expected codes follow from the construction; the
oracle supplies only the SR words (its Philox is pinned to rocRAND's)."""
import numpy as np


def sr_tie_tensor(oracle, rows, cols, col_blocks, seed, off):
    """fp32 [rows, cols] of E2M1 blocks (along each row, or down each column
    when col_blocks) whose first element is +-6 * 2^s, so that the block scale
    is 2^s, and whose other elements have |V / X| < 1 with a discarded fraction
    equal in its top 22 bits to the element's SR word: the word's low 10
    bits then decide the rounding.  Returns the tensor, the expected codes
    (codes[r, c]; -1 for the block maxima) and how many elements round up."""
    rng = np.random.default_rng(21)
    x = np.zeros((rows, cols), np.float32)
    codes = np.full((rows, cols), -1, np.int64)
    lay_id = 1 if col_blocks else 0
    n_up = 0
    for r in range(rows):
        for c in range(cols):
            k, blk, line = (r % 32, r // 32, c) if col_blocks else (c % 32, c // 32, r)
            scale = 2.0 ** ((blk * 7 + line * 3) % 40 - 20)
            sign = -1.0 if rng.integers(0, 2) else 1.0
            if k == 0:
                x[r, c] = sign * 6.0 * scale
                continue
            w = oracle.sr_word(seed, off, lay_id, r * cols + c)
            if rng.integers(0, 2):   # |V/X| in [0, 0.5): fraction 2|V/X| = t * 2^-24
                d = int(rng.integers(0, 4))
                t = ((w >> 10) << 2) | d
                y, lower = t * 2.0 ** -25, 0
            else:                    # [0.5, 1): fraction 2|V/X| - 1 = t * 2^-24, t even
                d = 2 * int(rng.integers(0, 2))
                t = ((w >> 10) << 2) | d
                y, lower = 0.5 + t * 2.0 ** -25, 1
            # top 32 bits of the fraction: t << 8; round up iff w < t << 8
            up = (w & 0x3FF) < (d << 8)
            n_up += int(up)
            x[r, c] = np.float32(sign * y * scale)
            codes[r, c] = (lower + int(up)) | (8 if sign < 0 else 0)
    return x, codes, n_up


def element_codes(q: dict, col_blocks: bool) -> np.ndarray:
    """E2M1 element codes [rows, cols] out of the packed row (or col-T) output."""
    p = (q["q_colt"] if col_blocks else q["q_row"])
    p = np.asarray(p).astype(np.int64)
    el = np.stack([p & 0xF, p >> 4], axis=2).reshape(p.shape[0], -1)  # element 2i in the low nibble
    return el.T if col_blocks else el
