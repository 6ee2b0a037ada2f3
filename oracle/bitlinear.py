"""Packed ternary (BitLinear) weights.  TEST INFRASTRUCTURE ONLY.

The pages run the decode layer's projections as BitLinear layers (Hesper
"FFN Backward GPU Kernels", executeFFNBackward takes wDown, wGate, wUp as
BitLinear; "Attention Backward GPU Kernels", Gradient Flow: "O projection
backward (BitLinear transpose)") but do not give a storage format.  This
module defines the one the library uses, and is the oracle for it:

  * a weight matrix W [out, in] holds values in {-s, 0, +s} with one scale s
    per matrix;
  * each value is coded in 2 bits by its sign: 0 -> 00, +s -> 01, -s -> 11
    (the 2-bit two's complement of -1, 0, +1; 10 never occurs);
  * four consecutive columns of a row share a byte, column 4c + j in bits
    2j .. 2j+1 of byte c; rows are stored one after another, so the packed
    matrix is uint8 [out, in / 4] (in a multiple of 4).

The transposed product of the backward, dx = dy W, is then
dx = s * (dy T) with T = unpack(packed) in {-1, 0, +1}: the dense product
on the unpacked values, which is what the oracle computes.
"""
import numpy as np

CODE = {0: 0b00, 1: 0b01, -1: 0b11}


def pack_ternary(w):
    """W [rows, cols] (values in {-s, 0, +s}, any s > 0) -> uint8 [rows, cols/4],
    coding each value by its sign, written element by element from the
    definition above."""
    w = np.asarray(w)
    rows, cols = w.shape
    assert cols % 4 == 0
    out = np.zeros((rows, cols // 4), np.uint8)
    for r in range(rows):
        for c in range(cols):
            code = CODE[int(np.sign(w[r, c]))]
            out[r, c // 4] |= np.uint8(code << (2 * (c % 4)))
    return out


def unpack_ternary(packed, cols):
    """uint8 [rows, cols/4] -> float64 [rows, cols] in {-1, 0, +1}."""
    packed = np.asarray(packed, np.uint8)
    rows = packed.shape[0]
    out = np.zeros((rows, cols))
    for j in range(4):
        code = (packed >> (2 * j)) & 0b11
        # 2-bit two's complement: 00 -> 0, 01 -> +1, 11 -> -1 (10 -> -2 never occurs)
        out[:, j::4] = np.where(code >= 2, code.astype(np.int64) - 4, code.astype(np.int64))[:, :cols // 4]
    return out


def bitlinear_t(dy, packed, scale, cols):
    """The transposed product dx = dy W for W = scale * unpack(packed):
    dy [n, rows] -> dx [n, cols]."""
    return float(scale) * (np.asarray(dy, np.float64) @ unpack_ternary(packed, cols))
