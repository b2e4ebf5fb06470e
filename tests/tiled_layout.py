"""The tiled table layout of include/mtp.h, written out with numpy from its
documented formula (used to check the library's packing kernel)."""

import numpy as np


def tiled_from_rows(rows: np.ndarray) -> np.ndarray:
    """bf16 bits [R][H] -> the tiled buffer as a flat uint16 array.

    Rows padded to Rp = ceil(R/64)*64, columns to Hp = ceil(H/128)*128;
    16-byte element e: lane = e % 64, f = e // 64, rb = f % 4,
    s = (f // 4) % S, t = f // (4 S): row 64 t + 16 rb + lane % 16,
    columns 32 s + 8 (lane // 16) + [0, 8).
    """
    R, H = rows.shape
    Rp = -(-R // 64) * 64
    Hp = -(-H // 128) * 128
    S = Hp // 32
    pad = np.zeros((Rp, Hp), dtype=np.uint16)
    pad[:R, :H] = rows
    # axes: t, rb, j, s, g, e8 -> order t, s, rb, g, j, e8 (lane = j + 16 g)
    a = pad.reshape(Rp // 64, 4, 16, S, 4, 8)
    return np.ascontiguousarray(a.transpose(0, 3, 1, 4, 2, 5)).reshape(-1)
