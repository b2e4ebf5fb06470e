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


def tiled_fp8_from_codes(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes [R][H] -> the fp8 tiled buffer as a flat uint8 array.

    Rows padded to Rp = ceil(R/64)*64, columns to Hp = ceil(H/128)*128;
    1 KiB fragment (t, p, rb) in that order, lane j + 16 g holding 16 bytes:
    row 64 t + 16 rb + j at columns 64 p + 8 g + [0, 8), then at columns
    64 p + 32 + 8 g + [0, 8).
    """
    R, H = codes.shape
    Rp = -(-R // 64) * 64
    Hp = -(-H // 128) * 128
    P = Hp // 64
    pad = np.zeros((Rp, Hp), dtype=np.uint8)
    pad[:R, :H] = codes
    # axes: t, rb, j, p, half, g, e8 -> order t, p, rb, g, j, half, e8
    a = pad.reshape(Rp // 64, 4, 16, P, 2, 4, 8)
    return np.ascontiguousarray(a.transpose(0, 3, 1, 5, 2, 4, 6)).reshape(-1)
