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


def tiled_mxfp4_from(q: np.ndarray, scales: np.ndarray):
    """Row-major MXFP4 codes [R][H/2] and scales [R][H/32] -> the MXFP4 tiled
    buffers (flat uint8): rows padded to ceil64(R), columns to ceil256(H);
    code fragment (t, p, rb), lane j + 16g, bytes 4u..4u+3 = bytes 4g..4g+3
    of block 4p + u of row 64t + 16rb + j; scale group (t, p), byte
    rb*64 + j*4 + u = scale of that row's block 4p + u (padding: zeros)."""
    R = q.shape[0]
    H = 2 * q.shape[1]
    Rp = -(-R // 64) * 64
    Hp = -(-H // 256) * 256
    SP = Hp // 128
    qp = np.zeros((Rp, Hp // 2), dtype=np.uint8)
    qp[:R, :H // 2] = q
    sp = np.zeros((Rp, Hp // 32), dtype=np.uint8)
    sp[:R, :H // 32] = scales
    # codes: axes t, rb, j, p, u, g, byte -> t, p, rb, g, j, u, byte
    a = qp.reshape(Rp // 64, 4, 16, SP, 4, 4, 4)
    codes = np.ascontiguousarray(a.transpose(0, 3, 1, 5, 2, 4, 6)).reshape(-1)
    # scales: axes t, rb, j, p, u -> t, p, rb, j, u
    b = sp.reshape(Rp // 64, 4, 16, SP, 4)
    sc = np.ascontiguousarray(b.transpose(0, 3, 1, 2, 4)).reshape(-1)
    return codes, sc
