"""Pins for the CPU oracle: checks against values fixed by the pages, by hand,
by exact arithmetic or by closed forms, never against the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle currently
selected in the ``oracle`` module breaks it. ``test_oracle_pins.py`` runs them
on the real oracle; ``test_oracle_mutants.py`` runs them on oracle builds with
a planted mistake and requires every mutant to fail at least one pin.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from speculative_decoding_argmax_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_exact(bits: int) -> Fraction:
    """Exact value of a bfloat16 bit pattern from its fields (sign, 8-bit
    exponent, 7-bit fraction); independent of any float reinterpretation."""
    bits = int(bits)
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite bfloat16")
    if e == 0:
        mag = Fraction(f, 128) * Fraction(1, 2 ** 126)
    else:
        mag = (1 + Fraction(f, 128)) * (Fraction(2) ** (e - 127))
    return sign * mag


def exact_dot(x_bits, w_bits) -> Fraction:
    return sum((bf16_exact(a) * bf16_exact(b) for a, b in zip(x_bits, w_bits)), Fraction(0))


def bits_of(values) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def _first_max(values):
    best = 0
    for i, v in enumerate(values):
        if v > values[best]:
            best = i
    return best


# ---------------------------------------------------------------------------

def pin_worked_logits(oracle):
    """Hand-summed logits and picks of tests/golden/logits_worked.json."""
    g = _golden("logits_worked.json")
    head = bits_of(g["head"])
    q = bits_of(g["queries"])
    # the fixture's values are exact in bfloat16
    assert np.array_equal(wl.bf16_bits_to_f32(head), np.asarray(g["head"], np.float32))
    z = oracle.logits(q, head)
    assert np.array_equal(z, np.asarray(g["logits"], np.float64)), z
    r = oracle.argmax(q, head)
    assert list(r["id"]) == g["full_argmax"], r["id"]
    assert list(r["runner_id"]) == g["full_runner_up"], r["runner_id"]
    ids = np.asarray(g["candidate_ids"], np.int32)
    d = oracle.draft(q, oracle.pack(head, ids), ids)
    assert list(d["id"]) == g["candidate_argmax_id"], d["id"]


def pin_exact_rational(oracle, seed=7):
    """fp64 logits against exact rational dot products, within the error bound
    of a sequential sum: |z - exact| <= (H+1) * 2^-53 * sum|x_j w_j|."""
    r = wl.rng(seed, 99)
    for H, scale_x, scale_w in ((1, 1.0, 1.0), (8, 1.0, 0.02), (37, 3.0, 0.5), (256, 1.0, 0.02)):
        x = bits_of(r.standard_normal((3, H)) * scale_x)
        w = bits_of(r.standard_normal((5, H)) * scale_w)
        z = oracle.logits(x, w)
        for m in range(3):
            for n in range(5):
                ex = exact_dot(x[m], w[n])
                bound = (H + 1) * Fraction(1, 2 ** 53) * sum(
                    abs(bf16_exact(a) * bf16_exact(b)) for a, b in zip(x[m], w[n]))
                assert abs(Fraction(z[m, n]) - ex) <= bound, (H, m, n, z[m, n], float(ex))
    # selected pairs: the same bound, rows and columns taken as given
    rows = np.array([0, 2, 1, 2], np.int64)
    cols = np.array([4, 0, 3, 3], np.int64)
    zp = oracle.pair_logits(x, w, rows, cols)
    for i in range(len(rows)):
        ex = exact_dot(x[rows[i]], w[cols[i]])
        bound = (x.shape[1] + 1) * Fraction(1, 2 ** 53) * sum(
            abs(bf16_exact(a) * bf16_exact(b)) for a, b in zip(x[rows[i]], w[cols[i]]))
        assert abs(Fraction(zp[i]) - ex) <= bound, (i, zp[i], float(ex))
    # widening covers the whole bfloat16 range: tiny, huge and subnormal values
    specials = np.array([0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80, 0x0000,
                         0x8000, 0x4049, 0x3C00], dtype=np.uint16)
    one = np.array([[0x3F80]], dtype=np.uint16)
    zs = oracle.logits(one, specials.reshape(-1, 1))[0]
    for b, v in zip(specials, zs):
        assert Fraction(v) == bf16_exact(b), (hex(int(b)), v)


def pin_exact_grid(oracle, seed=11):
    """Inputs on the grid q/16 (|q| <= 15): logits are exact integer sums
    sum(qx*qw)/256, so the oracle must match them bit for bit, and its pick
    must be the first maximum of those integers."""
    for H, N in ((4, 300), (64, 257), (5120, 40)):
        x = wl.exact_grid_bf16((2, H), seed, 1)
        w = wl.exact_grid_bf16((N, H), seed, 2)
        qx = np.rint(wl.bf16_bits_to_f32(x) * 16).astype(np.int64)
        qw = np.rint(wl.bf16_bits_to_f32(w) * 16).astype(np.int64)
        num = qx @ qw.T          # exact integer numerators over 256
        z = oracle.logits(x, w)
        assert np.array_equal(z * 256.0, num.astype(np.float64))
        r = oracle.argmax(x, w)
        for m in range(2):
            row = [int(v) for v in num[m]]
            best = _first_max(row)
            assert r["id"][m] == best, (H, m, r["id"][m], best)
            assert r["logit"][m] == np.float32(row[best] / 256.0)
            cand = [i for i in range(N) if i != best]
            second = max(cand, key=lambda i: (row[i], -i))
            assert r["runner_id"][m] == second
            assert r["runner_exact"][m] * 256.0 == row[second]


def pin_tie_break(oracle):
    """All-equal, max-at-end and repeated-max rows: the lowest index wins."""
    H = 2
    one = bits_of([[1.0, 0.0]])
    w = bits_of([[0.5, 9.0], [0.5, -3.0], [0.25, 0.0], [0.5, 0.0]])
    assert oracle.argmax(one, w)["id"][0] == 0
    w = bits_of([[0.25, 0.0], [0.125, 0.0], [0.5, 0.0]])
    assert oracle.argmax(one, w)["id"][0] == 2
    w = bits_of([[-1.0, 0.0], [2.0, 0.0], [-2.0, 0.0], [2.0, 1.0], [2.0, 0.0]])
    assert oracle.argmax(one, w)["id"][0] == 1
    # -0.0 and +0.0 are equal: lowest index
    zero_rows = np.array([[0x8000, 0x0000], [0x0000, 0x0000]], dtype=np.uint16)
    w = bits_of([[-1.0, 0.0]])
    w = np.concatenate([w, zero_rows])
    q = bits_of([[1.0, 1.0]])
    assert oracle.argmax(q, w)["id"][0] == 1
    # with an id map the pick is reported as the id of the first maximal row
    ids = np.array([3, 10, 11, 40, 41], np.int32)
    w = bits_of([[-1.0, 0.0], [2.0, 0.0], [-2.0, 0.0], [2.0, 1.0], [2.0, 0.0]])
    assert oracle.argmax(one, w, ids)["id"][0] == 10
    assert H == 2


def pin_candidate_vs_full(oracle, seed=5):
    """An argmax over the packed candidate table equals the full-table argmax
    restricted to the candidate ids (exact logits on the q/16 grid, so the
    restricted first maximum is known exactly)."""
    V, H, C = 3000, 48, 700
    W = wl.exact_grid_bf16((V, H), seed, 3)
    h = wl.exact_grid_bf16((4, H), seed, 4)
    ids = wl.candidate_ids(V, C, seed)
    table = oracle.pack(W, ids)
    assert table.shape == (C, H)
    d = oracle.draft(h, table, ids)
    qh = np.rint(wl.bf16_bits_to_f32(h) * 16).astype(np.int64)
    qW = np.rint(wl.bf16_bits_to_f32(W) * 16).astype(np.int64)
    full = qh @ qW.T
    for m in range(4):
        restricted = [int(full[m, i]) for i in ids]
        assert d["id"][m] == ids[_first_max(restricted)]
    # identity table: draft == full argmax of the same rows
    full_r = oracle.argmax(h, W)
    ident = np.arange(V, dtype=np.int32)
    d_id = oracle.draft(h, oracle.pack(W, ident), ident)
    assert np.array_equal(d_id["id"], full_r["id"])
    for m in range(4):
        assert full_r["id"][m] == _first_max([int(v) for v in full[m]])


def pin_gathered_candidates(oracle, seed=29):
    """Drafting over an id list (unsorted, repeated and out-of-range ids) picks
    the lowest id among the maximal exact logits of the valid distinct ids,
    computed here by brute force on the q/16 grid; a list of only invalid
    ids gives id -1."""
    V, H = 900, 40
    W = wl.exact_grid_bf16((V, H), seed, 1)
    h = wl.exact_grid_bf16((3, H), seed, 2)
    r = wl.rng(seed, 3)
    ids = r.integers(-50, V + 50, size=400).astype(np.int32)
    ids = np.concatenate([ids, ids[:60]])          # repeats
    r.shuffle(ids)
    # force an exact tie between two valid ids, the larger one listed first
    W[611] = W[87]
    ids = np.concatenate([[611], ids, [87]]).astype(np.int32)
    qh = np.rint(wl.bf16_bits_to_f32(h) * 16).astype(np.int64)
    qW = np.rint(wl.bf16_bits_to_f32(W) * 16).astype(np.int64)
    full = qh @ qW.T
    d = oracle.draft_gather(h, W, ids)
    valid = {int(i) for i in ids if 0 <= i < V}
    for m in range(3):
        best = max(full[m, i] for i in valid)
        expect = min(i for i in valid if full[m, i] == best)
        assert d["id"][m] == expect, (m, d["id"][m], expect)
        assert d["logit"][m] == np.float32(best / 256.0)
    # a row made to win by the duplicated pair: the lower id of the two
    h2 = W[[87]].copy()
    d2 = oracle.draft_gather(h2, W, ids)
    s2 = np.rint(wl.bf16_bits_to_f32(h2) * 16).astype(np.int64) @ qW.T
    best2 = max(s2[0, i] for i in valid)
    assert d2["id"][0] == min(i for i in valid if s2[0, i] == best2)
    if s2[0, 87] == best2:
        assert d2["id"][0] == 87
    # sorted distinct ids: the same as drafting over the packed table
    srt = np.array(sorted(valid), np.int32)
    assert np.array_equal(d["id"], oracle.draft(h, oracle.pack(W, srt), srt)["id"])
    none = oracle.draft_gather(h, W, np.array([-1, V, V + 7], np.int32))
    assert np.all(none["id"] == -1) and np.all(np.isnan(none["logit"]))


def _e4m3_table():
    """Values of the 256 E4M3 codes as torch's float8_e4m3fn decodes them."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _nearest_code_brute(x: float, table: np.ndarray) -> int:
    """Nearest finite E4M3 code by exhaustive search; ties to the code with
    mantissa bit 0 clear; beyond the largest magnitude, saturate."""
    finite = [c for c in range(256) if np.isfinite(table[c])]
    if abs(x) >= 448.0:
        return 0xFE if x < 0 else 0x7E
    best = None
    for c in finite:
        if (table[c] == 0.0) and (np.signbit(table[c]) != np.signbit(x)):
            continue                                   # keep the sign of zero
        d = abs(table[c] - x)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def pin_e4m3_format(oracle, seed=41):
    """The E4M3 decode equals torch's float8_e4m3fn for all 256 codes; the
    rounding equals torch's cast for in-range values and an exhaustive
    nearest-even search everywhere (including saturation at 448)."""
    import torch
    table = _e4m3_table()
    ours = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ours), np.isnan(table))
    fin = ~np.isnan(table)
    assert np.array_equal(ours[fin], table[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(table[fin]))
    r = wl.rng(seed, 1)
    mags = np.concatenate([
        r.uniform(0, 448, 3000), np.exp2(r.uniform(-12, 8.8, 3000)), r.uniform(0, 2 ** -6, 500)])
    # exact midpoints between neighbouring finite codes, and the codes themselves
    pos = np.sort(table[(table >= 0) & np.isfinite(table)])
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([mags, pos, mids])
    x = np.concatenate([x, -x]).astype(np.float32).astype(np.float64)
    got = oracle.e4m3_round(x)
    want_t = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(got, want_t.numpy()), "rounding differs from torch's cast"
    extra = np.array([448.0, 460.0, 464.0, 1e6, -500.0, 2 ** -10, -2 ** -10, 3 * 2 ** -10])
    for v in np.concatenate([x[::37], extra]):
        assert int(oracle.e4m3_round([v])[0]) == _nearest_code_brute(float(v), table), v


def pin_fp8_quantize(oracle, seed=43):
    """Per-row scale 2^e is the smallest power of two with max|w| <= 448 * 2^e;
    every element is the nearest E4M3 code of w * 2^-e (error at most half a
    step of its binade); values already on the scaled grid round-trip; an
    all-zero row has e = 0 and zero codes."""
    V, H = 40, 96
    W = wl.normal_bf16_rows(V, H, 0.02, seed, 1)
    W[3] = 0
    W[5] = wl.f32_to_bf16_bits(np.full(H, 448.0, np.float32))
    q, e = oracle.quantize_fp8(W)
    wf = wl.bf16_bits_to_f32(W).astype(np.float64)
    table = _e4m3_table()
    for i in range(V):
        amax = np.abs(wf[i]).max()
        if amax == 0:
            assert e[i] == 0 and not q[i].any()
            continue
        assert amax <= 448.0 * 2.0 ** int(e[i]) and amax > 448.0 * 2.0 ** (int(e[i]) - 1)
        deq = table[q[i]] * 2.0 ** int(e[i])
        y = wf[i] * 2.0 ** -int(e[i])
        step = np.where(np.abs(y) < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2 ** -6))) - 3))
        assert np.all(np.abs(deq - wf[i]) <= 0.5 * step * 2.0 ** int(e[i]) * (1 + 1e-12))
    assert e[5] == 0 and np.all(table[q[5]] == 448.0)
    # rows already on the scaled E4M3 grid come back exactly
    codes = wl.rng(seed, 2).integers(0, 126, size=(4, H)).astype(np.uint8)
    codes[:, 0] = 0x7E                                  # pins the scale to 2^-3
    vals = (table[codes] * 2.0 ** -3).astype(np.float32)
    Wg = wl.f32_to_bf16_bits(vals)
    assert np.array_equal(wl.bf16_bits_to_f32(Wg), vals)
    qg, eg = oracle.quantize_fp8(Wg)
    assert np.all(eg == -3) and np.array_equal(qg, codes)
    # with ids: the rows of the listed head rows
    ids = np.array([1, 3, 7, 30], np.int32)
    qi, ei = oracle.quantize_fp8(W, ids)
    assert np.array_equal(qi, q[ids]) and np.array_equal(ei, e[ids])


def pin_fp8_draft(oracle, seed=47):
    """Head rows of multiples of 1/8 up to 2 quantise exactly (scale 2^-7),
    so with hidden rows on the q/16 grid every fp8 logit is an exact integer
    sum over 128; the pick is the first maximum of those integers and equals
    the bf16 draft over the same rows."""
    V, H, C = 700, 64, 300
    r = wl.rng(seed, 1)
    kq = r.integers(-16, 17, size=(V, H))
    kq[:, 0] = 16                                       # max|w| = 2 in every row
    W = wl.f32_to_bf16_bits((kq / 8.0).astype(np.float32))
    h = wl.exact_grid_bf16((3, H), seed, 2)
    ids = wl.candidate_ids(V, C, seed)
    q, e = oracle.quantize_fp8(W, ids)
    assert np.all(e == -7)
    d8 = oracle.draft_fp8(h, q, e, ids)
    qh = np.rint(wl.bf16_bits_to_f32(h) * 16).astype(np.int64)
    num = qh @ kq[ids].T                                 # logits * 128
    for m in range(3):
        row = [int(v) for v in num[m]]
        best = _first_max(row)
        assert d8["id"][m] == ids[best]
        assert d8["logit"][m] == np.float32(row[best] / 128.0)
    assert np.array_equal(d8["id"], oracle.draft(h, oracle.pack(W, ids), ids)["id"])


def pin_fp8_gathered_candidates(oracle, seed=71):
    """Drafting over an id list on an fp8 head (unsorted, repeated and
    out-of-range ids) picks the lowest id among the maximal exact logits of
    the valid distinct ids. Head rows of multiples of 1/8 up to 2 quantise
    exactly (scale 2^-7), so every fp8 logit is an exact integer sum over 128,
    checked here by brute force; quantising the whole head and gathering rows
    equals quantising the gathered rows; an exact tie planted between two
    valid ids, the larger listed first, goes to the lower one; a list of only
    invalid ids gives id -1."""
    V, H = 800, 48
    r = wl.rng(seed, 1)
    kq = r.integers(-16, 17, size=(V, H))
    kq[:, 0] = 16                                       # max|w| = 2 in every row
    kq[517] = kq[44]                                    # the planted tie
    W = wl.f32_to_bf16_bits((kq / 8.0).astype(np.float32))
    h = wl.exact_grid_bf16((3, H), seed, 2)
    ids = r.integers(-30, V + 30, size=350).astype(np.int32)
    ids = np.concatenate([[517], ids, ids[:40], [44]]).astype(np.int32)
    q, e = oracle.quantize_fp8(W)
    assert np.all(e == -7)
    d = oracle.draft_fp8_gather(h, q, e, ids)
    num = np.rint(wl.bf16_bits_to_f32(h) * 16).astype(np.int64) @ kq.T    # logits * 128
    valid = sorted({int(i) for i in ids if 0 <= i < V})
    for m in range(3):
        best = max(int(num[m, i]) for i in valid)
        expect = min(i for i in valid if int(num[m, i]) == best)
        assert d["id"][m] == expect, (m, d["id"][m], expect)
        assert d["logit"][m] == np.float32(best / 128.0)
    srt = np.array(valid, np.int32)
    q2, e2 = oracle.quantize_fp8(W, srt)
    assert np.array_equal(q2, q[srt]) and np.array_equal(e2, e[srt])
    h2 = wl.f32_to_bf16_bits(np.sign(kq[[44]]).astype(np.float32))
    d2 = oracle.draft_fp8_gather(h2, q, e, ids)
    n2 = np.sign(kq[44]) @ kq.T
    best2 = max(n2[i] for i in valid)
    assert d2["id"][0] == min(i for i in valid if n2[i] == best2)
    if n2[44] == best2:
        assert d2["id"][0] == 44
    none = oracle.draft_fp8_gather(h, q, e, np.array([-3, V, V + 2], np.int32))
    assert np.all(none["id"] == -1) and np.all(np.isnan(none["logit"]))


def _minifloat_magnitudes(ebits: int, mbits: int, bias: int) -> np.ndarray:
    """Values of the non-negative codes of a sign / exponent / mantissa float
    without infinities, indexed by code: exponent field 0 holds the
    subnormals m * 2^(1 - bias - mbits), field e > 0 holds
    (1 + m / 2^mbits) * 2^(e - bias)."""
    vals = []
    for e in range(2 ** ebits):
        for m in range(2 ** mbits):
            vals.append(m * 2.0 ** (1 - bias - mbits) if e == 0
                        else (1 + m / 2 ** mbits) * 2.0 ** (e - bias))
    return np.array(vals)


def _nearest_even_code(x: float, mags: np.ndarray, sign_bit: int) -> int:
    """Brute force: the code of the magnitude nearest to |x| (past the largest,
    the largest; ties to the even code), with the sign bit set for x < 0."""
    a = abs(x)
    d = np.abs(mags - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
    return code | (sign_bit if x < 0 else 0)


def pin_e2m1_format(oracle, seed=53):
    """The field enumeration reproduces torch's E4M3 decode (all finite codes),
    which pins the enumeration; with 2 exponent bits, bias 1 and 1 mantissa
    bit it gives the E2M1 decode (sign in bit 3). Rounding equals a brute-force
    nearest-even search over the 8 magnitudes, at every midpoint and on
    random values, saturating at 6."""
    import torch
    e4 = _minifloat_magnitudes(4, 3, 7)
    t = torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(e4[:127], t[:127].astype(np.float64))
    mags = _minifloat_magnitudes(2, 1, 1)
    assert np.array_equal(mags, [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    got = oracle.e2m1_value(np.arange(16, dtype=np.uint8))
    assert np.array_equal(got[:8], mags) and np.array_equal(got[8:], -mags)
    assert np.all(np.signbit(got[8:]))
    mids = (mags[1:] + mags[:-1]) / 2
    r = wl.rng(seed, 1)
    x = np.concatenate([mags, mids, r.uniform(0, 8, 2000), np.exp2(r.uniform(-4, 3, 1000)),
                        [6.5, 7.0, 100.0, 1e9]])
    x = np.concatenate([x, -x[1:]])
    codes = oracle.e2m1_round(x)
    for v, c in zip(x, codes):
        assert int(c) == _nearest_even_code(float(v), mags, 8), (v, c)


def pin_mxfp4_quantize(oracle, seed=59):
    """Block scales follow the OCP MX rule 2^(e+2) <= max|w| < 2^(e+3) (clamped
    to [-127, 127]; -127 for an all-zero block); every element is the
    nearest-even E2M1 code of w * 2^-e; two codes per byte with the even
    element in the low nibble, one scale byte (e + 127) per 32 elements;
    rows on the scaled grid round-trip; ids select head rows."""
    V, H = 24, 128
    W = wl.normal_bf16_rows(V, H, 0.02, seed, 1)
    W[2] = 0
    W[3, 32:64] = 0                                      # one zero block
    W[4, :32] = 0x0001                                   # smallest subnormal: clamp at -127
    W[4, 32:64] = 0x7F7F                                 # largest finite bf16: e = 125
    q, sc = oracle.quantize_mxfp4(W)
    assert q.shape == (V, H // 2) and sc.shape == (V, H // 32)
    wf = wl.bf16_bits_to_f32(W).astype(np.float64)
    mags = _minifloat_magnitudes(2, 1, 1)
    for i in range(V):
        for b in range(H // 32):
            blk = wf[i, 32 * b:32 * b + 32]
            e = int(sc[i, b]) - 127
            amax = np.abs(blk).max()
            if amax == 0:
                assert e == -127
            elif 2.0 ** -125 <= amax < 2.0 ** 130:
                assert 2.0 ** (e + 2) <= amax < 2.0 ** (e + 3), (i, b, e, amax)
            assert e == oracle.mx_block_exponent(W[i, 32 * b:32 * b + 32])
            for j in range(32 * b, 32 * b + 32):
                byte = int(q[i, j // 2])
                code = byte & 15 if j % 2 == 0 else byte >> 4
                assert code == _nearest_even_code(float(wf[i, j] * 2.0 ** -e), mags, 8), (i, j)
    assert sc[4, 0] == 0 and sc[4, 1] == 125 + 127
    # a row on the scaled grid: element j = +-mags[j % 8] * 2^e_b, block max 6 * 2^e_b
    eb = np.array([-3, -5, 0, 2])
    vals = np.array([mags[j % 8] * (-1) ** (j // 8) * 2.0 ** eb[j // 32] for j in range(H)])
    Wg = wl.f32_to_bf16_bits(vals.astype(np.float32)[None, :])
    qg, sg = oracle.quantize_mxfp4(Wg)
    assert np.array_equal(sg[0], eb + 127)
    for j in range(H):
        code = (j % 8) | (8 if (j // 8) % 2 and j % 8 else 0)
        byte = int(qg[0, j // 2])
        assert (byte & 15 if j % 2 == 0 else byte >> 4) == code, j
    assert np.array_equal(oracle.mxfp4_values(qg, sg)[0], vals)
    ids = np.array([0, 4, 9, 23], np.int32)
    qi, si = oracle.quantize_mxfp4(W, ids)
    assert np.array_equal(qi, q[ids]) and np.array_equal(si, sc[ids])


def pin_mxfp4_fit_quantize(oracle, seed=67):
    """The fit scale rule: the smallest e with max|w| <= 6 * 2^e, i.e.
    6 * 2^(e-1) < max|w| <= 6 * 2^e (clamped to [-127, 127]; -127 for an
    all-zero block), so no element saturates and every code is the
    nearest-even E2M1 code of w * 2^-e. It equals the OCP rule's exponent
    where the OCP scale covers the block (max|w| <= 6 * 2^e_ocp) and is one
    larger where the OCP scale would saturate. Blocks at exactly 6 * 2^k and
    one bf16 step above it, at 7 * 2^k (saturating under the OCP rule), at
    both bf16 extremes and all-zero fix the boundaries; rule "ocp" is the
    default table."""
    V, H = 24, 128
    W = wl.normal_bf16_rows(V, H, 0.02, seed, 1)
    W[2] = 0
    W[3, 32:64] = 0                                      # one zero block
    W[4, :32] = 0x0001                                   # smallest subnormal: clamp at -127
    W[4, 32:64] = 0x7F7F                                 # largest finite bf16: e = 126
    six = wl.f32_to_bf16_bits(np.array([6.0 * 2.0 ** -7], np.float32))[0]
    W[5, :32] = 0
    W[5, 7] = six                                        # max exactly 6 * 2^-7: e = -7
    W[5, 32:64] = 0
    W[5, 40] = six + 1                                   # one bf16 step above: e = -6
    W[5, 64:96] = 0
    W[5, 70] = wl.f32_to_bf16_bits(np.array([-7.0 * 2.0 ** -9], np.float32))[0]  # 7 * 2^-9
    q, sc = oracle.quantize_mxfp4(W, rule="fit")
    q0, sc0 = oracle.quantize_mxfp4(W, rule="ocp")
    qd, scd = oracle.quantize_mxfp4(W)
    assert np.array_equal(q0, qd) and np.array_equal(sc0, scd)
    wf = wl.bf16_bits_to_f32(W).astype(np.float64)
    mags = _minifloat_magnitudes(2, 1, 1)
    raised = 0
    for i in range(V):
        for b in range(H // 32):
            blk = wf[i, 32 * b:32 * b + 32]
            e = int(sc[i, b]) - 127
            e0 = int(sc0[i, b]) - 127
            amax = np.abs(blk).max()
            assert e == oracle.mx_block_exponent(W[i, 32 * b:32 * b + 32], "fit")
            if amax == 0:
                assert e == -127
                continue
            if 2.0 ** -125 <= amax < 2.0 ** 127:
                assert 6.0 * 2.0 ** (e - 1) < amax <= 6.0 * 2.0 ** e, (i, b, e, amax)
                assert e == (e0 if amax <= 6.0 * 2.0 ** e0 else e0 + 1), (i, b, e, e0)
                raised += e != e0
            for j in range(32 * b, 32 * b + 32):
                x = float(wf[i, j] * 2.0 ** -e)
                if e > -127:
                    assert abs(x) <= 6.0
                byte = int(q[i, j // 2])
                code = byte & 15 if j % 2 == 0 else byte >> 4
                assert code == _nearest_even_code(x, mags, 8), (i, j)
    assert raised > 0
    assert sc[4, 0] == 0 and sc[4, 1] == 126 + 127 and sc0[4, 1] == 125 + 127
    assert sc[5, 0] == -7 + 127 and sc[5, 1] == -6 + 127
    assert sc[5, 2] == -8 + 127 and sc0[5, 2] == -9 + 127
    ids = np.array([0, 4, 5, 23], np.int32)
    qi, si = oracle.quantize_mxfp4(W, ids, rule="fit")
    assert np.array_equal(qi, q[ids]) and np.array_equal(si, sc[ids])


def pin_mxfp4_draft(oracle, seed=61):
    """Rows built on the scaled E2M1 grid (every block's max 6 * 2^e, so the
    scale rule returns e) quantise exactly; with hidden rows on the q/16 grid
    every logit is an exact multiple of 2^-8. The pick is the first maximum
    of the exact logits of the original rows, and equals the bf16 draft over
    the same rows, logit included."""
    V, H, C = 600, 96, 250
    r = wl.rng(seed, 1)
    mags = _minifloat_magnitudes(2, 1, 1)
    codes = r.integers(0, 16, size=(V, H))
    codes[:, ::32] = 7                                   # +6 leads every block
    e = r.integers(-3, 1, size=(V, H // 32))
    vals = np.where(codes >= 8, -1.0, 1.0) * mags[codes & 7] * np.exp2(np.repeat(e, 32, axis=1))
    W = wl.f32_to_bf16_bits(vals.astype(np.float32))
    h = wl.exact_grid_bf16((4, H), seed, 2)
    ids = wl.candidate_ids(V, C, seed)
    q, sc = oracle.quantize_mxfp4(W, ids)
    assert np.array_equal(sc.astype(np.int64) - 127, e[ids])
    d4 = oracle.draft_mxfp4(h, q, sc, ids)
    hf = wl.bf16_bits_to_f32(h).astype(np.float64)
    num = np.rint((hf @ vals[ids].T) * 256).astype(np.int64)
    assert np.array_equal(num / 256.0, hf @ vals[ids].T)
    for m in range(4):
        row = [int(v) for v in num[m]]
        best = _first_max(row)
        assert d4["id"][m] == ids[best]
        assert d4["logit"][m] == np.float32(row[best] / 256.0)
    d16 = oracle.draft(h, oracle.pack(W, ids), ids)
    assert np.array_equal(d4["id"], d16["id"]) and np.array_equal(d4["logit"], d16["logit"])


def pin_mxfp4_gathered_candidates(oracle, seed=67):
    """Drafting over an id list on an MXFP4 head (unsorted, repeated and
    out-of-range ids) picks the lowest id among the maximal exact logits of
    the valid distinct ids. Head rows are built on the scaled E2M1 grid, so
    quantisation is exact and every logit is a multiple of 2^-8, checked here
    by integer brute force; quantising the whole head and gathering rows
    equals quantising the gathered rows; an exact tie planted between two
    valid ids, the larger listed first, goes to the lower one; a list of only
    invalid ids gives id -1."""
    V, H = 700, 64
    r = wl.rng(seed, 1)
    mags = _minifloat_magnitudes(2, 1, 1)
    codes = r.integers(0, 16, size=(V, H))
    codes[:, ::32] = 7                                   # +6 leads every block
    e = r.integers(-3, 1, size=(V, H // 32))
    vals = np.where(codes >= 8, -1.0, 1.0) * mags[codes & 7] * np.exp2(np.repeat(e, 32, axis=1))
    vals[433] = vals[58]                                 # the planted tie
    W = wl.f32_to_bf16_bits(vals.astype(np.float32))
    h = wl.exact_grid_bf16((3, H), seed, 2)
    ids = r.integers(-40, V + 40, size=300).astype(np.int32)
    ids = np.concatenate([[433], ids, ids[:50], [58]]).astype(np.int32)
    q, sc = oracle.quantize_mxfp4(W)
    d = oracle.draft_mxfp4_gather(h, q, sc, ids)
    hf = wl.bf16_bits_to_f32(h).astype(np.float64)
    num = np.rint((hf @ vals.T) * 256).astype(np.int64)
    assert np.array_equal(num / 256.0, hf @ vals.T)
    valid = sorted({int(i) for i in ids if 0 <= i < V})
    for m in range(3):
        best = max(int(num[m, i]) for i in valid)
        expect = min(i for i in valid if int(num[m, i]) == best)
        assert d["id"][m] == expect, (m, d["id"][m], expect)
        assert d["logit"][m] == np.float32(best / 256.0)
    srt = np.array(valid, np.int32)
    q2, sc2 = oracle.quantize_mxfp4(W, srt)
    assert np.array_equal(q2, q[srt]) and np.array_equal(sc2, sc[srt])
    h2 = wl.f32_to_bf16_bits(np.sign(vals[[58]]).astype(np.float32))
    d2 = oracle.draft_mxfp4_gather(h2, q, sc, ids)
    n2 = np.sign(vals[58]) @ vals.T
    best2 = max(n2[i] for i in valid)
    assert d2["id"][0] == min(i for i in valid if n2[i] == best2)
    if n2[58] == best2:
        assert d2["id"][0] == 58
    none = oracle.draft_mxfp4_gather(h, q, sc, np.array([-1, V, V + 9], np.int32))
    assert np.all(none["id"] == -1) and np.all(np.isnan(none["logit"]))


def pin_pack(oracle):
    """Packing copies head rows ids[i]; invalid id lists are refused."""
    V, H = 50, 16
    head = (np.arange(V * H, dtype=np.uint32) % 65000).astype(np.uint16).reshape(V, H)
    ids = np.array([0, 7, 8, 31, 49], np.int32)
    t = oracle.pack(head, ids)
    for i, v in enumerate(ids):
        # row v of this head holds v*H .. v*H+H-1
        assert list(t[i]) == [int(v) * H + j for j in range(H)]
    for bad in ([1, 1], [3, 2], [-1, 4], [4, 50]):
        assert not oracle.check_ids(np.array(bad, np.int32), V)
        try:
            oracle.pack(head, np.array(bad, np.int32))
        except oracle.OracleError:
            pass
        else:
            raise AssertionError(f"pack accepted ids {bad}")
    assert oracle.check_ids(ids, V)


def pin_worked_accept(oracle):
    """Hand-worked acceptance cases of tests/golden/accept_worked.json."""
    g = _golden("accept_worked.json")
    total_acc = 0
    total_prop = 0
    for c in g["cases"]:
        k = len(c["draft"])
        tgt = np.asarray([c["target"]], np.int32)
        r = oracle.accept(np.asarray([c["draft"]], np.int32).reshape(1, k), tgt)
        assert int(r["accept"][0]) == c["accept"], c
        assert list(r["tokens"][0]) == c["tokens"], (c, r["tokens"])
        if k == g["acceptance_rate_example"]["k"]:
            total_acc += int(r["accept"][0])
            total_prop += k
    ex = g["acceptance_rate_example"]
    assert Fraction(total_acc, total_prop) == Fraction(ex["value_num"], ex["value_den"])


def pin_worked_verify(oracle):
    """Hand-worked verify steps of tests/golden/verify_worked.json: the rows
    of a [B*(k+1)][H] hidden block are read sequence-major (row b*(k+1)+p is
    position p of sequence b), each takes its full-head argmax (lowest id on
    ties), and acceptance runs on that [B][k+1] target. One case has B = k+1,
    so a position-major reading keeps the shape but fails the values."""
    g = _golden("verify_worked.json")
    perm = g["perm"]
    V = H = len(perm)
    head_f = np.zeros((V, H), np.float32)
    for v, col in enumerate(perm):
        head_f[v, col] = 1.0
    hidden_f = np.asarray(g["hidden"], np.float32)
    head, hidden = bits_of(head_f), bits_of(hidden_f)
    # the fixture's values are exact in bfloat16
    assert np.array_equal(wl.bf16_bits_to_f32(hidden), hidden_f)
    # the fixture's own arithmetic: the logit of id v is hidden[perm[v]]
    for r, row in enumerate(g["hidden"]):
        z = [row[perm[v]] for v in range(V)]
        assert _first_max(z) == g["row_argmax"][r] and max(z) == g["row_max_logit"][r]
    for c in g["cases"]:
        B, k = c["B"], c["k"]
        x = hidden[c["rows"]]
        out = oracle.verify(x, head, B, k, np.asarray(c["draft"], np.int32))
        assert out["id"].shape == (B, k + 1), out["id"].shape
        assert out["id"].tolist() == c["target"], (c["_note"], out["id"].tolist())
        want_logit = np.asarray(g["row_max_logit"], np.float32)[c["rows"]].reshape(B, k + 1)
        assert np.array_equal(out["logit"], want_logit), out["logit"]
        assert out["accept"].tolist() == c["accept"], out["accept"]
        assert out["tokens"].tolist() == c["tokens"], out["tokens"]


def pin_accept_invariants(oracle, seed=3):
    """0 <= n <= k; tokens[:n] == drafts[:n]; tokens[n] == target[n];
    if n < k the draft at n disagrees; slots after n are -1; p=1 accepts all,
    p=0 accepts none, k=0 is plain greedy."""
    r = wl.rng(seed, 17)
    ids = np.arange(0, 400, 3, dtype=np.int32)
    for B, k, p in ((64, 3, 0.55), (64, 4, 0.5), (16, 1, 0.9), (32, 6, 0.7)):
        t = r.integers(0, 400, size=(B, k + 1)).astype(np.int32)
        d = wl.select_drafts(t, wl.agreement_draws(B, k, p, len(ids), seed + k), ids)
        out = oracle.accept(d, t)
        for b in range(B):
            n = int(out["accept"][b])
            assert 0 <= n <= k
            assert list(out["tokens"][b, :n]) == list(d[b, :n])
            assert out["tokens"][b, n] == t[b, n]
            if n < k:
                assert d[b, n] != t[b, n]
            assert all(v == -1 for v in out["tokens"][b, n + 1:])
    B, k = 20, 3
    t = r.integers(0, 400, size=(B, k + 1)).astype(np.int32)
    assert np.all(oracle.accept(t[:, :k], t)["accept"] == k)
    d_all = wl.select_drafts(t, wl.agreement_draws(B, k, 0.0, len(ids), 1), ids)
    assert np.all(oracle.accept(d_all, t)["accept"] == 0)
    g = oracle.accept(np.zeros((B, 0), np.int32), t[:, :1])
    assert np.all(g["accept"] == 0) and np.array_equal(g["tokens"][:, 0], t[:, 0])


def pin_acceptance_law(oracle, seed=23):
    """With i.i.d. agreement p, P(n=j) = p^j (1-p) for j < k and P(n=k) = p^k
    (so E[n] = sum_{j=1..k} p^j). Chi-square over 40,000 seeded sequences."""
    B = 40_000
    ids = np.arange(1000, dtype=np.int32)
    r = wl.rng(seed, 5)
    for k, p in ((3, 0.55), (4, 0.5)):
        t = r.integers(0, 1000, size=(B, k + 1)).astype(np.int32)
        d = wl.select_drafts(t, wl.agreement_draws(B, k, p, len(ids), seed + k), ids)
        n = oracle.accept(d, t)["accept"]
        probs = [p ** j * (1 - p) for j in range(k)] + [p ** k]
        obs = np.bincount(n, minlength=k + 1)
        exp = np.asarray(probs) * B
        chi2 = float(((obs - exp) ** 2 / exp).sum())
        # 99.99th percentile of chi-square with k dof is below 26 for k <= 4
        assert chi2 < 26.0, (k, p, obs, exp, chi2)
        mean_expected = sum(p ** j for j in range(1, k + 1))
        assert abs(n.mean() - mean_expected) < 6 * math.sqrt(n.var() / B)


def pin_pages_layout(oracle):
    """The pages' printed sizes fix a dense [rows][hidden] bfloat16 table."""
    g = _golden("pages_layout.json")
    assert g["draft_rows"] == g["ranks"] * g["rows_per_rank"]
    rows, hidden = g["matched_shape"]
    assert rows == g["rows_per_rank"]
    V = rows  # one rank's share, identity ids: the table equals the head
    head = np.zeros((V, hidden), np.uint16)
    head[:, 0] = np.arange(V, dtype=np.uint16)
    t = oracle.pack(head, np.arange(V, dtype=np.int32))
    assert t.nbytes == g["extra_mib_per_rank"] * 2 ** 20
    assert t.shape == (rows, hidden) and t.dtype == np.uint16
    assert np.array_equal(t, head)


ALL_PINS = [
    pin_worked_logits,
    pin_exact_rational,
    pin_exact_grid,
    pin_tie_break,
    pin_candidate_vs_full,
    pin_gathered_candidates,
    pin_e4m3_format,
    pin_fp8_quantize,
    pin_fp8_draft,
    pin_fp8_gathered_candidates,
    pin_e2m1_format,
    pin_mxfp4_quantize,
    pin_mxfp4_fit_quantize,
    pin_mxfp4_draft,
    pin_mxfp4_gathered_candidates,
    pin_pack,
    pin_worked_accept,
    pin_worked_verify,
    pin_accept_invariants,
    pin_acceptance_law,
    pin_pages_layout,
]
