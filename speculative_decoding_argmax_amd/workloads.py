"""Seeded synthetic inputs for the MTP draft / verify LM-head path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no dot products, no argmax, no acceptance): wherever an
input depends on a result of the method (drafts that agree with the target's
argmax, rows forced into an exact logit tie) it returns the random draws and a
selection helper that takes that result as an argument. Both the CPU oracle
(tests) and the HIP path (tests, bench) take their inputs from here.

Sources of the workload shapes:
  * Qwen3.8 Flash dual-Spark tuning log (cnblogs), section "read one fewer big
    table" (少读一张大表): a 248,320-row output head, a 65,536-row draft table
    split 32,768 rows per rank, and the full-vocab / 64K / 32K ablation table.
    The candidate set there was built from the author's private corpus; a
    seeded, sorted random subset stands in for it (the 32K set nested in the
    64K set so the ablation shares one draw).
  * The same page, section "MTP guesses one more step": MTP3 and MTP4 draft
    depths (k = 3, k = 4).

Distributions: weights N(0, 0.02) and hidden states N(0, 1), drawn in fp32 and
rounded to bfloat16 with round-to-nearest-even. 0.02 is read as the standard
deviation. Random streams are numpy ``default_rng(SeedSequence([seed, stream,
...]))`` with one stream id per kind of draw, so every array is reproducible on
its own and independent of generation order or chunking.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

# Stream identifiers (second word of every SeedSequence).
STREAM_WEIGHTS = 1
STREAM_HIDDEN = 2
STREAM_SUBSET = 3
STREAM_DRAFTS = 4
STREAM_TIES = 5
STREAM_EXACT = 6

BASE_SEED = 20261202

# Rows of the weight matrix generated per random stream chunk. Fixed, so the
# head is the same whatever thread count generates it.
_ROWS_PER_CHUNK = 4096


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), *[int(s) for s in stream]]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even).

    Returns the bfloat16 bit patterns as uint16. Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_rows(n_rows: int, cols: int, std: float, seed: int, stream: int,
                     threads: int = 8) -> np.ndarray:
    """[n_rows][cols] bfloat16 bits, N(0, std^2), generated in fixed row chunks.

    Chunk c (rows c*4096 ...) uses SeedSequence([seed, stream, c]).
    """
    out = np.empty((n_rows, cols), dtype=np.uint16)
    n_chunks = (n_rows + _ROWS_PER_CHUNK - 1) // _ROWS_PER_CHUNK

    def one(c: int) -> None:
        r0 = c * _ROWS_PER_CHUNK
        r1 = min(n_rows, r0 + _ROWS_PER_CHUNK)
        g = rng(seed, stream, c)
        x = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(x)

    if n_chunks == 1 or threads <= 1:
        for c in range(n_chunks):
            one(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n_chunks)))
    return out


def head_weights(V: int, H: int, seed: int, threads: int = 8) -> np.ndarray:
    """Full output head [V][H] as bfloat16 bits, N(0, 0.02)."""
    return normal_bf16_rows(V, H, 0.02, seed, STREAM_WEIGHTS, threads)


def hidden_states(M: int, H: int, seed: int, block: int = 0) -> np.ndarray:
    """Hidden block [M][H] as bfloat16 bits, N(0, 1). ``block`` picks an
    independent block (e.g. the i-th sequential draft call)."""
    g = rng(seed, STREAM_HIDDEN, block)
    return f32_to_bf16_bits(g.standard_normal((M, H), dtype=np.float32))


def candidate_ids(V: int, C: int, seed: int) -> np.ndarray:
    """Sorted first C entries of a seeded permutation of [0, V) (int32).

    For a fixed seed, the C=32,768 set is contained in the C=65,536 set.
    """
    if not 0 < C <= V:
        raise ValueError("need 0 < C <= V")
    perm = rng(seed, STREAM_SUBSET).permutation(V)
    return np.sort(perm[:C]).astype(np.int32)


def exact_grid_bf16(shape: Sequence[int], seed: int, stream: int = 0) -> np.ndarray:
    """Values q/16 with q uniform in [-15, 15], as bfloat16 bits.

    Every such value and every product of two of them is exact in bf16 / fp32,
    and any sum of up to 5,120 products is a multiple of 1/256 below 2^24/256
    in magnitude, so it is exact in fp32 in every summation order.
    """
    g = rng(seed, STREAM_EXACT, stream)
    q = g.integers(-15, 16, size=tuple(shape))
    return f32_to_bf16_bits((q.astype(np.float32) / np.float32(16.0)))


# ---------------------------------------------------------------------------
# Drafts: random draws, then a selection that takes the target argmax as input.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DraftDraws:
    agree: np.ndarray   # [B][k] bool: draft equals the target's token
    alt: np.ndarray     # [B][k] int64 in [0, C-2]: which other candidate otherwise


def agreement_draws(B: int, k: int, p: float, C: int, seed: int) -> DraftDraws:
    g = rng(seed, STREAM_DRAFTS, 0)
    u = g.random((B, k))
    alt = g.integers(0, max(C - 1, 1), size=(B, k))
    return DraftDraws(agree=u < p, alt=alt)


def uniform_drafts(B: int, k: int, ids: np.ndarray, seed: int) -> np.ndarray:
    """Drafts drawn i.i.d. uniformly over the candidate ids (int32 [B][k])."""
    g = rng(seed, STREAM_DRAFTS, 1)
    return ids[g.integers(0, len(ids), size=(B, k))].astype(np.int32)


def select_drafts(target: np.ndarray, draws: DraftDraws, ids: np.ndarray) -> np.ndarray:
    """Build drafts d[b][p] from the target tokens t[b][p] (p < k).

    Where ``agree`` holds, d = t (even if t is not a candidate). Otherwise d is
    a candidate id different from t, uniform over the C-1 (or C) choices: the
    draw a in [0, C-2] is shifted past t's own position when t is a candidate.
    """
    B, k = draws.agree.shape
    t = np.asarray(target, dtype=np.int64)[:, :k]
    d = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        for p in range(k):
            if draws.agree[b, p]:
                d[b, p] = t[b, p]
                continue
            a = int(draws.alt[b, p])
            j = int(np.searchsorted(ids, t[b, p]))
            if j < len(ids) and ids[j] == t[b, p]:
                a = a + (1 if a >= j else 0)
            d[b, p] = ids[min(a, len(ids) - 1)]
    return d


# ---------------------------------------------------------------------------
# Exact ties: draws, then a row copy driven by the winners the caller found.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class TieDraws:
    rows: np.ndarray    # query rows chosen to hold a tie
    lower: np.ndarray   # bool per row: put the partner below the winner
    u: np.ndarray       # uniform [0,1) per row: where to put the partner


def tie_draws(n_rows: int, frac: float, seed: int, stream: int) -> TieDraws:
    """Choose ceil(frac * n_rows) rows (sorted) plus placement draws."""
    g = rng(seed, STREAM_TIES, stream)
    n = int(np.ceil(frac * n_rows))
    rows = np.sort(g.choice(n_rows, size=n, replace=False))
    return TieDraws(rows=rows, lower=g.random(n) < 0.5, u=g.random(n))


def tie_partner(winner: int, pool: np.ndarray, lower: bool, u: float) -> int:
    """A partner id from ``pool`` (sorted ids) strictly below or above
    ``winner`` (the other side if that side is empty), chosen by ``u``."""
    pool = np.asarray(pool)
    below = pool[pool < winner]
    above = pool[pool > winner]
    side = below if (lower and len(below)) or not len(above) else above
    if not len(side):
        raise ValueError("pool holds no id other than the winner")
    return int(side[min(int(u * len(side)), len(side) - 1)])


# ---------------------------------------------------------------------------
# Named workloads.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    index: int
    H: int
    V: int
    C: int                    # candidate rows of the draft table
    B: int                    # sequences
    k: int                    # drafts per sequence
    draft_calls: int          # sequential draft calls per MTP round
    p: Optional[float]        # draft agreement probability (None: uniform drafts)
    tie_frac: float = 0.0
    tables: Optional[List[int]] = None   # draft-table sizes timed (ablation)

    @property
    def Md(self) -> int:
        return self.B

    @property
    def Mv(self) -> int:
        return self.B * (self.k + 1)

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index


VOCAB = 248_320

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, H=256, V=4096, C=1024, B=1, k=3, draft_calls=3, p=None),
    "mtp3_single": Workload("mtp3_single", 1, H=2048, V=VOCAB, C=65_536, B=1, k=3,
                            draft_calls=3, p=0.55),
    "draft_ablation": Workload("draft_ablation", 2, H=2048, V=VOCAB, C=65_536, B=1, k=3,
                               draft_calls=1, p=None, tables=[VOCAB, 65_536, 32_768]),
    "batched_verify": Workload("batched_verify", 3, H=4096, V=VOCAB, C=65_536, B=8, k=3,
                               draft_calls=3, p=0.55),
    "mtp4_large": Workload("mtp4_large", 4, H=5120, V=VOCAB, C=65_536, B=32, k=4,
                           draft_calls=4, p=0.5, tie_frac=0.01),
}


def workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
