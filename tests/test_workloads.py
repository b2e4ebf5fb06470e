"""Seeded input generator: rounding, reproducibility, nesting, selection."""

import numpy as np
import torch

from speculative_decoding_argmax_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    r = wl.rng(1, 1)
    x = np.concatenate([r.standard_normal(100_000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40,
                                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_widen_is_exact():
    b = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    back = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(b))
    # -0.0 / +0.0 and every finite pattern round-trip
    assert np.array_equal(back, b)


def test_head_reproducible_and_chunk_independent():
    a = wl.head_weights(9000, 64, 5, threads=1)
    b = wl.head_weights(9000, 64, 5, threads=4)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, wl.head_weights(9000, 64, 6, threads=4))
    f = wl.bf16_bits_to_f32(a)
    assert abs(f.std() - 0.02) < 0.001 and abs(f.mean()) < 0.001


def test_candidate_ids_nested_sorted():
    V = 248_320
    a = wl.candidate_ids(V, 65_536, 20261204)
    b = wl.candidate_ids(V, 32_768, 20261204)
    assert np.all(np.diff(a) > 0) and a.min() >= 0 and a.max() < V
    assert np.isin(b, a).all()
    assert a.dtype == np.int32


def test_select_drafts_rule():
    ids = np.array([2, 5, 9, 14], np.int32)
    t = np.array([[5, 3, 9, 0]], np.int32)
    draws = wl.DraftDraws(agree=np.array([[False, False, True]]), alt=np.array([[1, 3, 0]]))
    d = wl.select_drafts(t, draws, ids)
    # t=5 is ids[1]: draw 1 shifts past it to ids[2]; t=3 is not a candidate:
    # draw 3 picks ids[3]; agreement copies the target.
    assert list(d[0]) == [9, 14, 9]
    B, k = 500, 3
    t = np.tile(np.array([[5, 5, 5, 5]], np.int32), (B, 1))
    d = wl.select_drafts(t, wl.agreement_draws(B, k, 0.0, len(ids), 3), ids)
    assert not np.any(d == 5) and set(np.unique(d)) == {2, 9, 14}


def test_exact_grid_values():
    g = wl.bf16_bits_to_f32(wl.exact_grid_bf16((64, 64), 1))
    q = g * 16
    assert np.array_equal(q, np.rint(q)) and np.abs(q).max() <= 15


def test_tie_partner():
    pool = np.array([1, 4, 6, 9], np.int32)
    assert wl.tie_partner(6, pool, True, 0.99) == 4
    assert wl.tie_partner(6, pool, False, 0.0) == 9
    assert wl.tie_partner(1, pool, True, 0.0) == 4   # nothing below: go above
    d = wl.tie_draws(160, 0.01, 7, 0)
    assert len(d.rows) == 2 and np.all(np.diff(d.rows) > 0)
