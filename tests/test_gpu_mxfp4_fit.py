"""GPU parity of the MXFP4 packs under the fit scale rule (the smallest e with
max|w| <= 6 * 2^e over a block, MTP_MX_SCALE_FIT) against the oracle's
quantize_mxfp4(rule="fit"), and of the MXFP4 drafts (packed, tiled and
gathered: the stored format is the same) on tables packed that way."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_mxfp4_rows, dev_bf16, dev_i32
from tests.test_gpu_mxfp4 import special_rows
from tests.tiled_layout import tiled_mxfp4_from

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a HIP device"
    return t


@pytest.fixture(scope="module")
def mtp(torch):
    from speculative_decoding_argmax_amd import mtp as m
    return m


def fit_rows(H: int) -> np.ndarray:
    """Blocks at the fit rule's boundaries (bf16 bits): largest magnitude
    exactly 6 * 2^k, one bf16 step above it, 7 * 2^k and -7.5 * 2^k (OCP
    scales saturate these), 1.5 * 2^k (the largest significand the OCP
    exponent covers) and one step above; subnormal maxima of both kinds."""
    rows = np.zeros((4, H), np.uint16)
    vals = [6.0, 7.0, -7.5, 1.5, 3.0, 5.0]
    for b in range(H // 32):
        k = (b % 9) - 4
        v = np.float32(vals[b % len(vals)] * 2.0 ** k)
        blk = np.linspace(-0.9, 0.9, 32).astype(np.float32) * abs(v) / 6
        rows[0, 32 * b:32 * b + 32] = wl.f32_to_bf16_bits(blk)
        rows[0, 32 * b + b % 32] = wl.f32_to_bf16_bits(np.array([v], np.float32))[0]
        rows[1, 32 * b:32 * b + 32] = rows[0, 32 * b:32 * b + 32]
        rows[1, 32 * b + b % 32] += 1                        # one bf16 step further out
    rows[2] = np.arange(H, dtype=np.uint16) % 0x80          # subnormal maxima
    rows[2, ::32] = 0x0061                                   # significand 0b1100001 > 1.5
    rows[3] = (np.arange(H, dtype=np.uint16) % 0x40) | 0x8000
    return rows


def gpu_pack4(torch, mtp, head, ids, rule):
    V, H = head.shape
    C = len(ids) if ids is not None else V
    q = torch.full((C, H // 2), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((C, H // 32), 0xA5, dtype=torch.uint8, device="cuda")
    mtp.mtp_pack_candidates_mxfp4(dev_bf16(head), None if ids is None else dev_i32(ids), q, s,
                                  C=C, rule=rule)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("V,H", [(300, 32), (2_000, 2_048), (700, 5_120), (64, 16_384), (97, 96)])
def test_pack_mxfp4_fit_bit_exact(torch, mtp, V, H):
    head = wl.normal_bf16_rows(V, H, 0.02, 91 + H, 1)
    head[:6] = special_rows(H)
    head[6:10] = fit_rows(H)
    ids = np.sort(wl.rng(V + H, 7).choice(V, size=min(V, 251), replace=False)).astype(np.int32)
    ids[:10] = np.arange(10)
    ids = np.unique(ids).astype(np.int32)
    for sel in (ids, None):
        q_d, s_d = gpu_pack4(torch, mtp, head, sel, mtp.MTP_MX_SCALE_FIT)
        q_ref, s_ref = oracle.quantize_mxfp4(head, sel, rule="fit")
        q_g, s_g = q_d.cpu().numpy(), s_d.cpu().numpy()
        bad = np.argwhere(q_g != q_ref)
        assert bad.size == 0, f"codes differ at {bad[:5].tolist()}"
        assert np.array_equal(s_g, s_ref)
        # the data reaches blocks where the two rules differ
        assert np.any(s_ref != oracle.quantize_mxfp4(head, sel, rule="ocp")[1])


@pytest.mark.parametrize("R,H", [(130, 2_048), (97, 96), (1_000, 5_120)])
def test_pack_tiled_mxfp4_fit_layout(torch, mtp, R, H):
    V = R + 37
    head = wl.normal_bf16_rows(V, H, 0.02, 47 + H, 1)
    head[:4] = fit_rows(H)
    ids = np.sort(wl.rng(R + H, 8).choice(V, size=R, replace=False)).astype(np.int32)
    q, s = mtp.alloc_tiled_mxfp4(R, H)
    q.fill_(0xA5)
    s.fill_(0xA5)
    mtp.mtp_pack_tiled_mxfp4(dev_bf16(head), dev_i32(ids), q, s, C=R, rule=mtp.MTP_MX_SCALE_FIT)
    torch.cuda.synchronize()
    want_q, want_s = tiled_mxfp4_from(*oracle.quantize_mxfp4(head, ids, rule="fit"))
    assert np.array_equal(q.cpu().numpy(), want_q)
    assert np.array_equal(s.cpu().numpy(), want_s)


def test_draft_mxfp4_fit_workload_data(torch, mtp):
    """N(0, 0.02) head, N(0, 1) hidden, H = 2,048, 32,768 candidate rows packed
    under the fit rule: the draft meets the near-tie rule against the oracle's
    MXFP4 draft over the oracle's fit table."""
    V, H, C = 60_000, 2_048, 32_768
    head = wl.head_weights(V, H, 797)
    ids = wl.candidate_ids(V, C, 797)
    q_d, s_d = gpu_pack4(torch, mtp, head, ids, mtp.MTP_MX_SCALE_FIT)
    q_ref, s_ref = oracle.quantize_mxfp4(head, ids, rule="fit")
    assert np.array_equal(q_d.cpu().numpy(), q_ref) and np.array_equal(s_d.cpu().numpy(), s_ref)
    for M in (1, 4):
        x = wl.hidden_states(M, H, 797, block=M)
        oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        mtp.mtp_draft_argmax_mxfp4(dev_bf16(x), q_d, s_d, dev_i32(ids), oi, ol)
        torch.cuda.synchronize()
        ref = oracle.draft_mxfp4(x, q_ref, s_ref, ids)
        check_mxfp4_rows(oi.cpu().numpy(), ol.cpu().numpy(), ref, x, q_ref, s_ref, ids)


def test_draft_tiled_mxfp4_fit_workload_data(torch, mtp):
    """32 hidden rows at H = 5,120 on a tiled table packed under the fit rule
    (matrix cores), against the oracle under the near-tie rule."""
    V, H, C, M = 20_000, 5_120, 8_192, 32
    head = wl.head_weights(V, H, 801)
    ids = wl.candidate_ids(V, C, 801)
    q, s = mtp.alloc_tiled_mxfp4(C, H)
    mtp.mtp_pack_tiled_mxfp4(dev_bf16(head), dev_i32(ids), q, s, C=C, rule=mtp.MTP_MX_SCALE_FIT)
    x = wl.hidden_states(M, H, 801, block=1)
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_tiled_mxfp4(dev_bf16(x), q, s, C, dev_i32(ids), oi, ol)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_mxfp4(head, ids, rule="fit")
    ref = oracle.draft_mxfp4(x, q_ref, s_ref, ids)
    check_mxfp4_rows(oi.cpu().numpy(), ol.cpu().numpy(), ref, x, q_ref, s_ref, ids)


def test_gather_mxfp4_fit_head(torch, mtp):
    """A head quantised under the fit rule, read through an unsorted id list
    with repeats and out-of-range ids (the gathered MXFP4 draft)."""
    V, H, M = 30_000, 2_048, 2
    head = wl.head_weights(V, H, 809)
    q_d, s_d = gpu_pack4(torch, mtp, head, None, mtp.MTP_MX_SCALE_FIT)
    q_ref, s_ref = oracle.quantize_mxfp4(head, rule="fit")
    r = wl.rng(809, 3)
    ids = r.choice(V, size=12_000, replace=True).astype(np.int32)
    ids[::997] = V + 5                                       # not candidates
    x = wl.hidden_states(M, H, 809, block=2)
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_mxfp4_gather(dev_bf16(x), q_d, s_d, dev_i32(ids), oi, ol)
    torch.cuda.synchronize()
    ref = oracle.draft_mxfp4_gather(x, q_ref, s_ref, ids)
    srt = np.unique(ids[(ids >= 0) & (ids < V)]).astype(np.int32)
    check_mxfp4_rows(oi.cpu().numpy(), ol.cpu().numpy(), ref, x, q_ref[srt], s_ref[srt], srt)
