"""GPU parity of the MXFP4 candidate table: the quantising pack must write
the oracle's E2M1 codes (nibble order included) and E8M0 block scales bit for
bit, and the MXFP4 draft must pick the oracle's ids (bit-exact logits on
exactly representable data, near-tie rule on random data)."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_mxfp4_rows, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a HIP device"
    return t


@pytest.fixture(scope="module")
def mtp(torch):
    from speculative_decoding_argmax_amd import mtp as m
    return m


def gpu_pack4(torch, mtp, head, ids, C=None):
    V, H = head.shape
    C = len(ids) if ids is not None else (V if C is None else C)
    q = torch.full((C, H // 2), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((C, H // 32), 0xA5, dtype=torch.uint8, device="cuda")
    mtp.mtp_pack_candidates_mxfp4(dev_bf16(head), None if ids is None else dev_i32(ids), q, s, C=C)
    torch.cuda.synchronize()
    return q, s


def gpu_draft4(torch, mtp, x, q_d, s_d, ids, **kw):
    M = x.shape[0]
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_mxfp4(dev_bf16(x), q_d, s_d, None if ids is None else dev_i32(ids), oi,
                               ol, **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ol.cpu().numpy()


def special_rows(H: int) -> np.ndarray:
    """Rows that reach the format's corners (bf16 bits): a zero row; every
    rounding midpoint of a block scaled by 2^-3; negatives that round to zero
    and -0; wide ranges that saturate; the smallest subnormals (scale clamped
    at 2^-127) and the largest finite bf16 (scale 2^125)."""
    rows = np.zeros((6, H), np.uint16)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0])
    v = np.tile(np.concatenate([mids, -mids]), H // 16)[:H] * 2.0 ** -3
    rows[1] = wl.f32_to_bf16_bits(v.astype(np.float32))
    v = np.full(H, -0.1)
    v[::32] = 4.0
    rows[2] = wl.f32_to_bf16_bits(v.astype(np.float32))
    rows[2, 1::7] = 0x8000                                   # -0
    rows[3] = wl.f32_to_bf16_bits(np.linspace(-3.0e4, 3.0e4, H).astype(np.float32))
    rows[4] = np.arange(H, dtype=np.uint16) % 0x80           # subnormals and zeros
    rows[5] = wl.f32_to_bf16_bits(np.linspace(-1, 1, H).astype(np.float32))
    rows[5, 0] = 0x7F7F                                      # largest finite bf16
    return rows


@pytest.mark.parametrize("V,H", [(300, 32), (2_000, 2_048), (700, 5_120), (64, 16_384),
                                 (97, 96), (1_500, 2_560)])
def test_pack_mxfp4_bit_exact(torch, mtp, V, H):
    head = wl.normal_bf16_rows(V, H, 0.02, 71 + H, 1)
    head[:6] = special_rows(H)
    ids = np.sort(wl.rng(V + H, 5).choice(V, size=min(V, 251), replace=False)).astype(np.int32)
    ids[:6] = np.arange(6)
    ids = np.unique(ids).astype(np.int32)
    for use_ids in (True, False):
        sel = ids if use_ids else None
        q_d, s_d = gpu_pack4(torch, mtp, head, sel)
        q_ref, s_ref = oracle.quantize_mxfp4(head, sel)
        q_g, s_g = q_d.cpu().numpy(), s_d.cpu().numpy()
        bad = np.argwhere(q_g != q_ref)
        assert bad.size == 0, f"codes differ at {bad[:5].tolist()}: {q_g[tuple(bad[0])]:#x} vs {q_ref[tuple(bad[0])]:#x}"
        assert np.array_equal(s_g, s_ref)


def test_pack_mxfp4_out_of_range_id_gives_zero_row(torch, mtp):
    head = wl.normal_bf16_rows(50, 64, 0.02, 5, 1)
    ids = np.array([3, 60, 7], np.int32)                     # 60 >= V
    q_d, s_d = gpu_pack4(torch, mtp, head, ids)
    q, s = q_d.cpu().numpy(), s_d.cpu().numpy()
    assert not q[1].any() and not s[1].any()
    q_ref, s_ref = oracle.quantize_mxfp4(head, np.array([3, 7], np.int32))
    assert np.array_equal(q[[0, 2]], q_ref) and np.array_equal(s[[0, 2]], s_ref)


def grid_rows(V: int, H: int, seed: int) -> np.ndarray:
    """bf16 rows on the scaled E2M1 grid: every block of 32 leads with
    6 * 2^e (e in -3..0), so the block scale is 2^e and every element
    quantises exactly."""
    r = wl.rng(seed, 7)
    codes = r.integers(0, 16, size=(V, H))
    codes[:, ::32] = 7
    e = r.integers(-3, 1, size=(V, H // 32))
    vals = np.where(codes >= 8, -1.0, 1.0) * E2M1[codes & 7] * np.exp2(np.repeat(e, 32, axis=1))
    return wl.f32_to_bf16_bits(vals.astype(np.float32))


GRID = [  # (M, C, H)
    (1, 1, 32), (1, 3_000, 2_048), (2, 999, 5_120), (3, 4_097, 1_024), (4, 2_000, 4_096),
    (8, 1_500, 2_048), (9, 800, 1_024), (17, 300, 256), (1, 257, 16_384), (5, 600, 2_560),
    (3, 333, 96),
]


@pytest.mark.parametrize("M,C,H", GRID)
@pytest.mark.parametrize("with_ids", [False, True])
def test_draft_mxfp4_exact_grid(torch, mtp, M, C, H, with_ids):
    """Rows on the scaled E2M1 grid quantise exactly and hidden rows on the
    q/16 grid make every partial sum exact: ids and logits bit-exact, exact
    ties included (the lower id wins)."""
    head = grid_rows(C, H, M * 11 + C + H)
    x = wl.exact_grid_bf16((M, H), M + C + H, 4)
    r = wl.rng(M + 3 * C + H, 8)
    ids = np.sort(r.choice(3 * C + 7, size=C, replace=False)).astype(np.int32) if with_ids \
        else None
    q_d, s_d = gpu_pack4(torch, mtp, head, None)
    q_ref, s_ref = oracle.quantize_mxfp4(head)
    assert np.array_equal(q_d.cpu().numpy(), q_ref) and np.array_equal(s_d.cpu().numpy(), s_ref)
    g_ids, g_logit = gpu_draft4(torch, mtp, x, q_d, s_d, ids)
    ref = oracle.draft_mxfp4(x, q_ref, s_ref, ids)
    assert np.array_equal(g_ids, ref["id"]), (g_ids, ref["id"])
    assert np.array_equal(g_logit, ref["logit"])


def test_draft_mxfp4_workload_data(torch, mtp):
    """N(0, 0.02) head, N(0, 1) hidden, H = 2,048, 32,768 candidate rows."""
    V, H, C = 60_000, 2_048, 32_768
    head = wl.head_weights(V, H, 779)
    ids = wl.candidate_ids(V, C, 779)
    q_d, s_d = gpu_pack4(torch, mtp, head, ids)
    q_ref, s_ref = oracle.quantize_mxfp4(head, ids)
    assert np.array_equal(q_d.cpu().numpy(), q_ref) and np.array_equal(s_d.cpu().numpy(), s_ref)
    for M in (1, 2, 4, 8):
        x = wl.hidden_states(M, H, 779, block=M)
        g_ids, g_logit = gpu_draft4(torch, mtp, x, q_d, s_d, ids)
        assert np.isin(g_ids, ids).all()
        ref = oracle.draft_mxfp4(x, q_ref, s_ref, ids)
        check_mxfp4_rows(g_ids, g_logit, ref, x, q_ref, s_ref, ids)


def test_draft_mxfp4_duplicate_rows_tie(torch, mtp):
    """Identical rows quantise to identical codes and scales, score
    bit-identically, and the lower id wins."""
    V, H = 4_000, 2_048
    head = wl.head_weights(V, H, 13)
    x = wl.hidden_states(1, H, 13, block=3)
    q, s = oracle.quantize_mxfp4(head)
    w = int(oracle.draft_mxfp4(x, q, s)["id"][0])
    partner = 5 if w != 5 else 6
    head[partner] = head[w]
    q_d, s_d = gpu_pack4(torch, mtp, head, None)
    g_ids, _ = gpu_draft4(torch, mtp, x, q_d, s_d, None)
    assert g_ids[0] == min(w, partner)


def test_draft_mxfp4_refuses_matrix_core_path(torch, mtp):
    head = wl.normal_bf16_rows(10, 64, 0.02, 1, 1)
    q_d, s_d = gpu_pack4(torch, mtp, head, None)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MTPError):
        mtp.mtp_draft_argmax_mxfp4(dev_bf16(wl.hidden_states(1, 64, 1)), q_d, s_d, None, out,
                                   path=mtp.MTP_PATH_MFMA)
