"""GPU parity of the FP8 candidate table: the quantising pack must write the
oracle's E4M3 codes and power-of-two scales bit for bit, and the fp8 draft
must pick the oracle's ids (near-tie rule on random data, bit-exact logits on
exactly representable data)."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_fp8_rows, dev_bf16, dev_i32

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


def gpu_pack(torch, mtp, head, ids, C=None):
    V, H = head.shape
    C = len(ids) if ids is not None else (V if C is None else C)
    q = torch.empty((C, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(C, dtype=torch.float32, device="cuda")
    mtp.mtp_pack_candidates_fp8(dev_bf16(head), None if ids is None else dev_i32(ids), q, s, C=C)
    torch.cuda.synchronize()
    return q, s


def gpu_draft8(torch, mtp, x, q_d, s_d, ids, **kw):
    M = x.shape[0]
    out_ids = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    out_logit = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_fp8(dev_bf16(x), q_d, s_d, None if ids is None else dev_i32(ids),
                             out_ids, out_logit, **kw)
    torch.cuda.synchronize()
    return out_ids.cpu().numpy(), out_logit.cpu().numpy()


def special_rows(H: int) -> np.ndarray:
    """Rows that reach the format's corners: zero, saturation, a maximum
    exactly 448 * 2^k, and magnitudes in the scaled subnormal range."""
    f = np.zeros((5, H), np.float32)
    f[1, :] = np.linspace(-3.0e4, 3.0e4, H)
    f[2, :] = 0.5
    f[2, 0] = 448.0 * 2.0 ** -7
    f[3, :] = np.linspace(-1, 1, H) * 2.0 ** -20
    f[3, 1] = 2.0 ** -12
    f[4, ::2] = 1.0                                      # scale 2^-8
    f[4, 1::2] = 2.0 ** -16                              # 2^-8 after scaling: subnormal code 2
    f[4, 1:8:2] = 3 * 2.0 ** -18                         # halfway between codes 1 and 2
    return wl.f32_to_bf16_bits(f)


@pytest.mark.parametrize("V,H", [(300, 16), (2_000, 2_048), (700, 5_120), (64, 16_384),
                                 (1_500, 2_560), (97, 48)])
def test_pack_fp8_bit_exact(torch, mtp, V, H):
    head = wl.normal_bf16_rows(V, H, 0.02, 31 + H, 1)
    head[:5] = special_rows(H)
    ids = np.sort(wl.rng(V + H, 2).choice(V, size=min(V, 251), replace=False)).astype(np.int32)
    ids[:5] = np.arange(5)
    ids = np.unique(ids).astype(np.int32)
    for use_ids in (True, False):
        sel = ids if use_ids else None
        q_d, s_d = gpu_pack(torch, mtp, head, sel)
        q_ref, e_ref = oracle.quantize_fp8(head, sel)
        assert np.array_equal(q_d.cpu().numpy(), q_ref)
        assert np.array_equal(s_d.cpu().numpy(), np.ldexp(np.float32(1), e_ref).astype(np.float32))


def test_pack_fp8_out_of_range_id_gives_zero_row(torch, mtp):
    head = wl.normal_bf16_rows(50, 64, 0.02, 5, 1)
    ids = np.array([3, 60, 7], np.int32)            # 60 >= V
    q_d, s_d = gpu_pack(torch, mtp, head, ids)
    q = q_d.cpu().numpy()
    assert not q[1].any() and s_d.cpu().numpy()[1] == 1.0
    q_ref, _ = oracle.quantize_fp8(head, np.array([3, 7], np.int32))
    assert np.array_equal(q[[0, 2]], q_ref)


GRID = [  # (M, C, H)
    (1, 1, 16), (1, 3_000, 2_048), (2, 999, 5_120), (3, 4_097, 1_024), (4, 2_000, 4_096),
    (8, 1_500, 2_048), (9, 800, 1_024), (17, 300, 256), (1, 257, 16_384), (5, 600, 2_560),
]


@pytest.mark.parametrize("M,C,H", GRID)
@pytest.mark.parametrize("with_ids", [False, True])
def test_draft_fp8_exact_grid(torch, mtp, M, C, H, with_ids):
    """Rows of multiples of 1/8 (max 2) quantise exactly and hidden rows on
    the q/16 grid make every partial sum exact: ids and logits bit-exact."""
    r = wl.rng(M * 13 + C + H, 1)
    kq = r.integers(-16, 17, size=(C, H))
    kq[:, 0] = 16
    head = wl.f32_to_bf16_bits((kq / 8.0).astype(np.float32))
    x = wl.exact_grid_bf16((M, H), M + C + H, 2)
    ids = np.sort(r.choice(3 * C + 7, size=C, replace=False)).astype(np.int32) if with_ids \
        else None
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    q_ref, e_ref = oracle.quantize_fp8(head)
    g_ids, g_logit = gpu_draft8(torch, mtp, x, q_d, s_d, ids)
    ref = oracle.draft_fp8(x, q_ref, e_ref, ids)
    assert np.array_equal(g_ids, ref["id"]), (g_ids, ref["id"])
    assert np.array_equal(g_logit, ref["logit"])


def test_draft_fp8_workload_data(torch, mtp):
    """N(0, 0.02) head, N(0, 1) hidden, H = 2,048, 32,768 candidate rows."""
    V, H, C = 60_000, 2_048, 32_768
    head = wl.head_weights(V, H, 777)
    ids = wl.candidate_ids(V, C, 777)
    q_d, s_d = gpu_pack(torch, mtp, head, ids)
    q_ref, e_ref = oracle.quantize_fp8(head, ids)
    assert np.array_equal(q_d.cpu().numpy(), q_ref)
    for M in (1, 2, 4, 8):
        x = wl.hidden_states(M, H, 777, block=M)
        g_ids, g_logit = gpu_draft8(torch, mtp, x, q_d, s_d, ids)
        ref = oracle.draft_fp8(x, q_ref, e_ref, ids)
        check_fp8_rows(g_ids, g_logit, ref, x, q_ref, e_ref, ids)


def test_draft_fp8_duplicate_rows_tie(torch, mtp):
    """Identical rows quantise to identical codes and scales, score
    bit-identically, and the lower id wins."""
    V, H = 4_000, 2_048
    head = wl.head_weights(V, H, 12)
    x = wl.hidden_states(1, H, 12, block=3)
    q, e = oracle.quantize_fp8(head)
    w = int(oracle.draft_fp8(x, q, e)["id"][0])
    partner = 5 if w != 5 else 6
    head[partner] = head[w]
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    g_ids, _ = gpu_draft8(torch, mtp, x, q_d, s_d, None)
    assert g_ids[0] == min(w, partner)


def test_draft_fp8_refuses_matrix_core_path(torch, mtp):
    head = wl.normal_bf16_rows(10, 64, 0.02, 1, 1)
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MTPError):
        mtp.mtp_draft_argmax_fp8(dev_bf16(wl.hidden_states(1, 64, 1)), q_d, s_d, None, out,
                                 path=mtp.MTP_PATH_MFMA)
