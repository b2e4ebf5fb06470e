"""GPU parity of the fp8 candidate table in the tiled layout (batched drafts
on the matrix cores): the pack must write the oracle's E4M3 codes in the
documented fragment order (zero padding included) and its power-of-two
scales bit for bit, and the draft must pick the oracle's ids (bit-exact on
exactly representable data, near-tie rule on workload data), over one and
several 64-row passes of hidden rows."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_fp8_rows, dev_bf16, dev_i32
from tests.test_gpu_fp8 import special_rows
from tests.tiled_layout import tiled_fp8_from_codes

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


def tiled_pack(torch, mtp, head_d, ids, C, H):
    """fp8 tiled table of C rows; the buffer starts as 0xA5 so that padding
    the pack fails to clear shows up."""
    q, s = mtp.alloc_tiled_fp8(C, H)
    q.fill_(0xA5)
    s.fill_(-3.0)
    mtp.mtp_pack_tiled_fp8(head_d, None if ids is None else dev_i32(ids), q, s, C=C)
    torch.cuda.synchronize()
    return q, s


def tiled_draft8(torch, mtp, x, q, s, C, ids, **kw):
    M = x.shape[0]
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_tiled_fp8(dev_bf16(x), q, s, C, None if ids is None else dev_i32(ids),
                                   oi, ol, **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ol.cpu().numpy()


@pytest.mark.parametrize("R,H", [(300, 16), (64, 128), (130, 2_048), (1_000, 5_120), (97, 48),
                                 (65, 2_560), (1, 144)])
@pytest.mark.parametrize("with_ids", [False, True])
def test_pack_tiled_fp8_layout(torch, mtp, R, H, with_ids):
    V = R + 37
    head = wl.normal_bf16_rows(V, H, 0.02, 41 + H, 1)
    head[:5] = special_rows(H)[: min(5, V)]
    ids = None
    if with_ids:
        ids = np.sort(wl.rng(R + H, 3).choice(V, size=R, replace=False)).astype(np.int32)
    q_d, s_d = tiled_pack(torch, mtp, dev_bf16(head), ids, R, H)
    codes, exps = oracle.quantize_fp8(head if ids is not None else head[:R], ids)
    want = tiled_fp8_from_codes(codes)
    got = q_d.cpu().numpy()
    assert got.size == want.size == mtp.mtp_tiled_fp8_bytes(R, H)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
    assert np.array_equal(s_d.cpu().numpy(), np.ldexp(np.float32(1), exps).astype(np.float32))


GRID = [  # (M, C, H): 1..4 row blocks, several 64-row passes, ragged tiles and columns
    (1, 1, 16), (1, 3_000, 2_048), (2, 999, 5_120), (3, 4_097, 1_024), (8, 2_000, 4_096),
    (16, 1_500, 2_048), (17, 800, 1_024), (33, 300, 256), (48, 257, 2_560), (64, 2_100, 768),
    (65, 700, 1_024), (100, 1_030, 512), (130, 513, 2_048), (5, 64, 16_384), (40, 129, 48),
]


@pytest.mark.parametrize("M,C,H", GRID)
@pytest.mark.parametrize("with_ids", [False, True])
def test_draft_tiled_fp8_exact_grid(torch, mtp, M, C, H, with_ids):
    """Head rows of multiples of 1/8 (max 2) quantise exactly and hidden rows
    on the q/16 grid make every partial sum exact: ids and logits bit-exact,
    exact ties included (the lower id wins)."""
    r = wl.rng(M * 17 + C + H, 4)
    kq = r.integers(-16, 17, size=(C, H))
    kq[:, 0] = 16
    head = wl.f32_to_bf16_bits((kq / 8.0).astype(np.float32))
    x = wl.exact_grid_bf16((M, H), M + C + H, 3)
    ids = np.sort(r.choice(3 * C + 7, size=C, replace=False)).astype(np.int32) if with_ids \
        else None
    q_d, s_d = tiled_pack(torch, mtp, dev_bf16(head), None, C, H)
    codes, exps = oracle.quantize_fp8(head)
    g_ids, g_logit = tiled_draft8(torch, mtp, x, q_d, s_d, C, ids)
    ref = oracle.draft_fp8(x, codes, exps, ids)
    assert np.array_equal(g_ids, ref["id"]), (g_ids, ref["id"])
    assert np.array_equal(g_logit, ref["logit"])


@pytest.mark.parametrize("M", [1, 8, 32, 64, 80])
def test_draft_tiled_fp8_workload_data(torch, mtp, M):
    """N(0, 0.02) head, N(0, 1) hidden, H = 2,048, 16,384 candidate rows of a
    40,000-row head."""
    V, H, C = 40_000, 2_048, 16_384
    head = wl.head_weights(V, H, 901)
    ids = wl.candidate_ids(V, C, 901)
    q_d, s_d = tiled_pack(torch, mtp, dev_bf16(head), ids, C, H)
    codes, exps = oracle.quantize_fp8(head, ids)
    x = wl.hidden_states(M, H, 901, block=M)
    g_ids, g_logit = tiled_draft8(torch, mtp, x, q_d, s_d, C, ids)
    assert np.isin(g_ids, ids).all()
    ref = oracle.draft_fp8(x, codes, exps, ids)
    check_fp8_rows(g_ids, g_logit, ref, x, codes, exps, ids)


def test_draft_tiled_fp8_duplicate_rows_tie(torch, mtp):
    """Identical rows quantise and score identically; the lower id wins, with
    the partner in another 64-row tile."""
    V, H = 4_000, 2_048
    head = wl.head_weights(V, H, 13)
    x = wl.hidden_states(4, H, 13, block=2)
    codes, exps = oracle.quantize_fp8(head)
    w = oracle.draft_fp8(x, codes, exps)["id"]
    for m, wm in enumerate(w):
        partner = (int(wm) + 700 + 64 * m) % V
        head[partner] = head[wm]
    q_d, s_d = tiled_pack(torch, mtp, dev_bf16(head), None, V, H)
    g_ids, _ = tiled_draft8(torch, mtp, x, q_d, s_d, V, None)
    codes, exps = oracle.quantize_fp8(head)
    ref = oracle.draft_fp8(x, codes, exps)
    assert np.array_equal(g_ids, ref["id"])


@pytest.mark.parametrize("name", ["batched_verify", "mtp4_large"])
@pytest.mark.timeout(600)
def test_draft_tiled_fp8_workload_sizes(torch, mtp, name):
    """The workload's draft shape (65,536 candidates of the 248,320-row head;
    8 rows at H=4,096, 32 rows at H=5,120) in the benchmark's launch
    configuration: every row of the first call checked against the oracle."""
    wk = wl.workload(name)
    print(f"[{name}] fp8 tiled draft M={wk.Md} C={wk.C} H={wk.H}", flush=True)
    W = wl.head_weights(wk.V, wk.H, wk.seed)
    ids = wl.candidate_ids(wk.V, wk.C, wk.seed)
    q_d, s_d = tiled_pack(torch, mtp, dev_bf16(W), ids, wk.C, wk.H)
    codes, exps = oracle.quantize_fp8(W, ids)
    del W
    sample = np.arange(0, wk.C, 997)
    got = q_d.cpu().numpy()
    want = tiled_fp8_from_codes(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(s_d.cpu().numpy()[sample],
                          np.ldexp(np.float32(1), exps[sample]).astype(np.float32))
    x = wl.hidden_states(wk.Md, wk.H, wk.seed, block=0)
    g_ids, g_logit = tiled_draft8(torch, mtp, x, q_d, s_d, wk.C, ids)
    ref = oracle.draft_fp8(x, codes, exps, ids)
    check_fp8_rows(g_ids, g_logit, ref, x, codes, exps, ids)


def test_draft_tiled_fp8_refuses_valu_path(torch, mtp):
    head = wl.normal_bf16_rows(10, 64, 0.02, 1, 1)
    q_d, s_d = tiled_pack(torch, mtp, dev_bf16(head), None, 10, 64)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MTPError):
        mtp.mtp_draft_argmax_tiled_fp8(dev_bf16(wl.hidden_states(1, 64, 1)), q_d, s_d, 10, None,
                                       out, path=mtp.MTP_PATH_VALU)
