"""GPU parity of the MXFP4 candidate table in the tiled layout (batched
drafts on the matrix cores): the pack must write the oracle's codes and
block scales in the documented fragment and scale-group order (zero padding
included); each step's codes are converted with their block's scale into an
exact bf16 operand, so the draft must equal the bf16 tiled draft over the
dequantised rows bit for bit, and pick the oracle's ids (bit-exact on exactly
representable data, near-tie rule on workload data), over one and several
64-row passes of hidden rows."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_mxfp4_rows, dev_bf16, dev_i32
from tests.test_gpu_mxfp4 import grid_rows, special_rows
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


def tiled_pack4(torch, mtp, head_d, ids, C, H):
    """MXFP4 tiled table of C rows; buffers start as 0xA5 so that padding the
    pack fails to write shows up."""
    q, s = mtp.alloc_tiled_mxfp4(C, H)
    q.fill_(0xA5)
    s.fill_(0xA5)
    mtp.mtp_pack_tiled_mxfp4(head_d, None if ids is None else dev_i32(ids), q, s, C=C)
    torch.cuda.synchronize()
    return q, s


def tiled_draft4(torch, mtp, x, q, s, C, ids, **kw):
    M = x.shape[0]
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_tiled_mxfp4(dev_bf16(x), q, s, C, None if ids is None else dev_i32(ids),
                                     oi, ol, **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ol.cpu().numpy()


@pytest.mark.parametrize("R,H", [(300, 32), (64, 256), (130, 2_048), (1_000, 5_120), (97, 96),
                                 (65, 2_560), (1, 288)])
@pytest.mark.parametrize("with_ids", [False, True])
def test_pack_tiled_mxfp4_layout(torch, mtp, R, H, with_ids):
    V = R + 37
    head = wl.normal_bf16_rows(V, H, 0.02, 43 + H, 1)
    head[:6] = special_rows(H)[: min(6, V)]
    ids = None
    if with_ids:
        ids = np.sort(wl.rng(R + H, 6).choice(V, size=R, replace=False)).astype(np.int32)
    q_d, s_d = tiled_pack4(torch, mtp, dev_bf16(head), ids, R, H)
    q, sc = oracle.quantize_mxfp4(head if ids is not None else head[:R], ids)
    want_q, want_s = tiled_mxfp4_from(q, sc)
    got_q, got_s = q_d.cpu().numpy(), s_d.cpu().numpy()
    assert got_q.size == want_q.size and got_s.size == want_s.size
    bad = np.flatnonzero(got_q != want_q)
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:8]}"
    bad = np.flatnonzero(got_s != want_s)
    assert bad.size == 0, f"{bad.size} scale bytes differ, first at {bad[:8]}"


GRID = [  # (M, C, H): 1..4 row blocks, several 64-row passes, ragged tiles and columns
    (1, 1, 32), (1, 3_000, 2_048), (2, 999, 5_120), (3, 4_097, 1_024), (8, 2_000, 4_096),
    (16, 1_500, 2_048), (17, 800, 1_024), (33, 300, 256), (48, 257, 2_560), (64, 2_100, 768),
    (65, 700, 1_024), (100, 1_030, 512), (130, 513, 2_048), (5, 64, 16_384), (40, 129, 96),
]


@pytest.mark.parametrize("M,C,H", GRID)
@pytest.mark.parametrize("with_ids", [False, True])
def test_draft_tiled_mxfp4_exact_grid(torch, mtp, M, C, H, with_ids):
    """Rows on the scaled E2M1 grid quantise exactly and hidden rows on the
    q/16 grid make every partial sum exact: ids and logits bit-exact, exact
    ties included (the lower id wins)."""
    head = grid_rows(C, H, M * 13 + C + H)
    x = wl.exact_grid_bf16((M, H), M + C + H, 5)
    r = wl.rng(M * 5 + C + H, 9)
    ids = np.sort(r.choice(3 * C + 7, size=C, replace=False)).astype(np.int32) if with_ids \
        else None
    q_d, s_d = tiled_pack4(torch, mtp, dev_bf16(head), None, C, H)
    q, sc = oracle.quantize_mxfp4(head)
    g_ids, g_logit = tiled_draft4(torch, mtp, x, q_d, s_d, C, ids)
    ref = oracle.draft_mxfp4(x, q, sc, ids)
    assert np.array_equal(g_ids, ref["id"]), (g_ids, ref["id"])
    assert np.array_equal(g_logit, ref["logit"])


@pytest.mark.parametrize("M", [1, 8, 32, 64, 80])
def test_draft_tiled_mxfp4_equals_bf16_over_dequantised_rows(torch, mtp, M):
    """On N(0, 0.02) rows the MXFP4 tiled draft equals, bit for bit, the bf16
    tiled draft over the dequantised rows (the operands are the same bf16
    values and the MFMA sequence is the same), and meets the near-tie rule
    against the oracle's MXFP4 logits."""
    V, H, C = 40_000, 2_048, 16_384
    head = wl.head_weights(V, H, 903)
    ids = wl.candidate_ids(V, C, 903)
    q_d, s_d = tiled_pack4(torch, mtp, dev_bf16(head), ids, C, H)
    q, sc = oracle.quantize_mxfp4(head, ids)
    deq = wl.f32_to_bf16_bits(oracle.mxfp4_values(q, sc).astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(deq).astype(np.float64), oracle.mxfp4_values(q, sc))
    t16 = mtp.alloc_tiled(C, H)
    mtp.mtp_pack_tiled(dev_bf16(deq), None, t16, C=C)
    x = wl.hidden_states(M, H, 903, block=M)
    g_ids, g_logit = tiled_draft4(torch, mtp, x, q_d, s_d, C, ids)
    oi = torch.empty(M, dtype=torch.int32, device="cuda")
    ol = torch.empty(M, dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_tiled(dev_bf16(x), t16, C, dev_i32(ids), oi, ol)
    torch.cuda.synchronize()
    assert np.array_equal(g_ids, oi.cpu().numpy())
    assert np.array_equal(g_logit.view(np.uint32), ol.cpu().numpy().view(np.uint32))
    ref = oracle.draft_mxfp4(x, q, sc, ids)
    check_mxfp4_rows(g_ids, g_logit, ref, x, q, sc, ids)


def test_draft_tiled_mxfp4_duplicate_rows_tie(torch, mtp):
    """Identical rows quantise and score identically; the lower id wins, with
    the partner in another 64-row tile."""
    V, H = 4_000, 2_048
    head = wl.head_weights(V, H, 17)
    x = wl.hidden_states(4, H, 17, block=2)
    q, sc = oracle.quantize_mxfp4(head)
    w = oracle.draft_mxfp4(x, q, sc)["id"]
    for m, wm in enumerate(w):
        head[(int(wm) + 700 + 64 * m) % V] = head[wm]
    q_d, s_d = tiled_pack4(torch, mtp, dev_bf16(head), None, V, H)
    g_ids, _ = tiled_draft4(torch, mtp, x, q_d, s_d, V, None)
    q, sc = oracle.quantize_mxfp4(head)
    assert np.array_equal(g_ids, oracle.draft_mxfp4(x, q, sc)["id"])


@pytest.mark.parametrize("name", ["batched_verify", "mtp4_large"])
@pytest.mark.timeout(600)
def test_draft_tiled_mxfp4_workload_sizes(torch, mtp, name):
    """The workload's draft shape (65,536 candidates of the 248,320-row head;
    8 rows at H = 4,096, 32 rows at H = 5,120) in the benchmark's launch
    configuration: layout checked, every row of the first call checked
    against the oracle."""
    wk = wl.workload(name)
    print(f"[{name}] mxfp4 tiled draft M={wk.Md} C={wk.C} H={wk.H}", flush=True)
    W = wl.head_weights(wk.V, wk.H, wk.seed)
    ids = wl.candidate_ids(wk.V, wk.C, wk.seed)
    q_d, s_d = tiled_pack4(torch, mtp, dev_bf16(W), ids, wk.C, wk.H)
    q, sc = oracle.quantize_mxfp4(W, ids)
    del W
    want_q, want_s = tiled_mxfp4_from(q, sc)
    assert np.array_equal(q_d.cpu().numpy(), want_q)
    assert np.array_equal(s_d.cpu().numpy(), want_s)
    x = wl.hidden_states(wk.Md, wk.H, wk.seed, block=0)
    g_ids, g_logit = tiled_draft4(torch, mtp, x, q_d, s_d, wk.C, ids)
    ref = oracle.draft_mxfp4(x, q, sc, ids)
    check_mxfp4_rows(g_ids, g_logit, ref, x, q, sc, ids)


def test_draft_tiled_mxfp4_refuses_valu_path(torch, mtp):
    head = wl.normal_bf16_rows(10, 64, 0.02, 1, 1)
    q_d, s_d = tiled_pack4(torch, mtp, dev_bf16(head), None, 10, 64)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MTPError):
        mtp.mtp_draft_argmax_tiled_mxfp4(dev_bf16(wl.hidden_states(1, 64, 1)), q_d, s_d, 10, None,
                                         out, path=mtp.MTP_PATH_VALU)
