"""GPU parity of the tiled-table path (matrix cores fed by LDS DMA): layout of
the packing kernel, bit-exact logits on exact-arithmetic inputs, ties,
determinism. Every call goes through the C ABI."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_rows, dev_bf16, dev_i32, exact_logit_match
from tests.tiled_layout import tiled_from_rows

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


def tile_on_gpu(torch, mtp, head, ids=None, C=None):
    V, H = head.shape
    C = len(ids) if ids is not None else (V if C is None else C)
    t = mtp.alloc_tiled(C, H)
    mtp.mtp_pack_tiled(dev_bf16(head), None if ids is None else dev_i32(ids), t, C=C)
    torch.cuda.synchronize()
    return t


def tiled_draft(torch, mtp, h, tiled, C, ids, **kw):
    M = h.shape[0]
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_tiled(dev_bf16(h), tiled, C, None if ids is None else dev_i32(ids), oi,
                               ol, **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ol.cpu().numpy()


@pytest.mark.parametrize("R,H,with_ids", [(1, 8, False), (64, 128, False), (100, 24, False),
                                          (1000, 2560, True), (777, 4096, True),
                                          (65, 5120, False)])
def test_pack_tiled_layout(torch, mtp, R, H, with_ids):
    V = 3 * R + 7 if with_ids else R
    head = wl.head_weights(V, H, R + H)
    ids = wl.candidate_ids(V, R, R) if with_ids else None
    t = tile_on_gpu(torch, mtp, head, ids, R)
    rows = head[ids] if with_ids else head[:R]
    got = t.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, tiled_from_rows(rows))


def test_pack_tiled_bad_ids_are_zero(torch, mtp):
    V, H = 50, 256
    head = wl.head_weights(V, H, 3)
    ids = np.array([3, -1, 60, 7], np.int32)
    t = tile_on_gpu(torch, mtp, head, ids)
    rows = np.stack([head[3], np.zeros(H, np.uint16), np.zeros(H, np.uint16), head[7]])
    assert np.array_equal(t.cpu().numpy().view(np.uint16), tiled_from_rows(rows))


TILED_SHAPES = [  # (M, N, H)
    (1, 1, 8), (1, 1000, 8), (3, 4097, 256), (8, 3001, 4096), (2, 999, 5120), (16, 1025, 640),
    (17, 333, 1032), (32, 5000, 1024), (48, 2049, 4096), (64, 4000, 2048), (100, 700, 512),
    (160, 1111, 5120), (161, 300, 256), (1, 257, 16384), (90, 1500, 1024), (130, 2100, 768),
    # more than 128 rows: the register-ring kernel over the packed hidden block
    (129, 64, 8), (144, 70, 1000), (200, 513, 2056), (320, 257, 136), (4096, 65, 64),
]


@pytest.mark.parametrize("M,N,H", TILED_SHAPES)
@pytest.mark.parametrize("with_ids", [False, True])
def test_tiled_draft_exact_grid(torch, mtp, M, N, H, with_ids):
    seed = 500 + M * 7 + N + H
    x = wl.exact_grid_bf16((M, H), seed, 1)
    w = wl.exact_grid_bf16((N, H), seed, 2)
    ids = np.sort(wl.rng(seed, 3).choice(3 * N + 5, size=N, replace=False)).astype(np.int32) \
        if with_ids else None
    t = tile_on_gpu(torch, mtp, w)
    g_ids, g_logit = tiled_draft(torch, mtp, x, t, N, ids)
    exact_logit_match(g_ids, g_logit, x, w, ids)


@pytest.mark.parametrize("B,k,H,V", [(1, 3, 256, 4096), (8, 3, 4096, 20000), (32, 4, 5120, 3000),
                                     (1, 0, 2048, 777), (40, 3, 1024, 999), (64, 3, 1000, 1234),
                                     (256, 15, 256, 3000)])  # B * (k + 1) = MTP_MAX_ROWS
def test_tiled_verify_exact_grid(torch, mtp, B, k, H, V):
    seed = 91 + B + k + H + V
    hv = wl.exact_grid_bf16((B * (k + 1), H), seed, 1)
    W = wl.exact_grid_bf16((V, H), seed, 2)
    orc = oracle.argmax(hv, W)
    t = orc["id"].reshape(B, k + 1)
    drafts = wl.select_drafts(t, wl.agreement_draws(B, k, 0.6, V, seed),
                              np.arange(V, dtype=np.int32))
    Wt = tile_on_gpu(torch, mtp, W)
    a = torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda")
    lg = torch.full((B, k + 1), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda")
    mtp.mtp_verify_accept_tiled(dev_bf16(hv), Wt, V, dev_i32(drafts) if k else None, B, k, a, acc,
                                tok, lg)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().ravel(), orc["id"])
    assert np.array_equal(lg.cpu().numpy().ravel(), orc["logit"])
    exp = oracle.accept(drafts, t)
    assert np.array_equal(acc.cpu().numpy(), exp["accept"])
    assert np.array_equal(tok.cpu().numpy(), exp["tokens"])


@pytest.mark.parametrize("M", [3, 40, 160])
def test_tiled_duplicate_rows_tie_to_lowest_id(torch, mtp, M):
    V, H = 30000, 2048
    W = wl.head_weights(V, H, 42)
    h = wl.hidden_states(M, H, 42)
    win = oracle.argmax(h, W)["id"]
    for m in range(M):
        j1 = int(win[m])
        lo = (j1 * 7919 + 13) % max(j1, 1) if j1 > 0 else None
        hi = j1 + 1 + (j1 * 104729) % (V - j1 - 1) if j1 < V - 1 else None
        for j2 in (lo, hi):
            if j2 is not None and j2 != j1:
                W[j2] = W[j1]
    orc = oracle.argmax(h, W)
    strict = [m for m in range(M) if orc["runner_exact"][m] == orc["exact"][m]]
    assert len(strict) >= M // 2   # copies for one row can undo another row's tie
    t = tile_on_gpu(torch, mtp, W)
    g_ids, g_logit = tiled_draft(torch, mtp, h, t, V, None)
    check_rows(g_ids, g_logit, orc, h, W, None, strict=strict)


@pytest.mark.parametrize("M", [4, 33, 150])
def test_tiled_determinism_across_grids(torch, mtp, M):
    V, H = 50000, 2048
    W = wl.head_weights(V, H, 9)
    h = wl.hidden_states(M, H, 9)
    t = tile_on_gpu(torch, mtp, W)
    ref = None
    for bpc in (0, 1, 2, 3, 8, 0):
        r = tiled_draft(torch, mtp, h, t, V, None, blocks_per_cu=bpc)
        if ref is None:
            ref = r
        assert np.array_equal(r[0], ref[0])
        assert np.array_equal(r[1].view(np.uint32), ref[1].view(np.uint32))
    check_rows(ref[0], ref[1], oracle.argmax(h, W), h, W, None)


def test_tiled_workspace_left_zeroed(torch, mtp):
    V, H, M = 9000, 1024, 37
    W = wl.head_weights(V, H, 3)
    t = tile_on_gpu(torch, mtp, W)
    nbytes = mtp.mtp_draft_workspace_bytes(M, V, H)
    ws = torch.zeros((nbytes // 8,), dtype=torch.int64, device="cuda")
    out = torch.empty(M, dtype=torch.int32, device="cuda")
    for _ in range(3):
        mtp.mtp_draft_argmax_tiled(dev_bf16(wl.hidden_states(M, H, 3)), t, V, None, out, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.abs().sum()) == 0


def test_tiled_wide_calls_share_one_workspace(torch, mtp):
    """The staging area of the wide calls is scratch that never overlaps any
    call's counters: one workspace, sized for the widest call, serves calls
    of 320, 140, 200 and 40 rows in turn (a narrower call's staging data
    must not sit where a wider call's keys go); each matches the oracle bit
    for bit and leaves its counters zeroed."""
    N, H = 900, 1032
    w = wl.exact_grid_bf16((N, H), 77, 2)
    t = tile_on_gpu(torch, mtp, w)
    ws = mtp.alloc_workspace(mtp.mtp_draft_workspace_bytes(320, N, H))
    for M in (320, 140, 200, 40):
        x = wl.exact_grid_bf16((M, H), 77 + M, 1)
        g_ids, g_logit = tiled_draft(torch, mtp, x, t, N, None, ws=ws)
        exact_logit_match(g_ids, g_logit, x, w, None)
        # every counter a call of up to 4,096 rows could use (256-byte
        # header, one 8-byte key per row) is left zeroed; the staging area
        # past them is scratch
        assert int(ws[:(256 + 4096 * 8) // 8].abs().sum()) == 0
