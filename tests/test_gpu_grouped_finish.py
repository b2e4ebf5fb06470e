"""GPU tests of the grouped cross-workgroup finish. A launch whose workgroups
each stream less than 448 KiB of the table, given the workspace's full size,
merges its winners through 8 group tickets and key sets; given only the
least size (header and one key per row) the same call runs the one-level
finish. Both must return the same bits, match the oracle, and leave the
workspace zeroed, also when calls of both kinds share one workspace."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import (check_accept, check_mxfp4_rows, check_rows, dev_bf16, dev_i32,
                          gpu_draft, gpu_verify)

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


def least_ws(mtp, M):
    """Header and M keys: the smallest workspace a call accepts."""
    return mtp.alloc_workspace(256 + -(-M * 8 // 256) * 256)


def full_ws(mtp, M, N, H):
    return mtp.alloc_workspace(mtp.mtp_draft_workspace_bytes(M, N, H))


def zeroed(torch, ws):
    torch.cuda.synchronize()
    return not bool(ws.cpu().numpy().any())


def same_bits(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.parametrize("M,N,H,bpc", [(1, 16384, 2048, 0), (2, 20000, 2048, 0),
                                       (1, 40, 2048, 0), (1, 9001, 1024, 3), (3, 30001, 256, 7),
                                       (8, 12000, 4096, 0)])
def test_bf16_draft_grouped_equals_one_level(torch, mtp, M, N, H, bpc):
    """Row-major bf16 drafts: full and least workspace give the same bits and
    the oracle's winners; 40 rows make fewer workgroups than groups, 3 and 7
    workgroups per CU make grids that are no multiple of 8."""
    seed = 900 + M + N + H
    W = wl.head_weights(N, H, seed)
    h = wl.hidden_states(M, H, seed)
    W_d, h_d = dev_bf16(W), dev_bf16(h)
    ws_f, ws_l = full_ws(mtp, M, N, H), least_ws(mtp, M)
    g = gpu_draft(h_d, W_d, None, ws=ws_f, blocks_per_cu=bpc)
    o = gpu_draft(h_d, W_d, None, ws=ws_l, blocks_per_cu=bpc)
    same_bits(g, o)
    check_rows(g[0], g[1], oracle.argmax(h, W), h, W, None)
    assert zeroed(torch, ws_f) and zeroed(torch, ws_l)


def test_bf16_verify_grouped_equals_one_level(torch, mtp):
    """Verify of B = 2 sequences with k = 3 over a 20,000-row head (320 KiB
    per workgroup): same argmax, logits, acceptance and tokens both ways,
    and the oracle's acceptance of the oracle's argmax."""
    B, k, V, H = 2, 3, 20000, 2048
    W = wl.head_weights(V, H, 77)
    hv = wl.hidden_states(B * (k + 1), H, 77)
    orc = oracle.argmax(hv, W)
    drafts = wl.select_drafts(orc["id"].reshape(B, k + 1), wl.agreement_draws(B, k, 0.5, V, 77),
                              np.arange(V, dtype=np.int32))
    W_d, hv_d = dev_bf16(W), dev_bf16(hv)
    ws_f = mtp.alloc_workspace(mtp.mtp_verify_workspace_bytes(B, k, V, H))
    ws_l = least_ws(mtp, B * (k + 1))
    g = gpu_verify(hv_d, W_d, drafts, B, k, ws=ws_f)
    o = gpu_verify(hv_d, W_d, drafts, B, k, ws=ws_l)
    for key in ("argmax", "accept", "tokens"):
        assert np.array_equal(g[key], o[key])
    assert np.array_equal(g["logit"].view(np.uint32), o["logit"].view(np.uint32))
    check_rows(g["argmax"].ravel(), g["logit"].ravel(), orc, hv, W, None)
    check_accept(g, drafts, B, k)
    assert zeroed(torch, ws_f) and zeroed(torch, ws_l)


@pytest.mark.parametrize("M", [1, 4])
def test_mxfp4_draft_grouped_equals_one_level(torch, mtp, M):
    """MXFP4 drafts at 32,768 x 2,048 (two workgroups per CU, 70 KiB each):
    the same bits both ways, and the winners of the oracle's MXFP4 draft."""
    N, H = 32768, 2048
    head = wl.head_weights(N, H, 811)
    q = torch.empty((N, H // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((N, H // 32), dtype=torch.uint8, device="cuda")
    mtp.mtp_pack_candidates_mxfp4(dev_bf16(head), None, q, s, C=N)
    x = wl.hidden_states(M, H, 811, block=M)
    x_d = dev_bf16(x)
    outs = []
    for ws in (full_ws(mtp, M, N, H), least_ws(mtp, M)):
        oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        mtp.mtp_draft_argmax_mxfp4(x_d, q, s, None, oi, ol, ws=ws)
        assert zeroed(torch, ws)
        outs.append((oi.cpu().numpy(), ol.cpu().numpy()))
    same_bits(*outs)
    q_ref, s_ref = oracle.quantize_mxfp4(head, None)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    ref = oracle.draft_mxfp4(x, q_ref, s_ref, np.arange(N, dtype=np.int32))
    check_mxfp4_rows(outs[0][0], outs[0][1], ref, x, q_ref, s_ref, np.arange(N, dtype=np.int32))


def test_fp8_draft_grouped_equals_one_level(torch, mtp):
    """fp8 draft, M = 1 at 32,768 x 2,048 (262 KiB per workgroup)."""
    N, H = 32768, 2048
    head = wl.head_weights(N, H, 812)
    q = torch.empty((N, H), dtype=torch.uint8, device="cuda")
    s = torch.empty((N,), dtype=torch.float32, device="cuda")
    mtp.mtp_pack_candidates_fp8(dev_bf16(head), None, q, s, C=N)
    x_d = dev_bf16(wl.hidden_states(1, H, 812))
    outs = []
    for ws in (full_ws(mtp, 1, N, H), least_ws(mtp, 1)):
        oi = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        ol = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        mtp.mtp_draft_argmax_fp8(x_d, q, s, None, oi, ol, ws=ws)
        assert zeroed(torch, ws)
        outs.append((oi.cpu().numpy(), ol.cpu().numpy()))
    same_bits(*outs)


def test_tiled_draft_grouped_equals_one_level(torch, mtp):
    """Tiled bf16 draft, M = 8 at 8,192 x 4,096 (matrix cores, 256 KiB per
    workgroup): the same bits both ways and the oracle's winners."""
    M, N, H = 8, 8192, 4096
    W = wl.head_weights(N, H, 813)
    h = wl.hidden_states(M, H, 813)
    tiled = mtp.alloc_tiled(N, H)
    mtp.mtp_pack_tiled(dev_bf16(W), None, tiled, C=N)
    h_d = dev_bf16(h)
    outs = []
    for ws in (full_ws(mtp, M, N, H), least_ws(mtp, M)):
        oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        mtp.mtp_draft_argmax_tiled(h_d, tiled, N, None, oi, ol, ws=ws)
        assert zeroed(torch, ws)
        outs.append((oi.cpu().numpy(), ol.cpu().numpy()))
    same_bits(*outs)
    check_rows(outs[0][0], outs[0][1], oracle.argmax(h, W), h, W, None)


def test_one_workspace_alternating_finishes(torch, mtp):
    """One full-size workspace serves a long call (one-level finish: 1 MiB
    per workgroup) and short calls (grouped) in turn; every call returns the
    oracle's winner and the workspace ends zeroed."""
    H = 2048
    big, small = 65536, 8192
    Wb = wl.head_weights(big, H, 814)
    ids = np.arange(0, 3 * small, 3, dtype=np.int32)
    table = oracle.pack(Wb, ids)
    Wb_d, t_d, ids_d = dev_bf16(Wb), dev_bf16(table), dev_i32(ids)
    ws = full_ws(mtp, 1, big, H)
    for i in range(6):
        h = wl.hidden_states(1, H, 814, block=i)
        h_d = dev_bf16(h)
        if i % 2 == 0:
            g = gpu_draft(h_d, Wb_d, None, ws=ws)
            check_rows(g[0], g[1], oracle.argmax(h, Wb), h, Wb, None)
        else:
            g = gpu_draft(h_d, t_d, ids_d, ws=ws)
            check_rows(g[0], g[1], oracle.draft(h, table, ids), h, table, ids)
        assert zeroed(torch, ws)
