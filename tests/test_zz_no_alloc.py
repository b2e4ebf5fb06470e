"""The allocation-free verify (mtp_verify_accept_noalloc) against the verify
with a caller workspace (mtp_verify_accept) and against the oracle, through
the C ABI. Calls come in a row on one stream, each later one smaller than the
one before, so a call that relied on what the previous call left in the
shared scratch would show it."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_accept, check_rows, dev_bf16, dev_i32

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


def _outs(torch, B, k):
    return (torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda"),
            torch.full((B,), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, k + 1), float("nan"), dtype=torch.float32, device="cuda"))


def _host(o):
    a, acc, tok, lg = o
    return {"argmax": a.cpu().numpy(), "accept": acc.cpu().numpy(),
            "tokens": tok.cpu().numpy(), "logit": lg.cpu().numpy()}


# (B, k, V, H, seed): each case smaller than the one before; the first runs the
# matrix-core kernel (32 rows), the second the vector-ALU kernel (4 rows)
CASES = [(8, 3, 60_013, 2048, 11), (1, 3, 20_011, 1024, 12)]


def test_noalloc_verify_matches_workspace_verify(torch, mtp):
    """Random N(0, 0.02) heads: the no-alloc call gives the workspace call's
    outputs bit for bit, and both meet the oracle's near-tie and logit rules;
    acceptance equals the oracle's acceptance of the GPU argmax."""
    results = []
    for B, k, V, H, seed in CASES:
        print(f"[noalloc] B={B} k={k} V={V} H={H}", flush=True)
        W = wl.head_weights(V, H, seed)
        hv = wl.hidden_states(B * (k + 1), H, seed, block=100)
        orc = oracle.argmax(hv, W)
        ids = np.arange(V, dtype=np.int32)
        drafts = wl.select_drafts(orc["id"].reshape(B, k + 1),
                                  wl.agreement_draws(B, k, 0.55, V, seed), ids)
        W_d, hv_d, d_d = dev_bf16(W), dev_bf16(hv), dev_i32(drafts)
        o_ws = _outs(torch, B, k)
        mtp.mtp_verify_accept(hv_d, W_d, d_d, B, k, o_ws[0], o_ws[1], o_ws[2], o_ws[3])
        o_na = _outs(torch, B, k)
        mtp.mtp_verify_accept_noalloc(hv_d, W_d, d_d, B, k, o_na[0], o_na[1], o_na[2], o_na[3])
        torch.cuda.synchronize()
        g_ws, g_na = _host(o_ws), _host(o_na)
        for key in ("argmax", "accept", "tokens"):
            assert np.array_equal(g_na[key], g_ws[key]), key
        assert np.array_equal(g_na["logit"].view(np.uint32), g_ws["logit"].view(np.uint32))
        check_rows(g_na["argmax"].ravel(), g_na["logit"].ravel(), orc, hv, W, None)
        check_accept(g_na, drafts, B, k)
        results.append(g_na)
    assert len(results) == len(CASES)


def test_noalloc_verify_exact_grid_and_limit(torch, mtp):
    """q/16-grid inputs (every fp32 sum exact, many exact ties): ids and logits
    equal the oracle's bit for bit, at the largest call the scratch takes
    (MTP_NOALLOC_MAX_ROWS rows) and then at a single row; one row more is
    refused before anything is enqueued."""
    for B, k, V, H in [(256, 3, 3001, 256), (1, 0, 5003, 512)]:
        print(f"[noalloc exact] B={B} k={k} V={V} H={H}", flush=True)
        M = B * (k + 1)
        x = wl.exact_grid_bf16((M, H), 500 + M, 1)
        w = wl.exact_grid_bf16((V, H), 500 + M, 2)
        orc = oracle.argmax(x, w)
        t = orc["id"].reshape(B, k + 1)
        drafts = t[:, :k].copy()
        if k > 0:
            drafts[::2, k - 1] = -1  # every other sequence disagrees at its last draft
        o = _outs(torch, B, k)
        mtp.mtp_verify_accept_noalloc(dev_bf16(x), dev_bf16(w),
                                      dev_i32(drafts) if k > 0 else None, B, k,
                                      o[0], o[1], o[2], o[3])
        torch.cuda.synchronize()
        g = _host(o)
        assert np.array_equal(g["argmax"].ravel(), orc["id"])
        assert np.array_equal(g["logit"].ravel(), orc["logit"])
        exp = oracle.accept(drafts.reshape(B, k), t)
        assert np.array_equal(g["accept"], exp["accept"])
        assert np.array_equal(g["tokens"], exp["tokens"])
    with pytest.raises(mtp.MTPError) as e:
        B, k = 257, 3
        o = _outs(torch, B, k)
        mtp.mtp_verify_accept_noalloc(
            torch.zeros((B * (k + 1), 256), dtype=torch.int16, device="cuda"),
            torch.zeros((100, 256), dtype=torch.int16, device="cuda"),
            torch.zeros((B, k), dtype=torch.int32, device="cuda"), B, k, o[0], o[1], o[2], o[3])
    assert e.value.status == mtp.MTP_ERR_WORKSPACE
