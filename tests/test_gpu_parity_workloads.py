"""GPU parity at the full workload sizes (248,320-row head), through the C ABI
in the launch configuration the benchmark uses. Every draft row and every
verify row of every workload is checked against the oracle (the largest,
mtp4_large, is about ten seconds of oracle work per layout on the GPU host's
cores), and acceptance is checked exactly against the oracle's acceptance of
the GPU's validated argmax."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import (check_accept, check_rows, dev_bf16, dev_i32, gpu_draft, gpu_verify,
                          make_drafts)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a HIP device"
    return t


@pytest.fixture(scope="module")
def mtp(torch):
    from speculative_decoding_argmax_amd import mtp as m
    return m


def _pack(torch, mtp, W_d, ids, H):
    t = torch.empty((len(ids), H), dtype=torch.int16, device="cuda")
    mtp.mtp_pack_candidates(W_d, dev_i32(ids), t)
    return t


class _Tiled:
    """Draft/verify through the tiled-table entry points."""

    def __init__(self, torch, mtp, W_d, ids_d, C, V, H):
        self.torch, self.mtp, self.C, self.V = torch, mtp, C, V
        self.table = mtp.alloc_tiled(C, H)
        mtp.mtp_pack_tiled(W_d, ids_d, self.table)
        self.head = mtp.alloc_tiled(V, H)
        mtp.mtp_pack_tiled(W_d, None, self.head, C=V)

    def draft(self, h_d, ids_d):
        torch = self.torch
        M = h_d.shape[0]
        oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        ol = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        self.mtp.mtp_draft_argmax_tiled(h_d, self.table, self.C, ids_d, oi, ol)
        torch.cuda.synchronize()
        return oi.cpu().numpy(), ol.cpu().numpy()

    def verify(self, hv_d, drafts, B, k):
        torch = self.torch
        a = torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda")
        lg = torch.full((B, k + 1), float("nan"), dtype=torch.float32, device="cuda")
        acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        tok = torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda")
        self.mtp.mtp_verify_accept_tiled(hv_d, self.head, self.V, dev_i32(drafts), B, k, a, acc,
                                         tok, lg)
        torch.cuda.synchronize()
        return {"argmax": a.cpu().numpy(), "logit": lg.cpu().numpy(),
                "accept": acc.cpu().numpy(), "tokens": tok.cpu().numpy()}


def _drafts_and_verify(torch, mtp, wk, W, draft_rows=None, verify_seqs=None, strict_draft=(),
                       strict_verify=(), layout="rows"):
    """Run the workload's draft calls and its verify call; check the rows
    against the oracle (draft_rows / verify_seqs None: every row)."""
    print(f"[{wk.name}] H={wk.H} V={wk.V} C={wk.C} B={wk.B} k={wk.k} layout={layout}", flush=True)
    ids = wl.candidate_ids(wk.V, wk.C, wk.seed)
    table = oracle.pack(W, ids)
    W_d = dev_bf16(W)
    table_d = _pack(torch, mtp, W_d, ids, wk.H)
    assert np.array_equal(table_d[:64].cpu().numpy().view(np.uint16), table[:64])
    assert np.array_equal(table_d[-64:].cpu().numpy().view(np.uint16), table[-64:])
    ids_d = dev_i32(ids)
    tiled = _Tiled(torch, mtp, W_d, ids_d, wk.C, wk.V, wk.H) if layout == "tiled" else None
    reports = []
    for call in range(wk.draft_calls):
        h = wl.hidden_states(wk.Md, wk.H, wk.seed, block=call)
        if tiled is None:
            g_ids, g_logit = gpu_draft(dev_bf16(h), table_d, ids_d)
        else:
            g_ids, g_logit = tiled.draft(dev_bf16(h), ids_d)
        assert np.isin(g_ids, ids).all()
        rows = list(range(wk.Md)) if draft_rows is None else sorted(
            set(draft_rows) | {r for c, r in strict_draft if c == call})
        orc = oracle.draft(h[rows], table, ids)
        strict = [i for i, r in enumerate(rows) if (call, r) in set(strict_draft)]
        sub_ids, sub_logit = g_ids[rows], g_logit[rows]
        reports.append(check_rows(sub_ids, sub_logit, orc, h[rows], table, ids, strict=strict))
    hv = wl.hidden_states(wk.Mv, wk.H, wk.seed, block=100)
    seqs = list(range(wk.B)) if verify_seqs is None else sorted(
        set(verify_seqs) | {r // (wk.k + 1) for r in strict_verify})
    vrows = [b * (wk.k + 1) + p for b in seqs for p in range(wk.k + 1)]
    orc_v = oracle.argmax(hv[vrows], W)
    t_sub = orc_v["id"].reshape(len(seqs), wk.k + 1)
    # drafts: the workload's agreement law against the oracle's target for the
    # checked sequences; uniform candidates for the others
    t_full = np.zeros((wk.B, wk.k + 1), np.int32)
    t_full[seqs] = t_sub
    drafts = make_drafts(t_full, wk, ids)
    if verify_seqs is not None:
        others = [b for b in range(wk.B) if b not in seqs]
        drafts[others] = wl.uniform_drafts(wk.B, wk.k, ids, wk.seed + 1)[others]
    if tiled is None:
        g = gpu_verify(dev_bf16(hv), W_d, drafts, wk.B, wk.k)
    else:
        g = tiled.verify(dev_bf16(hv), drafts, wk.B, wk.k)
    strict = [i for i, r in enumerate(vrows) if r in set(strict_verify)]
    reports.append(check_rows(g["argmax"].ravel()[vrows], g["logit"].ravel()[vrows], orc_v,
                              hv[vrows], W, None, strict=strict))
    assert ((g["argmax"] >= 0) & (g["argmax"] < wk.V)).all()
    check_accept(g, drafts, wk.B, wk.k)
    acc = g["accept"][seqs]
    print(f"[{wk.name}] checked rows {sum(r.rows for r in reports)} "
          f"({sum(r.rows for r in reports[:-1])} draft, {reports[-1].rows} verify), near-tie rows "
          f"{sum(r.near_tie_rows for r in reports)}, near-tie picks differing "
          f"{sum(r.near_tie_diff for r in reports)}, max logit rel err "
          f"{max(r.max_logit_rel for r in reports):.2e}; accepted {acc.tolist()}", flush=True)
    return g, sum(r.rows for r in reports)


@pytest.mark.timeout(600)
def test_mtp3_single_stream(torch, mtp):
    """MTP3 single stream: H=2048, 65,536-row table, 3 draft calls (M=1),
    verify M=4 against the 248,320-row head, agreement p=0.55."""
    wk = wl.workload("mtp3_single")
    W = wl.head_weights(wk.V, wk.H, wk.seed)
    _drafts_and_verify(torch, mtp, wk, W)


@pytest.mark.timeout(600)
def test_draft_head_ablation(torch, mtp):
    """Draft GEMV+argmax over the full 248,320-row head (identity map, both as
    ids=NULL and as explicit ids), the 65,536-row and the nested 32,768-row
    subsets; plus the 32,768 x 2,560 per-rank shape."""
    wk = wl.workload("draft_ablation")
    W = wl.head_weights(wk.V, wk.H, wk.seed)
    W_d = dev_bf16(W)
    h = wl.hidden_states(wk.Md, wk.H, wk.seed, block=0)
    h_d = dev_bf16(h)
    full = oracle.argmax(h, W)
    g_ids, g_logit = gpu_draft(h_d, W_d, None)
    check_rows(g_ids, g_logit, full, h, W, None)
    ident = np.arange(wk.V, dtype=np.int32)
    g2 = gpu_draft(h_d, W_d, dev_i32(ident))
    assert np.array_equal(g2[0], g_ids) and np.array_equal(g2[1].view(np.uint32),
                                                            g_logit.view(np.uint32))
    # identity table: the draft pick equals the verify argmax of the same row
    hv = np.repeat(h, 4, axis=0)
    gv = gpu_verify(dev_bf16(hv), W_d, np.zeros((1, 3), np.int32), 1, 3)
    assert np.all(gv["argmax"].ravel() == g_ids[0])
    for C in (65_536, 32_768):
        ids = wl.candidate_ids(wk.V, C, wk.seed)
        table = oracle.pack(W, ids)
        t_d = _pack(torch, mtp, W_d, ids, wk.H)
        g = gpu_draft(h_d, t_d, dev_i32(ids))
        check_rows(g[0], g[1], oracle.draft(h, table, ids), h, table, ids)
    # the pages' per-rank shape: 32,768 candidate rows of hidden size 2,560
    V2, H2 = 65_536, 2560
    W2 = wl.head_weights(V2, H2, wk.seed + 100)
    ids2 = wl.candidate_ids(V2, 32_768, wk.seed + 100)
    t2 = oracle.pack(W2, ids2)
    h2 = wl.hidden_states(1, H2, wk.seed + 100)
    g = gpu_draft(dev_bf16(h2), dev_bf16(t2), dev_i32(ids2))
    check_rows(g[0], g[1], oracle.draft(h2, t2, ids2), h2, t2, ids2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_batched_verify(torch, mtp, layout):
    """H=4096: draft calls with 8 rows (x3), verify 8 sequences x 4 = 32 rows."""
    wk = wl.workload("batched_verify")
    W = wl.head_weights(wk.V, wk.H, wk.seed)
    _drafts_and_verify(torch, mtp, wk, W, layout=layout)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_mtp4_large_with_exact_ties(torch, mtp, layout):
    """H=5120: draft calls with 32 rows (x4), verify 32 x 5 = 160 rows, p=0.5;
    1% of verify rows and of first-call draft rows hold an exact tie (the
    winner's head row copied to a partner id before packing, half of the
    partners below the winner), which must resolve to the lower id."""
    wk = wl.workload("mtp4_large")
    W = wl.head_weights(wk.V, wk.H, wk.seed)
    ids = wl.candidate_ids(wk.V, wk.C, wk.seed)
    # exact ties in verify rows
    hv = wl.hidden_states(wk.Mv, wk.H, wk.seed, block=100)
    vt = wl.tie_draws(wk.Mv, wk.tie_frac, wk.seed, 0)
    win = oracle.argmax(hv[vt.rows], W)["id"]
    all_ids = np.arange(wk.V, dtype=np.int32)
    pairs = []
    for j1, lower, u in zip(win, vt.lower, vt.u):
        j2 = wl.tie_partner(int(j1), all_ids, bool(lower), float(u))
        W[j2] = W[int(j1)]
        pairs.append((int(j1), j2))
    # exact ties in draft rows of the first call (partner among the candidates)
    h0 = wl.hidden_states(wk.Md, wk.H, wk.seed, block=0)
    dt = wl.tie_draws(wk.Md, wk.tie_frac, wk.seed, 1)
    dwin = oracle.draft(h0[dt.rows], oracle.pack(W, ids), ids)["id"]
    for j1, lower, u in zip(dwin, dt.lower, dt.u):
        j2 = wl.tie_partner(int(j1), ids, bool(lower), float(u))
        W[j2] = W[int(j1)]
        pairs.append((int(j1), j2))
    print(f"[mtp4_large] tie pairs (winner, partner): {pairs}", flush=True)
    # the injected ties hold on the modified head
    chk = oracle.argmax(hv[vt.rows], W)
    assert np.array_equal(chk["exact"], chk["runner_exact"])
    assert list(chk["id"]) == [min(p) for p in pairs[:len(vt.rows)]]
    strict_draft = [(0, int(r)) for r in dt.rows]
    _, checked = _drafts_and_verify(torch, mtp, wk, W, strict_draft=strict_draft,
                                    strict_verify=[int(r) for r in vt.rows], layout=layout)
    assert checked == wk.draft_calls * wk.Md + wk.Mv == 288
