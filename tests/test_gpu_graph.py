"""A whole MTP round (three draft calls, then verify with acceptance) captured
into one HIP graph through the C ABI (mtp_graph_begin / end / launch), then
replayed with new inputs written into the captured buffers.

Every replay must equal the same calls made eagerly, bit for bit (same
kernels, same grid, same summation order), with eager work and host
synchronisations between replays; one replay is also checked against the CPU
oracle."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_accept, check_rows, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu

V, C, H, B, K = 12_000, 3_000, 1_024, 2, 3
DRAFTS = 3


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a HIP device"
    return t


@pytest.fixture(scope="module")
def mtp(torch):
    from speculative_decoding_argmax_amd import mtp as m
    return m


class Step:
    """Static device buffers of one MTP round and the calls that use them."""

    def __init__(self, torch, mtp, head, ids, tiled: bool, M: int):
        self.torch, self.mtp, self.tiled, self.M = torch, mtp, tiled, M
        self.head_np = head
        self.ids_np = ids
        self.head = dev_bf16(head)
        self.ids = dev_i32(ids)
        if tiled:
            self.table = mtp.alloc_tiled(C, H)
            mtp.mtp_pack_tiled(self.head, self.ids, self.table, C=C)
            self.head_t = mtp.alloc_tiled(V, H)
            mtp.mtp_pack_tiled(self.head, None, self.head_t, C=V)
        else:
            self.table = torch.empty((C, H), dtype=torch.int16, device="cuda")
            mtp.mtp_pack_candidates(self.head, self.ids, self.table)
        i16, i32, f32 = torch.int16, torch.int32, torch.float32
        self.h = [torch.zeros((M, H), dtype=i16, device="cuda") for _ in range(DRAFTS)]
        self.hv = torch.zeros((B * (K + 1), H), dtype=i16, device="cuda")
        self.draft = torch.zeros((B, K), dtype=i32, device="cuda")
        nws = max(mtp.mtp_draft_workspace_bytes(M, C, H), mtp.mtp_verify_workspace_bytes(B, K, V, H))
        self.ws = mtp.alloc_workspace(nws)
        self.outs = self._outputs()
        torch.cuda.synchronize()

    def _outputs(self):
        torch = self.torch
        i32, f32 = torch.int32, torch.float32
        return {
            "ids": [torch.full((self.M,), -7, dtype=i32, device="cuda") for _ in range(DRAFTS)],
            "dlogit": [torch.full((self.M,), -1.0, dtype=f32, device="cuda") for _ in range(DRAFTS)],
            "argmax": torch.full((B, K + 1), -7, dtype=i32, device="cuda"),
            "vlogit": torch.full((B, K + 1), -1.0, dtype=f32, device="cuda"),
            "accept": torch.full((B,), -7, dtype=i32, device="cuda"),
            "tokens": torch.full((B, K + 1), -7, dtype=i32, device="cuda"),
        }

    def calls(self, o):
        mtp = self.mtp
        for i in range(DRAFTS):
            if self.tiled:
                mtp.mtp_draft_argmax_tiled(self.h[i], self.table, C, self.ids, o["ids"][i],
                                           o["dlogit"][i], ws=self.ws)
            else:
                mtp.mtp_draft_argmax(self.h[i], self.table, self.ids, o["ids"][i],
                                     o["dlogit"][i], ws=self.ws)
        if self.tiled:
            mtp.mtp_verify_accept_tiled(self.hv, self.head_t, V, self.draft, B, K, o["argmax"],
                                        o["accept"], o["tokens"], o["vlogit"], ws=self.ws)
        else:
            mtp.mtp_verify_accept(self.hv, self.head, self.draft, B, K, o["argmax"], o["accept"],
                                  o["tokens"], o["vlogit"], ws=self.ws)

    def set_inputs(self, seed: int):
        torch = self.torch
        hs = [wl.hidden_states(self.M, H, seed, 10 + i) for i in range(DRAFTS)]
        hv = wl.hidden_states(B * (K + 1), H, seed, 20)
        rng = wl.rng(seed, 30)
        d = self.ids_np[rng.integers(0, C, size=(B, K))].astype(np.int32)
        for i in range(DRAFTS):
            self.h[i].copy_(dev_bf16(hs[i]))
        self.hv.copy_(dev_bf16(hv))
        self.draft.copy_(dev_i32(d))
        return hs, hv, d

    @staticmethod
    def snapshot(o):
        return {k: ([t.cpu().numpy().copy() for t in v] if isinstance(v, list) else v.cpu().numpy().copy())
                for k, v in o.items()}


def _equal(a, b):
    for k in a:
        x, y = a[k], b[k]
        if isinstance(x, list):
            for p, q in zip(x, y):
                assert np.array_equal(p.view(np.uint32) if p.dtype == np.float32 else p,
                                      q.view(np.uint32) if q.dtype == np.float32 else q), k
        else:
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y), k


# (True, 160) and (False, 160): wide drafts on a tiled table and on row-major
# rows, two kernels per call (hidden pack into the workspace's staging area,
# then the register-ring kernel) recorded into the graph
@pytest.mark.parametrize("tiled,M", [(False, 1), (False, B), (True, 8), (True, 160), (False, 160)])
def test_graph_replays_equal_eager(torch, mtp, tiled, M):
    head = wl.head_weights(V, H, 9101)
    ids = wl.candidate_ids(V, C, 9101)
    step = Step(torch, mtp, head, ids, tiled, M)
    s = torch.cuda.Stream()
    g = mtp.Graph()
    with torch.cuda.stream(s):
        step.set_inputs(1)
        s.synchronize()
        g.begin()
        step.calls(step.outs)
        g.end()
        eager_outs = step._outputs()
        for rep, seed in enumerate((11, 12, 13, 14)):
            hs, hv, d = step.set_inputs(seed)
            g.launch()
            s.synchronize()
            got = Step.snapshot(step.outs)
            step.calls(eager_outs)            # the same calls, eagerly, same inputs
            s.synchronize()
            _equal(got, Step.snapshot(eager_outs))
            if rep == 0:
                # parity of the replayed round against the CPU oracle
                table = oracle.pack(head, ids)
                for i in range(DRAFTS):
                    ref = oracle.draft(hs[i], table, ids)
                    check_rows(got["ids"][i], got["dlogit"][i], ref, hs[i], table, ids)
                vref = oracle.argmax(hv, head)
                check_rows(got["argmax"].reshape(-1), got["vlogit"].reshape(-1), vref, hv, head,
                           None)
                check_accept({"argmax": got["argmax"], "accept": got["accept"],
                              "tokens": got["tokens"]}, d, B, K)
            # unrelated eager work between replays
            x = torch.randn(1 << 16, device="cuda")
            _ = float((x * 2).sum())
    g.destroy()


def test_capture_refuses_implicit_workspace(torch, mtp):
    """Inside a capture the binding refuses to allocate a workspace."""
    head = wl.head_weights(2_000, 64, 5)
    ids = wl.candidate_ids(2_000, 500, 5)
    h = dev_bf16(wl.hidden_states(1, 64, 5, 1))
    table = torch.empty((500, 64), dtype=torch.int16, device="cuda")
    mtp.mtp_pack_candidates(dev_bf16(head), dev_i32(ids), table)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = mtp.Graph()
    with torch.cuda.stream(s):
        g.begin()
        try:
            with pytest.raises(ValueError):
                mtp.mtp_draft_argmax(h, table, None, out)
        finally:
            try:
                g.end()          # ends the (empty) capture
            except mtp.MTPError:
                pass             # an empty graph may not instantiate; capture has ended
    g.destroy()


def test_graph_api_argument_errors(torch, mtp):
    import ctypes
    assert mtp.lib.mtp_graph_begin(None) == mtp.MTP_ERR_INVALID_ARG
    assert mtp.lib.mtp_graph_launch(None, None) == mtp.MTP_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert mtp.lib.mtp_graph_end(None, ctypes.byref(h)) == mtp.MTP_ERR_INVALID_ARG
    assert not h
    mtp.lib.mtp_graph_destroy(None)


@pytest.mark.parametrize("kind", ["fp8", "mxfp4", "gather_bf16", "gather_fp8", "gather_mxfp4"])
def test_graph_replays_quantised_and_gathered_drafts(torch, mtp, kind):
    """Three draft calls on an fp8 or MXFP4 table, or through per-call id
    lists (bf16, fp8 or MXFP4 head), captured into one graph. Each replay
    runs with new hidden rows and, for gathered drafts, new id lists written
    into the captured list buffers; it must equal the same calls made
    eagerly bit for bit, and the first replay meets the oracle's rule."""
    from tests.parity import check_fp8_rows, check_mxfp4_rows
    head = wl.head_weights(V, H, 9202)
    ids = wl.candidate_ids(V, C, 9202)
    head_d, ids_d = dev_bf16(head), dev_i32(ids)
    fmt = kind.split("_")[-1]
    gather = kind.startswith("gather")
    rows = V if gather else C
    sel = None if gather else ids_d
    u8, i16, i32, f32 = torch.uint8, torch.int16, torch.int32, torch.float32
    q = s8 = None
    if fmt == "fp8":
        q = torch.empty((rows, H), dtype=u8, device="cuda")
        s8 = torch.empty(rows, dtype=f32, device="cuda")
        mtp.mtp_pack_candidates_fp8(head_d, sel, q, s8, C=rows)
    elif fmt == "mxfp4":
        q = torch.empty((rows, H // 2), dtype=u8, device="cuda")
        s8 = torch.empty((rows, H // 32), dtype=u8, device="cuda")
        mtp.mtp_pack_candidates_mxfp4(head_d, sel, q, s8, C=rows)
    h = [torch.zeros((1, H), dtype=i16, device="cuda") for _ in range(DRAFTS)]
    lists = [torch.zeros(C, dtype=i32, device="cuda") for _ in range(DRAFTS)] if gather else None
    ws = mtp.alloc_workspace(mtp.mtp_draft_workspace_bytes(1, C, H))

    def outputs():
        return {"ids": [torch.full((1,), -7, dtype=i32, device="cuda") for _ in range(DRAFTS)],
                "dlogit": [torch.full((1,), -1.0, dtype=f32, device="cuda")
                           for _ in range(DRAFTS)]}

    def calls(o):
        for i in range(DRAFTS):
            a = (o["ids"][i], o["dlogit"][i])
            if kind == "fp8":
                mtp.mtp_draft_argmax_fp8(h[i], q, s8, ids_d, *a, ws=ws)
            elif kind == "mxfp4":
                mtp.mtp_draft_argmax_mxfp4(h[i], q, s8, ids_d, *a, ws=ws)
            elif kind == "gather_bf16":
                mtp.mtp_draft_argmax_gather(h[i], head_d, lists[i], *a, ws=ws)
            elif kind == "gather_fp8":
                mtp.mtp_draft_argmax_fp8_gather(h[i], q, s8, lists[i], *a, ws=ws)
            else:
                mtp.mtp_draft_argmax_mxfp4_gather(h[i], q, s8, lists[i], *a, ws=ws)

    def set_inputs(seed):
        hs = [wl.hidden_states(1, H, seed, 10 + i) for i in range(DRAFTS)]
        ls = []
        for i in range(DRAFTS):
            h[i].copy_(dev_bf16(hs[i]))
            if gather:
                lst = wl.candidate_ids(V, C, seed * 10 + i)
                wl.rng(seed, 40 + i).shuffle(lst)
                lists[i].copy_(dev_i32(lst))
                ls.append(lst)
        return hs, ls

    outs = outputs()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = mtp.Graph()
    with torch.cuda.stream(s):
        set_inputs(1)
        s.synchronize()
        g.begin()
        calls(outs)
        g.end()
        eager = outputs()
        for rep, seed in enumerate((21, 22, 23)):
            hs, ls = set_inputs(seed)
            g.launch()
            s.synchronize()
            got = Step.snapshot(outs)
            calls(eager)
            s.synchronize()
            _equal(got, Step.snapshot(eager))
            if rep == 0:
                if fmt != "bf16":
                    quant = oracle.quantize_fp8 if fmt == "fp8" else oracle.quantize_mxfp4
                    qr, sr = quant(head, None if gather else ids)
                for i in range(DRAFTS):
                    gi, gl = got["ids"][i], got["dlogit"][i]
                    srt = np.unique(ls[i]).astype(np.int32) if gather else ids
                    if fmt == "bf16":
                        w = oracle.pack(head, srt)
                        check_rows(gi, gl, oracle.draft(hs[i], w, srt), hs[i], w, srt)
                        continue
                    qs, ss = (qr[srt], sr[srt]) if gather else (qr, sr)
                    if fmt == "fp8":
                        check_fp8_rows(gi, gl, oracle.draft_fp8(hs[i], qs, ss, srt), hs[i], qs,
                                       ss, srt)
                    else:
                        check_mxfp4_rows(gi, gl, oracle.draft_mxfp4(hs[i], qs, ss, srt), hs[i],
                                         qs, ss, srt)
            x = torch.randn(1 << 16, device="cuda")
            _ = float((x * 2).sum())
    g.destroy()
