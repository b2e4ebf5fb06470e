"""Host logic of bench.py that runs without a GPU: the one-GPU guard, and the
parity summary that sets the GPU's outputs against the oracle's."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from speculative_decoding_argmax_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _tiny():
    wk = wl.workload("tiny")
    head = wl.head_weights(wk.V, wk.H, wk.seed)
    ids = wl.candidate_ids(wk.V, wk.C, wk.seed)
    hiddens = [wl.hidden_states(wk.Md, wk.H, wk.seed, block=c) for c in range(wk.draft_calls)]
    hv = wl.hidden_states(wk.Mv, wk.H, wk.seed, block=100)
    drafts = wl.uniform_drafts(wk.B, wk.k, ids, wk.seed)
    base, orc = bench.cpu_baseline(wk, head, ids, hiddens, hv, drafts, 0.0)
    return wk, head, ids, hiddens, hv, drafts, base, orc


def _as_gpu(wk, orc, drafts):
    """Outputs shaped like the GPU's, copied from the oracle's."""
    g_drafts = [(d["id"].copy(), d["logit"].copy()) for d in orc["drafts"]]
    v = orc["verify"]
    import oracle
    acc = oracle.accept(drafts, v["id"])
    g_verify = {"argmax": v["id"].copy(), "logit": v["logit"].copy(),
                "accept": acc["accept"].copy(), "tokens": acc["tokens"].copy()}
    return g_drafts, g_verify


def test_parity_summary_passes_the_oracle_itself():
    wk, head, ids, hiddens, hv, drafts, base, orc = _tiny()
    assert base["kind"] == "oracle" and base["cores"] >= 1
    g_drafts, g_verify = _as_gpu(wk, orc, drafts)
    p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g_drafts, g_verify)
    assert p["ok"] and p["accept_equal"]
    assert p["draft"]["rows"] == wk.draft_calls * wk.Md == p["draft"]["exact"]
    assert p["verify"]["rows"] == wk.Mv == p["verify"]["exact"]
    assert p["draft"]["violations"] == p["verify"]["violations"] == 0


def test_parity_summary_flags_wrong_picks_logits_and_acceptance():
    wk, head, ids, hiddens, hv, drafts, base, orc = _tiny()
    # a draft pick that is a candidate but far from the maximum
    g_drafts, g_verify = _as_gpu(wk, orc, drafts)
    ref = orc["drafts"][0]
    far = next(int(i) for i in ids if int(i) != int(ref["id"][0]) and
               bench_logit(hiddens[0], head, int(i)) < ref["exact"][0] - 0.1)
    g_drafts[0][0][0] = far
    p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g_drafts, g_verify)
    assert not p["ok"] and p["draft"]["violations"] == 1
    # a logit off by 1%
    g_drafts, g_verify = _as_gpu(wk, orc, drafts)
    g_verify["logit"].reshape(-1)[1] *= 1.01
    p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g_drafts, g_verify)
    assert not p["ok"] and p["verify"]["violations"] == 1
    # acceptance that does not follow the verify argmax
    g_drafts, g_verify = _as_gpu(wk, orc, drafts)
    g_verify["accept"][0] = (int(g_verify["accept"][0]) + 1) % (wk.k + 1)
    p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g_drafts, g_verify)
    assert not p["ok"] and not p["accept_equal"]


def test_parity_summary_on_quantised_and_gathered_drafts():
    """fp8 and MXFP4 tables, and gathered lists, are checked against the
    oracle's own quantisation and candidate sets: the oracle's outputs pass,
    and a pick that is not in the call's candidate set is a violation."""
    import oracle
    wk, head, ids, hiddens, hv, drafts, base, orc = _tiny()
    _, g_verify = _as_gpu(wk, orc, drafts)
    q8, e8 = oracle.quantize_fp8(head, ids)
    q4, s4 = oracle.quantize_mxfp4(head, ids)
    cases = {
        "fp8": [oracle.draft_fp8(h, q8, e8, ids) for h in hiddens],
        "mxfp4": [oracle.draft_mxfp4(h, q4, s4, ids) for h in hiddens],
    }
    for table, refs in cases.items():
        g = [(r["id"].copy(), r["logit"].copy()) for r in refs]
        p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g, g_verify, table)
        assert p["ok"] and p["draft"]["exact"] == p["draft"]["rows"], (table, p)
    lists = [np.sort(wl.rng(5, c).choice(wk.V, size=300, replace=False)).astype(np.int32)
             for c in range(wk.draft_calls)]
    qa8, ea8 = oracle.quantize_fp8(head)
    qa4, sa4 = oracle.quantize_mxfp4(head)
    gathered = {
        "bf16": [oracle.draft_gather(h, head, lst) for h, lst in zip(hiddens, lists)],
        "fp8": [oracle.draft_fp8_gather(h, qa8, ea8, lst) for h, lst in zip(hiddens, lists)],
        "mxfp4": [oracle.draft_mxfp4_gather(h, qa4, sa4, lst) for h, lst in zip(hiddens, lists)],
    }
    for table, refs in gathered.items():
        g = [(r["id"].copy(), r["logit"].copy()) for r in refs]
        p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g, g_verify, table, lists)
        assert p["ok"] and p["draft_source"] == "gather", (table, p)
        outside = next(i for i in range(wk.V) if i not in set(lists[0].tolist()))
        g[0][0][0] = outside
        p = bench.oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g, g_verify, table, lists)
        assert not p["ok"] and p["draft"]["violations"] == 1, (table, p)


def bench_logit(h, head, token):
    """fp64 logit of one head row (bf16 bits widened exactly)."""
    x = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64).ravel()
    w = (head[token].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return float(x @ w)


def test_source_hash_ignores_comments_and_layout_only():
    """Profile summaries carry a hash of their kernels' code: editing a
    comment or the layout keeps it, editing code (or a string) changes it."""
    src = 'int f(int a) {  // the sum\n  /* twice */ return a + a; }\nconst char *s = "x // y";\n'
    same = 'int f(int a) {\n  return a + a;   // twice, reworded\n}\nconst char *s = "x // y";\n'
    code = 'int f(int a) {  // the sum\n  /* twice */ return a + 2; }\nconst char *s = "x // y";\n'
    text = 'int f(int a) {  // the sum\n  /* twice */ return a + a; }\nconst char *s = "x // z";\n'
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(code)
    assert bench.code_text(src) != bench.code_text(text)
    assert bench.code_text("char c = '\\'';  // q") == "char c = '\\'';"
    for fam in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_hash(fam)) == 16
