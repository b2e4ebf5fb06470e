"""GPU parity of the draft over gathered candidates on an fp8 head
(mtp_draft_argmax_fp8_gather): every head row quantised once by the fp8 pack,
candidates named per call by an id list that may be unsorted, repeat ids and
hold out-of-range ids, against the CPU oracle's draft_fp8_gather. The
packed-table fp8 draft runs the same kernel and keeps its own tests."""

import numpy as np
import pytest

import oracle
from speculative_decoding_argmax_amd import workloads as wl
from tests.parity import check_fp8_rows, dev_bf16, dev_i32
from tests.test_gpu_fp8 import gpu_pack
from tests.test_gpu_gather import messy_ids

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


def gpu_gather8(torch, mtp, x, q_d, s_d, ids, **kw):
    M = x.shape[0]
    oi = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ol = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    mtp.mtp_draft_argmax_fp8_gather(dev_bf16(x), q_d, s_d, dev_i32(ids), oi, ol, **kw)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), ol.cpu().numpy()


GRID_SHAPES = [  # (M, V, C, H)
    (1, 1, 1, 16), (1, 5000, 3000, 256), (3, 20000, 9000, 2048), (8, 3001, 4000, 4096),
    (2, 700, 65, 5120), (5, 999, 777, 2560), (1, 300, 257, 16384), (9, 4000, 2500, 48),
]


@pytest.mark.parametrize("M,V,C,H", GRID_SHAPES)
def test_fp8_gather_exact_grid(torch, mtp, M, V, C, H):
    """Head rows of multiples of 1/8 (max 2) quantise exactly and hidden rows
    on the q/16 grid make every partial sum exact: ids and logits bit-exact,
    exact ties included (the lowest id wins whatever the list order)."""
    seed = 97 + M + V + C + H
    r = wl.rng(seed, 1)
    kq = r.integers(-16, 17, size=(V, H))
    kq[:, 0] = 16
    head = wl.f32_to_bf16_bits((kq / 8.0).astype(np.float32))
    x = wl.exact_grid_bf16((M, H), seed, 2)
    ids = messy_ids(V, C, seed)
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    q_ref, e_ref = oracle.quantize_fp8(head)
    assert np.array_equal(q_d.cpu().numpy(), q_ref)
    assert np.array_equal(s_d.cpu().numpy(), np.ldexp(1.0, e_ref).astype(np.float32))
    g_ids, g_logit = gpu_gather8(torch, mtp, x, q_d, s_d, ids)
    ref = oracle.draft_fp8_gather(x, q_ref, e_ref, ids)
    assert np.array_equal(g_ids, ref["id"]), (g_ids, ref["id"])
    ok = ref["id"] >= 0
    assert np.array_equal(g_logit[ok], ref["logit"][ok])
    assert np.all(np.isnan(g_logit[~ok]))


def test_fp8_gather_fixed_plus_dynamic_rows(torch, mtp):
    """N(0, 0.02) head, N(0, 1) hidden, H = 2,048: a fixed set of 32,768
    candidates plus 16,384 rows chosen for this call, the whole list shuffled,
    against the oracle under the near-tie rule (fp8 logits)."""
    V, H = 120_000, 2_048
    head = wl.head_weights(V, H, 787)
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    q_ref, e_ref = oracle.quantize_fp8(head)
    fixed = wl.candidate_ids(V, 32_768, 787)
    rest = np.setdiff1d(np.arange(V, dtype=np.int32), fixed)
    for call in range(2):
        r = wl.rng(787, 20 + call)
        dyn = r.choice(rest, size=16_384, replace=False).astype(np.int32)
        ids = np.concatenate([fixed, dyn])
        r.shuffle(ids)
        for M in (1, 2, 4):
            x = wl.hidden_states(M, H, 787, block=10 * call + M)
            g_ids, g_logit = gpu_gather8(torch, mtp, x, q_d, s_d, ids)
            assert np.isin(g_ids, ids).all()
            ref = oracle.draft_fp8_gather(x, q_ref, e_ref, ids)
            srt = np.sort(ids)
            check_fp8_rows(g_ids, g_logit, ref, x, q_ref[srt], e_ref[srt], srt)


def test_fp8_gather_all_invalid_and_tie(torch, mtp):
    """A list of only invalid ids gives id -1 and a NaN logit; identical
    rows listed high id first tie exactly and the lower id wins."""
    V, H = 3_000, 2_048
    head = wl.head_weights(V, H, 19)
    x = wl.hidden_states(1, H, 19, block=5)
    q, e = oracle.quantize_fp8(head)
    w = int(oracle.draft_fp8(x, q, e)["id"][0])
    partner = 11 if w != 11 else 12
    head[partner] = head[w]
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    hi, lo = max(w, partner), min(w, partner)
    ids = np.array([hi, 40, 41, 2000, lo, V + 3, -2], np.int32)
    g_ids, _ = gpu_gather8(torch, mtp, x, q_d, s_d, ids)
    assert g_ids[0] == lo
    g_ids, g_logit = gpu_gather8(torch, mtp, x, q_d, s_d, np.array([-1, V, V + 9], np.int32))
    assert g_ids[0] == -1 and np.isnan(g_logit[0])


def test_fp8_gather_refuses_matrix_core_path(torch, mtp):
    head = wl.normal_bf16_rows(10, 64, 0.02, 1, 1)
    q_d, s_d = gpu_pack(torch, mtp, head, None)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MTPError):
        mtp.mtp_draft_argmax_fp8_gather(dev_bf16(wl.hidden_states(1, 64, 1)), q_d, s_d,
                                        dev_i32(np.array([1, 2], np.int32)), out,
                                        path=mtp.MTP_PATH_MFMA)
