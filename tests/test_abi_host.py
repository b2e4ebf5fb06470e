"""The C ABI on the host: the library loads, exports every entry point the
header declares, and refuses bad arguments before anything reaches the GPU.
No call here passes validation, so nothing is ever launched."""

import ctypes

import numpy as np
import pytest

from speculative_decoding_argmax_amd import mtp

P = ctypes.c_void_p
FAKE = P(0x10000)        # non-null, 64 KiB aligned; never dereferenced
FAKE_ODD = P(0x10002)    # 2-byte aligned only


def test_exports_every_header_symbol():
    names = mtp.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(mtp.lib, n), n


def test_status_strings_and_version():
    for s in range(6):
        assert mtp.status_string(s).startswith("MTP_")
    assert mtp.lib.mtp_version() >= 100
    assert mtp.last_hip_error() == 0


def test_validate_ids():
    assert mtp.mtp_validate_ids(np.array([0, 5, 9]), 10) == mtp.MTP_OK
    assert mtp.mtp_validate_ids(np.array([0, 5, 5]), 10) == mtp.MTP_ERR_IDS
    assert mtp.mtp_validate_ids(np.array([3, 2]), 10) == mtp.MTP_ERR_IDS
    assert mtp.mtp_validate_ids(np.array([0, 10]), 10) == mtp.MTP_ERR_IDS
    assert mtp.mtp_validate_ids(np.array([-1, 4]), 10) == mtp.MTP_ERR_IDS
    assert mtp.lib.mtp_validate_ids(None, 3, 10) == mtp.MTP_ERR_INVALID_ARG


def counters(M):
    """Header and the grouped finish's 8 regions (64 bytes of group ticket,
    then M keys, rounded up to 256 bytes each)."""
    return 256 + 8 * (-(-(64 + 8 * M) // 256) * 256)


def least_counters(M):
    """The least workspace a call accepts: header and M keys (one-level
    finish)."""
    return 256 + -(-M * 8 // 256) * 256


def test_workspace_sizes():
    assert mtp.mtp_draft_workspace_bytes(1, 65536, 2048) == 2304 == counters(1)
    assert mtp.mtp_draft_workspace_bytes(24, 65536, 5120) == 2304
    assert mtp.mtp_draft_workspace_bytes(25, 65536, 5120) == 4352 == counters(25)
    assert mtp.mtp_draft_workspace_bytes(128, 65536, 5120) == counters(128) == 10496
    # 160 rows: the counters of the largest call, then the tiled calls'
    # staging area (see below)
    assert counters(4096) == 264448
    assert mtp.mtp_verify_workspace_bytes(32, 4, 248320, 5120) == \
        counters(4096) + 160 * 10 * 1024 + 256
    assert mtp.mtp_verify_workspace_bytes(1, 0, 10, 8) == counters(1)
    for bad in ((0, 10, 8), (1, 0, 8), (1, 10, 12), (1, 10, 4), (4097, 10, 8), (1, 10, 16392)):
        assert mtp.mtp_draft_workspace_bytes(*bad) == 0, bad
    assert mtp.mtp_verify_workspace_bytes(1, 16, 10, 8) == 0
    assert mtp.mtp_verify_workspace_bytes(1, -1, 10, 8) == 0
    assert mtp.mtp_verify_workspace_bytes(0, 3, 10, 8) == 0


def _draft(hidden=FAKE, M=1, H=64, table=FAKE, ids=FAKE, C=100, out_ids=FAKE, out_logit=None,
           ws=FAKE, ws_bytes=4096, cfg=None):
    args = [hidden, M, H, table, ids, C, out_ids, out_logit, ws, ws_bytes, None]
    if cfg is None:
        return mtp.lib.mtp_draft_argmax(*args)
    return mtp.lib.mtp_draft_argmax_cfg(*args, ctypes.byref(cfg))


def _verify(hidden=FAKE, B=1, k=3, H=64, head=FAKE, V=100, draft=FAKE, out_argmax=FAKE,
            out_logit=None, out_accept=FAKE, out_tokens=FAKE, ws=FAKE, ws_bytes=4096, cfg=None):
    args = [hidden, B, k, H, head, V, draft, out_argmax, out_logit, out_accept, out_tokens, ws,
            ws_bytes, None]
    if cfg is None:
        return mtp.lib.mtp_verify_accept(*args)
    return mtp.lib.mtp_verify_accept_cfg(*args, ctypes.byref(cfg))


INVALID = mtp.MTP_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(hidden=None), dict(table=None), dict(out_ids=None), dict(M=0), dict(M=4097),
    dict(C=0), dict(C=2 ** 31), dict(H=0), dict(H=12), dict(H=16392), dict(hidden=FAKE_ODD),
    dict(table=FAKE_ODD), dict(out_ids=P(0x10001)), dict(ids=P(0x10002)),
    dict(out_logit=P(0x10003)),
])
def test_draft_rejects_bad_arguments(kw):
    assert _draft(**kw) == INVALID


def test_draft_workspace_errors():
    assert _draft(ws=None) == mtp.MTP_ERR_WORKSPACE
    assert _draft(ws=P(0x10004)) == mtp.MTP_ERR_WORKSPACE
    assert _draft(M=33, ws_bytes=512) == mtp.MTP_ERR_WORKSPACE


def test_draft_rejects_bad_config():
    c = mtp.mtp_config()
    c.path = 7
    assert _draft(cfg=c) == INVALID
    c = mtp.mtp_config()
    c.blocks_per_cu = 17
    assert _draft(cfg=c) == INVALID
    c = mtp.mtp_config()
    c.reserved[2] = 1
    assert _draft(cfg=c) == INVALID


@pytest.mark.parametrize("kw", [
    dict(hidden=None), dict(head=None), dict(out_argmax=None), dict(out_accept=None),
    dict(out_tokens=None), dict(B=0), dict(k=-1), dict(k=16), dict(draft=None),
    dict(B=1025, k=3), dict(V=0), dict(H=20), dict(head=FAKE_ODD), dict(out_tokens=P(0x10001)),
])
def test_verify_rejects_bad_arguments(kw):
    assert _verify(**kw) == INVALID


def test_verify_workspace_errors():
    assert _verify(ws=None) == mtp.MTP_ERR_WORKSPACE
    assert _verify(B=64, k=3, ws_bytes=2048) == mtp.MTP_ERR_WORKSPACE


def _verify_noalloc(hidden=FAKE, B=1, k=3, H=64, head=FAKE, V=100, draft=FAKE, out_argmax=FAKE,
                    out_logit=None, out_accept=FAKE, out_tokens=FAKE):
    return mtp.lib.mtp_verify_accept_noalloc(hidden, B, k, H, head, V, draft, out_argmax,
                                             out_logit, out_accept, out_tokens, None)


@pytest.mark.parametrize("kw", [
    dict(hidden=None), dict(head=None), dict(out_argmax=None), dict(out_accept=None),
    dict(out_tokens=None), dict(B=0), dict(k=-1), dict(k=16), dict(draft=None),
    dict(B=1025, k=3), dict(V=0), dict(H=20), dict(head=FAKE_ODD), dict(out_tokens=P(0x10001)),
])
def test_verify_noalloc_rejects_bad_arguments(kw):
    """The allocation-free verify checks its arguments as mtp_verify_accept
    does, before it looks up its scratch or enqueues anything."""
    assert _verify_noalloc(**kw) == INVALID


def test_verify_noalloc_rejects_calls_beyond_its_scratch():
    """More than MTP_NOALLOC_MAX_ROWS verify rows do not fit the static
    scratch: MTP_ERR_WORKSPACE, nothing enqueued (no GPU needed)."""
    assert mtp.MTP_NOALLOC_MAX_ROWS == 1024
    assert _verify_noalloc(B=257, k=3) == mtp.MTP_ERR_WORKSPACE    # 1,028 rows
    assert _verify_noalloc(B=65, k=15) == mtp.MTP_ERR_WORKSPACE    # 1,040 rows
    assert _verify_noalloc(B=1025, k=0) == mtp.MTP_ERR_WORKSPACE
    header = open(mtp.HEADER).read()
    assert "#define MTP_NOALLOC_MAX_ROWS 1024" in header


def test_pack_and_init_reject_bad_arguments():
    f = mtp.lib.mtp_pack_candidates
    assert f(None, 10, 8, FAKE, 2, FAKE, None) == INVALID
    assert f(FAKE, 10, 12, FAKE, 2, FAKE, None) == INVALID
    assert f(FAKE, 0, 8, FAKE, 2, FAKE, None) == INVALID
    assert f(FAKE, 10, 8, FAKE, 0, FAKE, None) == INVALID
    assert f(FAKE_ODD, 10, 8, FAKE, 2, FAKE, None) == INVALID
    g = mtp.lib.mtp_workspace_init
    assert g(None, 64, None) == INVALID
    assert g(FAKE, 0, None) == INVALID
    assert g(FAKE, 12, None) == INVALID
    assert g(P(0x10004), 64, None) == INVALID


def test_tiled_sizes():
    assert mtp.mtp_tiled_bytes(65536, 2048) == 65536 * 2048 * 2
    assert mtp.mtp_tiled_bytes(248320, 5120) == 248320 * 5120 * 2
    assert mtp.mtp_tiled_bytes(100, 24) == 128 * 128 * 2
    assert mtp.mtp_tiled_bytes(1, 2560) == 64 * 2560 * 2
    assert mtp.mtp_tiled_bytes(0, 8) == 0
    assert mtp.mtp_tiled_bytes(10, 12) == 0
    assert mtp.mtp_tiled_bytes(10, 16392) == 0


def test_tiled_entry_points_reject_bad_arguments():
    f = mtp.lib.mtp_pack_tiled
    need = mtp.mtp_tiled_bytes(100, 64)
    assert f(None, 100, 64, None, 100, FAKE, need, None) == INVALID
    assert f(FAKE, 100, 64, None, 101, FAKE, need, None) == INVALID     # C > V without ids
    assert f(FAKE, 100, 64, None, 100, FAKE, need - 16, None) == INVALID
    assert f(FAKE, 100, 60, None, 100, FAKE, need, None) == INVALID
    assert f(FAKE_ODD, 100, 64, None, 100, FAKE, need, None) == INVALID
    d = mtp.lib.mtp_draft_argmax_tiled
    assert d(None, 1, 64, FAKE, None, 100, FAKE, None, FAKE, 4096, None) == INVALID
    assert d(FAKE, 0, 64, FAKE, None, 100, FAKE, None, FAKE, 4096, None) == INVALID
    assert d(FAKE, 1, 64, FAKE_ODD, None, 100, FAKE, None, FAKE, 4096, None) == INVALID
    assert d(FAKE, 1, 64, FAKE, None, 100, FAKE, None, None, 4096, None) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_VALU
    assert mtp.lib.mtp_draft_argmax_tiled_cfg(FAKE, 1, 64, FAKE, None, 100, FAKE, None, FAKE,
                                              4096, None, ctypes.byref(c)) == \
        mtp.MTP_ERR_UNSUPPORTED
    v = mtp.lib.mtp_verify_accept_tiled
    assert v(FAKE, 1, 16, 64, FAKE, 100, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4096, None) == INVALID
    assert v(FAKE, 1, 3, 64, None, 100, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4096, None) == INVALID
    assert v(FAKE, 1, 3, 64, FAKE, 100, FAKE, FAKE, None, FAKE, FAKE, FAKE, 16, None) == \
        mtp.MTP_ERR_WORKSPACE


def test_one_hip_runtime_per_process():
    """Importing the binding first must not load a second HIP runtime next to
    torch's own (the library's launches would then find no device)."""
    import subprocess
    import sys
    code = ("from speculative_decoding_argmax_amd import mtp\n"
            "import torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths), sorted(paths))\n")
    root = __import__("os").path.dirname(__import__("os").path.dirname(__file__))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    n = int(out.stdout.split()[0])
    assert n == 1, out.stdout


def test_gather_rejects_bad_arguments():
    f = mtp.lib.mtp_draft_argmax_gather
    ok = (FAKE, 1, 64, FAKE, 100, FAKE, 50, FAKE, None, FAKE, 4096, None)
    assert f(*ok[:5], None, *ok[6:]) == INVALID                 # no id list
    assert f(*ok[:4], 0, *ok[5:]) == INVALID                    # V < 1
    assert f(*ok[:4], 2 ** 31, *ok[5:]) == INVALID              # V too large
    assert f(*ok[:6], 0, *ok[7:]) == INVALID                    # C < 1
    assert f(None, *ok[1:]) == INVALID
    assert f(*ok[:3], FAKE_ODD, *ok[4:]) == INVALID             # head alignment
    assert f(*ok[:5], P(0x10002), *ok[6:]) == INVALID           # ids alignment
    assert f(*ok[:9], None, *ok[10:]) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_MFMA
    g = mtp.lib.mtp_draft_argmax_gather_cfg
    assert g(*ok, ctypes.byref(c)) == mtp.MTP_ERR_UNSUPPORTED


def test_fp8_entry_points_reject_bad_arguments():
    assert mtp.mtp_fp8_table_bytes(100, 2048) == 100 * 2048
    assert mtp.mtp_fp8_table_bytes(100, 24) == 0          # H % 16 != 0
    assert mtp.mtp_fp8_table_bytes(0, 32) == 0
    p = mtp.lib.mtp_pack_candidates_fp8
    ok = (FAKE, 100, 64, FAKE, 50, FAKE, FAKE, None)
    assert p(None, *ok[1:]) == INVALID
    assert p(*ok[:2], 24, *ok[3:]) == INVALID            # H % 16
    assert p(*ok[:3], None, 101, *ok[5:]) == INVALID     # C > V without ids
    assert p(*ok[:5], P(0x10008), *ok[6:]) == INVALID    # codes not 16-byte aligned
    assert p(*ok[:6], P(0x10002), None) == INVALID       # scales not 4-byte aligned
    d = mtp.lib.mtp_draft_argmax_fp8
    dk = (FAKE, 1, 64, FAKE, FAKE, None, 100, FAKE, None, FAKE, 4096, None)
    assert d(*dk[:2], 24, *dk[3:]) == INVALID
    assert d(*dk[:4], None, *dk[5:]) == INVALID          # no scales
    assert d(*dk[:9], None, *dk[10:]) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_MFMA
    assert mtp.lib.mtp_draft_argmax_fp8_cfg(*dk, ctypes.byref(c)) == mtp.MTP_ERR_UNSUPPORTED


def test_tiled_fp8_entry_points_reject_bad_arguments():
    assert mtp.mtp_tiled_fp8_bytes(100, 2048) == 128 * 2048
    assert mtp.mtp_tiled_fp8_bytes(65, 16) == 128 * 128
    assert mtp.mtp_tiled_fp8_bytes(100, 24) == 0         # H % 16 != 0
    assert mtp.mtp_tiled_fp8_bytes(0, 32) == 0
    p = mtp.lib.mtp_pack_tiled_fp8
    need = mtp.mtp_tiled_fp8_bytes(50, 64)
    ok = (FAKE, 100, 64, FAKE, 50, FAKE, need, FAKE, None)
    assert p(None, *ok[1:]) == INVALID
    assert p(*ok[:2], 24, *ok[3:]) == INVALID            # H % 16
    assert p(*ok[:3], None, 101, *ok[5:]) == INVALID     # C > V without ids
    assert p(*ok[:6], need - 1, *ok[7:]) == INVALID      # buffer too small
    assert p(*ok[:5], P(0x10008), *ok[6:]) == INVALID    # codes not 16-byte aligned
    assert p(*ok[:7], P(0x10002), None) == INVALID       # scales not 4-byte aligned
    assert p(*ok[:7], None, None) == INVALID             # no scales
    d = mtp.lib.mtp_draft_argmax_tiled_fp8
    dk = (FAKE, 1, 64, FAKE, FAKE, None, 100, FAKE, None, FAKE, 4096, None)
    assert d(*dk[:2], 24, *dk[3:]) == INVALID
    assert d(*dk[:4], None, *dk[5:]) == INVALID          # no scales
    assert d(*dk[:4], P(0x10002), *dk[5:]) == INVALID    # scales alignment
    assert d(*dk[:9], None, *dk[10:]) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_VALU
    assert mtp.lib.mtp_draft_argmax_tiled_fp8_cfg(*dk, ctypes.byref(c)) == \
        mtp.MTP_ERR_UNSUPPORTED


def test_stream_read_rejects_bad_arguments():
    f = mtp.lib.mtp_stream_read
    assert f(None, 1024, FAKE, None) == INVALID
    assert f(FAKE, 1024, None, None) == INVALID
    assert f(FAKE, 0, FAKE, None) == INVALID
    assert f(FAKE, 1000, FAKE, None) == INVALID          # not a multiple of 16
    assert f(P(0x10008), 1024, FAKE, None) == INVALID    # buffer not 16-byte aligned
    assert f(FAKE, 1024, P(0x10002), None) == INVALID    # sink not 4-byte aligned


def test_probe_atomic_rejects_bad_arguments():
    f = mtp.lib.mtp_probe_atomic
    assert f(None, 1, 1, 0, FAKE, None) == INVALID
    assert f(FAKE, 1, 1, 0, None, None) == INVALID
    assert f(FAKE, 0, 1, 0, FAKE, None) == INVALID                       # no workgroup
    assert f(FAKE, mtp.MTP_PROBE_MAX_WGS + 1, 1, 0, FAKE, None) == INVALID
    assert f(FAKE, 1, 0, 0, FAKE, None) == INVALID                       # no iteration
    assert f(FAKE, 1, mtp.MTP_PROBE_MAX_ITERS + 1, 0, FAKE, None) == INVALID
    assert f(FAKE, 1, 1, 2, FAKE, None) == INVALID                       # same is 0 or 1
    assert f(P(0x10002), 1, 1, 0, FAKE, None) == INVALID                 # words not 4-byte aligned
    assert f(FAKE, 1, 1, 0, P(0x10004), None) == INVALID                 # ticks not 8-byte aligned


def test_wide_tiled_calls_need_the_staging_area():
    """Above 128 hidden rows the workspace query adds the packed-hidden
    staging area (S steps x 10 row blocks x 1 KiB per 160-row pass, plus
    256 bytes of alignment slack) past the counters of the largest possible
    call, and a tiled call given only the counters' size is refused before
    anything is enqueued."""
    assert mtp.mtp_draft_workspace_bytes(128, 1000, 5120) == counters(128)
    base = counters(4096)
    stage160 = (5120 // 32) * 10 * 1024 + 256
    assert mtp.mtp_draft_workspace_bytes(160, 1000, 5120) == base + stage160
    assert mtp.mtp_verify_workspace_bytes(32, 4, 248320, 5120) == base + stage160
    # 161 rows: two 160-row passes; H = 1000 pads to 1024 columns (32 steps)
    assert mtp.mtp_draft_workspace_bytes(161, 1000, 1000) == base + 32 * 20 * 1024 + 256
    assert mtp.mtp_draft_workspace_bytes(4096, 1000, 64) == base + 4 * 260 * 1024 + 256
    d = mtp.lib.mtp_draft_argmax_tiled
    assert d(FAKE, 160, 5120, FAKE, None, 1000, FAKE, None, FAKE, counters(160), None) == \
        mtp.MTP_ERR_WORKSPACE
    v = mtp.lib.mtp_verify_accept_tiled
    assert v(FAKE, 32, 4, 5120, FAKE, 248320, FAKE, FAKE, None, FAKE, FAKE, FAKE, counters(160),
             None) == mtp.MTP_ERR_WORKSPACE


def test_mxfp4_entry_points_reject_bad_arguments():
    assert mtp.mtp_mxfp4_table_bytes(100, 2048) == 100 * 1024
    assert mtp.mtp_mxfp4_scale_bytes(100, 2048) == 100 * 64
    assert mtp.mtp_mxfp4_table_bytes(100, 48) == 0       # H % 32 != 0
    assert mtp.mtp_mxfp4_table_bytes(0, 64) == 0
    assert mtp.mtp_mxfp4_scale_bytes(100, 16) == 0
    p = mtp.lib.mtp_pack_candidates_mxfp4
    ok = (FAKE, 100, 64, FAKE, 50, FAKE, FAKE, None)
    assert p(None, *ok[1:]) == INVALID
    assert p(*ok[:2], 48, *ok[3:]) == INVALID            # H % 32
    assert p(*ok[:3], None, 101, *ok[5:]) == INVALID     # C > V without ids
    assert p(*ok[:5], P(0x10008), *ok[6:]) == INVALID    # codes not 16-byte aligned
    assert p(*ok[:6], None, None) == INVALID             # no scales
    r = mtp.lib.mtp_pack_candidates_mxfp4_rule
    okr = ok[:7] + (mtp.MTP_MX_SCALE_FIT, None)
    assert r(None, *okr[1:]) == INVALID
    assert r(*okr[:2], 48, *okr[3:]) == INVALID          # H % 32
    assert r(*okr[:7], 2, None) == INVALID               # no such scale rule
    assert r(*okr[:7], -1, None) == INVALID
    d = mtp.lib.mtp_draft_argmax_mxfp4
    dk = (FAKE, 1, 64, FAKE, FAKE, None, 100, FAKE, None, FAKE, 4096, None)
    assert d(*dk[:2], 48, *dk[3:]) == INVALID
    assert d(*dk[:4], None, *dk[5:]) == INVALID          # no scales
    assert d(*dk[:9], None, *dk[10:]) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_MFMA
    assert mtp.lib.mtp_draft_argmax_mxfp4_cfg(*dk, ctypes.byref(c)) == mtp.MTP_ERR_UNSUPPORTED


def test_tiled_mxfp4_entry_points_reject_bad_arguments():
    assert mtp.mtp_tiled_mxfp4_bytes(100, 2048) == 128 * 1024
    assert mtp.mtp_tiled_mxfp4_scale_bytes(100, 2048) == 128 * 64
    assert mtp.mtp_tiled_mxfp4_bytes(65, 96) == 128 * 128      # columns pad to 256
    assert mtp.mtp_tiled_mxfp4_bytes(100, 48) == 0              # H % 32 != 0
    assert mtp.mtp_tiled_mxfp4_scale_bytes(0, 64) == 0
    p = mtp.lib.mtp_pack_tiled_mxfp4
    nq, ns = mtp.mtp_tiled_mxfp4_bytes(50, 64), mtp.mtp_tiled_mxfp4_scale_bytes(50, 64)
    ok = (FAKE, 100, 64, FAKE, 50, FAKE, nq, FAKE, ns, None)
    assert p(None, *ok[1:]) == INVALID
    assert p(*ok[:2], 48, *ok[3:]) == INVALID                   # H % 32
    assert p(*ok[:3], None, 101, *ok[5:]) == INVALID            # C > V without ids
    assert p(*ok[:6], nq - 1, *ok[7:]) == INVALID               # codes buffer too small
    assert p(*ok[:8], ns - 1, None) == INVALID                  # scale buffer too small
    assert p(*ok[:7], None, ns, None) == INVALID                # no scales
    assert p(*ok[:5], P(0x10008), *ok[6:]) == INVALID           # codes not 16-byte aligned
    r = mtp.lib.mtp_pack_tiled_mxfp4_rule
    okr = ok[:9] + (mtp.MTP_MX_SCALE_OCP, None)
    assert r(None, *okr[1:]) == INVALID
    assert r(*okr[:6], nq - 1, *okr[7:]) == INVALID             # codes buffer too small
    assert r(*okr[:9], 3, None) == INVALID                      # no such scale rule
    d = mtp.lib.mtp_draft_argmax_tiled_mxfp4
    dk = (FAKE, 1, 64, FAKE, FAKE, None, 100, FAKE, None, FAKE, 4096, None)
    assert d(*dk[:2], 48, *dk[3:]) == INVALID
    assert d(*dk[:4], None, *dk[5:]) == INVALID                 # no scales
    assert d(*dk[:9], None, *dk[10:]) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_VALU
    assert mtp.lib.mtp_draft_argmax_tiled_mxfp4_cfg(*dk, ctypes.byref(c)) == \
        mtp.MTP_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With no built library the binding refuses to import (no CPU fallback):
    a copy of the package's Python files without lib/ raises ImportError
    naming the missing library."""
    import os
    import shutil
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = os.path.join(root, "speculative_decoding_argmax_amd")
    dst = tmp_path / "speculative_decoding_argmax_amd"
    dst.mkdir()
    for name in os.listdir(src):
        if name.endswith(".py"):
            shutil.copy(os.path.join(src, name), dst / name)
    code = "from speculative_decoding_argmax_amd import mtp\n"
    out = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True,
                         text=True, timeout=300, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert out.returncode != 0
    assert "ImportError" in out.stderr and "not built" in out.stderr, out.stderr[-2000:]


def test_mxfp4_gather_rejects_bad_arguments():
    f = mtp.lib.mtp_draft_argmax_mxfp4_gather
    # hidden, M, H, head_q, head_scales, V, ids, C, out_ids, out_logit, ws, ws_bytes, stream
    ok = [FAKE, 1, 64, FAKE, FAKE, 100, FAKE, 50, FAKE, None, FAKE, 4096, None]

    def call(changes):
        a = list(ok)
        for k, v in changes.items():
            a[k] = v
        return f(*a)

    assert call({6: None}) == INVALID                          # no id list
    assert call({5: 0}) == INVALID                             # V < 1
    assert call({5: 2 ** 31}) == INVALID                       # V too large
    assert call({7: 0}) == INVALID                             # C < 1
    assert call({2: 48}) == INVALID                            # H % 32
    assert call({4: None}) == INVALID                          # no scales
    assert call({3: FAKE_ODD}) == INVALID                      # codes alignment
    assert call({0: None}) == INVALID
    assert call({10: None}) == mtp.MTP_ERR_WORKSPACE
    assert call({11: 8}) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_MFMA
    assert mtp.lib.mtp_draft_argmax_mxfp4_gather_cfg(*ok, ctypes.byref(c)) == \
        mtp.MTP_ERR_UNSUPPORTED


def test_fp8_gather_rejects_bad_arguments():
    f = mtp.lib.mtp_draft_argmax_fp8_gather
    # hidden, M, H, head_q, head_scales, V, ids, C, out_ids, out_logit, ws, ws_bytes, stream
    ok = [FAKE, 1, 64, FAKE, FAKE, 100, FAKE, 50, FAKE, None, FAKE, 4096, None]

    def call(changes):
        a = list(ok)
        for k, v in changes.items():
            a[k] = v
        return f(*a)

    assert call({6: None}) == INVALID                            # no id list
    assert call({5: 0}) == INVALID                               # V < 1
    assert call({5: 2 ** 31}) == INVALID                         # V too large
    assert call({7: 0}) == INVALID                               # C < 1
    assert call({2: 40}) == INVALID                              # H % 16
    assert call({4: None}) == INVALID                            # no scales
    assert call({4: P(0x10002)}) == INVALID                      # scales alignment
    assert call({3: FAKE_ODD}) == INVALID                        # codes alignment
    assert call({10: None}) == mtp.MTP_ERR_WORKSPACE
    c = mtp.mtp_config()
    c.path = mtp.MTP_PATH_MFMA
    assert mtp.lib.mtp_draft_argmax_fp8_gather_cfg(*ok, ctypes.byref(c)) == \
        mtp.MTP_ERR_UNSUPPORTED
