"""CPU oracle for the MTP draft / verify LM-head path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package. It is a ctypes wrapper over ``mtp_oracle.c`` (plain C, fp64
accumulation, fp32 argmax decision); it shares no code with the HIP library
and never imports it.

Functions follow the method's steps (see ``mtp_oracle.c`` for the passages of
the pages each one follows):
  pack(head, ids)             candidate sub-table rows head[ids[i]]
  logits(x, w)                [M][N] fp64 logits
  argmax(x, w, ids=None)      per-row first maximum of the fp32-rounded logits
  draft(h, table, ids)        argmax over the candidate table, mapped to ids
  draft_gather(h, head, ids)  argmax over head rows named by an id list (any
                              order, repeats; out-of-range ids are no candidates)
  e4m3_value(codes), e4m3_round(x)
                              the OCP E4M3 format: exact values, nearest code
  quantize_fp8(head, ids)     fp8 candidate table: E4M3 rows and per-row
                              power-of-two scale exponents
  draft_fp8(h, q, exps, ids)  argmax over the fp8 table, mapped to ids
  draft_fp8_gather(h, q, exps, ids)
                              draft_gather's candidates on an fp8 head
  e2m1_value(codes), e2m1_round(x), mx_block_exponent(w, rule)
                              the OCP E2M1 element and the MX block scale rule
  quantize_mxfp4(head, ids, rule)  MXFP4 candidate table: packed E2M1 codes and
                              E8M0 scales per block of 32
  draft_mxfp4(h, q, scales, ids)
                              argmax over the MXFP4 table, mapped to ids
  draft_mxfp4_gather(h, q, scales, ids)
                              draft_gather's candidates on an MXFP4 head
  verify(hv, head, B, k)      argmax over the full head, shaped [B][k+1]
  accept(draft, target)       greedy acceptance plus bonus token
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mtp_oracle.c")
_LIB = os.path.join(_HERE, "libmtp_oracle.so")

ORC_OK = 0


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, out)
    return out


class _Lib:
    """The compiled oracle at one path (tests may load other builds)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.mtp_oracle_threads.restype = ctypes.c_int
        lib.mtp_oracle_logits.argtypes = [P, I64, P, I64, I64, P]
        lib.mtp_oracle_pair_logits.argtypes = [P, P, I64, P, P, I64, P]
        lib.mtp_oracle_argmax.argtypes = [P, I64, P, P, I64, I64, P, P, P, P, P]
        lib.mtp_oracle_accept.argtypes = [P, P, I64, I64, P, P]
        lib.mtp_oracle_check_ids.argtypes = [P, I64, I64]
        lib.mtp_oracle_pack.argtypes = [P, I64, I64, P, I64, P]
        lib.mtp_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.mtp_oracle_e4m3_value.restype = ctypes.c_double
        lib.mtp_oracle_e4m3_round.argtypes = [ctypes.c_double]
        lib.mtp_oracle_e4m3_round.restype = ctypes.c_uint8
        lib.mtp_oracle_e4m3_round_array.argtypes = [P, I64, P]
        lib.mtp_oracle_fp8_row_exponent.argtypes = [P, I64, P]
        lib.mtp_oracle_quantize_fp8.argtypes = [P, I64, I64, P, I64, P, P]
        lib.mtp_oracle_fp8_argmax.argtypes = [P, I64, P, P, P, I64, I64, P, P, P, P, P]
        lib.mtp_oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.mtp_oracle_e2m1_value.restype = ctypes.c_double
        lib.mtp_oracle_e2m1_round.argtypes = [ctypes.c_double]
        lib.mtp_oracle_e2m1_round.restype = ctypes.c_uint8
        lib.mtp_oracle_e2m1_round_array.argtypes = [P, I64, P]
        lib.mtp_oracle_mx_block_exponent.argtypes = [P, I64, P]
        lib.mtp_oracle_mx_block_exponent_fit.argtypes = [P, I64, P]
        lib.mtp_oracle_quantize_mxfp4.argtypes = [P, I64, I64, P, I64, P, P]
        lib.mtp_oracle_quantize_mxfp4_rule.argtypes = [P, I64, I64, P, I64, P, P, ctypes.c_int]
        lib.mtp_oracle_mxfp4_argmax.argtypes = [P, I64, P, P, P, I64, I64, P, P, P, P, P]
        for f in ("mtp_oracle_logits", "mtp_oracle_pair_logits", "mtp_oracle_argmax",
                  "mtp_oracle_accept", "mtp_oracle_check_ids", "mtp_oracle_pack",
                  "mtp_oracle_e4m3_round_array", "mtp_oracle_fp8_row_exponent",
                  "mtp_oracle_quantize_fp8", "mtp_oracle_fp8_argmax",
                  "mtp_oracle_e2m1_round_array", "mtp_oracle_mx_block_exponent",
                  "mtp_oracle_mx_block_exponent_fit", "mtp_oracle_quantize_mxfp4",
                  "mtp_oracle_quantize_mxfp4_rule", "mtp_oracle_mxfp4_argmax"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib
        self.path = path


_default: Optional[_Lib] = None
_current: Optional[_Lib] = None


def _load():
    global _default
    if _current is not None:
        return _current.lib
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _default = _Lib(_LIB)
    return _default.lib


class use_library:
    """Context manager: route this module's functions to another oracle build."""

    def __init__(self, path: str):
        self._lib = _Lib(path)
        self._prev: Optional[_Lib] = None

    def __enter__(self):
        global _current
        self._prev, _current = _current, self._lib
        return self

    def __exit__(self, *exc):
        global _current
        _current = self._prev
        return False


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != ORC_OK:
        raise OracleError(f"{what} failed with code {rc}")


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bfloat16 inputs are passed as uint16 bit patterns")
    return a


def threads() -> int:
    return int(_load().mtp_oracle_threads())


def logits(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    x = _bf16(np.atleast_2d(x))
    w = _bf16(np.atleast_2d(w))
    M, H = x.shape
    N, H2 = w.shape
    if H != H2:
        raise ValueError("hidden sizes differ")
    z = np.empty((M, N), dtype=np.float64)
    _check(_load().mtp_oracle_logits(_p(x), M, _p(w), N, H, _p(z)), "logits")
    return z


def pair_logits(x: np.ndarray, w: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """z[i] = dot(x[rows[i]], w[cols[i]]) in fp64."""
    x = _bf16(np.atleast_2d(x))
    w = _bf16(np.atleast_2d(w))
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if len(rows) and (rows.min() < 0 or rows.max() >= x.shape[0] or cols.min() < 0
                      or cols.max() >= w.shape[0]):
        raise IndexError("pair index out of range")
    z = np.empty(len(rows), dtype=np.float64)
    _check(_load().mtp_oracle_pair_logits(_p(x), _p(w), x.shape[1], _p(rows), _p(cols),
                                          len(rows), _p(z)), "pair_logits")
    return z


def argmax(x: np.ndarray, w: np.ndarray, ids: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    x = _bf16(np.atleast_2d(x))
    w = _bf16(np.atleast_2d(w))
    M, H = x.shape
    N = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("hidden sizes differ")
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        if ids.shape != (N,):
            raise ValueError("ids must have one entry per table row")
    out = {
        "id": np.empty(M, np.int32),
        "logit": np.empty(M, np.float32),
        "exact": np.empty(M, np.float64),
        "runner_id": np.empty(M, np.int32),
        "runner_exact": np.empty(M, np.float64),
    }
    _check(_load().mtp_oracle_argmax(_p(x), M, _p(w), _p(ids), N, H, _p(out["id"]),
                                     _p(out["logit"]), _p(out["exact"]), _p(out["runner_id"]),
                                     _p(out["runner_exact"])), "argmax")
    return out


def check_ids(ids: np.ndarray, V: int) -> bool:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    return _load().mtp_oracle_check_ids(_p(ids), len(ids), V) == ORC_OK


def pack(head: np.ndarray, ids: np.ndarray) -> np.ndarray:
    head = _bf16(head)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    V, H = head.shape
    table = np.empty((len(ids), H), dtype=np.uint16)
    _check(_load().mtp_oracle_pack(_p(head), V, H, _p(ids), len(ids), _p(table)), "pack")
    return table


def draft(h: np.ndarray, table: np.ndarray, ids: np.ndarray) -> Dict[str, np.ndarray]:
    """Draft step: argmax of each hidden row over the candidate table, as global ids."""
    return argmax(h, table, ids)


def draft_gather(h: np.ndarray, head: np.ndarray, ids: np.ndarray) -> Dict[str, np.ndarray]:
    """Draft over a candidate set given as an id list (Qwen3.8 Flash dual-Spark
    tuning log, section "read one fewer big table": a fixed candidate set plus
    rows chosen per step). The candidates are the distinct ids of the list that
    name a head row; the result is the draft over that set, i.e. the pinned
    argmax over the sorted set's packed rows, so ties go to the lowest id
    whatever the order of the list. With no valid id: id -1, logit NaN."""
    head = _bf16(head)
    V = head.shape[0]
    ids = np.asarray(ids, dtype=np.int64).ravel()
    valid = np.unique(ids[(ids >= 0) & (ids < V)]).astype(np.int32)
    M = np.atleast_2d(h).shape[0]
    if valid.size == 0:
        return {"id": np.full(M, -1, np.int32), "logit": np.full(M, np.nan, np.float32),
                "exact": np.full(M, np.nan), "runner_id": np.full(M, -1, np.int32),
                "runner_exact": np.full(M, np.nan)}
    return argmax(h, pack(head, valid), valid)


def accept(draft_ids: np.ndarray, target: np.ndarray) -> Dict[str, np.ndarray]:
    target = np.ascontiguousarray(target, dtype=np.int32)
    B, k1 = target.shape
    k = k1 - 1
    d = np.ascontiguousarray(np.asarray(draft_ids, dtype=np.int32).reshape(B, k))
    n = np.empty(B, np.int32)
    tok = np.empty((B, k + 1), np.int32)
    _check(_load().mtp_oracle_accept(_p(d), _p(target), B, k, _p(n), _p(tok)), "accept")
    return {"accept": n, "tokens": tok}


def verify(hv: np.ndarray, head: np.ndarray, B: int, k: int,
           draft_ids: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Verify step: full-head argmax of the B*(k+1) rows (row b*(k+1)+p),
    reshaped [B][k+1]; with drafts given, also the acceptance result."""
    r = argmax(hv, head, None)
    out = {key: v.reshape(B, k + 1) for key, v in r.items()}
    if draft_ids is not None:
        out.update(accept(draft_ids, out["id"]))
    return out


# ---- FP8 (E4M3) candidate table ---------------------------------------------


def e4m3_value(codes) -> np.ndarray:
    """Exact values of E4M3 codes (NaN for S.1111.111)."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.mtp_oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to even, saturating at 448)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _check(_load().mtp_oracle_e4m3_round_array(_p(x), x.size, _p(out)), "e4m3_round")
    return out


def fp8_row_exponent(w_row: np.ndarray) -> int:
    w = _bf16(np.atleast_1d(w_row))
    e = np.zeros(1, np.int32)
    _check(_load().mtp_oracle_fp8_row_exponent(_p(w), w.size, _p(e)), "fp8_row_exponent")
    return int(e[0])


def quantize_fp8(head: np.ndarray, ids: Optional[np.ndarray] = None):
    """The fp8 candidate table of head rows ids (None: every row): E4M3 codes
    [C][H] and the per-row scale exponents [C] (scale 2^e)."""
    head = _bf16(head)
    V, H = head.shape
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
    C = V if ids is None else len(ids)
    q = np.empty((C, H), dtype=np.uint8)
    exps = np.empty(C, dtype=np.int32)
    _check(_load().mtp_oracle_quantize_fp8(_p(head), V, H, _p(ids), C, _p(q), _p(exps)),
           "quantize_fp8")
    return q, exps


def draft_fp8(h: np.ndarray, q: np.ndarray, exps: np.ndarray,
              ids: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Draft over an fp8 candidate table: first maximum of the fp32-rounded
    logits 2^e[n] * sum_j h[j] * value(q[n][j]), reported as ids."""
    x = _bf16(np.atleast_2d(h))
    q = np.ascontiguousarray(q, dtype=np.uint8)
    exps = np.ascontiguousarray(exps, dtype=np.int32)
    M, H = x.shape
    N = q.shape[0]
    if q.shape[1] != H or exps.shape != (N,):
        raise ValueError("shapes differ")
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = {
        "id": np.empty(M, np.int32),
        "logit": np.empty(M, np.float32),
        "exact": np.empty(M, np.float64),
        "runner_id": np.empty(M, np.int32),
        "runner_exact": np.empty(M, np.float64),
    }
    _check(_load().mtp_oracle_fp8_argmax(_p(x), M, _p(q), _p(exps), _p(ids), N, H,
                                         _p(out["id"]), _p(out["logit"]), _p(out["exact"]),
                                         _p(out["runner_id"]), _p(out["runner_exact"])),
           "fp8_argmax")
    return out


def draft_fp8_gather(h: np.ndarray, q_head: np.ndarray, exps_head: np.ndarray,
                     ids: np.ndarray) -> Dict[str, np.ndarray]:
    """Draft over a candidate id list on an fp8 head (codes [V][H], row scale
    exponents [V], every head row quantised once): the candidate set of
    draft_gather with the fp8 logit of draft_fp8. Qwen3.8 Flash dual-Spark
    tuning log, section "read one fewer big table": a fixed candidate set plus
    rows chosen per step, in a low-precision float format. Ties go to the
    lowest id whatever the order of the list; with no valid id: id -1,
    logit NaN."""
    q_head = np.asarray(q_head, dtype=np.uint8)
    exps_head = np.asarray(exps_head, dtype=np.int32)
    V = q_head.shape[0]
    ids = np.asarray(ids, dtype=np.int64).ravel()
    valid = np.unique(ids[(ids >= 0) & (ids < V)]).astype(np.int32)
    M = np.atleast_2d(h).shape[0]
    if valid.size == 0:
        return {"id": np.full(M, -1, np.int32), "logit": np.full(M, np.nan, np.float32),
                "exact": np.full(M, np.nan), "runner_id": np.full(M, -1, np.int32),
                "runner_exact": np.full(M, np.nan)}
    return draft_fp8(h, q_head[valid], exps_head[valid], valid)


# ---- MXFP4 candidate table --------------------------------------------------


def e2m1_value(codes) -> np.ndarray:
    """Exact values of E2M1 codes (low 4 bits)."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.mtp_oracle_e2m1_value(c) for c in range(16)], dtype=np.float64)
    return table[codes & 15]


def e2m1_round(x) -> np.ndarray:
    """Nearest E2M1 code of each value (ties to even, saturating at 6)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _check(_load().mtp_oracle_e2m1_round_array(_p(x), x.size, _p(out)), "e2m1_round")
    return out


MX_SCALE_RULES = {"ocp": 0, "fit": 1}


def mx_block_exponent(w_block: np.ndarray, rule: str = "ocp") -> int:
    """Scale exponent of one block of bf16 values: the OCP MX rule
    floor(log2 max|w|) - 2, or the fit rule, the smallest e with
    max|w| <= 6 * 2^e (both clamped to [-127, 127], -127 for a zero block)."""
    w = _bf16(np.atleast_1d(w_block))
    e = np.zeros(1, np.int32)
    fn = {"ocp": _load().mtp_oracle_mx_block_exponent,
          "fit": _load().mtp_oracle_mx_block_exponent_fit}[rule]
    _check(fn(_p(w), w.size, _p(e)), "mx_block_exponent")
    return int(e[0])


def quantize_mxfp4(head: np.ndarray, ids: Optional[np.ndarray] = None, rule: str = "ocp"):
    """The MXFP4 candidate table of head rows ids (None: every row): packed
    E2M1 codes [C][H/2] (element 2i in the low nibble) and E8M0 block scales
    [C][H/32] (code e + 127), block scales by the OCP rule or the fit rule."""
    head = _bf16(head)
    V, H = head.shape
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
    C = V if ids is None else len(ids)
    q = np.empty((C, H // 2), dtype=np.uint8)
    scales = np.empty((C, H // 32), dtype=np.uint8)
    _check(_load().mtp_oracle_quantize_mxfp4_rule(_p(head), V, H, _p(ids), C, _p(q), _p(scales),
                                                  MX_SCALE_RULES[rule]),
           "quantize_mxfp4")
    return q, scales


def mxfp4_values(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The table's element values [C][H] (float64): value(code) * 2^(scale - 127)."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)
    e = np.repeat(np.asarray(scales, dtype=np.int64) - 127, 32, axis=1)
    return np.ldexp(e2m1_value(codes), e)


def draft_mxfp4_gather(h: np.ndarray, q_head: np.ndarray, scales_head: np.ndarray,
                       ids: np.ndarray) -> Dict[str, np.ndarray]:
    """Draft over a candidate id list on an MXFP4 head (codes [V][H/2], block
    scales [V][H/32], every head row quantised once). Qwen3.8 Flash dual-Spark
    tuning log, section "read one fewer big table": the upstream work pairs a
    fixed candidate set with rows chosen per step, stored in a 4-bit float
    format. The candidates are the distinct ids of the list that name a head
    row; the result is the MXFP4 draft over that set's rows in ascending id
    order, so ties go to the lowest id whatever the order of the list. With no
    valid id: id -1, logit NaN."""
    q_head = np.asarray(q_head, dtype=np.uint8)
    scales_head = np.asarray(scales_head, dtype=np.uint8)
    V = q_head.shape[0]
    ids = np.asarray(ids, dtype=np.int64).ravel()
    valid = np.unique(ids[(ids >= 0) & (ids < V)]).astype(np.int32)
    M = np.atleast_2d(h).shape[0]
    if valid.size == 0:
        return {"id": np.full(M, -1, np.int32), "logit": np.full(M, np.nan, np.float32),
                "exact": np.full(M, np.nan), "runner_id": np.full(M, -1, np.int32),
                "runner_exact": np.full(M, np.nan)}
    return draft_mxfp4(h, q_head[valid], scales_head[valid], valid)


def draft_mxfp4(h: np.ndarray, q: np.ndarray, scales: np.ndarray,
                ids: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Draft over an MXFP4 candidate table: first maximum of the fp32-rounded
    logits sum_j h[j] * 2^e(j/32) * value(q[n][j]), reported as ids."""
    x = _bf16(np.atleast_2d(h))
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M, H = x.shape
    N = q.shape[0]
    if q.shape[1] * 2 != H or scales.shape != (N, H // 32):
        raise ValueError("shapes differ")
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = {
        "id": np.empty(M, np.int32),
        "logit": np.empty(M, np.float32),
        "exact": np.empty(M, np.float64),
        "runner_id": np.empty(M, np.int32),
        "runner_exact": np.empty(M, np.float64),
    }
    _check(_load().mtp_oracle_mxfp4_argmax(_p(x), M, _p(q), _p(scales), _p(ids), N, H,
                                           _p(out["id"]), _p(out["logit"]), _p(out["exact"]),
                                           _p(out["runner_id"]), _p(out["runner_exact"])),
           "mxfp4_argmax")
    return out
