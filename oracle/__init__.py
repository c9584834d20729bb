"""CPU oracle of the DeepSeek-V4.1-Flash Engram forward (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The arithmetic lives in ``engram_oracle.cc`` (plain C++, built by
``__graft_entry__.build()`` into ``oracle/liboracle.so``, never linked into the product
library); this module only loads that library with ctypes and moves numpy arrays in and out.
Its header states what is computed and which passage of the pages each step follows.

bf16 tensors are carried as uint16 bit patterns.  Tokens are independent, so any subset of a
batch can be evaluated alone; the library spreads tokens over threads (``ORACLE_THREADS``, by
default the CPUs this process may run on, at most 16) and gives the same bits for any count.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
_sig = {
    "orc_e4m3_values": ([_vp, _i64, _vp], None),
    "orc_e8m0_values": ([_vp, _i64, _vp], None),
    "orc_round_fp32": ([_vp, _i64, _vp], None),
    "orc_bf16_from_double": ([_vp, _i64, _vp], None),
    "orc_bf16_values": ([_vp, _i64, _vp], None),
    "orc_gather_dequant": ([_vp, _i64, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i32],
                           ctypes.c_int),
    "orc_wkv_mxfp8_bits": ([_vp, _vp, _i64, _i64, _vp], None),
    "orc_kv_proj": ([_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _i32], None),
    "orc_gate_apply": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _f64, _f64, _vp, _vp, _vp, _vp,
                        _vp, _vp, _vp, _i32], None),
    "orc_residual": ([_vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp], None),
    "orc_forward": ([_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp,
                     _i64, _vp, _vp, _vp, _vp, _f64, _f64, _vp, _vp, _vp, _vp, _vp, _i32],
                    ctypes.c_int),
    "orc_hash_ids": ([_vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64,
                      _vp, _i64, _i64, _i32, _vp], ctypes.c_int64),
    "orc_param_counts": ([_i64, _i64, _i64, _i64, _i64, _vp], None),
    "orc_bytes_per_token": ([_i64, _i64, _i64, _i64, _vp], None),
}
for _name, (_args, _res) in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def threads() -> int:
    """Threads the oracle uses: ORACLE_THREADS, else the CPUs this process may run on (at most
    16, the CPU share of one GPU on the GPU hosts)."""
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------------


def e4m3fn_value(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 "fn" codes as float64 (NaN for 0x7F / 0xFF)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _lib.orc_e4m3_values(_p(c), c.size, _p(out))
    return out


def e8m0_value(exps) -> np.ndarray:
    """Values of E8M0 scale bytes, 2^(e - 127), NaN for 0xFF."""
    e = _c(exps, np.uint8)
    out = np.empty(e.shape, np.float64)
    _lib.orc_e8m0_values(_p(e), e.size, _p(out))
    return out


def round_fp32(x) -> np.ndarray:
    """Doubles rounded to the nearest fp32 (ties to even), returned as float64."""
    v = _c(x, np.float64)
    out = np.empty(v.shape, np.float64)
    _lib.orc_round_fp32(_p(v), v.size, _p(out))
    return out


def bf16_bits_from_fp32(x) -> np.ndarray:
    """bf16 bit patterns of values rounded to fp32 and then to bf16 (nearest even both times);
    NaN becomes 0x7FC0."""
    v = _c(x, np.float64)
    out = np.empty(v.shape, np.uint16)
    _lib.orc_bf16_from_double(_p(v), v.size, _p(out))
    return out


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    _lib.orc_bf16_values(_p(b), b.size, _p(out))
    return out


# ----------------------------------------------------------------------------------------
# the table as the oracle holds it
# ----------------------------------------------------------------------------------------

RowFetch = Callable[[np.ndarray], Tuple[np.ndarray, np.ndarray]]


class DenseRows:
    """Every row of a table held in memory: codes uint8 [n_rows, hd], scales [n_rows, nb] (fp32,
    or uint8 E8M0 exponents)."""

    def __init__(self, table, scales):
        self.table, self.scales = table, scales

    def __call__(self, rows):
        return self.table[rows], self.scales[rows]


def array_fetch(table, scales) -> DenseRows:
    return DenseRows(table, scales)


def _held_rows(ids: np.ndarray, fetch, n_rows: int, scale_format: str):
    """(codes, scales, row_ids or None, n_held) for the C library.  A DenseRows table is passed
    whole; any other row provider (a generator that regenerates rows on demand) is asked for the
    rows the tokens name, in ascending order, and the library finds each token's rows in that
    list."""
    sdt = np.uint8 if scale_format == "e8m0" else np.float32
    if isinstance(fetch, DenseRows):
        codes, scales = _c(fetch.table, np.uint8), _c(fetch.scales, sdt)
        if scales.shape[0] != codes.shape[0]:
            raise ValueError("table and scales hold different numbers of rows")
        return codes, scales, None, codes.shape[0]
    flat = ids.reshape(-1)
    need = np.unique(flat[(flat >= 0) & (flat < n_rows)])
    if need.size == 0:  # every id is out of range: no row is read
        return np.zeros((1, 1), np.uint8), np.zeros((1, 1), sdt), np.zeros(1, np.int64), 0
    codes, scales = fetch(need)
    codes, scales = _c(codes, np.uint8), _c(scales, sdt)
    if codes.shape[0] != need.size or scales.shape[0] != need.size:
        raise ValueError(f"row provider returned {codes.shape[0]} code rows and {scales.shape[0]} "
                         f"scale rows for {need.size} row ids")
    return codes, scales, _c(need, np.int64), need.size


def _scale_code(scale_format: str) -> int:
    if scale_format not in ("fp32", "e8m0"):
        raise ValueError(scale_format)
    return 1 if scale_format == "e8m0" else 0


# ----------------------------------------------------------------------------------------
# S1 + S2, S3, S4 - S6
# ----------------------------------------------------------------------------------------


def gather_dequant(hash_ids, fetch, n_rows: int, head_dim: int, scale_block: int,
                   scale_format: str = "fp32") -> np.ndarray:
    """emb bf16 bits [M, C * head_dim] for global row ids hash_ids [M, C]; ids outside
    [0, n_rows) give zero rows."""
    ids = _c(hash_ids, np.int64)
    M, C = ids.shape
    codes, scales, row_ids, n_held = _held_rows(ids, fetch, n_rows, scale_format)
    emb = np.empty((M, C * head_dim), np.uint16)
    rc = _lib.orc_gather_dequant(_p(ids), M, C, n_rows, head_dim, scale_block,
                                 _scale_code(scale_format), _p(codes), _p(scales), _p(row_ids),
                                 n_held, _p(emb), threads())
    if rc != 0:
        raise RuntimeError("oracle gather: a row the tokens name is not held")
    return emb


def _weights(wkv):
    """(bf16 bits, fp32 values): wkv given as uint16 bit patterns or as values that are bf16
    numbers (any float dtype; converted to fp32, which holds them exactly)."""
    w = np.asarray(wkv)
    if w.dtype == np.uint16:
        return _c(w, np.uint16), None
    return None, _c(w, np.float32)


def kv_proj(emb_bits, wkv, with_exact: bool = False):
    """kv bf16 bits [M, N] = bf16(emb @ wkv^T), wkv [N, K] in the Linear [out, in] layout; with
    ``with_exact`` the unrounded double sums as well."""
    emb = _c(emb_bits, np.uint16)
    wb, wf = _weights(wkv)
    M, K = emb.shape
    N = (wb if wb is not None else wf).shape[0]
    out = np.empty((M, N), np.uint16)
    exact = np.empty((M, N), np.float64) if with_exact else None
    _lib.orc_kv_proj(_p(emb), _p(wb), _p(wf), M, N, K, _p(out), _p(exact), threads())
    return (out, exact) if with_exact else out


def wkv_mxfp8_bits(codes, scales) -> np.ndarray:
    """bf16 bit patterns [N, K] of a wkv stored as e4m3fn codes [N, K] with one E8M0 scale per
    32 consecutive inputs [N, K / 32]."""
    c = _c(codes, np.uint8)
    N, K = c.shape
    e = _c(scales, np.uint8).reshape(N, K // 32)
    out = np.empty((N, K), np.uint16)
    _lib.orc_wkv_mxfp8_bits(_p(c), _p(e), N, K, _p(out))
    return out


def _mask(token_mask, M):
    return None if token_mask is None else _c(np.asarray(token_mask).reshape(M).astype(bool), np.uint8)


def gate_apply(x_bits, kv_bits, q_weight, k_weight, token_mask, eps, clamp) -> dict:
    """S4 - S6 from a given kv: gate [M, hc] and its sums (A, Kq, D, dot), the unrounded output
    out_f [M, hc, dim] and its bf16 rounding out_bits."""
    x = _c(x_bits, np.uint16)
    M, hc, dim = x.shape
    kv = _c(kv_bits, np.uint16)
    q, k = _c(q_weight, np.float32), _c(k_weight, np.float32)
    mask = _mask(token_mask, M)
    r = {n: np.empty((M, hc), np.float64) for n in ("gate", "A", "Kq", "D", "dot")}
    out_f = np.empty((M, hc, dim), np.float64)
    out_bits = np.empty((M, hc, dim), np.uint16)
    _lib.orc_gate_apply(_p(x), _p(kv), _p(q), _p(k), _p(mask), M, hc, dim, float(eps), float(clamp),
                        _p(r["gate"]), _p(r["A"]), _p(r["Kq"]), _p(r["D"]), _p(r["dot"]),
                        _p(out_f), _p(out_bits), threads())
    return {**r, "out_f": out_f, "out_bits": out_bits}


def gate(x_bits, kv_bits, q_weight, k_weight, token_mask, eps, clamp) -> dict:
    """S4 + S5: gate [M, hc] and its sums."""
    r = gate_apply(x_bits, kv_bits, q_weight, k_weight, token_mask, eps, clamp)
    return {n: r[n] for n in ("gate", "A", "Kq", "D", "dot")}


def residual(x_bits, kv_bits, g, token_mask) -> dict:
    """S6 with a given gate [M, hc]: out_f and out_bits."""
    x = _c(x_bits, np.uint16)
    M, hc, dim = x.shape
    kv = _c(kv_bits, np.uint16)
    gg = _c(g, np.float64)
    mask = _mask(token_mask, M)
    out_f = np.empty((M, hc, dim), np.float64)
    out_bits = np.empty((M, hc, dim), np.uint16)
    _lib.orc_residual(_p(x), _p(kv), _p(gg), _p(mask), M, hc, dim, _p(out_f), _p(out_bits))
    return {"out_f": out_f, "out_bits": out_bits}


def forward(x_bits, hash_ids, token_mask, fetch, n_rows: int, head_dim: int, scale_block: int,
            wkv, q_weight, k_weight, eps: float = 1e-20, clamp: float = 1e-6,
            scale_format: str = "fp32", want: Tuple[str, ...] = ("emb", "kv", "gate", "out_f",
                                                                 "out_bits")) -> dict:
    """Engram.forward for tokens x_bits [M, hc, dim] with hash_ids [M, C] and token_mask [M]
    (None = all open).  ``want`` names the outputs to return (emb, kv, gate, out_f, out_bits)."""
    x = _c(x_bits, np.uint16)
    M, hc, dim = x.shape
    ids = _c(hash_ids, np.int64).reshape(M, -1)
    C = ids.shape[1]
    codes, scales, row_ids, n_held = _held_rows(ids, fetch, n_rows, scale_format)
    wb, wf = _weights(wkv)
    q, k = _c(q_weight, np.float32), _c(k_weight, np.float32)
    mask = _mask(token_mask, M)
    K, N = C * head_dim, (hc + 1) * dim
    shapes = {"emb": ((M, K), np.uint16), "kv": ((M, N), np.uint16), "gate": ((M, hc), np.float64),
              "out_f": ((M, hc, dim), np.float64), "out_bits": ((M, hc, dim), np.uint16)}
    res = {n: np.empty(s, dt) for n, (s, dt) in shapes.items() if n in want}
    rc = _lib.orc_forward(_p(x), _p(ids), _p(mask), M, hc, dim, C, head_dim, scale_block,
                          _scale_code(scale_format), n_rows, _p(codes), _p(scales), _p(row_ids),
                          n_held, _p(wb), _p(wf), _p(q), _p(k), float(eps), float(clamp),
                          _p(res.get("emb")), _p(res.get("kv")), _p(res.get("gate")),
                          _p(res.get("out_f")), _p(res.get("out_bits")), threads())
    if rc != 0:
        raise RuntimeError("oracle forward: a row the tokens name is not held")
    return res


# ----------------------------------------------------------------------------------------
# the hash step in front of the path
# ----------------------------------------------------------------------------------------


def hash_ids(input_ids, token_map, multipliers, primes, offsets, pad_id: int, history,
             start_pos: int = 0, token_mask=None, dead: int = -1, wide: Optional[bool] = None):
    """Row ids [B, L, n_layers, (max_ngram - 1) * n_heads] of tokens input_ids [B, L] at positions
    start_pos.. of their sequences; ``history`` [B, S] int64 is read and written in place.

    multipliers [n_layers, max_ngram] (int64 bit patterns or non-negative Python ints), primes
    [n_layers, max_ngram - 1, n_heads], offsets [n_layers, n_cols].  ``wide`` keeps products
    exact in 128 bits (Python-integer semantics); by default it is chosen when the inputs are
    object arrays of Python ints, else products wrap modulo 2^64 as int64 tensors do."""
    ids = np.asarray(input_ids)
    if wide is None:
        wide = ids.dtype == object or np.asarray(multipliers).dtype == object
    B, L = ids.shape
    mult = np.asarray(multipliers)
    if mult.dtype == object:
        mult = np.array([[int(v) & ((1 << 64) - 1) for v in row] for row in mult], dtype=np.uint64)
    else:
        mult = _c(mult, np.int64).view(np.uint64)
    n_layers, max_ngram = mult.shape
    pr = _c(np.asarray(primes).astype(np.int64), np.int64)
    n_heads = pr.shape[-1]
    off = _c(np.asarray(offsets).astype(np.int64), np.int64)
    tm = _c(np.asarray(token_map).astype(np.int64), np.int64)
    idv = _c(ids.astype(np.int64), np.int64)
    mask = None if token_mask is None else _c(np.asarray(token_mask).astype(bool), np.uint8)
    hist = _c(np.asarray(history).astype(np.int64), np.int64)
    out = np.empty((B, L, n_layers, (max_ngram - 1) * n_heads), np.int64)
    rc = _lib.orc_hash_ids(_p(idv), _p(mask), B, L, _p(tm), tm.size, _p(_c(mult, np.uint64)),
                           _p(pr), _p(off), n_layers, max_ngram, n_heads, int(pad_id), int(dead),
                           _p(hist), hist.shape[1], start_pos, int(bool(wide)), _p(out))
    if rc < 0:
        raise ValueError("oracle hash: invalid arguments")
    history[...] = hist
    if wide:
        return out.astype(object)
    return out


# ----------------------------------------------------------------------------------------
# layout accounting
# ----------------------------------------------------------------------------------------


def param_counts(n_rows: int, head_dim: int, n_cols: int, hc: int, dim: int) -> dict:
    """Learned element counts of one Engram instance: table, wkv, gate weights, total."""
    out = np.zeros(4, np.int64)
    _lib.orc_param_counts(n_rows, head_dim, n_cols, hc, dim, _p(out))
    return {"table": int(out[0]), "wkv": int(out[1]), "gate": int(out[2]), "total": int(out[3])}


def bytes_per_token(n_cols: int, head_dim: int, scale_block: int, scale_bytes: int) -> dict:
    """Table bytes one token reads in one module: fp8 codes and block scales."""
    out = np.zeros(2, np.int64)
    _lib.orc_bytes_per_token(n_cols, head_dim, scale_block, scale_bytes, _p(out))
    return {"codes": int(out[0]), "scales": int(out[1])}


__all__ = [
    "e4m3fn_value", "e8m0_value", "round_fp32", "bf16_bits_from_fp32", "bf16_value", "array_fetch",
    "DenseRows", "gather_dequant", "kv_proj", "wkv_mxfp8_bits", "gate", "residual", "gate_apply",
    "forward", "hash_ids", "param_counts", "bytes_per_token", "threads",
]
