"""CPU oracle for the DeepSeek-V4.1-Flash Engram forward (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run this module.  The product path (the HIP library and its Python binding) never
touches it and shares no code with it.

What it computes is the plain definition of the Engram block, written from the pages:

* "DeepSeek-V4.1 / blocks / engram-second" (atlas.klimoza.dev), code panel, ``Engram.forward``
  and ``ParallelEngramEmbedding.forward``: gather fp8 rows and their block scales, multiply in
  fp32, round to bf16, flatten the hash columns, project with ``wkv`` into four keys and one
  value, gate each stream by a normalised dot product, add gate x value to every stream.
* "DeepSeek's Other Modules" (monishver11.github.io), section "Engram", subsections "The lookup
  pipeline" (context-aware gating, shared value and per-stream key) and "V4.1's two tables,
  reconciled" (24 columns of 256 fp8 features, the 6,144 -> 25,600 projection).
* "Engram in DeepSeek V4.1 Flash" (zhuai.tech), "Step 3: Inject memory at the correct layer
  boundary": the same gate formula restated, per stream, with q and k weights used as a product.

Precision: every floating-point step is carried out in IEEE double, except where the pages fix
a narrower type, which is then applied as an explicit rounding:
  * the dequantisation product is an fp32 multiply (fp8 value times fp32 scale);
  * table rows are rounded to bf16 before the projection;
  * the projection output (kv) is rounded to bf16 (reading: the Linear keeps the bf16
    activation dtype; its accumulation is exact here, then rounded once via fp32);
  * q_weight * k_weight is an fp32 product;
  * the output streams are rounded to bf16 (through fp32).
Reductions over ``dim`` start from +0 so that an all-zero sum is +0.

All arrays are numpy; bf16 tensors are carried as uint16 bit patterns.
"""
from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np

# ----------------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------------


def e4m3fn_value(codes: np.ndarray) -> np.ndarray:
    """Value of OCP FP8 E4M3 "fn" codes (torch.float8_e4m3fn; table dtype on the engram-second
    page, ParallelEngramEmbedding): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
    no infinities; exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal (m * 2^-9)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2((e - 10).astype(np.float64)))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e8m0_value(exps: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale bytes, the block scale of the MXFP8 tables ("Engram in DeepSeek V4.1
    Flash", Step 2; "DeepSeek's Other Modules", V4.1's two tables, reconciled: E4M3 codes with
    one E8M0 scale per 32 values).  The format is the OCP Microscaling (MX) v1.0 scale: an 8-bit
    unsigned biased exponent, value 2^(e - 127) for e = 0 .. 254; e = 255 is NaN."""
    e = np.asarray(exps, dtype=np.uint8).astype(np.int64)
    val = np.exp2((e - 127).astype(np.float64))
    return np.where(e == 255, np.nan, val)


def round_fp32(x: np.ndarray) -> np.ndarray:
    """Round doubles to the nearest fp32 (ties to even); returned as float64."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits_from_fp32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bit patterns.
    NaN becomes the canonical quiet NaN 0x7FC0; overflow past the largest bf16 gives inf."""
    with np.errstate(invalid="ignore", over="ignore"):
        f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------
# S1 + S2: row gather and dequantisation
# ----------------------------------------------------------------------------------------

RowFetch = Callable[[np.ndarray], Tuple[np.ndarray, np.ndarray]]


def array_fetch(table: np.ndarray, scales: np.ndarray) -> RowFetch:
    """Row provider over in-memory arrays: table uint8 [n_rows, hd], scales [n_rows, nb] (fp32,
    or uint8 E8M0 exponents)."""

    def fetch(rows: np.ndarray):
        return table[rows], scales[rows]

    return fetch


def scale_value(scales: np.ndarray, scale_format: str) -> np.ndarray:
    """Block scales as float64 values: fp32 scales as stored, or E8M0 exponent bytes."""
    if scale_format == "fp32":
        return np.asarray(scales, dtype=np.float32).astype(np.float64)
    if scale_format == "e8m0":
        return e8m0_value(scales)
    raise ValueError(scale_format)


def gather_dequant(hash_ids: np.ndarray, fetch: RowFetch, n_rows: int, head_dim: int,
                   scale_block: int, scale_format: str = "fp32") -> np.ndarray:
    """emb bf16 bits [M, C * head_dim] for hash_ids [M, C] (global row ids).

    engram-second page, ParallelEngramEmbedding.forward with a single shard: rows outside
    [0, n_rows) are replaced by row 0 for the lookup and then zeroed; the fp8 value of every
    feature is multiplied in fp32 by the scale of its block (feature c uses scale c //
    scale_block) and the product is rounded to bf16.  Engram.forward then flattens the
    columns: feature c of column j lands at position j * head_dim + c.  Scales are fp32 (the
    benchmark workloads' tables) or E8M0 (the official MXFP8 tables, ``scale_format="e8m0"``).
    """
    ids = np.asarray(hash_ids, dtype=np.int64)
    M, C = ids.shape
    out_of_range = (ids < 0) | (ids >= n_rows)
    local = np.where(out_of_range, 0, ids)
    codes, scales = fetch(local.reshape(-1))
    codes = np.asarray(codes, dtype=np.uint8).reshape(M, C, head_dim)
    scales = scale_value(scales, scale_format).reshape(M, C, head_dim // scale_block)
    block_of_feature = np.arange(head_dim) // scale_block
    with np.errstate(invalid="ignore", over="ignore"):
        prod = e4m3fn_value(codes) * scales[:, :, block_of_feature]
    bits = bf16_bits_from_fp32(round_fp32(prod))
    bits[out_of_range] = 0
    return bits.reshape(M, C * head_dim)


# ----------------------------------------------------------------------------------------
# S3: wkv projection
# ----------------------------------------------------------------------------------------


def kv_proj(emb_bits: np.ndarray, wkv: np.ndarray, chunk: int = 4096,
            with_exact: bool = False):
    """kv bf16 bits [M, N] = bf16(emb @ wkv^T).

    wkv is the Linear weight in [out, in] = [(hc + 1) * dim, C * head_dim] layout (the
    engram-second page, ``self.wkv = Linear(n_hash_cols * head_dim, dim * (hc_mult + 1))``).
    ``wkv`` is given either as bf16 bit patterns (uint16) or as float values that are exactly
    bf16 numbers.  The products of two bf16 numbers are exact in double and 6,144-term sums
    stay far inside double precision, so the accumulation is effectively exact; the result
    is rounded to fp32 and then to bf16.  With ``with_exact`` the unrounded sums are returned
    as well (for error bounds).
    """
    a = bf16_value(emb_bits)
    M = a.shape[0]
    N = wkv.shape[0]
    out = np.empty((M, N), dtype=np.uint16)
    exact = np.empty((M, N), dtype=np.float64) if with_exact else None
    for lo in range(0, N, chunk):
        hi = min(N, lo + chunk)
        w = wkv[lo:hi]
        w = bf16_value(w) if w.dtype == np.uint16 else np.asarray(w, dtype=np.float64)
        with np.errstate(invalid="ignore", over="ignore"):
            acc = a @ w.T
            out[:, lo:hi] = bf16_bits_from_fp32(round_fp32(acc))
        if with_exact:
            exact[:, lo:hi] = acc
    return (out, exact) if with_exact else out


def wkv_mxfp8_bits(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [N, K] of a wkv stored in FP8.

    "DeepSeek's Other Modules", section Engram: the four key projections and the value
    projection fuse into one FP8 matmul ("The lookup pipeline"), and the projections are FP8
    like the tables ("V4.1's two tables, reconciled"); the pages give no scale layout for the
    projection.  Reading: the tables' MXFP8 form applied along the projection's input features,
    e4m3fn codes [N, K] with one E8M0 scale per 32 consecutive inputs [N, K / 32], dequantised
    by the tables' rule (fp32 product, then bf16).  The projection is then the bf16 one of
    ``kv_proj`` over these weights.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    scale = e8m0_value(np.asarray(scales, dtype=np.uint8).reshape(N, K // 32))
    with np.errstate(invalid="ignore", over="ignore"):
        prod = e4m3fn_value(codes) * np.repeat(scale, 32, axis=1)
    return bf16_bits_from_fp32(round_fp32(prod))


# ----------------------------------------------------------------------------------------
# S4 + S5: per-(token, stream) gate
# ----------------------------------------------------------------------------------------


def gate(x_bits: np.ndarray, kv_bits: np.ndarray, q_weight: np.ndarray, k_weight: np.ndarray,
         token_mask: Optional[np.ndarray], eps: float, clamp: float) -> dict:
    """Gate [M, hc] (float64) and its intermediate sums.

    engram-second page, Engram.forward: keys are the first hc * dim columns of kv, one per
    stream; with w = q_weight * k_weight (an fp32 product) and h = x as float,
        rstd = rsqrt(mean_d h^2 + eps) * rsqrt(mean_d key^2 + eps)
        dot  = (sum_d h * w * key) * rstd * dim^-1/2
        gate = sigmoid(copysign(sqrt(max(|dot|, clamp)), dot))
    normalised per (token, stream), not across streams; the gate is 0 where token_mask is
    false.  The zhuai.tech page (Step 3) restates the same gate with q * k precomputed.
    """
    x = bf16_value(x_bits)
    M, hc, dim = x.shape
    key = bf16_value(kv_bits[:, :hc * dim]).reshape(M, hc, dim)
    w = round_fp32(np.asarray(q_weight, np.float64) * np.asarray(k_weight, np.float64))
    A = 0.0 + np.sum(x * x, axis=-1)
    Kq = 0.0 + np.sum(key * key, axis=-1)
    D = 0.0 + np.sum((x * w[None]) * key, axis=-1)
    rstd = (1.0 / np.sqrt(A / dim + eps)) * (1.0 / np.sqrt(Kq / dim + eps))
    dot = D * rstd * (dim ** -0.5)
    z = np.copysign(np.sqrt(np.maximum(np.abs(dot), clamp)), dot)
    g = 1.0 / (1.0 + np.exp(-z))
    if token_mask is not None:
        g = np.where(np.asarray(token_mask).reshape(M, 1).astype(bool), g, 0.0)
    return {"gate": g, "A": A, "Kq": Kq, "D": D, "dot": dot}


# ----------------------------------------------------------------------------------------
# S6: residual add
# ----------------------------------------------------------------------------------------


def residual(x_bits: np.ndarray, kv_bits: np.ndarray, g: np.ndarray,
             token_mask: Optional[np.ndarray]) -> dict:
    """out = h + gate * value on every stream, value shared (engram-second page, last line of
    Engram.forward; zhuai.tech Step 3: hidden += gate x value).  Returns the unrounded result
    (float64) and its bf16 rounding; tokens whose mask is false keep x bit for bit, as the
    Engram.forward docstring says they pass through untouched."""
    x = bf16_value(x_bits)
    M, hc, dim = x.shape
    value = bf16_value(kv_bits[:, hc * dim:(hc + 1) * dim])
    out_f = x + g[:, :, None] * value[:, None, :]
    out_bits = bf16_bits_from_fp32(round_fp32(out_f))
    if token_mask is not None:
        keep = ~np.asarray(token_mask).reshape(M).astype(bool)
        out_bits[keep] = x_bits[keep]
        out_f[keep] = x[keep]
    return {"out_f": out_f, "out_bits": out_bits}


def gate_apply(x_bits, kv_bits, q_weight, k_weight, token_mask, eps, clamp) -> dict:
    """S4-S6 from a given kv (the split the zhuai.tech page makes between projection and
    gating)."""
    g = gate(x_bits, kv_bits, q_weight, k_weight, token_mask, eps, clamp)
    r = residual(x_bits, kv_bits, g["gate"], token_mask)
    return {**g, **r}


# ----------------------------------------------------------------------------------------
# whole forward
# ----------------------------------------------------------------------------------------


def forward(x_bits: np.ndarray, hash_ids: np.ndarray, token_mask: Optional[np.ndarray],
            fetch: RowFetch, n_rows: int, head_dim: int, scale_block: int, wkv: np.ndarray,
            q_weight: np.ndarray, k_weight: np.ndarray, eps: float = 1e-20,
            clamp: float = 1e-6, scale_format: str = "fp32") -> dict:
    """Engram.forward for tokens x_bits [M, hc, dim] with hash_ids [M, C] and token_mask [M]
    (None = all true).  Tokens are independent, so any subset of a batch can be evaluated
    alone."""
    emb = gather_dequant(hash_ids, fetch, n_rows, head_dim, scale_block, scale_format)
    kv = kv_proj(emb, wkv)
    res = gate_apply(x_bits, kv, q_weight, k_weight, token_mask, eps, clamp)
    return {"emb": emb, "kv": kv, **res}


# ----------------------------------------------------------------------------------------
# The hash step in front of the path: token ids -> the 24 global row ids of each Engram layer
# ----------------------------------------------------------------------------------------


def hash_ids(input_ids: np.ndarray, token_map: np.ndarray, multipliers: np.ndarray,
             primes: np.ndarray, offsets: np.ndarray, pad_id: int, history: np.ndarray,
             start_pos: int = 0, token_mask: Optional[np.ndarray] = None,
             dead: int = -1) -> np.ndarray:
    """Hash ids [B, L, n_layers, (max_ngram - 1) * n_heads] of tokens input_ids [B, L] at
    positions start_pos .. start_pos + L - 1 (engram-second page, code panel, the hash module's
    forward; "DeepSeek's Other Modules", Engram, The lookup pipeline: compressed ids, one odd
    multiplier per look-back, XOR, modulo a prime per head).

    token_map [vocab] maps raw ids to compressed ids; tokens whose mask is false become ``dead``
    (image spans).  ``history`` [B, S] holds the compressed ids of earlier positions of each
    sequence and receives those of this call (in place).  For each look-back ``shift`` the
    source id is the history at position - shift; once a source lies before the sequence start
    or is dead, it and every longer look-back read ``pad_id``.  products = tokens * multipliers
    [n_layers, max_ngram]; the running XOR over look-backs 0..i is the (i+1)-gram's hash, taken
    modulo primes[layer, i - 1, head] (floor modulo) and offset by offsets[layer, column].

    Integer dtype decides the arithmetic: int64 arrays wrap modulo 2^64 as the page's int64
    tensors do; object arrays of Python ints give unbounded products."""
    ids = np.asarray(input_ids)
    B, L = ids.shape
    n_layers, max_ngram = multipliers.shape
    compressed = np.asarray(token_map)[ids.astype(np.int64)]
    if token_mask is not None:
        compressed = np.where(np.asarray(token_mask).astype(bool), compressed, dead)
    history[:B, start_pos:start_pos + L] = compressed
    positions = np.arange(start_pos, start_pos + L)
    blocked = np.zeros((B, L), dtype=bool)
    tokens = []
    for shift in range(max_ngram):
        source = history[:B, np.maximum(positions - shift, 0)]
        blocked = blocked | (positions < shift)[None, :] | (source == dead)
        tokens.append(np.where(blocked, pad_id, source))
    tokens = np.stack(tokens, axis=-1)                          # [B, L, max_ngram]
    with np.errstate(over="ignore"):
        products = tokens[:, :, None, :] * multipliers[None, None]  # [B, L, n_layers, max_ngram]
    rolling = products[..., 0]
    hashes = []
    for i in range(1, max_ngram):
        rolling = rolling ^ products[..., i]
        hashes.append(np.mod(rolling[..., None], primes[None, None, :, i - 1, :]))
    return np.concatenate(hashes, axis=-1) + offsets[None, None]


# ----------------------------------------------------------------------------------------
# layout accounting
# ----------------------------------------------------------------------------------------


def param_counts(n_rows: int, head_dim: int, n_cols: int, hc: int, dim: int) -> dict:
    """Learned element counts of one Engram instance (engram-second page, parameter table):
    table rows x features, the wkv projection, and the q/k gate weights."""
    table = n_rows * head_dim
    wkv = (n_cols * head_dim) * (dim * (hc + 1))
    gate_w = 2 * hc * dim
    return {"table": table, "wkv": wkv, "gate": gate_w, "total": table + wkv + gate_w}


def bytes_per_token(n_cols: int, head_dim: int, scale_block: int, scale_bytes: int) -> dict:
    """Table traffic of one token in one module: one fp8 byte per feature of each gathered row
    plus one scale per block ("DeepSeek's Other Modules", Serving cost)."""
    codes = n_cols * head_dim
    scales = n_cols * (head_dim // scale_block) * scale_bytes
    return {"codes": codes, "scales": scales}


__all__ = [
    "e4m3fn_value", "e8m0_value", "scale_value", "round_fp32", "bf16_bits_from_fp32", "bf16_value",
    "array_fetch",
    "gather_dequant", "kv_proj", "wkv_mxfp8_bits", "gate", "residual", "gate_apply", "forward", "hash_ids",
    "param_counts",
    "bytes_per_token",
]
