"""Seeded synthetic inputs for the Engram forward (test and benchmark infrastructure).

This module draws inputs; it holds none of the Engram method's arithmetic (no fp8 decode,
no dequantisation, no projection, no gate).  Both the CPU oracle and the HIP path take
their inputs from here, and nothing else is shared between them.

Generator definition (the same on the host, in numpy, and on the device, in
``synth/fill.hip``):

* ``mix64(z)`` is the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014): ``z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
  z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31``, all modulo 2**64.
* A tensor gets a 64-bit ``key`` (derived on the host from the seed and a stream id); its
  i-th draw is ``draw(key, i) = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``, i.e. the i-th
  output of a SplitMix64 sequence started at ``key``.  Any element can be regenerated alone.
* fp8-e4m3 codes ``~ RNE_e4m3(U(-4, 4))``: with ``d = draw(key, r*hd + c)``, the sign is bit
  63 and the magnitude is ``v = r24 * 2**-22`` with ``r24 = (d >> 32) & 0xFFFFFF``; ``v`` is
  rounded to the nearest e4m3 magnitude (ties to even) with integer arithmetic only.
* uniform fp32 ``U(lo, hi)``: ``u = d >> 40``; ``v = lo + (hi - lo) * (u * 2**-24)`` in IEEE
  double with every operation rounded separately (no fused multiply-add), then rounded to
  fp32 (nearest even).
* approximately normal ``N(mean, std)``: Irwin-Hall sum of twelve 16-bit uniforms taken
  from draws ``3i, 3i+1, 3i+2`` (four 16-bit fields each): ``z = (S + 6 - 393216) / 65536``
  (exact), ``v = mean + std * z`` in double without fusion, then fp32, then bf16 with
  round-to-nearest-even.  Tails are bounded at 6 sigma.
* hash ids, token masks and the outlier-token choice are drawn on the host only and copied
  to the device (they are small).  Zipf ranks use Hoermann and Derflinger's
  rejection-inversion method ("Rejection-inversion to generate variates from monotone
  discrete distributions", ACM TOMACS 6(3), 1996).
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import dataclasses
import math
import os
from typing import List, Optional, Sequence

import numpy as np

_U64 = np.uint64
GOLDEN = _U64(0x9E3779B97F4A7C15)
_M1 = _U64(0xBF58476D1CE4E5B9)
_M2 = _U64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

# stream ids (one per tensor kind); an instance index is folded in as stream + 64 * inst
S_CODES, S_SCALES, S_WKV, S_X, S_QW, S_KW, S_HASH, S_MASK, S_OUTLIER, S_PERM = range(1, 11)
S_TOKMAP, S_MULT, S_IDS, S_SPAN = range(11, 15)  # hash-step inputs
S_WKV8, S_WKV8S = range(15, 17)  # MXFP8 wkv: codes, E8M0 scales


# ----------------------------------------------------------------------------------------
# counter-based generator
# ----------------------------------------------------------------------------------------
def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=_U64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _U64(30))) * _M1
        z = (z ^ (z >> _U64(27))) * _M2
    return z ^ (z >> _U64(31))


def mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int, inst: int = 0) -> int:
    """64-bit key of one tensor's draw sequence."""
    s = stream + 64 * inst
    return mix64_int(((seed & 0xFFFFFFFF) << 24 | (s & 0xFFFFFF)) * 0x9E3779B97F4A7C15)


def draw(key: int, idx: np.ndarray) -> np.ndarray:
    """draw(key, i) for a uint64/int64 index array."""
    i = np.asarray(idx).astype(_U64)
    with np.errstate(over="ignore"):
        return mix64(_U64(key) + (i + _U64(1)) * GOLDEN)


def _f32_to_bf16_bits(v32: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 bit patterns, nearest even (generator's own copy)."""
    b = np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + _U64(0x7FFF) + ((b >> _U64(16)) & _U64(1))
    return (b >> _U64(16)).astype(np.uint16)


def e4m3_magnitude_code(r24: np.ndarray) -> np.ndarray:
    """Nearest-even e4m3 magnitude code of v = r24 * 2**-22 (0 <= r24 < 2**24), integer-only."""
    r = np.asarray(r24, dtype=np.int64)
    p = np.zeros_like(r)
    nz = r > 0
    p[nz] = np.floor(np.log2(r[nz].astype(np.float64))).astype(np.int64)
    # guard log2 rounding at exact powers of two
    p = np.where((np.int64(1) << np.clip(p, 0, 62)) > r, p - 1, p)
    p = np.where((np.int64(1) << np.clip(p + 1, 0, 62)) <= r, p + 1, p)
    sub = p < 16                      # v < 2**-6: subnormal grid of 2**-9 = 2**13 units
    q = np.where(sub, 13, p - 3)      # quantum exponent in units of 2**-22
    t = r >> q
    rem = r & ((np.int64(1) << q) - 1)
    half = np.int64(1) << (q - 1)
    up = (rem > half) | ((rem == half) & ((t & 1) == 1))
    t = t + up.astype(np.int64)
    # subnormal: code = t (t == 8 is the smallest normal, code 0x08)
    e = p - 15
    carry = t == 16
    e = np.where(carry, e + 1, e)
    t = np.where(carry, 8, t)
    normal_code = (e << 3) | (t - 8)
    return np.where(sub, t, normal_code).astype(np.uint8)


def codes_from_draws(d: np.ndarray) -> np.ndarray:
    sign = (d >> _U64(63)).astype(np.uint8)
    r24 = ((d >> _U64(32)) & _U64(0xFFFFFF)).astype(np.int64)
    return (sign << np.uint8(7)) | e4m3_magnitude_code(r24)


def uniform_f32_from_draws(d: np.ndarray, lo: float, hi: float) -> np.ndarray:
    u = (d >> _U64(40)).astype(np.float64) * (2.0 ** -24)
    w = np.float64(hi) - np.float64(lo)
    return (np.float64(lo) + w * u).astype(np.float32)


def e8m0_from_draws(d: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """E8M0 exponent bytes, uniform integers in [lo, hi] (integer-only, as on the device)."""
    span = np.uint64(hi - lo + 1)
    return (np.uint64(lo) + (((d >> _U64(40)) * span) >> _U64(24))).astype(np.uint8)


def normal_f32_from_draws(d3: np.ndarray, mean: float, std) -> np.ndarray:
    """d3: [..., 3] uint64 draws -> approximately N(mean, std) rounded to fp32."""
    s = np.zeros(d3.shape[:-1], dtype=np.int64)
    for k in range(3):
        dk = d3[..., k]
        for f in range(4):
            s += ((dk >> _U64(16 * f)) & _U64(0xFFFF)).astype(np.int64)
    z = (s + 6 - 393216).astype(np.float64) / 65536.0
    v = np.float64(mean) + np.asarray(std, dtype=np.float64) * z
    return v.astype(np.float32)


def normal_bf16(key: int, i0: int, n: int, mean: float, std) -> np.ndarray:
    """Elements i0 .. i0+n-1 of an approximately-normal bf16 tensor (uint16 bit patterns)."""
    idx = np.arange(i0, i0 + n, dtype=np.int64)
    d = draw(key, (3 * idx)[:, None] + np.arange(3, dtype=np.int64)[None, :])
    return _f32_to_bf16_bits(normal_f32_from_draws(d, mean, std))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------
# layouts and workloads
# ----------------------------------------------------------------------------------------
def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    f = 3
    while f * f <= n:
        if n % f == 0:
            return False
        f += 2
    return True


def primes_from(start: int, count: int) -> List[int]:
    """The first `count` primes >= start, ascending."""
    out, n = [], start
    while len(out) < count:
        if _is_prime(n):
            out.append(n)
        n += 1
    return out


def model_primes(module: int, n_cols: int = 24) -> List[int]:
    """Row-range lengths of an Engram module: primes above 16,000,000 taken in order and
    never reused, 24 per module (module 0 takes the first 24, module 1 the next 24)."""
    return primes_from(16_000_001, n_cols * (module + 1))[n_cols * module:]


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    hc: int
    dim: int
    n_cols: int
    head_dim: int
    scale_block: int
    primes: Sequence[int]
    seed: int
    wkv_std: float = 0.02
    qk_std: float = 0.0               # 0 -> q = k = 1 exactly
    x_std: float = 1.0
    outlier_frac: float = 0.0         # fraction of tokens whose x is drawn with std x outlier_scale
    outlier_scale: float = 50.0
    mask_false_frac: float = 0.0
    masked_positions: Sequence[int] = ()
    hash_dist: str = "uniform"        # or "zipf"
    zipf_s: float = 1.1
    n_instances: int = 1
    scale_lo: float = 0.01
    scale_hi: float = 0.1
    scale_format: str = "fp32"        # or "e8m0": one exponent byte per block (MXFP8 tables)
    e8m0_lo: int = 120                # E8M0 exponents drawn uniformly in [lo, hi] (2^-7 .. 2^-3)
    e8m0_hi: int = 124
    wkv_format: str = "bf16"          # or "mxfp8": e4m3fn codes + one E8M0 scale per 32 inputs
    wkv_e8m0_lo: int = 119            # wkv scale exponents uniform in [lo, hi] (2^-8 .. 2^-6)
    wkv_e8m0_hi: int = 121
    eps: float = 1e-20
    clamp: float = 1e-6

    # derived sizes
    @property
    def M(self) -> int:
        return self.B * self.T

    @property
    def K(self) -> int:
        return self.n_cols * self.head_dim

    @property
    def N(self) -> int:
        return (self.hc + 1) * self.dim

    @property
    def n_blocks(self) -> int:
        return self.head_dim // self.scale_block

    @property
    def n_rows(self) -> int:
        return int(sum(self.primes))

    @property
    def offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.primes)[:-1]]).astype(np.int64)

    def key(self, stream: int, inst: int = 0) -> int:
        return stream_key(self.seed, stream, inst)

    # ---------------- host-side generation ----------------
    def codes_rows(self, rows: np.ndarray, inst: int = 0) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64)
        c = np.arange(self.head_dim, dtype=np.int64)
        d = draw(self.key(S_CODES, inst), rows[:, None] * self.head_dim + c[None, :])
        return codes_from_draws(d)

    def scales_rows(self, rows: np.ndarray, inst: int = 0) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64)
        b = np.arange(self.n_blocks, dtype=np.int64)
        d = draw(self.key(S_SCALES, inst), rows[:, None] * self.n_blocks + b[None, :])
        if self.scale_format == "e8m0":
            return e8m0_from_draws(d, self.e8m0_lo, self.e8m0_hi)
        return uniform_f32_from_draws(d, self.scale_lo, self.scale_hi)

    def wkv_rows(self, n_lo: int, n_hi: int, inst: int = 0) -> np.ndarray:
        """bf16 bit patterns of wkv rows [n_lo, n_hi), shape [n_hi - n_lo, K]."""
        n = (n_hi - n_lo) * self.K
        return normal_bf16(self.key(S_WKV, inst), n_lo * self.K, n, 0.0, self.wkv_std).reshape(
            n_hi - n_lo, self.K)

    def wkv8_rows(self, n_lo: int, n_hi: int, inst: int = 0):
        """MXFP8 wkv rows [n_lo, n_hi): e4m3fn codes [n, K] (the table codes' distribution) and
        E8M0 exponents [n, K / 32] uniform in [wkv_e8m0_lo, wkv_e8m0_hi]."""
        rows = np.arange(n_lo, n_hi, dtype=np.int64)
        k = np.arange(self.K, dtype=np.int64)
        codes = codes_from_draws(draw(self.key(S_WKV8, inst), rows[:, None] * self.K + k[None, :]))
        b = np.arange(self.K // 32, dtype=np.int64)
        d = draw(self.key(S_WKV8S, inst), rows[:, None] * (self.K // 32) + b[None, :])
        return codes, e8m0_from_draws(d, self.wkv_e8m0_lo, self.wkv_e8m0_hi)

    def wkv8(self, inst: int = 0, chunk_rows: int = 512, threads: int = 0):
        """All MXFP8 wkv rows: (codes [N, K] uint8, scales [N, K / 32] uint8)."""
        codes = np.empty((self.N, self.K), dtype=np.uint8)
        scales = np.empty((self.N, self.K // 32), dtype=np.uint8)

        def fill(lo):
            hi = min(self.N, lo + chunk_rows)
            codes[lo:hi], scales[lo:hi] = self.wkv8_rows(lo, hi, inst)

        n = threads or min(16, os.cpu_count() or 1)
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as pool:
            list(pool.map(fill, range(0, self.N, chunk_rows)))
        return codes, scales

    def wkv_f32(self, inst: int = 0, chunk_rows: int = 512, threads: int = 0) -> np.ndarray:
        """All of wkv as fp32 values; chunks of rows are generated on a thread pool (numpy
        releases the GIL inside its array operations)."""
        out = np.empty((self.N, self.K), dtype=np.float32)

        def fill(lo):
            hi = min(self.N, lo + chunk_rows)
            out[lo:hi] = bf16_bits_to_f32(self.wkv_rows(lo, hi, inst))

        n = threads or min(16, os.cpu_count() or 1)
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as pool:
            list(pool.map(fill, range(0, self.N, chunk_rows)))
        return out

    def outlier_tokens(self) -> np.ndarray:
        """bool [M]: tokens whose streams are drawn with the outlier std."""
        if self.outlier_frac <= 0:
            return np.zeros(self.M, dtype=bool)
        thr = int(round(self.outlier_frac * (1 << 24)))
        d = draw(self.key(S_OUTLIER), np.arange(self.M, dtype=np.int64))
        return (d >> _U64(40)).astype(np.int64) < thr

    def outlier_threshold(self) -> int:
        return int(round(self.outlier_frac * (1 << 24))) if self.outlier_frac > 0 else 0

    def x_tokens(self, tokens: np.ndarray) -> np.ndarray:
        """bf16 bit patterns of x for the given flat token indices, shape [len, hc, dim]."""
        tokens = np.asarray(tokens, dtype=np.int64)
        per = self.hc * self.dim
        out = np.empty((len(tokens), per), dtype=np.uint16)
        outl = self.outlier_tokens()
        key = self.key(S_X)
        for i, t in enumerate(tokens):
            std = self.x_std * (self.outlier_scale if outl[t] else 1.0)
            out[i] = normal_bf16(key, int(t) * per, per, 0.0, std)
        return out.reshape(len(tokens), self.hc, self.dim)

    def qk(self, inst: int = 0):
        """q_weight, k_weight as fp32 [hc, dim] (bf16-representable values)."""
        n = self.hc * self.dim
        if self.qk_std == 0.0:
            one = np.ones((self.hc, self.dim), dtype=np.float32)
            return one, one.copy()
        q = bf16_bits_to_f32(normal_bf16(self.key(S_QW, inst), 0, n, 1.0, self.qk_std))
        k = bf16_bits_to_f32(normal_bf16(self.key(S_KW, inst), 0, n, 1.0, self.qk_std))
        return q.reshape(self.hc, self.dim).copy(), k.reshape(self.hc, self.dim).copy()

    def token_mask(self) -> np.ndarray:
        """uint8 [B, T]: 1 where the token takes part (gate open)."""
        m = np.ones(self.M, dtype=np.uint8)
        for p in self.masked_positions:
            m[p] = 0
        if self.mask_false_frac > 0:
            thr = int(round(self.mask_false_frac * (1 << 24)))
            d = draw(self.key(S_MASK), np.arange(self.M, dtype=np.int64))
            m[(d >> _U64(40)).astype(np.int64) < thr] = 0
        return m.reshape(self.B, self.T)

    def hash_ids(self, inst: int = 0) -> np.ndarray:
        """int64 [B, T, n_cols] global row ids; column j lies in [offset_j, offset_j + p_j)."""
        M, C = self.M, self.n_cols
        p = np.asarray(self.primes, dtype=np.int64)
        off = self.offsets
        key = self.key(S_HASH, inst)
        if self.hash_dist == "uniform":
            d = draw(key, np.arange(M * C, dtype=np.int64)).reshape(M, C)
            hi32 = (d >> _U64(32)).astype(np.uint64)
            local = ((hi32 * p[None, :].astype(np.uint64)) >> _U64(32)).astype(np.int64)
        elif self.hash_dist == "zipf":
            local = np.empty((M, C), dtype=np.int64)
            pk = self.key(S_PERM, inst)
            for j in range(C):
                ranks = zipf_ranks(key, j * M, M, int(p[j]), self.zipf_s)
                da, dc = draw(pk, np.array([2 * j, 2 * j + 1], dtype=np.int64))
                a = 1 + int(da) % (int(p[j]) - 1)
                c = int(dc) % int(p[j])
                local[:, j] = ((ranks - 1) * a + c) % int(p[j])
        else:
            raise ValueError(self.hash_dist)
        return (local + off[None, :]).reshape(self.B, self.T, C)


def zipf_ranks(key: int, i0: int, n: int, N: int, s: float, max_tries: int = 32) -> np.ndarray:
    """n Zipf(s) ranks on {1..N} by rejection-inversion; sample i uses draws (i0+i)*max_tries+t."""
    om = 1.0 - s

    def H(x):
        lx = np.log(x)
        return np.expm1(om * lx) / om

    def Hinv(y):
        return np.exp(np.log1p(om * y) / om)

    def h(x):
        return np.exp(-s * np.log(x))

    hx1 = H(1.5) - 1.0
    hn = H(N + 0.5)
    sthr = 2.0 - Hinv(H(2.5) - h(2.0))
    out = np.zeros(n, dtype=np.int64)
    todo = np.arange(n, dtype=np.int64)
    for t in range(max_tries):
        if todo.size == 0:
            break
        d = draw(key, (i0 + todo) * max_tries + t)
        u01 = (d >> _U64(11)).astype(np.float64) * (2.0 ** -53)
        u = hn + u01 * (hx1 - hn)
        x = Hinv(u)
        k = np.clip(np.floor(x + 0.5), 1, N)
        ok = (k - x <= sthr) | (u >= H(k + 0.5) - h(k))
        if t == max_tries - 1:
            ok[:] = True
        out[todo[ok]] = k[ok].astype(np.int64)
        todo = todo[~ok]
    return out


def hash_inputs(seed: int, B: int, L: int, n_layers: int = 2, max_ngram: int = 4, n_heads: int = 8,
                vocab: int = 129_280, compressed_vocab: int = 99_092, primes=None,
                span_frac: float = 0.0, span_len: int = 16) -> dict:
    """Seeded inputs of the hash step at the model's sizes (config.json: vocab 129,280 raw ids,
    99,092 compressed; 2 layers, 4-grams, 8 heads).  The real token map and multipliers are not
    available: token_map is a seeded surjection onto the compressed range (every compressed id
    hit, the rest uniform), multipliers are seeded odd 64-bit values (int64 bit patterns), the
    primes are the model's (module y takes the y-th 24 primes above 16,000,000) unless given,
    offsets are the per-module cumulative range starts.  Input ids are uniform; a fraction
    span_frac of positions starts a dead span (an image) of span_len tokens (token_mask 0)."""
    key = lambda s: stream_key(seed, s)
    n_cols = (max_ngram - 1) * n_heads
    d = draw(key(S_TOKMAP), np.arange(vocab, dtype=np.int64))
    token_map = ((d >> _U64(32)) * _U64(compressed_vocab) >> _U64(32)).astype(np.int64)
    token_map[np.arange(min(vocab, compressed_vocab))] = np.arange(min(vocab, compressed_vocab))
    perm = (draw(key(S_TOKMAP + 64), np.arange(vocab, dtype=np.int64)) >> _U64(11)).argsort(kind="stable")
    token_map = token_map[perm].astype(np.uint32)
    mult = (draw(key(S_MULT), np.arange(n_layers * max_ngram, dtype=np.int64)) | _U64(1))
    mult = mult.view(np.int64).reshape(n_layers, max_ngram)
    if primes is None:
        primes = [model_primes(y, n_cols) for y in range(n_layers)]
    primes = np.asarray(primes, dtype=np.int64).reshape(n_layers, max_ngram - 1, n_heads)
    flat = primes.reshape(n_layers, n_cols)
    offsets = np.concatenate([np.zeros((n_layers, 1), np.int64), np.cumsum(flat, axis=1)[:, :-1]],
                             axis=1)
    ids = ((draw(key(S_IDS), np.arange(B * L, dtype=np.int64)) >> _U64(32)) * _U64(vocab)
           >> _U64(32)).astype(np.int64).reshape(B, L)
    mask = np.ones((B, L), dtype=np.uint8)
    if span_frac > 0:
        start = (draw(key(S_SPAN), np.arange(B * L, dtype=np.int64)) >> _U64(40)).astype(np.int64)
        starts = np.argwhere(start.reshape(B, L) < int(round(span_frac * (1 << 24))))
        for b, t in starts:
            mask[b, t:t + span_len] = 0
    return {"token_map": token_map, "multipliers": mult, "primes": primes, "offsets": offsets,
            "input_ids": ids, "token_mask": mask, "pad_id": 2, "n_layers": n_layers,
            "max_ngram": max_ngram, "n_heads": n_heads, "vocab": vocab}


_SEED0 = 0x454E4752


def workloads() -> dict:
    """Named workloads; shapes and distributions follow the benchmark configurations."""
    tiny = Workload("tiny", B=1, T=16, hc=4, dim=256, n_cols=6, head_dim=64, scale_block=32,
                    primes=[1009, 1013, 1019, 1021, 1031, 1033], seed=_SEED0 + 0,
                    masked_positions=(3, 9))
    decode = Workload("decode_b64", B=64, T=1, hc=4, dim=5120, n_cols=24, head_dim=256,
                      scale_block=128, primes=primes_from(700_001, 24), seed=_SEED0 + 1,
                      qk_std=0.05)
    prefill = Workload("prefill_t8192", B=1, T=8192, hc=4, dim=5120, n_cols=24, head_dim=256,
                       scale_block=128, primes=primes_from(4_166_671, 24), seed=_SEED0 + 2,
                       qk_std=0.05, hash_dist="zipf", mask_false_frac=0.10)
    full = Workload("fulltable_b4_t4096", B=4, T=4096, hc=4, dim=5120, n_cols=24, head_dim=256,
                    scale_block=128, primes=model_primes(1), seed=_SEED0 + 3, qk_std=0.05,
                    hash_dist="zipf", mask_false_frac=0.20, outlier_frac=0.01)
    two_p = Workload("two_instance_t32768", B=1, T=32768, hc=4, dim=5120, n_cols=24,
                     head_dim=256, scale_block=128, primes=model_primes(1), seed=_SEED0 + 4,
                     qk_std=0.05, hash_dist="zipf", n_instances=2)
    two_d = dataclasses.replace(two_p, name="two_instance_decode_b256", B=256, T=1)
    # the decode workload over a table in the pages' MXFP8 format (E8M0 scale per 32 features)
    decode_mx = dataclasses.replace(decode, name="decode_b64_mxfp8", scale_block=32,
                                    scale_format="e8m0")
    # ... and with the projection stored in FP8 as well (MXFP8 along its input features)
    decode_fp8 = dataclasses.replace(decode_mx, name="decode_b64_fp8", wkv_format="mxfp8")
    # FP8 weights with the benchmark tables' fp32 scales (the weights are dequantised to bf16)
    decode_w8 = dataclasses.replace(decode, name="decode_b64_w8", wkv_format="mxfp8")
    # the decode layout at 128 tokens (two 64-token blocks per pass over the weights)
    decode_b128 = dataclasses.replace(decode, name="decode_b128", B=128, seed=_SEED0 + 7)
    prefill_fp8 = dataclasses.replace(prefill, name="prefill_t8192_fp8", scale_block=32,
                                      scale_format="e8m0", wkv_format="mxfp8")
    return {w.name: w for w in (tiny, decode, prefill, full, two_p, two_d, decode_mx, decode_fp8,
                                prefill_fp8, decode_w8, decode_b128)}


def get(name: str) -> Workload:
    return workloads()[name]


def small_variant(base: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (test sizes)."""
    return dataclasses.replace(base, **kw)


# ----------------------------------------------------------------------------------------
# device-side fill (HIP), same element definitions as above
# ----------------------------------------------------------------------------------------
_HERE = os.path.dirname(os.path.abspath(__file__))
FILL_LIB_PATH = os.path.join(_HERE, "libsynth_fill.so")


class DeviceFill:
    """ctypes binding of libsynth_fill.so (device pointers and a HIP stream handle)."""

    def __init__(self, path: str = FILL_LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp, i64, i32, u64, f64, u32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_uint64, ctypes.c_double, ctypes.c_uint32)
        lib.synth_fill_codes.argtypes = [vp, i64, i64, i32, u64, vp]
        lib.synth_fill_scales.argtypes = [vp, i64, i64, i32, u64, f64, f64, vp]
        lib.synth_fill_normal_bf16.argtypes = [vp, i64, i64, u64, f64, f64, vp]
        lib.synth_fill_x.argtypes = [vp, i64, i64, i64, u64, u64, u32, f64, f64, vp]
        lib.synth_fill_e8m0.argtypes = [vp, i64, i64, i32, u64, u32, u32, vp]
        for f in (lib.synth_fill_codes, lib.synth_fill_scales, lib.synth_fill_normal_bf16,
                  lib.synth_fill_x, lib.synth_fill_e8m0):
            f.restype = ctypes.c_int
        self.lib = lib

    @staticmethod
    def _chk(rc: int, what: str):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def codes(self, ptr: int, row0: int, nrows: int, head_dim: int, key: int, stream: int):
        self._chk(self.lib.synth_fill_codes(ptr, row0, nrows, head_dim, key, stream), "fill codes")

    def scales(self, ptr, row0, nrows, n_blocks, key, lo, hi, stream):
        self._chk(self.lib.synth_fill_scales(ptr, row0, nrows, n_blocks, key, lo, hi, stream),
                  "fill scales")

    def e8m0(self, ptr, row0, nrows, n_blocks, key, lo, hi, stream):
        self._chk(self.lib.synth_fill_e8m0(ptr, row0, nrows, n_blocks, key, lo, hi, stream),
                  "fill e8m0")

    def normal_bf16(self, ptr, i0, n, key, mean, std, stream):
        self._chk(self.lib.synth_fill_normal_bf16(ptr, i0, n, key, mean, std, stream),
                  "fill normal")

    def x(self, ptr, tok0, ntok, per_tok, key_x, key_outlier, thr, std, outlier_std, stream):
        self._chk(self.lib.synth_fill_x(ptr, tok0, ntok, per_tok, key_x, key_outlier, thr, std,
                                        outlier_std, stream), "fill x")


def device_inputs(w: Workload, inst: int = 0, device: str = "cuda", with_table: bool = True) -> dict:
    """Allocate and fill the inputs of one Engram call on the device (torch tensors).

    Large tensors (table, scales, wkv, x) are written by the device fill from the same
    definitions as the host generator; hash ids and the token mask are drawn on the host and
    copied.  Returns x, hash_ids, token_mask, table, scales, wkv, q_weight, k_weight."""
    import torch

    fill = DeviceFill()
    dev = torch.device(device)
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = {}
    x = torch.empty((w.B, w.T, w.hc, w.dim), dtype=torch.bfloat16, device=dev)
    fill.x(x.data_ptr(), 0, w.M, w.hc * w.dim, w.key(S_X), w.key(S_OUTLIER),
           w.outlier_threshold(), w.x_std, w.x_std * w.outlier_scale, stream)
    out["x"] = x
    out["hash_ids"] = torch.from_numpy(w.hash_ids(inst)).to(dev)
    out["token_mask"] = torch.from_numpy(w.token_mask()).to(dev)
    if with_table:
        table = torch.empty((w.n_rows, w.head_dim), dtype=torch.uint8, device=dev)
        fill.codes(table.data_ptr(), 0, w.n_rows, w.head_dim, w.key(S_CODES, inst), stream)
        if w.scale_format == "e8m0":
            scales = torch.empty((w.n_rows, w.n_blocks), dtype=torch.uint8, device=dev)
            fill.e8m0(scales.data_ptr(), 0, w.n_rows, w.n_blocks, w.key(S_SCALES, inst),
                      w.e8m0_lo, w.e8m0_hi, stream)
        else:
            scales = torch.empty((w.n_rows, w.n_blocks), dtype=torch.float32, device=dev)
            fill.scales(scales.data_ptr(), 0, w.n_rows, w.n_blocks, w.key(S_SCALES, inst),
                        w.scale_lo, w.scale_hi, stream)
        out["table"], out["scales"] = table, scales
    if w.wkv_format == "mxfp8":
        # one buffer: codes [N, K], then scales [N, K / 32]
        wkv = torch.empty(w.N * w.K + w.N * (w.K // 32), dtype=torch.uint8, device=dev)
        fill.codes(wkv.data_ptr(), 0, w.N, w.K, w.key(S_WKV8, inst), stream)
        fill.e8m0(wkv.data_ptr() + w.N * w.K, 0, w.N, w.K // 32, w.key(S_WKV8S, inst),
                  w.wkv_e8m0_lo, w.wkv_e8m0_hi, stream)
    else:
        wkv = torch.empty((w.N, w.K), dtype=torch.bfloat16, device=dev)
        fill.normal_bf16(wkv.data_ptr(), 0, w.N * w.K, w.key(S_WKV, inst), 0.0, w.wkv_std, stream)
    out["wkv"] = wkv
    q, k = w.qk(inst)
    out["q_weight"] = torch.from_numpy(q).to(dev)
    out["k_weight"] = torch.from_numpy(k).to(dev)
    return out


def host_fetch(w: Workload, inst: int = 0):
    """Row provider for the oracle: regenerates table rows and their scales on the host."""

    def fetch(rows):
        rows = np.asarray(rows, dtype=np.int64)
        return w.codes_rows(rows, inst), w.scales_rows(rows, inst)

    return fetch
