"""Pins of the CPU oracle (oracle/engram_oracle.cc) against things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form, a number printed on the
pages, or a brute-force evaluation on tiny inputs written in a different way (scalar loops,
exact rational arithmetic, struct-based rounding).
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_layout.json")))


def g(name):
    return GOLDEN[name]["value"]


# ---------------------------------------------------------------- number formats


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_special_values():
    v = oracle.e4m3fn_value(np.array([0x7E, 0x7F, 0xFF, 0x01, 0x08, 0x00, 0x80, 0xFE], np.uint8))
    assert v[0] == g("fp8_e4m3_max") and v[7] == -448.0
    assert math.isnan(v[1]) and math.isnan(v[2])
    assert v[3] == 2.0 ** -9 and v[4] == 2.0 ** -6
    assert v[5] == 0.0 and not np.signbit(v[5]) and v[6] == 0.0 and np.signbit(v[6])
    assert int(np.isnan(oracle.e4m3fn_value(np.arange(256, dtype=np.uint8))).sum()) == 2


def _bf16_edge_fp32():
    rng = np.random.default_rng(7)
    bits = [0x3F808000, 0x3F818000, 0x3F80C000, 0x3F807FFF, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF,
            0x00000001, 0x00008000, 0x00018000, 0x80008000, 0x807FFFFF, 0x7F800000, 0xFF800000,
            0x00000000, 0x80000000, 0x7FC00000, 0xFFC00001, 0x7F800001]
    r = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([np.array(bits, np.uint32), r]).view(np.float32)


def test_bf16_rounding_matches_torch():
    """Bits agree for every non-NaN input; NaN gives a NaN (torch's vectorised CPU path writes
    0xFFFF, its scalar path 0x7FC0; the oracle uses 0x7FC0)."""
    f = _bf16_edge_fp32()
    with np.errstate(invalid="ignore"):
        ours = oracle.bf16_bits_from_fp32(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)
    assert np.all(np.isnan(oracle.bf16_value(ref[nan])))


def test_round_fp32_is_ieee_single():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1000) * 10.0 ** rng.integers(-40, 38, 1000)
    ours = oracle.round_fp32(x)
    ref = np.array([struct.unpack("f", struct.pack("f", float(v)))[0] for v in x])
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- S1 + S2 gather / dequant


def _torch_dequant_rows(codes_rows, scale_rows, scale_block):
    """fp8 rows through torch's own conversions: value as float, times fp32 scale, to bf16."""
    v = torch.from_numpy(codes_rows).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(scale_rows).float()
    blk = torch.arange(codes_rows.shape[-1]) // scale_block
    return (v * s[..., blk]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_dequant_matches_torch_conversions_all_codes():
    rng = np.random.default_rng(11)
    hd, sb, n = 64, 32, 40
    table = np.tile(np.arange(256, dtype=np.uint8), n * hd // 256 + 1)[: n * hd].reshape(n, hd)
    rng.shuffle(table.reshape(-1))
    scales = rng.uniform(0.01, 0.1, (n, hd // sb)).astype(np.float32)
    scales[0] = [1e-40, 2.0 ** -126]          # subnormal and smallest normal scale
    scales[1] = [3e38, -1.5]                  # overflow to inf, negative scale
    scales[2] = [np.float32(2.0 ** -149), 1.0]
    ids = np.arange(n, dtype=np.int64).reshape(-1, 1)
    ours = oracle.gather_dequant(ids, oracle.array_fetch(table, scales), n, hd, sb)
    ref = _torch_dequant_rows(table, scales, sb)
    ours = ours.reshape(n, hd)
    nan = np.isnan(oracle.bf16_value(ref))
    assert np.array_equal(nan, ours == 0x7FC0)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e8m0_decode_matches_torch_float8_e8m0fnu():
    # the library's E8M0 type (OCP MX scale: 2^(e - 127), 0xFF NaN) on all 256 bytes
    e = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(e).view(torch.float8_e8m0fnu).float().double().numpy()
    ours = oracle.e8m0_value(e)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    # closed forms: 2^0 at the bias, the extremes
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_dequant_e8m0_matches_torch_conversions_all_codes_and_exponents():
    # every e4m3 code against every E8M0 exponent: fp8 value x 2^(e - 127) rounded to fp32 and
    # then to bf16, as torch computes it (subnormal fp32 products, overflow to inf, NaN scales)
    hd, sb = 256, 32
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))           # row e: all codes
    exps = np.repeat(np.arange(256, dtype=np.uint8)[:, None], hd // sb, axis=1)
    ids = np.arange(256, dtype=np.int64).reshape(-1, 1)
    ours = oracle.gather_dequant(ids, oracle.array_fetch(codes, exps), 256, hd, sb,
                                 scale_format="e8m0").reshape(256, hd)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    sc = torch.from_numpy(exps).view(torch.float8_e8m0fnu).float()
    ref = (v * sc[:, torch.arange(hd) // sb]).to(torch.bfloat16).view(torch.int16).numpy()
    ref = ref.view(np.uint16)
    nan = np.isnan(oracle.bf16_value(ref))
    assert np.array_equal(nan, ours == 0x7FC0)
    assert np.array_equal(ours[~nan], ref[~nan])
    # with a power-of-two scale the product is exact wherever it stays a normal bf16 number:
    # code 0x38 (1.0) at exponent e reproduces 2^(e - 127)
    assert all(oracle.bf16_value(ours[e, 0x38]) == 2.0 ** (e - 127) for e in range(1, 255))


def test_wkv_mxfp8_matches_torch_conversions_all_codes_and_exponents():
    # FP8 projection weights: row e holds every e4m3 code (in a 256-wide row, 8 scale blocks)
    # with exponent e in every block; torch's float8 types give the reference values
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    exps = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 256 // 32, axis=1)
    ours = oracle.wkv_mxfp8_bits(codes, exps)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    sc = torch.from_numpy(exps).view(torch.float8_e8m0fnu).float()
    ref = (v * sc[:, torch.arange(256) // 32]).to(torch.bfloat16).view(torch.int16).numpy()
    ref = ref.view(np.uint16)
    nan = np.isnan(oracle.bf16_value(ref))
    assert np.array_equal(nan, ours == 0x7FC0)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_wkv_mxfp8_scale_of_each_input_block():
    # all weights 1.0 (code 0x38) at exponent 127, except one scale byte: only the 32 inputs
    # of that (row, block) change, a transposed or shifted scale index would move them
    N, K = 5, 256
    codes = np.full((N, K), 0x38, dtype=np.uint8)
    exps = np.full((N, K // 32), 127, dtype=np.uint8)
    exps[2, 5] = 130
    exps[4, 0] = 125
    w = oracle.bf16_value(oracle.wkv_mxfp8_bits(codes, exps))
    want = np.ones((N, K))
    want[2, 160:192] = 8.0
    want[4, 0:32] = 0.25
    assert np.array_equal(w, want)
    # and a projection through these weights is the bf16 projection of the same values
    emb = synth.normal_bf16(5, 0, 3 * K, 0.0, 1.0).reshape(3, K)
    got = oracle.kv_proj(emb, oracle.wkv_mxfp8_bits(codes, exps))
    ref = F.linear(torch.from_numpy(oracle.bf16_value(emb)), torch.from_numpy(want))
    assert np.array_equal(got, oracle.bf16_bits_from_fp32(ref.numpy()))


def test_gather_brute_force_flatten_and_scale_blocks():
    """Scalar loops with struct rounding: feature c of column j at j*hd + c, scale c // sb."""
    rng = np.random.default_rng(5)
    n_rows, hd, sb, C, M = 13, 8, 4, 3, 5
    table = rng.integers(0, 256, (n_rows, hd), dtype=np.uint8)
    table[(table & 0x7F) == 0x7F] = 0x11
    scales = rng.uniform(0.5, 2.0, (n_rows, hd // sb)).astype(np.float32)
    ids = rng.integers(0, n_rows, (M, C)).astype(np.int64)
    ids[1, 2] = -3
    ids[4, 0] = n_rows
    ours = oracle.gather_dequant(ids, oracle.array_fetch(table, scales), n_rows, hd, sb)

    def fp8(code):  # sign * 2^(E-7) * (1 + M/8), or M * 2^-9 for E == 0
        sgn = -1.0 if code & 0x80 else 1.0
        E, Mn = (code >> 3) & 0xF, code & 7
        return sgn * (math.ldexp(Mn, -9) if E == 0 else math.ldexp(1.0 + Mn / 8.0, E - 7))

    def to_f32(v):
        return struct.unpack("f", struct.pack("f", v))[0]

    def to_bf16_bits(v):
        u = struct.unpack("I", struct.pack("f", v))[0]
        top, low = u >> 16, u & 0xFFFF
        if low > 0x8000 or (low == 0x8000 and top & 1):
            top += 1
        return top & 0xFFFF

    for m in range(M):
        for j in range(C):
            r = int(ids[m, j])
            for c in range(hd):
                if 0 <= r < n_rows:
                    want = to_bf16_bits(to_f32(fp8(int(table[r, c])) * float(scales[r, c // sb])))
                else:
                    want = 0
                assert ours[m, j * hd + c] == want, (m, j, c)


def test_gather_matches_torch_embedding_lookup():
    rng = np.random.default_rng(9)
    n_rows, hd, sb = 50, 64, 32
    table = rng.integers(0, 256, (n_rows, hd), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.1, (n_rows, hd // sb)).astype(np.float32)
    ids = rng.integers(0, n_rows, (7, 6)).astype(np.int64)
    ours = oracle.gather_dequant(ids, oracle.array_fetch(table, scales), n_rows, hd, sb)
    rows_c = F.embedding(torch.from_numpy(ids), torch.from_numpy(table)).numpy()
    rows_s = F.embedding(torch.from_numpy(ids), torch.from_numpy(scales)).numpy()
    ref = _torch_dequant_rows(rows_c, rows_s, sb).reshape(7, -1)
    ok = ~np.isnan(oracle.bf16_value(ref))
    assert np.array_equal(ours[ok], ref[ok])


# ---------------------------------------------------------------- S3 projection


def test_kv_matches_torch_linear_bf16():
    rng = np.random.default_rng(2)
    M, K, N = 9, 384, 200
    emb = oracle.bf16_bits_from_fp32(rng.standard_normal((M, K)) * 0.1)
    wkv = oracle.bf16_bits_from_fp32(rng.standard_normal((N, K)) * 0.02)
    ours = oracle.kv_proj(emb, wkv)
    t_emb = torch.from_numpy(emb.view(np.int16)).view(torch.bfloat16)
    t_w = torch.from_numpy(wkv.view(np.int16)).view(torch.bfloat16)
    ref = F.linear(t_emb.double(), t_w.double()).float().to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # torch's bf16 Linear (fp32 accumulate) agrees to within one bf16 ulp
    lin = F.linear(t_emb, t_w).view(torch.int16).numpy().view(np.uint16).astype(np.int32)
    assert np.abs(lin - ours.astype(np.int32)).max() <= 1


def test_kv_exact_rational_brute_force_non_square():
    rng = np.random.default_rng(4)
    M, K, N = 3, 8, 5
    emb = oracle.bf16_bits_from_fp32(rng.standard_normal((M, K)))
    wkv = oracle.bf16_bits_from_fp32(rng.standard_normal((N, K)))
    ours = oracle.kv_proj(emb, wkv)
    ev, wv = oracle.bf16_value(emb), oracle.bf16_value(wkv)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(ev[m, k])) * Fraction(float(wv[n, k])) for k in range(K))
            f32 = struct.unpack("f", struct.pack("f", float(exact)))[0]
            assert ours[m, n] == oracle.bf16_bits_from_fp32(np.array([f32]))[0], (m, n)


# ---------------------------------------------------------------- S4 + S5 gate


def _bits(x):
    return oracle.bf16_bits_from_fp32(np.asarray(x, np.float64))


def _case(M=3, hc=4, dim=256, seed=0):
    rng = np.random.default_rng(seed)
    x = _bits(rng.standard_normal((M, hc, dim)))
    return x, rng


def _kv_from(key_vals, value_vals):
    M, hc, dim = key_vals.shape
    kv = np.concatenate([key_vals.reshape(M, hc * dim), value_vals.reshape(M, dim)], axis=1)
    return _bits(kv)


def _sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


ONES = np.ones((4, 256), np.float32)


def test_gate_zero_key_is_sigmoid_of_sqrt_clamp():
    """key = 0: the sum is +0, eps keeps rstd finite, so dot = +0 and the clamp gives
    sigmoid(+sqrt(1e-6)); without eps the zero key would give 0 * inf = NaN."""
    x, _ = _case()
    kv = _kv_from(np.zeros((3, 4, 256)), np.ones((3, 256)))
    r = oracle.gate(x, kv, ONES, ONES, None, 1e-20, 1e-6)
    assert np.allclose(r["gate"], _sigmoid(math.sqrt(1e-6)), rtol=0, atol=1e-15)
    z = np.zeros((3, 4, 256), np.uint16)
    r0 = oracle.gate(z, kv, ONES, ONES, None, 1e-20, 1e-6)
    assert np.allclose(r0["gate"], 0.5002499999791667, rtol=0, atol=1e-15)


@pytest.mark.parametrize("dim", [256, 5120])
def test_gate_key_equal_stream_closed_form(dim):
    """key = h, w = 1: dot = sum(h^2) / mean(h^2) / sqrt(dim) = sqrt(dim)."""
    x, _ = _case(dim=dim)
    key = oracle.bf16_value(x)
    kv = _kv_from(key, np.zeros((3, dim)))
    one = np.ones((4, dim), np.float32)
    r = oracle.gate(x, kv, one, one, None, 1e-20, 1e-6)
    assert np.allclose(r["dot"], math.sqrt(dim), rtol=1e-12)
    assert np.allclose(r["gate"], _sigmoid(dim ** 0.25), rtol=0, atol=1e-12)
    # negated key: sigmoid symmetry
    kvn = _kv_from(-key, np.zeros((3, dim)))
    rn = oracle.gate(x, kvn, one, one, None, 1e-20, 1e-6)
    assert np.allclose(rn["gate"], 1.0 - _sigmoid(dim ** 0.25), rtol=0, atol=1e-12)


def test_gate_page_values_at_model_width():
    assert abs(_sigmoid(5120 ** 0.25) - 0.99978805) < 5e-9
    assert abs(_sigmoid(256 ** 0.25) - 0.98201379) < 5e-9


def test_gate_weight_is_product_of_q_and_k():
    """q = 2, k = 3 and key = h: dot = 6 sqrt(dim) (a sum q + k would give 5 sqrt(dim))."""
    x, _ = _case()
    kv = _kv_from(oracle.bf16_value(x), np.zeros((3, 256)))
    q = np.full((4, 256), 2.0, np.float32)
    k = np.full((4, 256), 3.0, np.float32)
    r = oracle.gate(x, kv, q, k, None, 1e-20, 1e-6)
    assert np.allclose(r["dot"], 6 * 16.0, rtol=1e-12)
    assert np.allclose(r["gate"], _sigmoid(math.sqrt(96.0)), rtol=0, atol=1e-12)


def test_gate_is_cosine_similarity_times_sqrt_dim():
    """With w = 1 and eps negligible, dot = cos(h, key) * sqrt(dim) (torch cosine_similarity)."""
    x, rng = _case(M=5, seed=3)
    key = rng.standard_normal((5, 4, 256)) * 0.3 + 0.5 * oracle.bf16_value(x)
    kv = _kv_from(key, np.zeros((5, 256)))
    r = oracle.gate(x, kv, ONES, ONES, None, 1e-20, 1e-6)
    h = torch.from_numpy(oracle.bf16_value(x))
    kk = torch.from_numpy(oracle.bf16_value(kv[:, :1024]).reshape(5, 4, 256))
    cos = F.cosine_similarity(h, kk, dim=-1, eps=0.0).numpy()
    assert np.allclose(r["dot"], cos * 16.0, rtol=1e-10, atol=1e-12)
    ref = torch.sigmoid(torch.sign(torch.from_numpy(cos * 16)) *
                        torch.sqrt(torch.from_numpy(np.maximum(np.abs(cos * 16), 1e-6)))).numpy()
    assert np.allclose(r["gate"], ref, rtol=0, atol=1e-12)


def test_gate_normalises_each_stream_alone_and_is_scale_invariant():
    x, rng = _case(M=2, seed=8)
    base = oracle.bf16_value(x)[:, 0]
    streams = np.stack([base * 2.0 ** s for s in range(4)], axis=1)   # exact scalings
    key = rng.standard_normal((2, 256))
    kv = _kv_from(np.stack([key * 2.0 ** (-s) for s in range(4)], axis=1), np.zeros((2, 256)))
    r = oracle.gate(_bits(streams), kv, ONES, ONES, None, 1e-20, 1e-6)
    assert np.allclose(r["gate"], r["gate"][:, :1], rtol=0, atol=1e-13)


def test_mask_closes_gate_and_passes_tokens_through():
    x, rng = _case(M=4, seed=2)
    x[1, 2, 5] = 0x8000                                   # a -0.0 survives untouched
    kv = _kv_from(rng.standard_normal((4, 4, 256)), rng.standard_normal((4, 256)))
    mask = np.array([1, 0, 1, 0], np.uint8)
    r = oracle.gate_apply(x, kv, ONES, ONES, mask, 1e-20, 1e-6)
    assert np.all(r["gate"][[1, 3]] == 0.0) and np.all(r["gate"][[0, 2]] > 0.0)
    assert np.array_equal(r["out_bits"][[1, 3]], x[[1, 3]])


def test_residual_adds_shared_value_times_gate():
    x, rng = _case(M=3, seed=6)
    kv = _kv_from(rng.standard_normal((3, 4, 256)), rng.standard_normal((3, 256)))
    r = oracle.gate_apply(x, kv, ONES, ONES, None, 1e-20, 1e-6)
    value = oracle.bf16_value(kv[:, 1024:])
    diff = r["out_f"] - oracle.bf16_value(x)
    for s in range(4):
        assert np.allclose(diff[:, s], r["gate"][:, s:s + 1] * value, rtol=1e-14, atol=1e-15)
    assert np.array_equal(r["out_bits"], oracle.bf16_bits_from_fp32(oracle.round_fp32(r["out_f"])))


# ---------------------------------------------------------------- whole forward, brute force


def test_forward_brute_force_tiny_layout():
    """Scalar re-evaluation with exact sums on a tiny random layout (hc=4, dim=8, C=3, hd=8)."""
    rng = np.random.default_rng(21)
    hc, dim, C, hd, sb, n_rows, M = 4, 8, 3, 8, 4, 11, 3
    table = rng.integers(0, 256, (n_rows, hd), dtype=np.uint8)
    table[(table & 0x7F) == 0x7F] = 0x30
    scales = rng.uniform(0.01, 0.1, (n_rows, hd // sb)).astype(np.float32)
    ids = rng.integers(0, n_rows, (M, C)).astype(np.int64)
    wkv = _bits(rng.standard_normal(((hc + 1) * dim, C * hd)) * 0.5)
    x = _bits(rng.standard_normal((M, hc, dim)))
    q = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    k = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    mask = np.array([1, 0, 1], np.uint8)
    r = oracle.forward(x, ids, mask, oracle.array_fetch(table, scales), n_rows, hd, sb, wkv, q, k)

    f8 = oracle.e4m3fn_value(np.arange(256, dtype=np.uint8))  # pinned above against torch
    wv, xv = oracle.bf16_value(wkv), oracle.bf16_value(x)
    for m in range(M):
        emb = []
        for j in range(C):
            for c in range(hd):
                p = struct.unpack("f", struct.pack("f", f8[table[ids[m, j], c]] *
                                                   float(scales[ids[m, j], c // sb])))[0]
                emb.append(float(torch.tensor(p).to(torch.bfloat16).float()))
        kv = []
        for n in range((hc + 1) * dim):
            s = sum(Fraction(emb[f]) * Fraction(float(wv[n, f])) for f in range(C * hd))
            kv.append(float(torch.tensor(float(s)).float().to(torch.bfloat16).float()))
        assert np.array_equal(oracle.bf16_value(r["kv"][m]), np.array(kv))
        for s_ in range(hc):
            h = [float(v) for v in xv[m, s_]]
            key = kv[s_ * dim:(s_ + 1) * dim]
            w = [struct.unpack("f", struct.pack("f", float(q[s_, d]) * float(k[s_, d])))[0]
                 for d in range(dim)]
            A = math.fsum(v * v for v in h) / dim
            Kq = math.fsum(v * v for v in key) / dim
            D = math.fsum(h[d] * w[d] * key[d] for d in range(dim))
            dot = D / math.sqrt(A + 1e-20) / math.sqrt(Kq + 1e-20) / math.sqrt(dim)
            gt = _sigmoid(math.copysign(math.sqrt(max(abs(dot), 1e-6)), dot)) if mask[m] else 0.0
            assert abs(r["gate"][m, s_] - gt) < 1e-12
            for d in range(dim):
                want = h[d] + gt * kv[hc * dim + d] if mask[m] else h[d]
                assert abs(r["out_f"][m, s_, d] - want) < 1e-12


# ---------------------------------------------------------------- layout accounting


def test_param_counts_match_page_table():
    pc = oracle.param_counts(g("table_rows_second_module"), g("engram_head_dim"),
                             (g("engram_max_ngram_size") - 1) * g("engram_n_heads"), g("hc_mult"),
                             g("dim"))
    assert pc["table"] == g("table_entries")
    assert pc["wkv"] == g("projection_params")
    assert pc["gate"] == g("gate_params")
    assert pc["total"] == g("instance_total")


def test_prime_layout_sums_match_config():
    p0, p1 = synth.model_primes(0), synth.model_primes(1)
    assert p0[0] == g("first_prime") and len(p0) == len(p1) == 24
    assert sum(p0) == g("table_rows_first_module")
    assert sum(p1) == g("table_rows_second_module")
    assert p1[0] > p0[-1]


def test_bytes_per_token_and_totals():
    C = (g("engram_max_ngram_size") - 1) * g("engram_n_heads")
    assert C * g("engram_head_dim") == g("values_per_token_per_layer")
    assert (g("hc_mult") + 1) * g("dim") == g("projection_outputs")
    e8m0 = oracle.bytes_per_token(C, 256, 32, 1)
    f32_128 = oracle.bytes_per_token(C, 256, 128, 4)
    assert e8m0["codes"] == g("code_bytes_per_token_per_module")
    assert e8m0["scales"] == f32_128["scales"] == g("scale_bytes_per_token_per_module")
    assert 256 // 32 == g("scale_bytes_per_row_e8m0_32")
    rows = g("table_rows_first_module") + g("table_rows_second_module")
    assert round(rows * (256 + 8) / 2 ** 30, 1) == g("both_modules_gib")
    assert int(rows * 256 / 2 ** 30) == g("codes_both_layers_gib")


# ---------------------------------------------------------------------------- hash step


def _hash_case(rng, B, L, n_layers=2, max_ngram=4, n_heads=8, vocab=5000, cvocab=3000):
    token_map = rng.integers(0, cvocab, vocab).astype(np.int64)
    mult = (rng.integers(0, 2 ** 63 - 1, (n_layers, max_ngram), dtype=np.int64) * 2 + 1)  # odd, wraps
    primes = np.array(synth.primes_from(16_000_001, n_layers * (max_ngram - 1) * n_heads),
                      dtype=np.int64).reshape(n_layers, max_ngram - 1, n_heads)
    offsets = np.concatenate([np.zeros((n_layers, 1), np.int64),
                              np.cumsum(primes.reshape(n_layers, -1), axis=1)[:, :-1]], axis=1)
    ids = rng.integers(0, vocab, (B, L)).astype(np.int64)
    return ids, token_map, mult, primes, offsets


def test_hash_big_int_reproduces_page_demo():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_hash_demo.json")))
    mult = np.array([[int(m, 16) for m in g["multipliers"]]], dtype=object)      # 1 layer
    n = g["ngram"]
    primes = np.array([[g["primes"], g["primes"]]], dtype=object)                 # orders 2 and 3
    offsets = np.zeros((1, 2 * len(g["primes"])), dtype=object)
    ids = np.array([g["compressed_ids"]], dtype=object)
    token_map = np.arange(max(g["compressed_ids"]) + 1, dtype=object)            # already compressed
    history = np.zeros((1, len(g["compressed_ids"])), dtype=object)
    out = oracle.hash_ids(ids, token_map, mult, primes, offsets, g["pad_id"], history)
    assert mult.shape[1] == n
    assert [int(v) for v in out[0, -1, 0, len(g["primes"]):]] == g["rows_at_last_token"]


def _hash_brute_force_int64(ids, token_map, mult, primes, offsets, pad_id, mask=None, dead=-1):
    """Scalar restatement with explicit two's-complement wrap, one token at a time, in the shape
    of the page demo's loop (look back, multiply, XOR, modulo each head's prime)."""
    B, L = ids.shape
    n_layers, max_ngram = mult.shape
    n_heads = primes.shape[2]
    out = np.zeros((B, L, n_layers, (max_ngram - 1) * n_heads), dtype=np.int64)
    for b in range(B):
        comp = [int(token_map[i]) for i in ids[b]]
        if mask is not None:
            comp = [c if mask[b, t] else dead for t, c in enumerate(comp)]
        for t in range(L):
            toks, blocked = [], False
            for sh in range(max_ngram):
                src = comp[t - sh] if t - sh >= 0 else None
                blocked = blocked or src is None or src == dead
                toks.append(pad_id if blocked else src)
            for layer in range(n_layers):
                h = 0
                for i in range(max_ngram):
                    prod = (toks[i] * int(mult[layer, i])) % (1 << 64)
                    h ^= prod
                    if i >= 1:
                        sh = h - (1 << 64) if h >= (1 << 63) else h   # as a signed 64-bit value
                        for k in range(n_heads):
                            p = int(primes[layer, i - 1, k])
                            col = (i - 1) * n_heads + k
                            out[b, t, layer, col] = sh % p + int(offsets[layer, col])
    return out


def test_hash_int64_matches_scalar_brute_force_with_masks():
    rng = np.random.default_rng(21)
    ids, tm, mult, primes, offsets = _hash_case(rng, 2, 11)
    mask = np.ones(ids.shape, dtype=bool)
    mask[0, 4] = mask[1, 0] = mask[1, 7] = False
    hist = np.zeros((2, 11), dtype=np.int64)
    got = oracle.hash_ids(ids, tm, mult, primes, offsets, 2, hist, token_mask=mask)
    ref = _hash_brute_force_int64(ids, tm, mult, primes, offsets, 2, mask=mask)
    assert np.array_equal(got, ref)
    # every id lies in its column's prime range of the module's table
    lo = offsets[None, None]
    assert np.all(got >= lo) and np.all(got < lo + primes.reshape(2, -1)[None, None])


def test_hash_chunked_calls_equal_one_call_and_dead_blocks_lookback():
    rng = np.random.default_rng(22)
    ids, tm, mult, primes, offsets = _hash_case(rng, 3, 40)
    mask = rng.random(ids.shape) > 0.1
    h1 = np.zeros((3, 40), dtype=np.int64)
    whole = oracle.hash_ids(ids, tm, mult, primes, offsets, 2, h1, token_mask=mask)
    h2 = np.zeros((3, 40), dtype=np.int64)
    parts = [oracle.hash_ids(ids[:, a:b], tm, mult, primes, offsets, 2, h2, start_pos=a,
                             token_mask=mask[:, a:b]) for a, b in ((0, 17), (17, 18), (18, 40))]
    assert np.array_equal(np.concatenate(parts, axis=1), whole) and np.array_equal(h1, h2)
    # a dead token: right after it, the n-gram sees only the current token, as at a sequence
    # start; at the dead position itself every look-back reads pad
    b, t = np.argwhere(~mask[:, 1:-1])[0] + [0, 1]
    if mask[b, t + 1]:
        fresh = oracle.hash_ids(ids[b:b + 1, t + 1:t + 2], tm, mult, primes, offsets, 2,
                                np.zeros((1, 1), dtype=np.int64))
        assert np.array_equal(whole[b, t + 1], fresh[0, 0])
    pads = oracle.hash_ids(np.zeros((1, 1), dtype=np.int64), np.array([2]), mult, primes, offsets,
                           2, np.zeros((1, 1), dtype=np.int64))
    assert np.array_equal(whole[b, t], pads[0, 0])


def _hash_brute_force_unbounded(ids, token_map, mult, primes, offsets, pad_id):
    """The page demo's loop over Python integers (no wrap): per token, the look-backs blocked at
    the sequence start, products summed with XOR, each order's value modulo each head's prime."""
    B, L = ids.shape
    n_layers, max_ngram = mult.shape
    n_heads = primes.shape[2]
    out = np.zeros((B, L, n_layers, (max_ngram - 1) * n_heads), dtype=object)
    for b in range(B):
        comp = [int(token_map[i]) for i in ids[b]]
        for t in range(L):
            toks = [comp[t - sh] if t - sh >= 0 else pad_id for sh in range(max_ngram)]
            for sh in range(1, max_ngram):
                if t - sh < 0:
                    toks[sh:] = [pad_id] * (max_ngram - sh)
                    break
            for layer in range(n_layers):
                h = 0
                for i in range(max_ngram):
                    h ^= toks[i] * int(mult[layer, i])
                    if i >= 1:
                        for k in range(n_heads):
                            col = (i - 1) * n_heads + k
                            out[b, t, layer, col] = h % int(primes[layer, i - 1, k]) + int(offsets[layer, col])
    return out


def test_hash_wide_mode_matches_unbounded_brute_force():
    # 64-bit odd multipliers above 2^63 (as on the page): the 128-bit mode keeps every product
    rng = np.random.default_rng(31)
    ids, tm, _, primes, offsets = _hash_case(rng, 2, 9)
    mult = np.array([[int(v) | 1 | (1 << 63) for v in rng.integers(0, 2 ** 62, 4)] for _ in range(2)],
                    dtype=object)
    got = oracle.hash_ids(ids.astype(object), tm, mult, primes.astype(object),
                          offsets.astype(object), 2, np.zeros((2, 9), dtype=object))
    ref = _hash_brute_force_unbounded(ids, tm, mult, primes, offsets, 2)
    assert np.array_equal(got.astype(object), ref)
    # and the 64-bit mode on the same inputs is the unbounded value's two's-complement reduction
    wrap = oracle.hash_ids(ids, tm, np.array([[v - (1 << 64) for v in r] for r in mult],
                                             dtype=np.int64), primes, offsets, 2,
                           np.zeros((2, 9), np.int64))
    assert np.array_equal(wrap, _hash_brute_force_int64(ids, tm, np.array(
        [[v - (1 << 64) for v in r] for r in mult], dtype=np.int64), primes, offsets, 2))
    assert not np.array_equal(wrap, got.astype(np.int64))  # the two readings do differ


def _tiny_forward_inputs(seed=41, M=7):
    rng = np.random.default_rng(seed)
    hc, dim, C, hd, sb, n_rows = 4, 64, 6, 32, 16, 97
    table = rng.integers(0, 256, (n_rows, hd), dtype=np.uint8)
    table[(table & 0x7F) == 0x7F] = 0x21        # no NaN codes: results compare bit for bit
    scales = rng.uniform(0.01, 0.1, (n_rows, hd // sb)).astype(np.float32)
    ids = rng.integers(0, n_rows, (M, C)).astype(np.int64)
    ids[2, 3] = n_rows + 5                      # out of range: a zero row
    wkv = _bits(rng.standard_normal(((hc + 1) * dim, C * hd)) * 0.05)
    x = _bits(rng.standard_normal((M, hc, dim)))
    q = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    k = rng.uniform(0.5, 1.5, (hc, dim)).astype(np.float32)
    mask = np.ones(M, np.uint8)
    mask[4] = 0
    return dict(x=x, ids=ids, mask=mask, table=table, scales=scales, n_rows=n_rows, hd=hd, sb=sb,
                wkv=wkv, q=q, k=k)


def _run_forward(a, fetch):
    return oracle.forward(a["x"], a["ids"], a["mask"], fetch, a["n_rows"], a["hd"], a["sb"],
                          a["wkv"], a["q"], a["k"])


def test_forward_same_bits_for_any_thread_count(monkeypatch):
    a = _tiny_forward_inputs()
    monkeypatch.setenv("ORACLE_THREADS", "1")
    one = _run_forward(a, oracle.array_fetch(a["table"], a["scales"]))
    monkeypatch.setenv("ORACLE_THREADS", "5")
    many = _run_forward(a, oracle.array_fetch(a["table"], a["scales"]))
    for key in one:
        assert np.array_equal(one[key], many[key]), key


def test_held_rows_lookup_equals_whole_table():
    """A row provider that hands over only the rows the tokens name (ascending) gives the same
    results as the whole table; a provider that leaves one out is an error."""
    a = _tiny_forward_inputs(seed=43)
    dense = _run_forward(a, oracle.array_fetch(a["table"], a["scales"]))
    asked = []

    def fetch(rows):
        asked.append(np.asarray(rows).copy())
        return a["table"][rows], a["scales"][rows]

    held = _run_forward(a, fetch)
    for key in dense:
        assert np.array_equal(dense[key], held[key]), key
    rows = asked[0]
    assert np.all(np.diff(rows) > 0) and rows.max() < a["n_rows"]   # in range, ascending, unique

    def lossy(rows):  # one row short: the last id the tokens name is not held
        return a["table"][rows[:-1]], a["scales"][rows[:-1]]

    with pytest.raises(ValueError):
        oracle.gather_dequant(a["ids"], lossy, a["n_rows"], a["hd"], a["sb"])
    # a whole-table view shorter than n_rows: an in-range id past its end is not held
    short = oracle.array_fetch(a["table"][:50], a["scales"][:50])
    assert a["ids"].max() >= 50
    with pytest.raises(RuntimeError):
        oracle.gather_dequant(a["ids"], short, a["n_rows"], a["hd"], a["sb"])
    with pytest.raises(RuntimeError):
        _run_forward(a, short)


def test_kv_full_width_against_torch_double_linear():
    """K = 6144 (the model's 24 x 256 inputs): the oracle's in-order double sums, rounded to fp32
    and then bf16, against torch's double Linear rounded the same way."""
    rng = np.random.default_rng(12)
    M, K, N = 3, 6144, 96
    emb = oracle.bf16_bits_from_fp32(rng.standard_normal((M, K)) * 0.05)
    wkv = oracle.bf16_bits_from_fp32(rng.standard_normal((N, K)) * 0.02)
    ours, exact = oracle.kv_proj(emb, wkv, with_exact=True)
    t_emb = torch.from_numpy(emb.view(np.int16)).view(torch.bfloat16).double()
    t_w = torch.from_numpy(wkv.view(np.int16)).view(torch.bfloat16).double()
    ref64 = F.linear(t_emb, t_w)
    assert np.allclose(exact, ref64.numpy(), rtol=1e-12, atol=1e-14)
    ref = ref64.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours != ref).mean() <= 1e-3
