"""Host-side checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest

import oracle
import synth


def test_splitmix64_reference_sequence():
    # SplitMix64 started at state 0 produces these first outputs (Vigna's reference code)
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [int(v) for v in synth.draw(0, np.arange(3))]
    assert got == want


def test_draws_are_counter_based():
    key = synth.stream_key(123, synth.S_WKV)
    a = synth.draw(key, np.arange(100))
    b = synth.draw(key, np.arange(50, 100))
    assert np.array_equal(a[50:], b)
    assert synth.stream_key(123, synth.S_WKV) != synth.stream_key(123, synth.S_X)
    assert synth.stream_key(123, synth.S_WKV, 1) != synth.stream_key(123, synth.S_WKV, 0)


def test_e4m3_encoder_rounds_to_nearest_even():
    r24 = np.concatenate([np.arange(0, 1 << 17, 97), np.arange((1 << 24) - 5000, 1 << 24),
                          np.random.default_rng(0).integers(0, 1 << 24, 20000)])
    codes = synth.e4m3_magnitude_code(r24)
    v = r24 * 2.0 ** -22
    grid = oracle.e4m3fn_value(np.arange(0x49, dtype=np.uint8))        # 0 .. 4.0
    got = oracle.e4m3fn_value(codes)
    err = np.abs(got - v)
    best = np.min(np.abs(grid[None, :] - v[:, None]), axis=1)
    assert np.all(err == best)
    ties = np.abs(np.abs(grid[None, :] - v[:, None]) - best[:, None]) == 0
    tie_rows = ties.sum(1) > 1
    assert np.all((codes[tie_rows] & 1) == 0)          # ties go to the even mantissa
    assert codes.max() <= 0x48


def test_codes_are_finite_and_roughly_uniform():
    w = synth.get("tiny")
    codes = w.codes_rows(np.arange(2000))
    vals = oracle.e4m3fn_value(codes)
    assert np.all(np.isfinite(vals)) and np.abs(vals).max() <= 4.0
    assert abs(vals.mean()) < 0.05 and abs(vals.std() - 4 / np.sqrt(3)) < 0.05


def test_normal_generator_moments():
    v = synth.bf16_bits_to_f32(synth.normal_bf16(99, 0, 200000, 0.0, 1.0)).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01 and np.abs(v).max() <= 6.0


def test_hash_ids_stay_in_their_column_ranges():
    for name in ("tiny", "decode_b64"):
        w = synth.get(name)
        ids = w.hash_ids().reshape(-1, w.n_cols)
        lo = w.offsets
        hi = lo + np.asarray(w.primes)
        assert np.all(ids >= lo[None]) and np.all(ids < hi[None])


def test_zipf_ranks_follow_the_pmf():
    N, s, n = 50, 1.1, 200000
    r = synth.zipf_ranks(77, 0, n, N, s)
    assert r.min() >= 1 and r.max() <= N
    pmf = np.arange(1, N + 1, dtype=np.float64) ** -s
    pmf /= pmf.sum()
    obs = np.bincount(r, minlength=N + 1)[1:]
    chi2 = np.sum((obs - n * pmf) ** 2 / (n * pmf))
    assert chi2 < 100.0          # 49 degrees of freedom; p ~ 1e-5 at 100


def test_masks_and_outliers():
    t = synth.get("tiny").token_mask().reshape(-1)
    assert list(np.nonzero(t == 0)[0]) == [3, 9]
    p = synth.get("prefill_t8192").token_mask()
    assert abs((p == 0).mean() - 0.10) < 0.02
    f = synth.get("fulltable_b4_t4096")
    assert abs(f.outlier_tokens().mean() - 0.01) < 0.004


@pytest.mark.parametrize("name,rows", [("decode_b64", 16_803_844), ("prefill_t8192", 100_006_264),
                                       ("fulltable_b4_t4096", 384_016_682)])
def test_workload_table_sizes(name, rows):
    assert synth.get(name).n_rows == rows


def test_fp8_projection_weights_spread_like_the_bf16_ones():
    # MXFP8 wkv of the decode layout with FP8 weights: rows regenerate identically in any chunk,
    # codes are finite, exponents stay in [lo, hi], and the weights' spread is that of the bf16
    # N(0, 0.02) weights within a factor (codes ~ U(-4, 4) x 2^(-8 .. -6))
    w = synth.get("decode_b64_fp8")
    codes, exps = w.wkv8_rows(100, 164)
    c2, e2 = w.wkv8_rows(130, 140)
    assert np.array_equal(codes[30:40], c2) and np.array_equal(exps[30:40], e2)
    assert codes.shape == (64, w.K) and exps.shape == (64, w.K // 32)
    assert not ((codes & 0x7F) == 0x7F).any()
    assert exps.min() >= w.wkv_e8m0_lo and exps.max() <= w.wkv_e8m0_hi
    assert set(np.unique(exps)) == set(range(w.wkv_e8m0_lo, w.wkv_e8m0_hi + 1))
    vals = oracle.bf16_value(oracle.wkv_mxfp8_bits(codes, exps))
    assert 0.01 < vals.std() < 0.03 and abs(vals.mean()) < 1e-3
