"""The projection stored in FP8 (MXFP8 along its input features) against the oracle (needs an
MI355X).

Up to 64 tokens the fused weight-streaming kernel reads the FP8 weights itself: with a table of
fp32 scales it dequantises them exactly to bf16 in registers (the bf16 MFMA, so results equal
the bf16 path on the oracle's dequantised weights bit for bit); with an MXFP8 table both
operands stay fp8 and meet the scaled fp8 MFMA (the same exact products summed in another
order, so results agree to rounding).  Above 64 tokens an MXFP8 table takes the fp8 tiled
kernel (scaled fp8 MFMA as well); otherwise the weights are expanded to bf16 in the staging area
for the bf16 schedules (bit for bit equal to the bf16 path).  Everything is checked against the
oracle at the forward tolerance.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_common import check_out, eg, forward, host_wkv, layout, oracle_for, say, u16  # noqa: E402
from test_gpu_parity import _kv_case  # noqa: E402

WORKLOADS = synth.workloads()
DECODE_FP8 = WORKLOADS["decode_b64_fp8"]
# decode layout with FP8 weights over a table of 24 ~1000-row ranges: 64 tokens (the fused
# kernel on FP8 weights), 100 tokens (expansion + the tiled schedule), 3 x 37 tokens for the
# projection alone (two token blocks)
SMALL_TABLE = synth.primes_from(1009, 24)
FP8_B64 = synth.small_variant(DECODE_FP8, name="decode_dims_fp8_b64", primes=SMALL_TABLE,
                              hash_dist="zipf", mask_false_frac=0.2, outlier_frac=0.05,
                              seed=DECODE_FP8.seed + 500)
FP8_T100 = synth.small_variant(FP8_B64, name="decode_dims_fp8_t100", B=1, T=100,
                               seed=DECODE_FP8.seed + 501)
FP8_KV = synth.small_variant(FP8_B64, name="decode_dims_fp8_b3_t37", B=3, T=37,
                             seed=DECODE_FP8.seed + 502)
# the fp8 tiled kernel without split K: three token blocks (the last one ragged), 300 tiles
FP8_T600 = synth.small_variant(FP8_B64, name="decode_dims_fp8_b2_t300", B=2, T=300,
                               seed=DECODE_FP8.seed + 506)
# fp32-scaled table, FP8 weights, a layout without a tiled schedule: 60 tokens (fused FP8
# kernel) and 150 tokens (expansion + weight streaming over three token blocks)
FP8_SMALL = synth.small_variant(WORKLOADS["tiny"], name="dim320_fp8_b2_t30", B=2, T=30, dim=320,
                                n_cols=4, head_dim=128, scale_block=32,
                                primes=synth.primes_from(1009, 4), hash_dist="zipf",
                                mask_false_frac=0.1, masked_positions=(), outlier_frac=0.05,
                                wkv_format="mxfp8", seed=DECODE_FP8.seed + 503)
FP8_SMALL_T75 = synth.small_variant(FP8_SMALL, name="dim320_fp8_b2_t75", T=75,
                                    seed=DECODE_FP8.seed + 504)


def _bf16_twin(w, d):
    """The same inputs with the oracle's bf16 dequantisation of the FP8 weights."""
    bits = oracle.wkv_mxfp8_bits(*w.wkv8())
    w16 = synth.small_variant(w, wkv_format="bf16")
    return w16, d | {"wkv": torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)}


def test_device_fill_mxfp8_wkv_matches_host_generator():
    say("[gpu] device fill of FP8 weights vs host generator")
    w = FP8_SMALL
    d = synth.device_inputs(w)
    codes, scales = w.wkv8()
    blob = d["wkv"].cpu().numpy()
    assert blob.size == w.N * w.K + w.N * (w.K // 32)
    assert np.array_equal(blob[: w.N * w.K].reshape(w.N, w.K), codes)
    assert np.array_equal(blob[w.N * w.K:].reshape(w.N, w.K // 32), scales)
    assert eg.wkv_bytes(layout(w)) == blob.size


def _fp8_kernels(w):
    """(the fused streaming kernel reads the FP8 weights, the fp8 tiled kernel does)"""
    native = w.M <= 64 and w.head_dim % 128 == 0 and (w.K // 4) % 128 == 0
    tiled8 = (w.M > 64 and w.scale_format == "e8m0" and w.scale_block % 32 == 0 and w.dim % 256 == 0
              and w.K % 128 == 0)
    return native, tiled8


@pytest.mark.parametrize("w", [FP8_B64, FP8_T100, FP8_T600, FP8_SMALL, FP8_SMALL_T75],
                         ids=lambda w: w.name)
def test_forward_fp8_wkv(w):
    say(f"[gpu] forward with FP8 weights: {w.name} (B={w.B} T={w.T}, dim {w.dim}, table "
        f"{w.scale_format}/{w.scale_block})")
    d = synth.device_inputs(w)
    lay = layout(w)
    ws = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    stg = eg.engram_forward_staging_bytes(lay, w.B, w.T)
    native, tiled8 = _fp8_kernels(w)
    # the expansion needs N x K bf16 of staging; the kernels that read FP8 weights need none
    assert (stg >= 2 * w.N * w.K) == (not native and not tiled8), (stg, w.N * w.K)
    buf = torch.zeros(ws + 4096, dtype=torch.uint8, device="cuda")
    buf[ws:] = 0xA5
    out = forward(w, d, ws=buf[:ws])
    torch.cuda.synchronize()
    assert bool((buf[ws:] == 0xA5).all()), "a kernel wrote past the workspace"
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
    w16, d16 = _bf16_twin(w, d)
    out16 = forward(w16, d16)
    torch.cuda.synchronize()
    if (native and w.scale_format == "e8m0") or tiled8:
        # scaled fp8 MFMA: equal up to the summation order of the projection
        diff = np.abs(u16(out).astype(np.int32) - u16(out16).astype(np.int32))
        say(f"    vs bf16 path: {float((diff > 0).mean()):.2e} of outputs differ, "
            f"{float((diff > 1).mean()):.2e} by more than one ulp")
        assert (diff > 1).mean() <= 1e-3
    else:
        assert torch.equal(out.view(torch.int16), out16.view(torch.int16))
    del d, d16
    torch.cuda.empty_cache()


def test_forward_fp8_wkv_mxfp8_table_bad_ids_nan_substitute_row():
    say("[gpu] FP8 weights and an MXFP8 table (scaled fp8 MFMA): out-of-range ids, the row they "
        "are replaced by has NaN scales, 64 features per scale")
    w = synth.small_variant(FP8_B64, name="decode_dims_fp8_sb64_bad", scale_block=64, B=2, T=32,
                            seed=DECODE_FP8.seed + 505)
    d = synth.device_inputs(w)
    ids = w.hash_ids().reshape(w.M, w.n_cols).copy()
    ids[ids == 0] = 1                       # row 0 is read only in place of bad ids
    ids[3, 5], ids[17, 0], ids[40, 23] = -1, w.n_rows, 1 << 40
    d["hash_ids"] = torch.from_numpy(ids.reshape(w.B, w.T, w.n_cols)).cuda()
    d["scales"][0] = 255                    # NaN scales in row 0
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = eg.engram_forward(layout(w), d["x"], d["hash_ids"], d["token_mask"], d["table"],
                            d["scales"], d["wkv"], d["q_weight"], d["k_weight"], err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 3
    assert not torch.isnan(out.float()).any()
    codes, scales = synth.host_fetch(w)(np.arange(w.n_rows))
    scales = scales.copy()
    scales[0] = 255
    q, k = w.qk()
    ref = oracle.forward(w.x_tokens(np.arange(w.M)), ids, w.token_mask().reshape(-1),
                         oracle.array_fetch(codes, scales), w.n_rows, w.head_dim, w.scale_block,
                         host_wkv(w), q, k, eps=w.eps, clamp=w.clamp, scale_format="e8m0")
    say("   ", check_out(w, np.arange(w.M), u16(out).reshape(w.M, w.hc, w.dim), ref))


@pytest.mark.slow
def test_forward_prefill_fp8_sampled():
    say("[gpu] forward prefill_t8192_fp8 (MXFP8 table and weights, fp8 tiled kernel), sampled tokens")
    w = WORKLOADS["prefill_t8192_fp8"]
    d = synth.device_inputs(w)
    out = forward(w, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    mask = w.token_mask().reshape(-1)
    closed = np.nonzero(mask == 0)[0][:4]
    sel = np.unique(np.concatenate([[0, 63, 64, 255, 256, w.M - 1], closed, rng.integers(0, w.M, 40)]))
    got = u16(out).reshape(w.M, w.hc, w.dim)[sel]
    del d, out
    torch.cuda.empty_cache()
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))


def test_kv_proj_fp8_wkv_two_token_blocks():
    say("[gpu] kv_proj with FP8 weights: decode dims, B=3 T=37")
    w = FP8_KV
    d = synth.device_inputs(w)
    emb, kv = _kv_case(w, d)
    w16, d16 = _bf16_twin(w, d)
    kv16 = eg.engram_kv_proj(layout(w16), emb, d16["wkv"])
    torch.cuda.synchronize()
    assert torch.equal(kv.view(torch.int16), kv16.view(torch.int16))
    del d, d16
    torch.cuda.empty_cache()


def test_kv_proj_fp8_wkv_shape_without_streaming_loop_is_rejected():
    say("[gpu] kv_proj with FP8 weights on tiny dims (K / 4 = 96): layout error, nothing launched")
    w = synth.small_variant(WORKLOADS["tiny"], wkv_format="mxfp8")
    d = synth.device_inputs(w)
    emb = torch.zeros((w.B, w.T, w.K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(eg.EngramError) as e:
        eg.engram_kv_proj(layout(w), emb, d["wkv"])
    assert e.value.status == -2
    # the whole forward still runs there (expansion + the narrow bf16 loop)
    out = forward(w, d)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))


def test_wrong_wkv_size_is_refused_by_the_binding():
    w = FP8_SMALL
    lay = layout(w)
    x = torch.zeros((1, 1, w.hc, w.dim), dtype=torch.bfloat16, device="cuda")
    emb = torch.zeros((1, 1, w.K), dtype=torch.bfloat16, device="cuda")
    short = torch.zeros(eg.wkv_bytes(lay) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        eg.engram_kv_proj(lay, emb, short)
    bf = torch.zeros((w.N, w.K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        eg.engram_kv_proj(lay, emb, bf)
    del x


def test_workspace_sizes_never_decrease_with_token_count_fp8():
    say("[gpu] workspace and staging sizes against the token count, FP8 weights")
    for w in (FP8_B64, FP8_SMALL, synth.small_variant(WORKLOADS["tiny"], wkv_format="mxfp8")):
        lay = layout(w)
        last_ws = last_stg = last_ctrl = 0
        for M in list(range(1, 300)) + [320, 511, 512, 513, 1000, 4096, 8192]:
            ws = eg.engram_forward_workspace_bytes(lay, 1, M)
            stg = eg.engram_forward_staging_bytes(lay, 1, M)
            assert ws >= last_ws and stg >= last_stg and ws - stg >= last_ctrl, (w.name, M)
            last_ws, last_stg, last_ctrl = ws, stg, ws - stg


def test_fp8_weight_dequantisation_every_code_and_exponent():
    say("[gpu] FP8 weights through the projection alone with one-hot rows: every code at every "
        "exponent 0..245 dequantised bit for bit")
    # dim 320, 4 columns of 128: N = 1600 weight rows of K = 512; scale block B = 16 n + b takes
    # exponent B % 246 and codes 32 ((B // 246) % 8) + 0..31, so every (code, exponent) pair occurs.
    # NaN codes are replaced by 0x00, and exponents stop at 245 so that no weight overflows bf16
    # (a zero times an infinite or NaN weight would poison every sum)
    w = synth.small_variant(FP8_SMALL, wkv_format="mxfp8")
    N, K = w.N, w.K
    blk = np.arange(N * (K // 32)).reshape(N, K // 32)
    exps = (blk % 246).astype(np.uint8)
    off = 32 * ((blk // 246) % 8)
    codes = (np.repeat(off, 32, axis=1) + np.tile(np.arange(32), K // 32)[None, :]).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    covered = {(int(c), int(e)) for c, e in zip(codes.reshape(-1), np.repeat(exps, 32, axis=1).reshape(-1))}
    assert len(covered) >= 254 * 246
    blob = torch.from_numpy(np.concatenate([codes.reshape(-1), exps.reshape(-1)])).cuda()
    # token m selects input feature m
    emb = torch.zeros((1, K, K), dtype=torch.bfloat16, device="cuda")
    emb[0, torch.arange(K), torch.arange(K)] = 1.0
    kv = eg.engram_kv_proj(layout(w), emb, blob)
    torch.cuda.synchronize()
    got = u16(kv).reshape(K, N).T
    want = oracle.wkv_mxfp8_bits(codes, exps)
    # a -0 weight comes out of the sum as +0 (-0 + +0 = +0): the one sign the projection loses
    want = np.where(want == 0x8000, np.uint16(0), want)
    assert (want != 0).mean() > 0.9
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], want[bad][:5])
