"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Every GPU call goes through the C ABI (the ctypes binding); the tolerances are those stated in
gpu_common.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_common import check_out, eg, forward, host_wkv, layout, oracle_for, say, u16  # noqa: E402


# ---------------------------------------------------------------------------- fixtures

WORKLOADS = synth.workloads()
TINY = WORKLOADS["tiny"]
DECODE = WORKLOADS["decode_b64"]
# decode layout, three sequences of 37 tokens: two token blocks and a ragged tail, skewed ids,
# closed tokens and outlier streams
RAGGED = synth.small_variant(DECODE, name="decode_dims_b3_t37", B=3, T=37, hash_dist="zipf",
                             mask_false_frac=0.2, outlier_frac=0.05, seed=DECODE.seed + 100)
# token counts that take the tiled (256 x 256) schedule: tiny dims with three token blocks (the
# last one ragged), and the decode layout with one full and one ragged token block
TILED_TINY = synth.small_variant(TINY, name="tiny_dims_b2_t300", B=2, T=300, hash_dist="zipf",
                                 mask_false_frac=0.15, outlier_frac=0.05, masked_positions=(),
                                 seed=TINY.seed + 200)
TILED_DECODE = synth.small_variant(DECODE, name="decode_dims_b1_t300", B=1, T=300,
                                   hash_dist="zipf", mask_false_frac=0.1, outlier_frac=0.02,
                                   seed=DECODE.seed + 200)


@pytest.fixture(scope="module")
def dev_tiny():
    say("[gpu] inputs: tiny")
    return synth.device_inputs(TINY)


@pytest.fixture(scope="module")
def dev_decode():
    say("[gpu] inputs: decode_b64 (4.3 GB table)")
    d = synth.device_inputs(DECODE)
    torch.cuda.synchronize()
    yield d
    del d
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------- generator


def test_device_fill_matches_host_generator(dev_tiny, dev_decode):
    say("[gpu] device fill vs host generator")
    w, d = TINY, dev_tiny
    assert np.array_equal(u16(d["x"]).reshape(w.M, w.hc, w.dim), w.x_tokens(np.arange(w.M)))
    assert np.array_equal(d["table"].cpu().numpy(), w.codes_rows(np.arange(w.n_rows)))
    assert np.array_equal(d["scales"].cpu().numpy(), w.scales_rows(np.arange(w.n_rows)))
    assert np.array_equal(u16(d["wkv"]), w.wkv_rows(0, w.N))
    w, d = DECODE, dev_decode
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, w.n_rows - 1], rng.integers(0, w.n_rows, 300)])
    assert np.array_equal(d["table"][torch.from_numpy(rows).cuda()].cpu().numpy(), w.codes_rows(rows))
    assert np.array_equal(d["scales"][torch.from_numpy(rows).cuda()].cpu().numpy(), w.scales_rows(rows))
    assert np.array_equal(u16(d["wkv"][:7]), w.wkv_rows(0, 7))
    assert np.array_equal(u16(d["wkv"][-5:]), w.wkv_rows(w.N - 5, w.N))
    toks = np.array([0, 17, 63])
    assert np.array_equal(u16(d["x"]).reshape(w.M, w.hc, w.dim)[toks], w.x_tokens(toks))


# ---------------------------------------------------------------------------- S1 + S2


def _gather_case(w, d, sel_tokens=None):
    emb = eg.engram_gather_dequant(layout(w), d["table"], d["scales"], d["hash_ids"])
    torch.cuda.synchronize()
    got = u16(emb).reshape(w.M, -1)
    ids = w.hash_ids().reshape(w.M, w.n_cols)
    sel = np.arange(w.M) if sel_tokens is None else sel_tokens
    ref = oracle.gather_dequant(ids[sel], synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block,
                                scale_format=w.scale_format)
    assert np.array_equal(got[sel], ref)


def test_gather_dequant_bit_exact_tiny(dev_tiny):
    say("[gpu] gather tiny")
    _gather_case(TINY, dev_tiny)


def test_gather_dequant_bit_exact_decode(dev_decode):
    say("[gpu] gather decode_b64")
    _gather_case(DECODE, dev_decode)


def test_gather_all_codes_special_scales_and_bad_ids():
    say("[gpu] gather: all 256 codes, special scales, out-of-range ids")
    hd, sb, n = 64, 32, 40
    rng = np.random.default_rng(12)
    table = np.tile(np.arange(256, dtype=np.uint8), n * hd // 256 + 1)[: n * hd].reshape(n, hd)
    rng.shuffle(table.reshape(-1))
    scales = rng.uniform(0.01, 0.1, (n, hd // sb)).astype(np.float32)
    scales[0] = [1e-40, 2.0 ** -126]
    scales[1] = [3e38, -1.5]
    scales[2] = [np.inf, np.nan]
    scales[3] = [0.0, -0.0]
    C = 6
    ids = rng.integers(0, n, (3, 5, C)).astype(np.int64)
    ids.reshape(-1)[:n] = np.arange(n)  # every row at least once
    ids[0, 0, 0] = -1
    ids[1, 2, 3] = n
    ids[2, 4, 5] = 1 << 40
    lay = eg.make_layout(4, 256, C, hd, sb, n)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    emb = eg.engram_gather_dequant(lay, torch.from_numpy(table).cuda(), torch.from_numpy(scales).cuda(),
                                   torch.from_numpy(ids).cuda(), err_count=err)
    torch.cuda.synchronize()
    ref = oracle.gather_dequant(ids.reshape(-1, C), oracle.array_fetch(table, scales), n, hd, sb)
    assert np.array_equal(u16(emb).reshape(15, -1), ref)
    bad = int(((ids < 0) | (ids >= n)).sum())
    assert int(err.item()) == bad == 3


# ---------------------------------------------------------------------------- S3


def _kv_case(w, d, sel=None):
    emb = eg.engram_gather_dequant(layout(w), d["table"], d["scales"], d["hash_ids"])
    kv = eg.engram_kv_proj(layout(w), emb, d["wkv"])
    torch.cuda.synchronize()
    got = u16(kv).reshape(w.M, -1)
    sel = np.arange(w.M) if sel is None else sel
    ids = w.hash_ids().reshape(w.M, w.n_cols)[sel]
    emb_ref = oracle.gather_dequant(ids, synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block,
                                    scale_format=w.scale_format)
    ref, exact = oracle.kv_proj(emb_ref, host_wkv(w), with_exact=True)
    # fp32 accumulation (any order) then one bf16 rounding: |got - exact| <= ulp(exact) plus the
    # classical sum-of-products bound K * 2^-24 * sum |a| |b|
    abs_sum = np.abs(oracle.bf16_value(emb_ref)) @ np.abs(host_wkv(w)).astype(np.float64).T
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
    err = np.abs(oracle.bf16_value(got[sel]) - exact)
    bound = ulp + w.K * 2.0 ** -24 * abs_sum
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    say(f"    kv: worst err/bound {float((err / bound)[worst]):.3f} at {worst}: exact "
        f"{exact[worst]:.6e} sum|ab| {abs_sum[worst]:.4e} err {err[worst]:.3e}; "
        f"bf16 bits differ on {float((got[sel] != ref).mean()):.2e} of entries")
    assert np.all(err <= bound)
    assert (got[sel] != ref).mean() < 0.01
    return emb, kv


def test_kv_proj_tiny(dev_tiny):
    say("[gpu] kv_proj tiny")
    _kv_case(TINY, dev_tiny)


def test_kv_proj_decode(dev_decode):
    say("[gpu] kv_proj decode_b64")
    _kv_case(DECODE, dev_decode)


# ---------------------------------------------------------------------------- S4 - S6


def _gate_case(w, d, in_place=False):
    ids = w.hash_ids().reshape(w.M, w.n_cols)
    emb_ref = oracle.gather_dequant(ids, synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block,
                                    scale_format=w.scale_format)
    kv_ref = oracle.kv_proj(emb_ref, host_wkv(w))
    x_bits = w.x_tokens(np.arange(w.M))
    q, k = w.qk()
    mask = w.token_mask().reshape(-1)
    ref = oracle.gate_apply(x_bits, kv_ref, q, k, mask, w.eps, w.clamp)
    kv = torch.from_numpy(kv_ref.view(np.int16)).cuda().view(torch.bfloat16)
    gate = torch.empty((w.M, w.hc), dtype=torch.float32, device="cuda")
    x = d["x"].clone()
    out = eg.engram_gate_apply(layout(w), x, kv, d["q_weight"], d["k_weight"], d["token_mask"],
                               out=x if in_place else None, gate=gate)
    torch.cuda.synchronize()
    g = gate.cpu().numpy().astype(np.float64)
    assert np.abs(g - ref["gate"]).max() <= 1e-4
    got = u16(out).reshape(w.M, w.hc, w.dim)
    d_ulp = np.abs(got.astype(np.int32) - ref["out_bits"].astype(np.int32))
    assert (d_ulp > 1).mean() <= 1e-4, (d_ulp > 1).mean()
    err = np.abs(oracle.bf16_value(got) - ref["out_f"])
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.array_equal(got[~mask.astype(bool)], x_bits[~mask.astype(bool)])


def test_gate_apply_tiny(dev_tiny):
    say("[gpu] gate_apply tiny")
    _gate_case(TINY, dev_tiny)
    _gate_case(TINY, dev_tiny, in_place=True)


def test_gate_apply_decode(dev_decode):
    say("[gpu] gate_apply decode_b64")
    _gate_case(DECODE, dev_decode)


# ---------------------------------------------------------------------------- whole forward


def test_forward_tiny(dev_tiny):
    say("[gpu] forward tiny")
    w = TINY
    out = forward(w, dev_tiny)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))


def test_forward_decode(dev_decode):
    say("[gpu] forward decode_b64")
    w = DECODE
    out = forward(w, dev_decode)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))


def test_forward_ragged_multi_block():
    say("[gpu] forward decode dims, B=3 T=37 (ragged, closed tokens, outliers)")
    w = RAGGED
    d = synth.device_inputs(w)
    out = forward(w, d)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
    del d
    torch.cuda.empty_cache()


def test_forward_equals_composition_in_place_and_deterministic(dev_decode):
    say("[gpu] forward: composed path, in place, reruns")
    w, d = DECODE, dev_decode
    lay = layout(w)
    ws = torch.zeros(eg.engram_forward_workspace_bytes(lay, w.B, w.T), dtype=torch.uint8, device="cuda")
    a = forward(w, d, ws=ws)
    b = forward(w, d, ws=ws)
    x2 = d["x"].clone()
    c = forward(w, d | {"x": x2}, out=x2, ws=ws)
    emb = eg.engram_gather_dequant(lay, d["table"], d["scales"], d["hash_ids"])
    kv = eg.engram_kv_proj(lay, emb, d["wkv"])
    e = eg.engram_gate_apply(lay, d["x"], kv, d["q_weight"], d["k_weight"], d["token_mask"])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    # no cross-workgroup wait timed out (word 0), every call left the workspace all zero, and a
    # fresh zero-filled workspace gives the same result as the reused one
    assert int(torch.count_nonzero(ws).item()) == 0
    fresh = forward(w, d, ws=torch.zeros_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(a, fresh)
    diff = np.abs(u16(a).astype(np.int32) - u16(e).astype(np.int32))
    assert (diff > 1).mean() <= 1e-4
    assert np.abs(oracle.bf16_value(u16(a)) - oracle.bf16_value(u16(e))).max() <= 2e-2


def test_split_phase_projection_on_a_side_stream_equals_fused(dev_decode):
    # The pages' serving schedule ("Engram in DeepSeek V4.1 Flash", the later optimisation that
    # separates lookup, projection and gating): rows and projection as soon as the hash ids are
    # known, on a stream of their own while other work runs, the gate at the layer's entry.
    say("[gpu] split phase: gather + projection on a side stream, gate on the main stream")
    w, d = DECODE, dev_decode
    lay = layout(w)
    fused = forward(w, d)
    torch.cuda.synchronize()
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    filler = torch.randn(4096, 4096, device="cuda")
    side.wait_stream(main)
    with torch.cuda.stream(side):
        emb = eg.engram_gather_dequant(lay, d["table"], d["scales"], d["hash_ids"])
        kv = eg.engram_kv_proj(lay, emb, d["wkv"])
        done = torch.cuda.Event()
        done.record(side)
    for _ in range(4):
        filler = filler @ filler / 64.0  # the backbone's work meanwhile
    main.wait_event(done)
    out = eg.engram_gate_apply(lay, d["x"], kv, d["q_weight"], d["k_weight"], d["token_mask"])
    torch.cuda.synchronize()
    diff = np.abs(u16(out).astype(np.int32) - u16(fused).astype(np.int32))
    assert (diff > 1).mean() <= 1e-4
    assert np.abs(oracle.bf16_value(u16(out)) - oracle.bf16_value(u16(fused))).max() <= 2e-2
    sel = np.arange(w.M)
    check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel))


def test_forward_bad_ids_read_zero_rows():
    say("[gpu] forward with out-of-range hash ids")
    w = synth.small_variant(TINY, name="tiny_bad_ids", seed=TINY.seed + 7)
    d = synth.device_inputs(w)
    ids = w.hash_ids()
    ids[0, 2, 1] = -5
    ids[0, 7, 4] = w.n_rows
    d["hash_ids"] = torch.from_numpy(ids).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    q, k = w.qk()
    ref = oracle.forward(w.x_tokens(np.arange(w.M)), ids.reshape(w.M, -1), w.token_mask().reshape(-1),
                         synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block, host_wkv(w), q, k)
    check_out(w, np.arange(w.M), u16(out).reshape(w.M, w.hc, w.dim), ref)


@pytest.mark.parametrize("B,T", [(1, 1), (1, 65), (0, 5)])
def test_forward_edge_token_counts(B, T):
    say(f"[gpu] forward tiny dims B={B} T={T}")
    w = synth.small_variant(TINY, name=f"tiny_{B}x{T}", B=B, T=T, masked_positions=())
    d = synth.device_inputs(w)
    out = forward(w, d)
    torch.cuda.synchronize()
    if w.M == 0:
        return
    sel = np.arange(w.M)
    check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel))


@pytest.mark.slow
def test_forward_prefill_sampled():
    say("[gpu] forward prefill_t8192 (25.6 GB table), sampled tokens")
    w = WORKLOADS["prefill_t8192"]
    d = synth.device_inputs(w)
    out = forward(w, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    mask = w.token_mask().reshape(-1)
    closed = np.nonzero(mask == 0)[0][:4]
    sel = np.unique(np.concatenate([[0, 63, 64, 255, 256, w.M - 1], closed, rng.integers(0, w.M, 40)]))
    got = u16(out).reshape(w.M, w.hc, w.dim)[sel]
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))
    del d, out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------- tiled schedule


def test_kv_proj_tiled_tiny_dims():
    say("[gpu] kv_proj tiled: tiny dims, B=2 T=300")
    w = TILED_TINY
    d = synth.device_inputs(w)
    _kv_case(w, d)


def test_forward_tiled_tiny_dims_bad_ids_in_place():
    say("[gpu] forward tiled: tiny dims, B=2 T=300 (ragged block, closed tokens, outliers, bad ids)")
    w = TILED_TINY
    d = synth.device_inputs(w)
    ids = w.hash_ids()
    ids[0, 5, 1] = -3
    ids[1, 299, 5] = w.n_rows
    ids[1, 40, 0] = 1 << 40
    d["hash_ids"] = torch.from_numpy(ids).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, err=err)
    x2 = d["x"].clone()
    out2 = forward(w, d | {"x": x2}, out=x2)
    torch.cuda.synchronize()
    assert int(err.item()) == 3
    assert torch.equal(out, out2)
    q, k = w.qk()
    sel = np.arange(w.M)
    ref = oracle.forward(w.x_tokens(sel), ids.reshape(w.M, -1), w.token_mask().reshape(-1),
                         synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block, host_wkv(w), q, k)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), ref))


def test_workspace_control_zero_and_shared_across_schedules():
    say("[gpu] workspace: control words zero after calls, shared by the streaming and tiled "
        "schedules and two tiled token counts")
    w_big, w_small = TILED_TINY, synth.small_variant(TILED_TINY, name="tiny_dims_b1_t40", B=1, T=40)
    w_mid = synth.small_variant(TILED_TINY, name="tiny_dims_b1_t260", B=1, T=260)
    lay = layout(w_big)
    cases = [w_big, w_small, w_mid]
    n = max(eg.engram_forward_workspace_bytes(lay, w.B, w.T) for w in cases)
    assert eg.engram_forward_staging_bytes(lay, w_small.B, w_small.T) == 0
    assert eg.engram_forward_staging_bytes(lay, w_big.B, w_big.T) >= w_big.M * w_big.K * 2
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    devs = {w.name: synth.device_inputs(w) for w in cases}
    outs = []
    for w in (w_big, w_small, w_mid, w_big, w_small, w_mid):
        outs.append(forward(w, devs[w.name], ws=ws))
        torch.cuda.synchronize()
        # below the largest staging area, every byte is a control word of some call: all zero
        ctrl = n - max(eg.engram_forward_staging_bytes(lay, v.B, v.T) for v in cases)
        assert int(torch.count_nonzero(ws[:ctrl]).item()) == 0, w.name
    fresh = [forward(w, devs[w.name], ws=torch.zeros_like(ws)) for w in cases]
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(outs[i], fresh[i]) and torch.equal(outs[i + 3], fresh[i]), cases[i].name


# a layout without a tiled schedule (dim not a multiple of 256): the whole forward streams wkv
# once per 64-token block at every token count; three blocks, the last one ragged
STREAM_ONLY = synth.small_variant(TINY, name="dim320_b2_t75", B=2, T=75, dim=320, n_cols=4,
                                  head_dim=128, scale_block=32, primes=synth.primes_from(1009, 4),
                                  hash_dist="zipf", mask_false_frac=0.1, masked_positions=(),
                                  outlier_frac=0.05, seed=TINY.seed + 300)


def test_forward_streaming_token_blocks_exact_workspace_with_guard():
    say("[gpu] forward, layout without a tiled schedule: three token blocks, workspace of exactly "
        "the reported size followed by guard bytes")
    w = STREAM_ONLY
    lay = layout(w)
    d = synth.device_inputs(w)
    need = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    assert eg.engram_forward_staging_bytes(lay, w.B, w.T) == 0
    buf = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    out = forward(w, d, ws=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "a kernel wrote past the workspace"
    assert int(torch.count_nonzero(buf[:need]).item()) == 0
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))


@pytest.mark.parametrize("T", [37, 64])
def test_forward_one_token_block_apply_workgroups_small_layout(T):
    """One token block on the layout without a tiled schedule: the weight-streaming kernel with
    apply workgroups at one or two 4-row groups per workgroup (value tiles of 4 or 8 features,
    shifted by 4 for half of them), a partial second token half at 37 tokens; a workspace of
    exactly the reported size followed by guard bytes, every control word (tiles included) left
    zero, in place as well."""
    w = synth.small_variant(STREAM_ONLY, name=f"dim320_b1_t{T}", B=1, T=T, seed=TINY.seed + 310 + T)
    say(f"[gpu] forward {w.name}: one token block, apply workgroups, small layout")
    lay = layout(w)
    d = synth.device_inputs(w)
    need = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    buf = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    out = forward(w, d, ws=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "a kernel wrote past the workspace"
    assert int(torch.count_nonzero(buf[:need]).item()) == 0
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
    x2 = d["x"].clone()
    forward(w, d | {"x": x2}, out=x2, ws=buf[:need])
    torch.cuda.synchronize()
    assert torch.equal(x2, out)


def test_kv_proj_streaming_two_token_blocks():
    say("[gpu] kv_proj decode dims, B=3 T=37 (weight streaming, two token blocks)")
    w = RAGGED
    d = synth.device_inputs(w)
    _kv_case(w, d)
    del d
    torch.cuda.empty_cache()


def test_workspace_sizes_never_decrease_with_token_count():
    say("[gpu] workspace and staging sizes against the token count")
    for w in (TINY, DECODE, STREAM_ONLY):
        lay = layout(w)
        last_ws = last_stg = last_ctrl = 0
        for M in list(range(1, 300)) + [320, 511, 512, 513, 1000, 4096, 8192]:
            ws = eg.engram_forward_workspace_bytes(lay, 1, M)
            stg = eg.engram_forward_staging_bytes(lay, 1, M)
            assert ws >= last_ws and stg >= last_stg and ws - stg >= last_ctrl, (w.name, M)
            last_ws, last_stg, last_ctrl = ws, stg, ws - stg


def test_binding_workspace_shared_by_two_layouts():
    say("[gpu] the binding's workspace across layouts: a four-token-block call (staged rows at the "
        "end) then streamed token blocks of another layout (control words over that staging)")
    # (five token blocks: their control words reach past the first call's control part, which
    # holds the streaming schedules' words up to 256 tokens, value tiles included)
    a, b = E8M0_TB4, synth.small_variant(STREAM_ONLY, name="dim320_b2_t150", T=150)
    assert (eg.engram_forward_workspace_bytes(layout(b), b.B, b.T) >
            eg.engram_forward_workspace_bytes(layout(a), a.B, a.T) - eg.engram_forward_staging_bytes(layout(a), a.B, a.T))
    da, db = synth.device_inputs(a), synth.device_inputs(b)
    wso = eg.Workspace()  # sized by the first call; the second fits without growing
    forward(a, da, ws=wso.get(layout(a), a.B, a.T))
    got = forward(b, db, ws=wso.get(layout(b), b.B, b.T))
    fresh = torch.zeros(eg.engram_forward_workspace_bytes(layout(b), b.B, b.T), dtype=torch.uint8, device="cuda")
    want = forward(b, db, ws=fresh)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    del da, db
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------- E8M0 scales
# MXFP8 tables (E8M0 block scales): the decode layout with one scale per 32 features (the
# pages' format; weight streaming, the two-token-block kernel at 100 tokens and the
# four-token-block kernel at 150), one per 64 features (a scale's byte position in its dword changes from chunk
# to chunk; also at 100 tokens), and tiny dims with 16 features per scale (the narrow streaming
# loop).  Exponents 120..124 (scales 2^-7 .. 2^-3, the
# magnitude of the fp32 workloads' scales); the gather test covers all 256 exponents.
E8M0_DECODE = synth.small_variant(DECODE, name="decode_dims_e8m0_sb32", B=2, T=3, scale_block=32,
                                  scale_format="e8m0", hash_dist="zipf", mask_false_frac=0.2,
                                  seed=DECODE.seed + 400)
E8M0_DECODE64 = synth.small_variant(E8M0_DECODE, name="decode_dims_e8m0_sb64", scale_block=64,
                                    seed=DECODE.seed + 401)
E8M0_TB2 = synth.small_variant(E8M0_DECODE, name="decode_dims_e8m0_t100", B=1, T=100,
                               seed=DECODE.seed + 402)
E8M0_TB2_64 = synth.small_variant(E8M0_DECODE64, name="decode_dims_e8m0_sb64_t100", B=1, T=100,
                                  seed=DECODE.seed + 404)
E8M0_TB4 = synth.small_variant(E8M0_DECODE, name="decode_dims_e8m0_t150", B=1, T=150,
                                 seed=DECODE.seed + 405)
E8M0_TINY = synth.small_variant(TINY, name="tiny_e8m0_sb16", scale_block=16, scale_format="e8m0",
                                seed=TINY.seed + 403)


def test_gather_e8m0_all_codes_all_exponents_bad_ids():
    say("[gpu] gather with E8M0 scales: all 256 codes x all 256 exponents, out-of-range ids")
    hd, sb = 256, 32
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    exps = np.repeat(np.arange(256, dtype=np.uint8)[:, None], hd // sb, axis=1)
    exps[7] = np.arange(8, dtype=np.uint8) + 120  # different exponents within one row
    C = 4
    rng = np.random.default_rng(13)
    ids = rng.integers(0, 256, (2, 40, C)).astype(np.int64)
    ids.reshape(-1)[:256] = np.arange(256)  # every row at least once
    ids[0, 1, 2] = -1
    ids[1, 39, 3] = 256
    lay = eg.make_layout(4, 256, C, hd, sb, 256, scale_format=eg.SCALE_E8M0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    emb = eg.engram_gather_dequant(lay, torch.from_numpy(codes).cuda(), torch.from_numpy(exps).cuda(),
                                   torch.from_numpy(ids).cuda(), err_count=err)
    torch.cuda.synchronize()
    ref = oracle.gather_dequant(ids.reshape(-1, C), oracle.array_fetch(codes, exps), 256, hd, sb,
                                scale_format="e8m0")
    assert np.array_equal(u16(emb).reshape(80, -1), ref)
    assert int(err.item()) == 2


def test_device_fill_e8m0_matches_host_generator():
    say("[gpu] device fill of E8M0 scales vs host generator")
    w = E8M0_TINY
    d = synth.device_inputs(w)
    assert d["scales"].dtype == torch.uint8
    assert np.array_equal(d["scales"].cpu().numpy(), w.scales_rows(np.arange(w.n_rows)))


@pytest.mark.parametrize("w", [E8M0_DECODE, E8M0_DECODE64, E8M0_TB2, E8M0_TB2_64, E8M0_TB4, E8M0_TINY],
                         ids=lambda w: w.name)
def test_forward_e8m0(w):
    say(f"[gpu] forward with E8M0 scales: {w.name} (B={w.B} T={w.T}, scale_block {w.scale_block})")
    d = synth.device_inputs(w)
    out = forward(w, d)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
    # the rows themselves, bit for bit
    emb = eg.engram_gather_dequant(layout(w), d["table"], d["scales"], d["hash_ids"])
    torch.cuda.synchronize()
    ids = w.hash_ids().reshape(w.M, w.n_cols)
    ref = oracle.gather_dequant(ids, synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block,
                                scale_format="e8m0")
    assert np.array_equal(u16(emb).reshape(w.M, -1), ref)
    del d
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def dev_tiled_decode():
    say("[gpu] inputs: decode layout, B=1 T=300")
    d = synth.device_inputs(TILED_DECODE)
    torch.cuda.synchronize()
    yield d
    del d
    torch.cuda.empty_cache()


def test_kv_proj_tiled_decode_dims(dev_tiled_decode):
    say("[gpu] kv_proj tiled: decode layout, B=1 T=300")
    _kv_case(TILED_DECODE, dev_tiled_decode)


def test_forward_tiled_decode_dims(dev_tiled_decode):
    say("[gpu] forward tiled: decode layout, B=1 T=300")
    w = TILED_DECODE
    out = forward(w, dev_tiled_decode)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
