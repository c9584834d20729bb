"""The whole forward at decode shapes (one token block at the model's dims: the weight-streaming
schedule) against the oracle (needs an MI355X).

Partial token blocks (1, 5, 33 tokens), closed tokens, x50 outlier streams, out-of-range ids,
fp32 and E8M0 table scales, in place; a workspace of exactly the reported size followed by guard
bytes; control words zero after every call; bitwise-identical reruns.  The decode loop's second
weight slot for the first row block at a layout of two row blocks per workgroup (dim 1024: 20
rows, one full block and four rows) with one, two and twelve 128-feature chunks per K quarter."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_common import check_out, eg, forward, host_wkv, layout, say, u16  # noqa: E402

DECODE = synth.workloads()["decode_b64"]
MX = synth.workloads()["decode_b64_mxfp8"]
CASES = [
    synth.small_variant(DECODE, name="decode_dims_b1", B=1, T=1, seed=DECODE.seed + 400),
    synth.small_variant(DECODE, name="decode_dims_b5_closed_outliers", B=5, T=1, seed=DECODE.seed + 401,
                        mask_false_frac=0.3, outlier_frac=0.3, hash_dist="zipf"),
    synth.small_variant(DECODE, name="decode_dims_b33", B=33, T=1, seed=DECODE.seed + 402,
                        mask_false_frac=0.1, outlier_frac=0.05),
    synth.small_variant(MX, name="decode_mxfp8_table_b64", seed=MX.seed + 403, mask_false_frac=0.1),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_decode_shapes_against_oracle(w):
    say(f"[gpu] decode shapes: {w.name} ({w.M} tokens, {w.scale_format} scales)")
    d = synth.device_inputs(w)
    ids = w.hash_ids()
    if w.M >= 5:   # two rows outside the table: zero rows, counted
        ids[1, 0, 3] = -7
        ids[w.B - 1, 0, 20] = w.n_rows + 3
        d["hash_ids"] = torch.from_numpy(ids).cuda()
    lay = layout(w)
    need = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    stg = eg.engram_forward_staging_bytes(lay, w.B, w.T)
    buf = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, ws=buf[:need], err=err)
    again = forward(w, d, ws=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "a kernel wrote past the workspace"
    assert int(torch.count_nonzero(buf[:need - stg]).item()) == 0, "control words left set"
    assert torch.equal(out, again)
    assert int(err.item()) == (2 if w.M >= 5 else 0)
    sel = np.arange(w.M)
    q, k = w.qk()
    ref = oracle.forward(w.x_tokens(sel), ids.reshape(w.M, -1), w.token_mask().reshape(-1),
                         synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block, host_wkv(w), q, k,
                         eps=w.eps, clamp=w.clamp, scale_format=w.scale_format)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), ref))
    # in place: out is x itself
    x2 = d["x"].clone()
    forward(w, d | {"x": x2}, out=x2, ws=buf[:need])
    torch.cuda.synchronize()
    assert torch.equal(x2, out)
    del d, buf
    torch.cuda.empty_cache()


def test_prepared_forward_equals_forward():
    """prepare_forward (checks once, then calls the entry point with the bound pointers) gives
    the bits of engram_forward, call after call, and still reports an error status."""
    w = CASES[1]
    say(f"[gpu] prepared forward: {w.name}")
    d = synth.device_inputs(w)
    lay = layout(w)
    ws = torch.zeros(eg.engram_forward_workspace_bytes(lay, w.B, w.T), dtype=torch.uint8, device="cuda")
    ref = forward(w, d, ws=ws)
    out = torch.empty_like(d["x"])
    call = eg.prepare_forward(lay, d["x"], d["hash_ids"], d["token_mask"], d["table"], d["scales"],
                              d["wkv"], d["q_weight"], d["k_weight"], out, ws)
    for _ in range(3):
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    with pytest.raises(ValueError):
        eg.prepare_forward(lay, d["x"], d["hash_ids"], d["token_mask"], d["table"], d["scales"],
                           d["wkv"], d["q_weight"], d["k_weight"], out, ws[:256])
    del d, ws
    torch.cuda.empty_cache()


# dim 1024: 5120 wkv rows over 256 workgroups, 20 each (a full 16-row block and four rows)
TWO_BLOCKS = [
    synth.small_variant(synth.workloads()["tiny"], name=f"dim1024_cols{nc}_hd{hd}_b{b}", B=b, T=1, dim=1024,
                        n_cols=nc, head_dim=hd, scale_block=sb, primes=synth.primes_from(1009, nc),
                        hash_dist="zipf", mask_false_frac=0.1, masked_positions=(), outlier_frac=0.05,
                        seed=DECODE.seed + 410 + nc + b)
    for nc, hd, sb, b in [(4, 128, 32, 7), (8, 128, 64, 64), (24, 256, 128, 40)]
]


@pytest.mark.parametrize("w", TWO_BLOCKS, ids=lambda w: w.name)
def test_decode_loop_two_row_blocks(w):
    say(f"[gpu] decode loop, two row blocks per workgroup: {w.name} (K quarter {w.n_cols * w.head_dim // 4})")
    d = synth.device_inputs(w)
    lay = layout(w)
    need = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    buf = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, ws=buf[:need], err=err)
    again = forward(w, d, ws=buf[:need])
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert bool((buf[need:] == 0xA5).all()), "a kernel wrote past the workspace"
    assert int(torch.count_nonzero(buf[:need]).item()) == 0
    assert torch.equal(out, again)
    sel = np.arange(w.M)
    q, k = w.qk()
    ref = oracle.forward(w.x_tokens(sel), w.hash_ids().reshape(w.M, -1), w.token_mask().reshape(-1),
                         synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block, host_wkv(w), q, k,
                         eps=w.eps, clamp=w.clamp, scale_format=w.scale_format)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), ref))
    del d, buf
    torch.cuda.empty_cache()
