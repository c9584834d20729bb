"""The two-token-block weight-streaming forward (65..128 tokens, bf16 weights) against the CPU
oracle: every workgroup reads its wkv rows once for both 64-token blocks.

The decode layout (seven row blocks per workgroup) at a ragged second block with out-of-range ids
in both blocks and the output written over x; a small layout where every workgroup owns one row
block (dim 320) and one where 16 workgroups own two and the rest one (dim 832: 1040 groups of
four rows over 256 workgroups), each with a workspace of exactly the reported size followed by
guard bytes, every token checked, control words left zero, and the in-place result identical;
fp32 scales per 32, 64 and 256 features at the decode layout (the scale gathers per chunk: two,
one, or one kept across a column's chunks); and one workspace shared in turn with the
four-token-block and one-block schedules of the decode layout.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_common import check_out, eg, forward, host_wkv, layout, oracle_for, say, u16  # noqa: E402

WORKLOADS = synth.workloads()
TINY = WORKLOADS["tiny"]
DECODE = WORKLOADS["decode_b64"]


def small_layout(dim, T, seed):
    return synth.small_variant(TINY, name=f"dim{dim}_b1_t{T}", B=1, T=T, dim=dim, n_cols=4,
                               head_dim=128, scale_block=32, primes=synth.primes_from(1009, 4),
                               hash_dist="zipf", mask_false_frac=0.1, masked_positions=(),
                               outlier_frac=0.05, seed=TINY.seed + seed)


@pytest.mark.parametrize("dim,T", [(320, 100), (832, 65), (832, 128)])
def test_forward_two_token_blocks_small_layouts(dim, T):
    w = small_layout(dim, T, 700 + dim + T)
    say(f"[gpu] forward {w.name}: two token blocks in one pass over wkv")
    lay = layout(w)
    d = synth.device_inputs(w)
    need = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    buf = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, ws=buf[:need], err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert bool((buf[need:] == 0xA5).all()), "a kernel wrote past the workspace"
    assert int(torch.count_nonzero(buf[:need]).item()) == 0
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
    x2 = d["x"].clone()
    forward(w, d | {"x": x2}, out=x2, ws=buf[:need])
    torch.cuda.synchronize()
    assert torch.equal(x2, out)
    assert int(torch.count_nonzero(buf[:need]).item()) == 0


@pytest.mark.parametrize("sb", [32, 64, 256])
def test_forward_two_token_blocks_scale_widths(sb):
    """fp32 scales per 32 features (two scale gathers per chunk), per 64 (one, a fresh word every
    chunk) and per 256 (one word for the four chunks of a column, kept across them), at 100
    tokens of the decode layout, every token checked."""
    w = synth.small_variant(DECODE, name=f"decode_dims_sb{sb}_t100", B=1, T=100, scale_block=sb,
                            hash_dist="zipf", mask_false_frac=0.1, seed=DECODE.seed + 730 + sb)
    say(f"[gpu] forward {w.name}: two token blocks, fp32 scales per {sb} features")
    d = synth.device_inputs(w)
    out = forward(w, d)
    torch.cuda.synchronize()
    sel = np.arange(w.M)
    got = u16(out).reshape(w.M, w.hc, w.dim)
    del d, out
    torch.cuda.empty_cache()
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))


def test_forward_two_token_blocks_decode_bad_ids_in_place():
    w = synth.small_variant(DECODE, name="decode_dims_b1_t100", B=1, T=100, hash_dist="zipf",
                            mask_false_frac=0.15, outlier_frac=0.03, seed=DECODE.seed + 710)
    say(f"[gpu] forward {w.name}: out-of-range ids in both token blocks, output over x")
    d = synth.device_inputs(w)
    ids = w.hash_ids()
    ids[0, 5, 0] = -3
    ids[0, 70, 23] = w.n_rows
    ids[0, 99, 11] = w.n_rows + 12345
    d["hash_ids"] = torch.from_numpy(ids).cuda()
    x_host = w.x_tokens(np.arange(w.M))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = d["x"]
    out = forward(w, d, out=x, err=err)
    torch.cuda.synchronize()
    assert out.data_ptr() == x.data_ptr()
    assert int(err.item()) == 3
    mask = w.token_mask().reshape(-1)
    sel = np.unique(np.concatenate([[0, 5, 15, 16, 63, 64, 70, 80, 99], np.nonzero(mask == 0)[0][:4]]))
    got = u16(out).reshape(w.M, w.hc, w.dim)[sel]
    del d, out, x
    torch.cuda.empty_cache()
    q, k = w.qk()
    ref = oracle.forward(x_host[sel], ids.reshape(w.M, -1)[sel], mask[sel], synth.host_fetch(w), w.n_rows,
                         w.head_dim, w.scale_block, host_wkv(w), q, k, eps=w.eps, clamp=w.clamp,
                         scale_format=w.scale_format)
    say("   ", check_out(w, sel, got, ref))


def test_workspace_shared_with_the_other_decode_schedules():
    """One workspace for 150 tokens (four token blocks: staged rows behind the control words), 100
    (two token blocks) and 64 (one token block) of the decode layout, twice in turn:
    every control word zero after each call, every result equal to a call on a fresh workspace."""
    w150 = synth.small_variant(DECODE, name="decode_dims_b150", B=150, T=1, seed=DECODE.seed + 720)
    say("[gpu] one workspace for the tiled, two-block and one-block schedules at the decode layout")
    d = synth.device_inputs(w150)
    lay = layout(w150)
    cases = []
    for n in (150, 100, 64):
        w = synth.small_variant(w150, name=f"decode_dims_b{n}", B=n)
        dn = dict(d)
        for k in ("x", "hash_ids", "token_mask"):
            dn[k] = d[k][:n].contiguous()
        cases.append((w, dn))
    sizes = [eg.engram_forward_workspace_bytes(lay, w.B, w.T) for w, _ in cases]
    n_ws = max(sizes)
    ctrl = n_ws - max(eg.engram_forward_staging_bytes(lay, w.B, w.T) for w, _ in cases)
    assert eg.engram_forward_staging_bytes(lay, 100, 1) == 0 and eg.engram_forward_staging_bytes(lay, 64, 1) == 0
    ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    outs = []
    for w, dn in cases + cases:
        outs.append(forward(w, dn, ws=ws))
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:ctrl]).item()) == 0, w.name
    for i, (w, dn) in enumerate(cases):
        fresh = forward(w, dn, ws=torch.zeros_like(ws))
        torch.cuda.synchronize()
        assert torch.equal(outs[i], fresh) and torch.equal(outs[i + 3], fresh), w.name
    del d, cases, outs, ws
    torch.cuda.empty_cache()
