"""The four-token-block weight-streaming forward (129..256 tokens, bf16 weights) against the CPU
oracle: the rows are gathered into the staging area, then every workgroup reads its wkv rows once
for all token blocks (copy waves filling a ring of weight stages, eight multiplying waves of 32
tokens each).

The decode layout at 129 (a last block of one token), 200 (out-of-range ids in three blocks, the
output written over x) and 256 tokens, each with a workspace of exactly the reported size followed
by guard bytes, every token checked, control words left zero and a bitwise-identical rerun; E8M0
table scales at 160 tokens; layouts of two row blocks per workgroup (dim 1024: 20 rows, the
last block's slot trimmed to its four rows) with four and eight table columns (four and eight
128-feature stages), and of three (dim 2048: 40 rows, every slot full size).
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
MX = WORKLOADS["decode_b64_mxfp8"]


def run_checked(w, d, **kw):
    """One forward on a workspace of exactly the reported size followed by guard bytes."""
    lay = layout(w)
    need = eg.engram_forward_workspace_bytes(lay, w.B, w.T)
    stg = eg.engram_forward_staging_bytes(lay, w.B, w.T)
    assert stg >= w.M * w.K * 2, "the staged rows need room"
    buf = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, ws=buf[:need], err=err, **kw)
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "a kernel wrote past the workspace"
    assert int(torch.count_nonzero(buf[:need - stg]).item()) == 0, "control words left set"
    return out, buf[:need], int(err.item())


@pytest.mark.parametrize("T", [129, 256])
def test_forward_four_token_blocks_decode_layout(T):
    w = synth.small_variant(DECODE, name=f"decode_dims_b1_t{T}", B=1, T=T, hash_dist="zipf",
                            mask_false_frac=0.1, outlier_frac=0.03, seed=DECODE.seed + 800 + T)
    say(f"[gpu] forward {w.name}: four token blocks in one pass over wkv")
    d = synth.device_inputs(w)
    out, ws, err = run_checked(w, d)
    assert err == 0
    again = forward(w, d, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    sel = np.arange(w.M)
    got = u16(out).reshape(w.M, w.hc, w.dim)
    del d, out, again, ws
    torch.cuda.empty_cache()
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))


def test_forward_four_token_blocks_bad_ids_in_place():
    w = synth.small_variant(DECODE, name="decode_dims_b2_t100", B=2, T=100, hash_dist="zipf",
                            mask_false_frac=0.15, outlier_frac=0.03, seed=DECODE.seed + 810)
    say(f"[gpu] forward {w.name}: out-of-range ids in three token blocks, output over x")
    d = synth.device_inputs(w)
    ids = w.hash_ids()
    ids[0, 5, 0] = -3
    ids[1, 30, 23] = w.n_rows          # token 130
    ids[1, 99, 11] = w.n_rows + 12345  # token 199, the last
    d["hash_ids"] = torch.from_numpy(ids).cuda()
    x_host = w.x_tokens(np.arange(w.M))
    x = d["x"]
    out, _, err = run_checked(w, d, out=x)
    assert out.data_ptr() == x.data_ptr()
    assert err == 3
    mask = w.token_mask().reshape(-1)
    sel = np.arange(w.M)
    got = u16(out).reshape(w.M, w.hc, w.dim)
    del d, out, x
    torch.cuda.empty_cache()
    q, k = w.qk()
    ref = oracle.forward(x_host, ids.reshape(w.M, -1), mask, synth.host_fetch(w), w.n_rows, w.head_dim,
                         w.scale_block, host_wkv(w), q, k, eps=w.eps, clamp=w.clamp, scale_format=w.scale_format)
    say("   ", check_out(w, sel, got, ref))


def test_forward_four_token_blocks_e8m0_scales():
    w = synth.small_variant(MX, name="decode_mxfp8_table_b160", B=160, T=1, mask_false_frac=0.1,
                            seed=MX.seed + 820)
    say(f"[gpu] forward {w.name}: E8M0 table scales, three token blocks")
    d = synth.device_inputs(w)
    out, _, err = run_checked(w, d)
    assert err == 0
    sel = np.arange(w.M)
    got = u16(out).reshape(w.M, w.hc, w.dim)
    del d, out
    torch.cuda.empty_cache()
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))


@pytest.mark.parametrize("dim,nc,T", [(1024, 4, 140), (1024, 8, 256), (2048, 8, 200)])
def test_forward_four_token_blocks_small_layouts(dim, nc, T):
    """dim 1024: 20 rows per workgroup (a full row block and one of four rows, whose slot holds
    only them); dim 2048: 40 rows (two full blocks and one of eight: every slot full size)."""
    w = synth.small_variant(TINY, name=f"dim{dim}_cols{nc}_b1_t{T}", B=1, T=T, dim=dim, n_cols=nc,
                            head_dim=128, scale_block=32, primes=synth.primes_from(1009, nc), hash_dist="zipf",
                            mask_false_frac=0.1, masked_positions=(), outlier_frac=0.05,
                            seed=TINY.seed + 830 + nc + T + dim)
    say(f"[gpu] forward {w.name}: four token blocks, small layout")
    d = synth.device_inputs(w)
    out, _, err = run_checked(w, d)
    assert err == 0
    sel = np.arange(w.M)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), oracle_for(w, sel)))
    del d, out
    torch.cuda.empty_cache()
