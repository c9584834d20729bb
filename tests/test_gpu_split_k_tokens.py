"""Token counts above one token block against the CPU oracle, on the schedules that take them.

The decode layout at 129..256 tokens: 256, 193 (a last 64-token block of one token), 150, which the
four-token-block weight-streaming kernel takes on this layout; skewed ids, closed tokens, outlier
streams, out-of-range ids, in-place output.  The same checks at 65 and 128 tokens (the
two-token-block kernel).  Split K in the tiled schedule at tiny dims and 13,300 tokens: 260 tiles
of 256 x 256, the last 4 (tiles mod the CU count; value tiles of the last four token blocks, the
ragged one among them) computed by two workgroups each over half of K (the second adds the
first one's fp32 partial tile), every token checked.  Every result is also checked for
run-to-run identity, control words left zero and no timed-out wait.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import hashed_gram_engram_amd as eg  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_common import check_out, forward, host_wkv, layout, oracle_for, say, u16  # noqa: E402

DECODE = synth.workloads()["decode_b64"]
TINY = synth.workloads()["tiny"]


def variant(B, T, seed):
    return synth.small_variant(DECODE, name=f"decode_dims_b{B}_t{T}", B=B, T=T, hash_dist="zipf",
                               mask_false_frac=0.15, outlier_frac=0.03, seed=DECODE.seed + seed)


def boundary_tokens(w, seed, n_random=24):
    """Tokens at every 16- and 64-token boundary, closed and outlier tokens, and random ones."""
    rng = np.random.default_rng(seed)
    fixed = [t for b in range(0, w.M, 64) for t in (b, b + 15, b + 16, b + 63)]
    mask = w.token_mask().reshape(-1)
    fixed += list(np.nonzero(mask == 0)[0][:4]) + list(np.nonzero(w.outlier_tokens())[0][:4])
    sel = np.concatenate([np.asarray(fixed, dtype=np.int64), rng.integers(0, w.M, n_random), [w.M - 1]])
    return np.unique(sel[sel < w.M])


def run_twice(w, d, err=None):
    lay = layout(w)
    ws = torch.zeros(eg.engram_forward_workspace_bytes(lay, w.B, w.T), dtype=torch.uint8, device="cuda")
    ctrl = ws.numel() - eg.engram_forward_staging_bytes(lay, w.B, w.T)
    assert ctrl > 0
    a = forward(w, d, ws=ws, err=err)
    b = forward(w, d, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "two runs differ"
    # word 0 counts timed-out waits; every control word (in front of the staging area) is left zero
    assert int(torch.count_nonzero(ws[:ctrl]).item()) == 0
    return a


@pytest.mark.parametrize("B,T,seed", [(4, 64, 501), (1, 193, 502), (1, 65, 503), (2, 64, 504)])
def test_forward_split_k_sampled(B, T, seed):
    w = variant(B, T, seed)
    say(f"[gpu] forward {w.name}: {w.M} tokens, " + ("split-K tiles" if w.M > 128 else "two token blocks"))
    d = synth.device_inputs(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_twice(w, d, err=err)
    assert int(err.item()) == 0
    sel = boundary_tokens(w, seed)
    got = u16(out).reshape(w.M, w.hc, w.dim)[sel]
    del d, out
    torch.cuda.empty_cache()
    say("   ", len(sel), "tokens:", check_out(w, sel, got, oracle_for(w, sel)))


def test_forward_split_k_bad_ids_in_place():
    w = variant(1, 150, 505)
    say(f"[gpu] forward {w.name}: out-of-range ids in blocks 0 and 2, output over x")
    d = synth.device_inputs(w)
    ids = w.hash_ids()
    ids[0, 3, 5] = -7
    ids[0, 140, 23] = w.n_rows
    d["hash_ids"] = torch.from_numpy(ids).cuda()
    x_host = w.x_tokens(np.arange(w.M))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = d["x"]
    out = forward(w, d, out=x, err=err)
    torch.cuda.synchronize()
    assert out.data_ptr() == x.data_ptr()
    assert int(err.item()) == 2
    sel = np.unique(np.concatenate([[0, 3, 63, 64, 127, 128, 140, 149], np.nonzero(w.token_mask().reshape(-1) == 0)[0][:4]]))
    got = u16(out).reshape(w.M, w.hc, w.dim)[sel]
    del d, out, x
    torch.cuda.empty_cache()
    q, k = w.qk()
    ref = oracle.forward(x_host[sel], ids.reshape(w.M, -1)[sel], w.token_mask().reshape(-1)[sel],
                         synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block, host_wkv(w), q, k,
                         eps=w.eps, clamp=w.clamp, scale_format=w.scale_format)
    say("   ", check_out(w, sel, got, ref))


def test_forward_last_round_split_tiny_dims():
    w = synth.small_variant(TINY, name="tiny_dims_b1_t13300", B=1, T=13300, hash_dist="zipf",
                            mask_false_frac=0.1, outlier_frac=0.02, masked_positions=(),
                            seed=TINY.seed + 506)
    n_tiles = -(-w.M // 256) * (w.N // 256)
    assert n_tiles == 260  # 256 CUs: one full round, then 4 tiles split over K
    say(f"[gpu] forward {w.name}: {n_tiles} tiles, the last {n_tiles % 256} split over K")
    d = synth.device_inputs(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_twice(w, d, err=err)
    assert int(err.item()) == 0
    sel = np.arange(w.M)
    got = u16(out).reshape(w.M, w.hc, w.dim)
    del d, out
    torch.cuda.empty_cache()
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))
