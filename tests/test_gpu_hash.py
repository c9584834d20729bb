"""Hash step on the device (engram_hash_ids) vs the oracle: bit-exact row ids and history, chunked
calls over one sequence, dead spans and out-of-map ids, and the row ids driving engram_forward."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_common import check_out, eg, forward, layout, say, u16, host_wkv  # noqa: E402


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def run_hash(h, ids, mask, history, start_pos=0, err=None):
    hl = eg.make_hash_layout(h["n_layers"], h["max_ngram"], h["n_heads"], h["pad_id"], h["vocab"],
                             history.shape[1])
    return eg.engram_hash_ids(hl, dev(h["token_map"], torch.int32), dev(h["multipliers"]),
                              dev(h["primes"]), dev(h["offsets"]), dev(ids), history,
                              start_pos=start_pos, token_mask=None if mask is None else dev(mask),
                              err_count=err)


def oracle_hash(h, ids, mask, hist, start_pos=0):
    return oracle.hash_ids(ids, h["token_map"].astype(np.int64), h["multipliers"], h["primes"],
                           h["offsets"], h["pad_id"], hist, start_pos=start_pos, token_mask=mask)


def test_hash_ids_match_oracle_with_dead_spans():
    say("[gpu] hash ids: B=3, L=300, 2 layers, dead spans")
    h = synth.hash_inputs(31, 3, 300, span_frac=0.02, span_len=9)
    hist = torch.zeros((3, 300), dtype=torch.int64, device="cuda")
    out = run_hash(h, h["input_ids"], h["token_mask"], hist)
    torch.cuda.synchronize()
    ref_hist = np.zeros((3, 300), dtype=np.int64)
    ref = oracle_hash(h, h["input_ids"], h["token_mask"], ref_hist)          # [B, L, layers, C]
    assert np.array_equal(out.cpu().numpy(), ref.transpose(2, 0, 1, 3))
    assert np.array_equal(hist.cpu().numpy(), ref_hist)
    assert (h["token_mask"] == 0).any()


def test_hash_ids_chunked_calls_equal_one_call():
    say("[gpu] hash ids: one sequence in chunks of 100, 1 and 199 positions (history)")
    h = synth.hash_inputs(32, 2, 300, span_frac=0.02, span_len=5)
    ids, mask = h["input_ids"], h["token_mask"]
    hist = torch.zeros((2, 512), dtype=torch.int64, device="cuda")
    parts = [run_hash(h, ids[:, a:b], mask[:, a:b], hist, start_pos=a).clone()
             for a, b in ((0, 100), (100, 101), (101, 300))]
    torch.cuda.synchronize()
    got = torch.cat(parts, dim=2).cpu().numpy()
    ref_hist = np.zeros((2, 512), dtype=np.int64)
    ref = oracle_hash(h, ids, mask, ref_hist)
    assert np.array_equal(got, ref.transpose(2, 0, 1, 3))
    assert np.array_equal(hist.cpu().numpy()[:, :300], ref_hist[:, :300])


def test_hash_ids_out_of_map_ids_are_dead_and_counted():
    say("[gpu] hash ids: ids outside the token map")
    h = synth.hash_inputs(33, 2, 64)
    ids = h["input_ids"].copy()
    ids[0, 5] = -7
    ids[1, 63] = h["vocab"]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hist = torch.zeros((2, 64), dtype=torch.int64, device="cuda")
    out = run_hash(h, ids, None, hist, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    # reading: an id outside the map takes no part in an n-gram, like a masked token
    mask = np.ones(ids.shape, dtype=np.uint8)
    mask[0, 5] = mask[1, 63] = 0
    ok = ids.copy()
    ok[0, 5] = ok[1, 63] = 0
    ref = oracle_hash(h, ok, mask, np.zeros((2, 64), dtype=np.int64))
    assert np.array_equal(out.cpu().numpy(), ref.transpose(2, 0, 1, 3))


def test_hash_ids_drive_the_forward():
    say("[gpu] hash ids -> engram_forward (decode dims, a 24-range table of ~1000-row primes)")
    base = synth.get("decode_b64")
    w = synth.small_variant(base, name="decode_dims_hashed", B=2, T=37,
                            primes=synth.primes_from(1009, 24), seed=base.seed + 500)
    h = synth.hash_inputs(34, w.B, w.T, n_layers=1, primes=[w.primes], span_frac=0.03,
                          span_len=3)
    hist = torch.zeros((w.B, w.T), dtype=torch.int64, device="cuda")
    hid = run_hash(h, h["input_ids"], h["token_mask"], hist)
    d = synth.device_inputs(w)
    d["hash_ids"] = hid[0]          # layer 0: a contiguous [B, T, 24] slice
    out = forward(w, d)
    torch.cuda.synchronize()
    ids = oracle_hash(h, h["input_ids"], h["token_mask"], np.zeros((w.B, w.T), np.int64))[:, :, 0]
    assert ids.min() >= 0 and ids.max() < w.n_rows
    q, k = w.qk()
    sel = np.arange(w.M)
    ref = oracle.forward(w.x_tokens(sel), ids.reshape(w.M, -1), w.token_mask().reshape(-1),
                         synth.host_fetch(w), w.n_rows, w.head_dim, w.scale_block, host_wkv(w), q, k)
    say("   ", check_out(w, sel, u16(out).reshape(w.M, w.hc, w.dim), ref))
