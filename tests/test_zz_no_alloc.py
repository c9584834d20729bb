"""engram_forward_noalloc: the forward with the library's fixed per-GPU scratch array as its
workspace, for callers that cannot allocate (needs an MI355X).

It must give engram_forward's output bit for bit (the same kernels): two calls in a row, the
second on fewer tokens, at the model's layout (the one-token-block weight-streaming schedule, and
the two-token-block one at 100 then 65 tokens) and at tiny dims; a call whose workspace would
exceed the scratch (200 tokens at the model's layout, tiled schedule) is refused before anything
is enqueued."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from gpu_common import eg, forward, layout, say  # noqa: E402

W = synth.workloads()
DECODE, TINY = W["decode_b64"], W["tiny"]
DECODE_B100 = synth.small_variant(DECODE, name="decode_dims_b100", B=100, T=1)


def _slice(d, n):
    """The first n tokens of a [B, 1, ...] (or [1, T, ...]) input set, as contiguous tensors."""
    out = dict(d)
    if d["x"].shape[1] == 1:
        out["x"] = d["x"][:n].contiguous()
        out["hash_ids"] = d["hash_ids"][:n].contiguous()
        out["token_mask"] = d["token_mask"][:n].contiguous()
    else:
        out["x"] = d["x"][:, :n].contiguous()
        out["hash_ids"] = d["hash_ids"][:, :n].contiguous()
        out["token_mask"] = d["token_mask"][:, :n].contiguous()
    return out


def _noalloc(w, d, err=None):
    out = torch.empty_like(d["x"])
    return eg.engram_forward_noalloc(layout(w), d["x"], d["hash_ids"], d["token_mask"], d["table"],
                                     d["scales"], d["wkv"], d["q_weight"], d["k_weight"], out,
                                     err_count=err)


@pytest.mark.parametrize("w,n2", [(DECODE, 17), (DECODE_B100, 65), (TINY, 5)],
                         ids=["decode_b64_then_17", "decode_b100_then_65", "tiny_t16_then_5"])
def test_noalloc_equals_forward_two_calls_second_smaller(w, n2):
    say(f"[gpu] no-allocation forward: {w.name} ({w.M} tokens), then {n2} tokens")
    d = synth.device_inputs(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for dd in (d, _slice(d, n2)):
        ref = forward(w, dd)
        got = _noalloc(w, dd, err)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), int((got != ref).sum().item())
    assert int(err.item()) == 0
    del d
    torch.cuda.empty_cache()


def test_noalloc_refuses_calls_beyond_its_scratch():
    say("[gpu] no-allocation forward refuses 200 tokens at the model's layout (tiled schedule)")
    w = synth.small_variant(DECODE, name="decode_dims_b200", B=200, T=1)
    d = synth.device_inputs(w)
    out = torch.full_like(d["x"], 7)
    with pytest.raises(eg.EngramError) as e:
        eg.engram_forward_noalloc(layout(w), d["x"], d["hash_ids"], d["token_mask"], d["table"],
                                  d["scales"], d["wkv"], d["q_weight"], d["k_weight"], out)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((out == 7).all())   # nothing ran
    del d
    torch.cuda.empty_cache()
