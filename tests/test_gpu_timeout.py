"""A cross-workgroup wait that gives up reaches the caller (needs an MI355X).

The host sets a tiny wait bound (engram_set_spin_budget), so the fused schedules' waits give up
while every kernel still runs to its end; engram_forward_check must then report
ENGRAM_E_TIMEOUT and leave the workspace zero-filled, and the next call with the default bound
must give the same bits as a call before the time-outs.  Covered: the weight-streaming schedule
(gates handed to the apply workgroups), the two-token-block kernel at 100 tokens and the
four-token-block kernel at 150 tokens (gates and value tiles of two and three blocks handed to
the apply workgroups), and the tiled schedule at 300 tokens (gates handed between tiles)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from gpu_common import eg, forward, layout, say  # noqa: E402

DECODE = synth.workloads()["decode_b64"]
CASES = [synth.small_variant(DECODE, name="decode_dims_b64", B=64, T=1),
         synth.small_variant(DECODE, name="decode_dims_b1_t100", B=1, T=100, seed=DECODE.seed + 300),
         synth.small_variant(DECODE, name="decode_dims_b1_t150", B=1, T=150, seed=DECODE.seed + 301),
         synth.small_variant(DECODE, name="decode_dims_b1_t300", B=1, T=300, seed=DECODE.seed + 302)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_timed_out_wait_is_reported_and_the_workspace_cleared(w):
    say(f"[gpu] wait time-out reported: {w.name} ({w.M} tokens)")
    d = synth.device_inputs(w)
    lay = layout(w)
    ws = torch.zeros(eg.engram_forward_workspace_bytes(lay, w.B, w.T), dtype=torch.uint8,
                     device="cuda")
    good = forward(w, d, ws=ws)                  # default bound: checked, no time-out
    old = eg.engram_set_spin_budget(1)
    try:
        forward(w, d, ws=ws, check=False)
        with pytest.raises(eg.EngramError) as e:
            eg.engram_forward_check(ws)
        assert e.value.status == eg.ENGRAM_E_TIMEOUT
    finally:
        eg.engram_set_spin_budget(old)
    assert int(torch.count_nonzero(ws).item()) == 0   # cleared by the check
    again = forward(w, d, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, good)
    del d, ws
    torch.cuda.empty_cache()
