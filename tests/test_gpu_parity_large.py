"""HIP path vs the CPU oracle at the largest workload sizes (needs an MI355X with ~210 GB free).

The full-table workload (B=4, T=4096 over a 384,016,682-row table, Zipf ids, closed tokens and
x50 outlier tokens) and the two-instance workloads (two such tables, each with its own wkv and
q/k; instance 2 consumes instance 1's output) run at full size in one call each, as the
benchmark runs them; the oracle evaluates sampled tokens one by one (tokens are independent).
For the chained instance, the oracle's input is the device's output of instance 1 for the same
tokens, so each instance is held to the forward tolerance on its actual input.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

import synth  # noqa: E402
from gpu_common import check_out, forward, oracle_for, say, u16  # noqa: E402

WORKLOADS = synth.workloads()
FULL = WORKLOADS["fulltable_b4_t4096"]
TWO_PREFILL = WORKLOADS["two_instance_t32768"]
TWO_DECODE = WORKLOADS["two_instance_decode_b256"]


def sample_tokens(w, seed, n_random=32):
    """Token ids at tile and sequence boundaries, some closed and outlier tokens, and random ones."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 255, 256, w.M - 1]
    fixed += [b * w.T + t for b in range(w.B) for t in (0, w.T - 1)][:8]
    mask = w.token_mask().reshape(-1)
    closed = np.nonzero(mask == 0)[0][:4]
    outl = np.nonzero(w.outlier_tokens())[0][:6]
    sel = np.concatenate([fixed, closed, outl, rng.integers(0, w.M, n_random)])
    return np.unique(np.asarray(sel, dtype=np.int64) % max(w.M, 1))


def free_device():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_forward_full_table_sampled():
    w = FULL
    say(f"[gpu] forward {w.name}: 98.3 GB table, B={w.B} T={w.T}, sampled tokens")
    d = synth.device_inputs(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = forward(w, d, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    sel = sample_tokens(w, 11)
    got = u16(out).reshape(w.M, w.hc, w.dim)[sel]
    del d, out
    free_device()
    assert w.outlier_tokens()[sel].any() and (w.token_mask().reshape(-1)[sel] == 0).any()
    say("   ", check_out(w, sel, got, oracle_for(w, sel)))


@pytest.fixture(scope="module")
def two_tables():
    """Tables, scales, wkv and q/k of both instances (shared by the prefill and decode
    workloads, which differ only in B and T)."""
    say("[gpu] inputs: two instances, 2 x 101.4 GB of tables")
    insts = []
    for inst in range(2):
        d = synth.device_inputs(TWO_PREFILL, inst=inst)
        d.pop("x")
        d.pop("hash_ids")
        d.pop("token_mask")
        insts.append(d)
    torch.cuda.synchronize()
    yield insts
    insts.clear()
    free_device()


def _two_instance_case(w, tables, seed):
    per_inst = []
    for inst in range(2):
        small = synth.device_inputs(w, inst=inst, with_table=False)
        per_inst.append(tables[inst] | {"hash_ids": small["hash_ids"],
                                        "token_mask": small["token_mask"], "x": small["x"]})
        del small["wkv"]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out1 = forward(w, per_inst[0], err=err)
    out2 = forward(w, per_inst[1] | {"x": out1}, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    sel = sample_tokens(w, seed)
    got1 = u16(out1).reshape(w.M, w.hc, w.dim)[sel]
    got2 = u16(out2).reshape(w.M, w.hc, w.dim)[sel]
    del per_inst, out1, out2
    free_device()
    say("    instance 1:", check_out(w, sel, got1, oracle_for(w, sel, inst=0, keep=2)))
    ref2 = oracle_for(w, sel, inst=1, x_bits=got1, keep=2)
    say("    instance 2:", check_out(w, sel, got2, ref2, x_bits=got1))


def test_forward_two_instance_prefill_sampled(two_tables):
    w = TWO_PREFILL
    say(f"[gpu] forward {w.name}: two chained instances, B={w.B} T={w.T}, sampled tokens")
    _two_instance_case(w, two_tables, 21)


def test_forward_two_instance_decode(two_tables):
    w = TWO_DECODE
    say(f"[gpu] forward {w.name}: two chained instances, B={w.B} T={w.T}, sampled tokens")
    _two_instance_case(w, two_tables, 22)
