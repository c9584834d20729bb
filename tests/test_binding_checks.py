"""The binding's argument checks (CPU, no GPU call): the library takes plain pointers, so every
tensor is checked against the layout before a call.  A wrong shape, size or dtype raises; so do
correctly shaped tensors in host memory (the last check before the library is called)."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import hashed_gram_engram_amd as eg  # noqa: E402
import synth  # noqa: E402

W = synth.workloads()["tiny"]  # hc 4, dim 256, 6 columns of 64 features, 32 per scale
LAY = eg.make_layout(W.hc, W.dim, W.n_cols, W.head_dim, W.scale_block, W.n_rows, W.eps, W.clamp)
B, T = 2, 3
K, N = W.n_cols * W.head_dim, (W.hc + 1) * W.dim


def inputs(**over):
    d = {
        "x": torch.zeros((B, T, W.hc, W.dim), dtype=torch.bfloat16),
        "hash_ids": torch.zeros((B, T, W.n_cols), dtype=torch.int64),
        "token_mask": torch.ones((B, T), dtype=torch.uint8),
        "table": torch.zeros(W.n_rows * W.head_dim, dtype=torch.uint8),
        "scales": torch.zeros((W.n_rows, W.head_dim // W.scale_block), dtype=torch.float32),
        "wkv": torch.zeros((N, K), dtype=torch.bfloat16),
        "q_weight": torch.ones((W.hc, W.dim), dtype=torch.float32),
        "k_weight": torch.ones((W.hc, W.dim), dtype=torch.float32),
    }
    d.update(over)
    return d


def forward(d, **kw):
    return eg.engram_forward(LAY, d["x"], d["hash_ids"], d["token_mask"], d["table"], d["scales"],
                             d["wkv"], d["q_weight"], d["k_weight"], **kw)


def test_forward_well_formed_host_tensors_stop_at_the_device_check():
    with pytest.raises(ValueError, match="must be on a GPU"):
        forward(inputs())


@pytest.mark.parametrize("name,bad,match", [
    ("hash_ids", torch.zeros((B, T, W.n_cols - 1), dtype=torch.int64), "hash_ids"),
    ("x", torch.zeros((B, T, W.hc, W.dim + 8), dtype=torch.bfloat16), "x has shape"),
    ("x", torch.zeros((B * T, W.hc, W.dim), dtype=torch.bfloat16), "x has shape"),
    ("table", torch.zeros(W.n_rows * W.head_dim - 1, dtype=torch.uint8), "table holds"),
    ("scales", torch.zeros((W.n_rows - 1, W.head_dim // W.scale_block), dtype=torch.float32), "scales holds"),
    ("token_mask", torch.ones((B, T + 1), dtype=torch.uint8), "token_mask"),
    ("q_weight", torch.ones((W.hc, W.dim - 1), dtype=torch.float32), "q_weight"),
    ("wkv", torch.zeros((N, K - 32), dtype=torch.bfloat16), "wkv holds"),
])
def test_forward_rejects_a_mismatched_tensor(name, bad, match):
    with pytest.raises(ValueError, match=match):
        forward(inputs(**{name: bad}))


def test_forward_rejects_bad_out_and_err_count():
    d = inputs()
    with pytest.raises(ValueError, match="out has shape"):
        forward(d, out=torch.zeros((B, T, W.hc, W.dim - 1), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out has dtype"):
        forward(d, out=torch.zeros((B, T, W.hc, W.dim), dtype=torch.float32))
    with pytest.raises(TypeError, match="err_count"):
        forward(d, err_count=torch.zeros(1, dtype=torch.int64))


def test_split_path_entry_points_check_their_tensors():
    d = inputs()
    with pytest.raises(ValueError, match="hash_ids"):
        eg.engram_gather_dequant(LAY, d["table"], d["scales"], torch.zeros((B, W.n_cols), dtype=torch.int64))
    with pytest.raises(ValueError, match="emb has shape"):
        eg.engram_gather_dequant(LAY, d["table"], d["scales"], d["hash_ids"],
                                 emb=torch.zeros((B, T, K - 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on a GPU"):
        eg.engram_gather_dequant(LAY, d["table"], d["scales"], d["hash_ids"])
    emb = torch.zeros((B, T, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="emb has shape"):
        eg.engram_kv_proj(LAY, torch.zeros((B, T, K + 64), dtype=torch.bfloat16), d["wkv"])
    with pytest.raises(ValueError, match="kv has shape"):
        eg.engram_kv_proj(LAY, emb, d["wkv"], kv=torch.zeros((B, T, N - 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on a GPU"):
        eg.engram_kv_proj(LAY, emb, d["wkv"])
    kv = torch.zeros((B, T, N), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="kv has shape"):
        eg.engram_gate_apply(LAY, d["x"], kv[:, :, :-256].contiguous(), d["q_weight"], d["k_weight"])
    with pytest.raises(ValueError, match="gate has shape"):
        eg.engram_gate_apply(LAY, d["x"], kv, d["q_weight"], d["k_weight"],
                             gate=torch.zeros((B, T), dtype=torch.float32))
    with pytest.raises(ValueError, match="must be on a GPU"):
        eg.engram_gate_apply(LAY, d["x"], kv, d["q_weight"], d["k_weight"], d["token_mask"])


def test_hash_entry_point_checks_its_tensors():
    h = synth.hash_inputs(34, 2, 5, n_layers=2)
    hl = eg.make_hash_layout(h["n_layers"], h["max_ngram"], h["n_heads"], h["pad_id"], h["vocab"], 8)
    args = dict(token_map=torch.from_numpy(np.ascontiguousarray(h["token_map"])).view(torch.int32),
                multipliers=torch.from_numpy(h["multipliers"]), primes=torch.from_numpy(h["primes"]),
                offsets=torch.from_numpy(h["offsets"]), input_ids=torch.from_numpy(h["input_ids"]),
                history=torch.zeros((2, 8), dtype=torch.int64))
    with pytest.raises(ValueError, match="must be on a GPU"):
        eg.engram_hash_ids(hl, **args)
    with pytest.raises(ValueError, match="primes has shape"):
        eg.engram_hash_ids(hl, **(args | {"primes": args["primes"][:, :2].contiguous()}))
    with pytest.raises(ValueError, match="history has shape"):
        eg.engram_hash_ids(hl, **(args | {"history": torch.zeros((2, 7), dtype=torch.int64)}))
    with pytest.raises(ValueError, match="token_map has shape"):
        eg.engram_hash_ids(hl, **(args | {"token_map": args["token_map"][:-1].contiguous()}))


def test_default_workspace_is_one_per_device_and_stream():
    """Calls on different streams may overlap in time and so must not share a workspace: the
    binding keeps one per (device, stream); the same pair gets the same one back."""
    saved = dict(eg._default_ws)
    eg._default_ws.clear()
    try:
        a = eg.workspace_for(0, 0x1000)
        assert eg.workspace_for(0, 0x1000) is a
        b = eg.workspace_for(0, 0x2000)
        c = eg.workspace_for(1, 0x1000)
        assert b is not a and c is not a and c is not b
        assert a.buf is None  # nothing is allocated before the first call
        eg.release_default_workspaces()
        assert not eg._default_ws
    finally:
        eg._default_ws.clear()
        eg._default_ws.update(saved)


def test_forward_check_validates_before_touching_the_device():
    lib = eg._lib
    assert lib.engram_forward_check(None, 256, None) == -1            # NULL workspace
    buf = (ctypes.c_uint8 * 64)()
    off = (16 - ctypes.addressof(buf) % 16) % 16
    assert lib.engram_forward_check(ctypes.c_void_p(ctypes.addressof(buf) + off + 1), 32, None) == -5
    assert lib.engram_forward_check(ctypes.c_void_p(ctypes.addressof(buf) + off), 2, None) == -5
    assert eg.STATUS[-8] == "timeout" and eg.ENGRAM_E_TIMEOUT == -8
    assert "timed out" in lib.engram_status_str(-8).decode()


def test_spin_budget_setter_returns_the_previous_bound():
    old = eg.engram_set_spin_budget(7)
    try:
        assert eg.engram_set_spin_budget(9) == 7
        assert eg.engram_set_spin_budget(0) == 9          # 0 restores the default ...
        assert eg.engram_set_spin_budget(0) == 1 << 22    # ... 2^22 polls
    finally:
        eg.engram_set_spin_budget(old)
