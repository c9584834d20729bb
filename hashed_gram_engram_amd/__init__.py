"""Python binding of libengram.so, the MI355X (gfx950) Engram forward library.

The functions here carry the C ABI's names (include/engram.h) and only marshal arguments:
torch tensors provide device memory, the current torch stream provides the HIP stream, and
every step of the computation runs in the library's HIP kernels.  If the shared library is
missing, importing the binding raises: there is no fallback path.
"""
from __future__ import annotations

import atexit
import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

ENGRAM_OK = 0
ENGRAM_E_TIMEOUT = -8
STATUS = {0: "ok", -1: "null pointer", -2: "layout", -3: "shape", -4: "alignment",
          -5: "workspace", -6: "hip", -7: "device", -8: "timeout"}


class EngramLayout(ctypes.Structure):
    _fields_ = [("hc", ctypes.c_int32), ("dim", ctypes.c_int32), ("n_cols", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("scale_block", ctypes.c_int32),
                ("scale_format", ctypes.c_int32), ("wkv_format", ctypes.c_int32),
                ("n_rows", ctypes.c_int64), ("eps", ctypes.c_float), ("clamp", ctypes.c_float)]


class HashLayout(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("max_ngram", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("pad_id", ctypes.c_int32), ("vocab", ctypes.c_int64),
                ("history_len", ctypes.c_int64)]


class EngramError(RuntimeError):
    def __init__(self, where: str, status: int):
        msg = _lib.engram_status_str(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_LP = ctypes.POINTER(EngramLayout)
_lib.engram_status_str.restype = ctypes.c_char_p
_lib.engram_status_str.argtypes = [ctypes.c_int]
_lib.engram_layout_check.argtypes = [_LP]
_lib.engram_param_counts.argtypes = [_LP, ctypes.POINTER(ctypes.c_int64)]
_lib.engram_forward_workspace_bytes.argtypes = [_LP, _i64, _i64]
_lib.engram_forward_workspace_bytes.restype = _sz
_lib.engram_forward_staging_bytes.argtypes = [_LP, _i64, _i64]
_lib.engram_forward_staging_bytes.restype = _sz
_lib.engram_gather_dequant.argtypes = [_LP, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp]
_lib.engram_kv_proj.argtypes = [_LP, _vp, _vp, _i64, _i64, _vp, _vp]
_lib.engram_gate_apply.argtypes = [_LP, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp]
_lib.engram_forward.argtypes = [_LP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                                _sz, _vp, _vp]
_lib.engram_hash_ids.argtypes = [ctypes.POINTER(HashLayout), _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                 _i64, _i64, _vp, _vp, _vp, _vp]
_lib.engram_forward_noalloc.argtypes = [_LP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp]
_lib.engram_forward_noalloc.restype = ctypes.c_int
_lib.engram_forward_check.argtypes = [_vp, _sz, _vp]
_lib.engram_set_spin_budget.argtypes = [ctypes.c_uint32]
_lib.engram_set_spin_budget.restype = ctypes.c_uint32
for _f in (_lib.engram_layout_check, _lib.engram_param_counts, _lib.engram_gather_dequant,
           _lib.engram_kv_proj, _lib.engram_gate_apply, _lib.engram_forward, _lib.engram_hash_ids,
           _lib.engram_forward_check):
    _f.restype = ctypes.c_int

EXPORTED = ["engram_layout_check", "engram_param_counts", "engram_forward_workspace_bytes",
            "engram_forward_staging_bytes",
            "engram_gather_dequant", "engram_kv_proj", "engram_gate_apply", "engram_forward",
            "engram_hash_ids", "engram_status_str", "engram_forward_check", "engram_set_spin_budget",
            "engram_forward_noalloc"]


SCALE_FP32, SCALE_E8M0 = 0, 1  # engram_scale_format
WKV_BF16, WKV_MXFP8 = 0, 1     # engram_wkv_format


def make_layout(hc: int, dim: int, n_cols: int, head_dim: int, scale_block: int, n_rows: int,
                eps: float = 1e-20, clamp: float = 1e-6, scale_format: int = SCALE_FP32,
                wkv_format: int = WKV_BF16) -> EngramLayout:
    return EngramLayout(hc, dim, n_cols, head_dim, scale_block, scale_format, wkv_format, n_rows,
                        eps, clamp)


def wkv_bytes(layout: EngramLayout) -> int:
    """Bytes of the wkv argument: N x K bf16, or for MXFP8 the codes [N, K] followed by the
    E8M0 scales [N, K / 32] in one uint8 buffer."""
    n, k = (layout.hc + 1) * layout.dim, layout.n_cols * layout.head_dim
    return n * k + n * (k // 32) if layout.wkv_format == WKV_MXFP8 else 2 * n * k


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(where: str, st: int):
    if st != ENGRAM_OK:
        raise EngramError(where, st)


def _contig(name: str, t: torch.Tensor, dtype=None) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


_BF16 = (torch.bfloat16, torch.int16)


# The library takes plain pointers and cannot see buffer sizes: every tensor's shape (or size) is
# checked here against the layout, so that a mismatch raises instead of reading or writing past
# a buffer on the device.
def _shape(name: str, t: torch.Tensor, shape: tuple):
    if t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _numel(name: str, t: torch.Tensor, shape: tuple):
    """t holds exactly the elements of `shape` (in any shape: the library sees a flat buffer)."""
    need = math.prod(shape)
    if t.numel() != need:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {need} elements {tuple(shape)}")


def _nbytes(name: str, t: torch.Tensor, need: int, exact: bool = True):
    have = t.numel() * t.element_size()
    if (have != need) if exact else (have < need):
        raise ValueError(f"{name} holds {have} bytes, expected {'' if exact else 'at least '}{need}")


def _same_device(ref: torch.Tensor, **ts):
    dev = ref.device
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")
    for name, t in ts.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _dims(layout: EngramLayout):
    """(K, N, scale bytes per table row) of a layout."""
    k, n = layout.n_cols * layout.head_dim, (layout.hc + 1) * layout.dim
    nb = layout.head_dim // layout.scale_block if layout.scale_block > 0 else 0
    return k, n, nb * (1 if layout.scale_format == SCALE_E8M0 else 4)


def _check_table(layout: EngramLayout, table: torch.Tensor, scales: torch.Tensor):
    _, _, sbytes = _dims(layout)
    _nbytes("table", table, layout.n_rows * layout.head_dim, exact=False)
    _nbytes("scales", scales, layout.n_rows * sbytes, exact=False)


def _check_err(err_count: Optional[torch.Tensor]):
    if err_count is not None:
        _contig("err_count", err_count, torch.int32)
        if err_count.numel() < 1:
            raise ValueError("err_count needs one int32")


def _check_wkv(layout: EngramLayout, wkv: torch.Tensor):
    _contig("wkv", wkv, torch.uint8 if layout.wkv_format == WKV_MXFP8 else _BF16)
    if wkv.numel() * wkv.element_size() != wkv_bytes(layout):
        raise ValueError(f"wkv holds {wkv.numel() * wkv.element_size()} bytes, the layout needs "
                         f"{wkv_bytes(layout)}")


def engram_layout_check(layout: EngramLayout) -> int:
    return _lib.engram_layout_check(ctypes.byref(layout))


def engram_param_counts(layout: EngramLayout):
    out = (ctypes.c_int64 * 3)()
    _check("engram_param_counts", _lib.engram_param_counts(ctypes.byref(layout), out))
    return int(out[0]), int(out[1]), int(out[2])


def engram_forward_workspace_bytes(layout: EngramLayout, B: int, T: int) -> int:
    return int(_lib.engram_forward_workspace_bytes(ctypes.byref(layout), B, T))


def engram_forward_staging_bytes(layout: EngramLayout, B: int, T: int) -> int:
    return int(_lib.engram_forward_staging_bytes(ctypes.byref(layout), B, T))


def engram_gather_dequant(layout: EngramLayout, table: torch.Tensor, scales: torch.Tensor,
                          hash_ids: torch.Tensor, emb: Optional[torch.Tensor] = None,
                          err_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """emb [B, T, n_cols * head_dim] bf16 from hash_ids [B, T, n_cols] int64."""
    if hash_ids.dim() != 3:
        raise ValueError(f"hash_ids has shape {tuple(hash_ids.shape)}, expected [B, T, n_cols]")
    B, T, C = hash_ids.shape
    _shape("hash_ids", hash_ids, (B, T, layout.n_cols))
    _contig("hash_ids", hash_ids, torch.int64)
    _contig("table", table, torch.uint8)
    _contig("scales", scales, torch.uint8 if layout.scale_format == SCALE_E8M0 else torch.float32)
    _check_table(layout, table, scales)
    _check_err(err_count)
    if emb is None:
        emb = torch.empty((B, T, C * layout.head_dim), dtype=torch.bfloat16, device=hash_ids.device)
    _numel("emb", emb, (B, T, C * layout.head_dim))
    _contig("emb", emb, _BF16)
    _same_device(hash_ids, table=table, scales=scales, emb=emb, err_count=err_count)
    _check("engram_gather_dequant", _lib.engram_gather_dequant(
        ctypes.byref(layout), _ptr(table), _ptr(scales), _ptr(hash_ids), B, T, _ptr(emb),
        _ptr(err_count), _stream()))
    return emb


def engram_kv_proj(layout: EngramLayout, emb: torch.Tensor, wkv: torch.Tensor,
                   kv: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kv [B, T, (hc + 1) * dim] bf16 = emb @ wkv^T (wkv in the layout's wkv_format)."""
    if emb.dim() != 3:
        raise ValueError(f"emb has shape {tuple(emb.shape)}, expected [B, T, n_cols * head_dim]")
    B, T, _ = emb.shape
    K, N, _ = _dims(layout)
    _shape("emb", emb, (B, T, K))
    _contig("emb", emb, _BF16)
    _check_wkv(layout, wkv)
    if kv is None:
        kv = torch.empty((B, T, N), dtype=torch.bfloat16, device=emb.device)
    _numel("kv", kv, (B, T, N))
    _contig("kv", kv, _BF16)
    _same_device(emb, wkv=wkv, kv=kv)
    _check("engram_kv_proj", _lib.engram_kv_proj(ctypes.byref(layout), _ptr(emb), _ptr(wkv), B, T,
                                                 _ptr(kv), _stream()))
    return kv


def make_hash_layout(n_layers: int, max_ngram: int, n_heads: int, pad_id: int, vocab: int,
                     history_len: int) -> HashLayout:
    return HashLayout(n_layers, max_ngram, n_heads, pad_id, vocab, history_len)


def engram_hash_ids(layout: HashLayout, token_map: torch.Tensor, multipliers: torch.Tensor,
                    primes: torch.Tensor, offsets: torch.Tensor, input_ids: torch.Tensor,
                    history: torch.Tensor, start_pos: int = 0,
                    token_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    err_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row ids [n_layers, B, L, (max_ngram - 1) * n_heads] int64 of tokens input_ids [B, L] at
    positions start_pos.. (engram_hash_ids in include/engram.h); history [B, history_len] int64
    is read and updated in place."""
    if input_ids.dim() != 2:
        raise ValueError(f"input_ids has shape {tuple(input_ids.shape)}, expected [B, L]")
    B, L = input_ids.shape
    _contig("token_map", token_map, (torch.int32, torch.uint32) if hasattr(torch, "uint32") else torch.int32)
    for name, t in (("multipliers", multipliers), ("primes", primes), ("offsets", offsets),
                    ("input_ids", input_ids), ("history", history)):
        _contig(name, t, torch.int64)
    n_cols = (layout.max_ngram - 1) * layout.n_heads
    _numel("token_map", token_map, (layout.vocab,))
    _numel("multipliers", multipliers, (layout.n_layers, layout.max_ngram))
    _numel("primes", primes, (layout.n_layers, layout.max_ngram - 1, layout.n_heads))
    _numel("offsets", offsets, (layout.n_layers, n_cols))
    _numel("history", history, (B, layout.history_len))
    if token_mask is not None:
        _contig("token_mask", token_mask, (torch.uint8, torch.bool))
        _numel("token_mask", token_mask, (B, L))
    _check_err(err_count)
    if out is None:
        out = torch.empty((layout.n_layers, B, L, n_cols), dtype=torch.int64, device=input_ids.device)
    _numel("out", out, (layout.n_layers, B, L, n_cols))
    _contig("out", out, torch.int64)
    _same_device(input_ids, token_map=token_map, multipliers=multipliers, primes=primes,
                 offsets=offsets, history=history, token_mask=token_mask, out=out, err_count=err_count)
    _check("engram_hash_ids", _lib.engram_hash_ids(
        ctypes.byref(layout), _ptr(token_map), _ptr(multipliers), _ptr(primes), _ptr(offsets),
        _ptr(input_ids), _ptr(token_mask), B, L, start_pos, _ptr(history), _ptr(out),
        _ptr(err_count), _stream()))
    return out


def engram_gate_apply(layout: EngramLayout, x: torch.Tensor, kv: torch.Tensor,
                      q_weight: torch.Tensor, k_weight: torch.Tensor,
                      token_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      gate: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out [B, T, hc, dim] bf16 = x + gate * value (gate per token and stream)."""
    if x.dim() != 4:
        raise ValueError(f"x has shape {tuple(x.shape)}, expected [B, T, hc, dim]")
    B, T = x.shape[0], x.shape[1]
    _, N, _ = _dims(layout)
    _shape("x", x, (B, T, layout.hc, layout.dim))
    _contig("x", x, _BF16)
    _numel("kv", kv, (B, T, N))
    _contig("kv", kv, _BF16)
    _contig("q_weight", q_weight, torch.float32)
    _contig("k_weight", k_weight, torch.float32)
    _numel("q_weight", q_weight, (layout.hc, layout.dim))
    _numel("k_weight", k_weight, (layout.hc, layout.dim))
    if token_mask is not None:
        _contig("token_mask", token_mask, (torch.uint8, torch.bool))
        _numel("token_mask", token_mask, (B, T))
    if out is None:
        out = torch.empty_like(x)
    _numel("out", out, tuple(x.shape))
    _contig("out", out, _BF16)
    if gate is not None:
        _numel("gate", gate, (B, T, layout.hc))
        _contig("gate", gate, torch.float32)
    _same_device(x, kv=kv, q_weight=q_weight, k_weight=k_weight, token_mask=token_mask, out=out,
                 gate=gate)
    _check("engram_gate_apply", _lib.engram_gate_apply(
        ctypes.byref(layout), _ptr(x), _ptr(kv), _ptr(q_weight), _ptr(k_weight), _ptr(token_mask),
        B, T, _ptr(out), _ptr(gate), _stream()))
    return out


def _layout_key(layout: EngramLayout) -> tuple:
    # the fields that place control words and staging data (not n_rows, eps, clamp: the two
    # Engram modules of the model differ only in n_rows and share a workspace without clearing)
    return (layout.hc, layout.dim, layout.n_cols, layout.head_dim, layout.scale_block,
            layout.scale_format, layout.wkv_format)


class Workspace:
    """Zero-filled device workspace for engram_forward, grown on demand.

    The library leaves its control words zero after every call (except the time-out counter
    in word 0), and the staging area at the buffer's end holds scratch data; calls with one
    layout never place control words where another call's staging lies.  Calls with another
    layout may, so when the layout changes the buffer is cleared again (a fill kernel on the
    current stream), keeping word 0."""

    def __init__(self, device=None):
        self.device = device
        self.buf: Optional[torch.Tensor] = None
        self.layout = None

    def get(self, layout: EngramLayout, B: int, T: int) -> torch.Tensor:
        need = max(256, engram_forward_workspace_bytes(layout, B, T))
        key = _layout_key(layout)
        if self.buf is None or self.buf.numel() < need:
            old = self.buf
            self.buf = torch.zeros(need, dtype=torch.uint8, device=self.device or "cuda")
            if old is not None:  # keep the time-out counter across growth
                self.buf[:4].copy_(old[:4])
        elif self.layout is not None and key != self.layout:
            self.buf[4:].zero_()
        self.layout = key
        return self.buf


# One default workspace per (device, stream): calls that overlap in time must not share one, and
# calls on different streams may overlap.
_default_ws: dict = {}


def workspace_for(dev: int, stream_handle: int) -> "Workspace":
    """The default Workspace of a (device index, HIP stream handle): one each, made on first use
    (it allocates nothing until its first get())."""
    key = (int(dev), int(stream_handle))
    if key not in _default_ws:
        _default_ws[key] = Workspace(torch.device("cuda", int(dev)))
    return _default_ws[key]


def default_workspace(layout: EngramLayout, B: int, T: int, device: torch.device) -> torch.Tensor:
    """The workspace engram_forward uses when the caller passes none: the one of x's device and
    the current stream, grown on demand."""
    dev = device.index if device.index is not None else torch.cuda.current_device()
    return workspace_for(dev, torch.cuda.current_stream(dev).cuda_stream).get(layout, B, T)


def release_default_workspaces() -> None:
    """Frees the default workspaces (after the work on them has finished).  Registered to run at
    interpreter exit, so that no device buffer of this module outlives the program's own
    teardown of the HIP runtime or of a profiler attached to it."""
    if _default_ws and torch.cuda.is_initialized():
        torch.cuda.synchronize()
    _default_ws.clear()


atexit.register(release_default_workspaces)


def engram_forward_check(workspace: torch.Tensor) -> None:
    """Waits for the current stream and raises EngramError (status ENGRAM_E_TIMEOUT) if a
    cross-workgroup wait of an engram_forward call on `workspace` gave up since the last check;
    the library then zero-fills the workspace, so it can be used again."""
    _contig("workspace", workspace)
    _check("engram_forward_check", _lib.engram_forward_check(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))


def engram_set_spin_budget(polls: int) -> int:
    """Bound of the cross-workgroup waits in polls (0 restores the default); returns the old one."""
    return int(_lib.engram_set_spin_budget(polls))


def engram_forward(layout: EngramLayout, x: torch.Tensor, hash_ids: torch.Tensor,
                   token_mask: Optional[torch.Tensor], table: torch.Tensor, scales: torch.Tensor,
                   wkv: torch.Tensor, q_weight: torch.Tensor, k_weight: torch.Tensor,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   err_count: Optional[torch.Tensor] = None, check: bool = False) -> torch.Tensor:
    """The whole Engram forward: out [B, T, hc, dim] bf16 (may be x itself).  With ``check`` the
    call waits for its stream and raises if a cross-workgroup wait timed out
    (engram_forward_check); without it the caller checks when it chooses to."""
    if out is None:
        out = torch.empty_like(x)
    B, T = _check_forward_args(layout, x, hash_ids, token_mask, table, scales, wkv, q_weight,
                               k_weight, out, err_count)
    if workspace is not None:
        _contig("workspace", workspace)
    _same_device(x, workspace=workspace)
    if workspace is None:
        workspace = default_workspace(layout, B, T, x.device)
    _check("engram_forward", _lib.engram_forward(
        ctypes.byref(layout), _ptr(x), _ptr(hash_ids), _ptr(token_mask), _ptr(table), _ptr(scales),
        _ptr(wkv), _ptr(q_weight), _ptr(k_weight), B, T, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(err_count), _stream()))
    if check:
        engram_forward_check(workspace)
    return out


class PreparedForward:
    """engram_forward with its arguments checked once (prepare_forward): each call passes the same
    tensors' pointers to the C entry point on the current stream, with no per-call Python checks,
    so that back-to-back calls queue faster than the kernels run.  The tensors must stay alive and
    keep their storage while the object is used."""

    def __init__(self, layout, x, hash_ids, token_mask, table, scales, wkv, q_weight, k_weight,
                 out, workspace, err_count):
        B, T = _check_forward_args(layout, x, hash_ids, token_mask, table, scales, wkv, q_weight,
                                   k_weight, out, err_count)
        _contig("workspace", workspace)
        _same_device(x, workspace=workspace)
        need = engram_forward_workspace_bytes(layout, B, T)
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, "
                             f"the call needs {need}")
        self._keep = (layout, x, hash_ids, token_mask, table, scales, wkv, q_weight, k_weight, out,
                      workspace, err_count)
        self._args = (ctypes.byref(layout), _ptr(x), _ptr(hash_ids), _ptr(token_mask), _ptr(table),
                      _ptr(scales), _ptr(wkv), _ptr(q_weight), _ptr(k_weight), B, T, _ptr(out),
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err_count))
        self._fn = _lib.engram_forward
        self.out = out
        self.workspace = workspace

    def __call__(self) -> torch.Tensor:
        st = self._fn(*self._args, _stream())
        if st != ENGRAM_OK:
            raise EngramError("engram_forward", st)
        return self.out


def prepare_forward(layout: EngramLayout, x: torch.Tensor, hash_ids: torch.Tensor,
                    token_mask: Optional[torch.Tensor], table: torch.Tensor, scales: torch.Tensor,
                    wkv: torch.Tensor, q_weight: torch.Tensor, k_weight: torch.Tensor,
                    out: torch.Tensor, workspace: torch.Tensor,
                    err_count: Optional[torch.Tensor] = None) -> PreparedForward:
    """A repeatable engram_forward on fixed tensors (checked here, once): returns a callable."""
    return PreparedForward(layout, x, hash_ids, token_mask, table, scales, wkv, q_weight, k_weight,
                           out, workspace, err_count)


def engram_forward_noalloc(layout: EngramLayout, x: torch.Tensor, hash_ids: torch.Tensor,
                           token_mask: Optional[torch.Tensor], table: torch.Tensor,
                           scales: torch.Tensor, wkv: torch.Tensor, q_weight: torch.Tensor,
                           k_weight: torch.Tensor, out: torch.Tensor,
                           err_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """engram_forward without a workspace argument and without any allocation: the library's
    fixed per-GPU scratch array serves as the workspace (at most 4 MiB of it: up to 128 tokens at
    the model's layout; larger calls raise with status ENGRAM_E_WORKSPACE).  `out` must be
    given; calls on one GPU that overlap in time race on the scratch."""
    B, T = _check_forward_args(layout, x, hash_ids, token_mask, table, scales, wkv, q_weight,
                               k_weight, out, err_count)
    _check("engram_forward_noalloc", _lib.engram_forward_noalloc(
        ctypes.byref(layout), _ptr(x), _ptr(hash_ids), _ptr(token_mask), _ptr(table), _ptr(scales),
        _ptr(wkv), _ptr(q_weight), _ptr(k_weight), B, T, _ptr(out), _ptr(err_count), _stream()))
    return out


def _check_forward_args(layout: EngramLayout, x, hash_ids, token_mask, table, scales, wkv,
                        q_weight, k_weight, out, err_count):
    """Checks the tensors of a whole forward against the layout; returns (B, T)."""
    if x.dim() != 4:
        raise ValueError(f"x has shape {tuple(x.shape)}, expected [B, T, hc, dim]")
    B, T = x.shape[0], x.shape[1]
    _shape("x", x, (B, T, layout.hc, layout.dim))
    _contig("x", x, _BF16)
    _numel("hash_ids", hash_ids, (B, T, layout.n_cols))
    _contig("hash_ids", hash_ids, torch.int64)
    _contig("table", table, torch.uint8)
    _contig("scales", scales, torch.uint8 if layout.scale_format == SCALE_E8M0 else torch.float32)
    _check_table(layout, table, scales)
    _check_wkv(layout, wkv)
    _contig("q_weight", q_weight, torch.float32)
    _contig("k_weight", k_weight, torch.float32)
    _numel("q_weight", q_weight, (layout.hc, layout.dim))
    _numel("k_weight", k_weight, (layout.hc, layout.dim))
    if token_mask is not None:
        _contig("token_mask", token_mask, (torch.uint8, torch.bool))
        _numel("token_mask", token_mask, (B, T))
    _check_err(err_count)
    _numel("out", out, tuple(x.shape))
    _contig("out", out, _BF16)
    _same_device(x, hash_ids=hash_ids, table=table, scales=scales, wkv=wkv, q_weight=q_weight,
                 k_weight=k_weight, token_mask=token_mask, out=out, err_count=err_count)
    return B, T
