"""The C-ABI library loads, exports every declared entry point, and validates arguments on
the host before touching a device (CPU only; no compute call reaches a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")

eg = pytest.importorskip("hashed_gram_engram_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("engram_gather_dequant", "engram_kv_proj", "engram_gate_apply", "engram_forward",
                 "engram_forward_workspace_bytes", "engram_layout_check", "engram_param_counts",
                 "engram_hash_ids", "engram_status_str"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(eg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(eg.EXPORTED) == declared_functions()


def good():
    return eg.make_layout(4, 5120, 24, 256, 128, 384016682)


def test_layout_checks():
    assert eg.engram_layout_check(good()) == 0
    assert eg.engram_layout_check(eg.make_layout(4, 256, 6, 64, 32, 6126)) == 0
    # MXFP8 tables: E8M0 scales, one per 32 features of a 256-feature row
    assert eg.engram_layout_check(eg.make_layout(4, 5120, 24, 256, 32, 16803844,
                                                 scale_format=eg.SCALE_E8M0)) == 0
    # FP8 projection weights (MXFP8 along the inputs), alone and with an MXFP8 table
    assert eg.engram_layout_check(eg.make_layout(4, 5120, 24, 256, 128, 16803844,
                                                 wkv_format=eg.WKV_MXFP8)) == 0
    assert eg.engram_layout_check(eg.make_layout(4, 5120, 24, 256, 32, 16803844,
                                                 scale_format=eg.SCALE_E8M0,
                                                 wkv_format=eg.WKV_MXFP8)) == 0
    bad = [dict(hc=3), dict(dim=5000), dict(head_dim=96), dict(scale_block=24),
           dict(scale_block=512), dict(n_rows=0), dict(eps=float("nan")), dict(n_cols=0),
           dict(scale_format=2), dict(scale_format=-1), dict(wkv_format=2), dict(wkv_format=-1),
           # E8M0 with 2 scales per row (not whole dwords)
           dict(scale_format=1, scale_block=128)]
    for change in bad:
        lay = good()
        for k, v in change.items():
            setattr(lay, k, v)
        assert eg.engram_layout_check(lay) == -2, change


def test_param_counts_on_host():
    assert eg.engram_param_counts(good()) == (98308270592, 157286400, 40960)
    # the counts are elements, whatever the storage of the projection
    fp8 = eg.make_layout(4, 5120, 24, 256, 128, 384016682, wkv_format=eg.WKV_MXFP8)
    assert eg.engram_param_counts(fp8) == (98308270592, 157286400, 40960)
    # bytes of the wkv argument: 2 per weight, or 1 per weight + 1 per 32 (codes then scales)
    assert eg.wkv_bytes(good()) == 2 * 157286400
    assert eg.wkv_bytes(fp8) == 157286400 + 157286400 // 32 == 162201600


def test_layout_struct_matches_the_header():
    # field order and offsets of engram_layout as declared in include/engram.h
    hdr = open(os.path.join(ROOT, "include", "engram.h")).read()
    body = hdr[hdr.index("typedef struct {", hdr.index("engram_wkv_format")):]
    body = body[:body.index("} engram_layout;")]
    names = [line.split(";")[0].split()[-1] for line in body.splitlines()[1:] if ";" in line]
    assert names == [f for f, _ in eg.EngramLayout._fields_]
    assert eg.EngramLayout.n_rows.offset == 32 and ctypes.sizeof(eg.EngramLayout) == 48


def test_entry_points_reject_bad_arguments_before_any_device_work():
    lib = eg._lib
    lay = good()
    L = ctypes.byref(lay)
    bad = eg.make_layout(4, 5120, 24, 256, 100, 10)
    Lb = ctypes.byref(bad)
    p = ctypes.c_void_p(16)
    assert lib.engram_forward(Lb, p, p, None, p, p, p, p, p, 1, 1, p, p, 1 << 20, None, None) == -2
    assert lib.engram_forward(L, None, p, None, p, p, p, p, p, 1, 1, p, p, 1 << 20, None, None) == -1
    assert lib.engram_forward(L, p, p, None, p, p, p, p, p, -1, 1, p, p, 1 << 20, None, None) == -3
    assert lib.engram_gather_dequant(L, p, p, None, 2, 3, p, None, None) == -1
    assert lib.engram_kv_proj(L, p, None, 2, 3, p, None) == -1
    assert lib.engram_gate_apply(L, p, p, p, None, None, 1, 1, p, None, None) == -1
    # empty batches are a no-op
    assert lib.engram_forward(L, None, None, None, None, None, None, None, None, 0, 7, None, None, 0,
                              None, None) == 0
    assert lib.engram_kv_proj(L, None, None, 5, 0, None, None) == 0
    odd = ctypes.c_void_p(24)
    assert lib.engram_kv_proj(L, odd, p, 1, 1, p, None) == -4
    assert eg.engram_forward_workspace_bytes(bad, 1, 1) == 0


def test_status_strings():
    for st in range(-7, 1):
        assert eg._lib.engram_status_str(st)


def test_hash_entry_point_rejects_bad_arguments_before_any_device_work():
    hl = eg.make_hash_layout(2, 4, 8, 2, 129280, 16)
    lib = eg._lib
    null = None
    assert lib.engram_hash_ids(None, null, null, null, null, null, null, 1, 1, 0, null, null,
                               null, null) == -1
    bad = eg.make_hash_layout(2, 1, 8, 2, 129280, 16)  # max_ngram < 2
    assert lib.engram_hash_ids(ctypes.byref(bad), null, null, null, null, null, null, 1, 1, 0,
                               null, null, null, null) == -2
    # positions past the history
    assert lib.engram_hash_ids(ctypes.byref(hl), null, null, null, null, null, null, 1, 10, 7,
                               null, null, null, null) == -3
    # nothing to do: no pointer is looked at
    assert lib.engram_hash_ids(ctypes.byref(hl), null, null, null, null, null, null, 0, 10, 0,
                               null, null, null, null) == 0
    # missing tensors
    assert lib.engram_hash_ids(ctypes.byref(hl), null, null, null, null, null, null, 1, 10, 0,
                               null, null, null, null) == -1
