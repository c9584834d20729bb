"""The benchmark's roofline accounting (CPU): algorithmic bytes and flops of the forward and of the
split path's entry points, against the per-token and per-call figures derived by hand from the
layer sizes (every input read once, every output written once), the kernel whose profile each
token count's roofline names, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytest.importorskip("torch")
import bench  # noqa: E402
import synth  # noqa: E402

W = synth.workloads()
DECODE, PREFILL = W["decode_b64"], W["prefill_t8192"]

WKV_BF16 = 25600 * 6144 * 2          # 314,572,800
QK = 2 * 4 * 5120 * 4                 # q_weight + k_weight, fp32
# per token: ids 24 x 8, codes 24 x 256, fp32 scales 24 x 2 (256 / 128) x 4, x and out 4 x 5120 x 2
# each, mask 1
PER_TOKEN = 192 + 6144 + 192 + 40960 + 40960 + 1


def test_forward_bytes_per_token_and_per_call():
    assert PER_TOKEN == 88449
    assert bench.algorithmic_bytes(DECODE) == WKV_BF16 + QK + 64 * PER_TOKEN == 320_397_376
    # 32 features per fp32 scale: 8 scales per row
    w32 = synth.small_variant(DECODE, name="sb32", scale_block=32)
    assert bench.algorithmic_bytes(w32) - bench.algorithmic_bytes(DECODE) == 64 * (24 * 8 * 4 - 192)
    assert (bench.algorithmic_bytes(w32) - WKV_BF16 - QK) // 64 == 89025
    # E8M0 scales: one byte per block
    we = synth.small_variant(DECODE, name="e8m0", scale_block=32, scale_format="e8m0")
    assert (bench.algorithmic_bytes(we) - WKV_BF16 - QK) // 64 == PER_TOKEN - 192 + 24 * 8


def test_fp8_projection_weight_bytes():
    w8 = W["decode_b64_fp8"]
    per_call = 25600 * 6144 + 25600 * 6144 // 32  # codes + one E8M0 byte per 32 inputs
    assert per_call == 162_201_600
    # its table has E8M0 scales per 32 features: 24 x 8 bytes, as many as the fp32 scales per 128
    assert (w8.scale_format, w8.scale_block, w8.wkv_format) == ("e8m0", 32, "mxfp8")
    assert bench.algorithmic_bytes(w8) == per_call + QK + 64 * PER_TOKEN


def test_projection_flops():
    assert bench.algorithmic_flops(PREFILL) == 2 * 8192 * 25600 * 6144 == 2_576_980_377_600
    assert bench.algorithmic_flops(DECODE) == 64 * 314_572_800


def test_split_path_bytes():
    b = bench.standalone_bytes(DECODE)
    # gather: ids + codes + scales read, bf16 rows (6144 x 2) written
    assert b["gather"] == 64 * (192 + 6144 + 192 + 12288) == 64 * 18816
    # projection: wkv + rows read, kv (25600 x 2) written
    assert b["proj"] == WKV_BF16 + 64 * (12288 + 51200)
    # gate and residual: x + kv + mask read, out written, q/k once
    assert b["gate"] == QK + 64 * (40960 + 51200 + 1 + 40960) == QK + 64 * 133121


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_kernel_of_token_ranges_at_the_decode_layout():
    """The profile each workload's roofline names follows the library's schedule choice: one
    token block streams, 65..128 tokens take the two-token-block kernel, 129..256 the
    four-token-block kernel (bf16 weights, every workgroup owning 100 rows), more the tiled one;
    MXFP8 weights never take the several-block streaming kernels."""
    dec = synth.get("decode_b64")
    cases = [(1, "k_stream_wide_fused"), (64, "k_stream_wide_fused"), (65, "k_stream_tb2"),
             (128, "k_stream_tb2"), (129, "k_stream_tb4"), (256, "k_stream_tb4"), (257, "k_tiled_fused")]
    for m, name in cases:
        assert bench.kernel_of(synth.small_variant(dec, B=m, T=1))[0] == name, m
    assert bench.tb4_layout(dec)
    assert not bench.tb4_layout(synth.small_variant(dec, wkv_format="mxfp8"))
    # 1600 wkv rows over 256 workgroups: 4 or 8 rows each, not one row count for all
    assert not bench.tb4_layout(synth.small_variant(dec, dim=320, n_cols=4, head_dim=128))
    assert bench.kernel_of(synth.small_variant(dec, B=200, T=1, wkv_format="mxfp8"))[0] != "k_stream_tb4"
    # the profile names the sources whose hash it was taken at
    assert bench.kernel_of(synth.small_variant(dec, B=256, T=1))[1] == ("stream.hip", "gather_gate.hip", "common.h")
