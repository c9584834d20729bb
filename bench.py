"""Engram forward benchmark on one MI355X.

One step = one engram_forward call (row gather + dequantisation, wkv projection, per-stream
gate, residual add) over one batch of seeded synthetic inputs already resident in HBM; for the
two-instance workloads, two calls, the second consuming the first one's output.
Prints one JSON line.  `value` is tokens per second of the whole job (one GPU).

  python bench.py [--steps K] [--warmup W] [--workload decode_b64|prefill_t8192|...]
                  [--prefill-workload prefill_t8192|none] [--flush-mib F] [--standalone]

By default the line reports the decode workload (64 tokens; `value`) and, in a nested object
"prefill", the prefill workload (8192 tokens), each with its roofline and CPU baseline: the
metric names both.

With --flush-mib, F MiB are written between steps (evicting the L2s and the Infinity Cache) and
each step is timed by its own event pair.  With --standalone the line also holds the three
entry points of the split path timed alone on the same inputs (first instance): the row gather
(engram_gather_dequant), the projection (engram_kv_proj) and the gate with the residual add
(engram_gate_apply), each against its roofline.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
WARMUP_MIN_MS = 100.0       # least wall time of untimed warm-up steps per workload (default)
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published


def algorithmic_bytes(w) -> int:
    """Bytes one launch must move at least: every input read once, every output written once."""
    scale_bytes = 1 if w.scale_format == "e8m0" else 4
    per_token = (w.n_cols * 8 + w.n_cols * w.head_dim + w.n_cols * w.n_blocks * scale_bytes +
                 2 * w.hc * w.dim * 2 + 1)
    wkv = w.N * w.K + w.N * (w.K // 32) if w.wkv_format == "mxfp8" else w.N * w.K * 2
    per_call = wkv + 2 * w.hc * w.dim * 4
    return per_call + w.M * per_token


def algorithmic_flops(w) -> int:
    return 2 * w.M * w.N * w.K


TILED_MIN_TOKENS = 65  # the whole forward switches from weight streaming to 256 x 256 tiles here,
TB2_MAX_TOKENS = 128   # except up to here with bf16 weights (the two-token-block streaming kernel)
TB4_MAX_TOKENS = 256   # and up to here where the layout admits the four-token-block kernel


def fp8_mfma(w) -> bool:
    """Both operands of the projection stay fp8 (MXFP8 table and weights: the scaled fp8 MFMA)."""
    return w.wkv_format == "mxfp8" and w.scale_format == "e8m0" and w.scale_block % 32 == 0


def tb4_layout(w, cus: int = 256) -> bool:
    """Whether the library's four-token-block kernel takes this layout (bf16 weights, every
    workgroup of the weight-streaming grid owning the same whole number of at most seven 16-row
    blocks, K a multiple of 128), as the library decides it on a GPU of `cus` compute units."""
    N = (w.hc + 1) * w.dim
    q = N // 4
    G = min(cus, q)
    blocks = lambda g: (4 * ((q + g - 1) // g) + 15) // 16
    while blocks(G) > 8:
        G += 1
    rows = 4 * ((q + G - 1) // G)
    return (w.wkv_format != "mxfp8" and q % G == 0 and w.K % 128 == 0 and rows <= w.dim and 1 <= blocks(G) <= 7)


def kernel_of(w):
    """(profile name, sources) of the kernels that engram_forward runs for this workload: the
    fused weight-streaming kernels for up to 256 tokens (above 128 the row gather into the
    staging area first, timed with it as one forward); for more, the row gather followed by the
    fused tiled kernel (one forward)."""
    if TILED_MIN_TOKENS <= w.M <= TB2_MAX_TOKENS and w.wkv_format != "mxfp8":
        return "k_stream_tb2", ("stream.hip", "common.h")
    if TB2_MAX_TOKENS < w.M <= TB4_MAX_TOKENS and tb4_layout(w):
        return "k_stream_tb4", ("stream.hip", "gather_gate.hip", "common.h")
    if w.M >= TILED_MIN_TOKENS:
        return ("k_tiled_mx_fused" if fp8_mfma(w) else "k_tiled_fused"), ("tiled.hip", "gather_gate.hip", "common.h")
    return "k_stream_wide_fused", ("stream.hip", "common.h")


KERNEL_LABEL = {"k_tiled_fused": "k_gather_dequant + k_tiled<true> (one forward)",
                "k_tiled_mx_fused": "k_gather_mx + k_tiled<true, true> (fp8 operands; one forward)",
                "k_stream_wide_fused": "k_stream_wide<.., true>",
                "k_stream_tb2": "k_stream_tb2 (two token blocks per pass over wkv)",
                "k_stream_tb4": "k_gather_dequant + k_stream_tb4 (four token blocks per pass over wkv; one forward)"}


def kernel_label(w) -> str:
    k = kernel_of(w)[0]
    if w.wkv_format == "mxfp8":
        if k == "k_tiled_fused":
            return "k_expand_mxfp8 + " + KERNEL_LABEL[k]
        if k == "k_stream_wide_fused":
            return ("k_stream_wide<.., true, .., W8, MX> (fp8 operands)" if fp8_mfma(w)
                    else "k_stream_wide<.., true, .., W8> (FP8 weights, bf16 MFMA)")
    return KERNEL_LABEL[k]


def measured_traffic(w):
    """HBM bytes per launch from the committed PMC summary of this kernel and workload, or None
    when there is none or the kernel sources changed since the counters were taken."""
    import hashlib
    kname, sources = kernel_of(w)
    path = os.path.join(ROOT, "profiles", f"{kname}_{w.name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, "hashed_gram_engram_amd", "csrc")
    now = " ".join(hashlib.sha256(open(os.path.join(src, f), "rb").read()).hexdigest()
                   for f in sources)
    if fields.get("kernel_sources_sha256") != now or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def standalone_bytes(w) -> dict:
    """Algorithmic bytes of the three split-path entry points: every input read once, every output
    written once."""
    scale_bytes = 1 if w.scale_format == "e8m0" else 4
    wkv = w.N * w.K + w.N * (w.K // 32) if w.wkv_format == "mxfp8" else w.N * w.K * 2
    gather = w.M * (w.n_cols * 8 + w.n_cols * w.head_dim + w.n_cols * w.n_blocks * scale_bytes + w.K * 2)
    proj = wkv + w.M * (w.K * 2 + w.N * 2)
    gate = 2 * w.hc * w.dim * 4 + w.M * (w.hc * w.dim * 2 + w.N * 2 + 1 + w.hc * w.dim * 2)
    return {"gather": gather, "proj": proj, "gate": gate}


def time_calls(fn, steps: int, warmup: int, stream) -> list:
    """Per-call milliseconds of `fn` over `steps` back-to-back calls (event pairs on `stream`)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def standalone(eg, lay, w, d, steps: int, warmup: int, stream) -> dict:
    """The split path's entry points timed alone (mean per call; HBM roofline for all three, bf16
    or fp8 MFMA roofline for the projection as well)."""
    emb = eg.engram_gather_dequant(lay, d["table"], d["scales"], d["hash_ids"])
    kv = eg.engram_kv_proj(lay, emb, d["wkv"])
    out = torch.empty_like(d["x"])
    calls = {
        "gather": ("engram_gather_dequant (k_gather_dequant)",
                   lambda: eg.engram_gather_dequant(lay, d["table"], d["scales"], d["hash_ids"], emb=emb)),
        "proj": ("engram_kv_proj", lambda: eg.engram_kv_proj(lay, emb, d["wkv"], kv=kv)),
        "gate": ("engram_gate_apply (k_gate_apply)",
                 lambda: eg.engram_gate_apply(lay, d["x"], kv, d["q_weight"], d["k_weight"],
                                              d["token_mask"], out=out)),
    }
    nbytes = standalone_bytes(w)
    res = {}
    for key, (label, fn) in calls.items():
        ms = float(np.mean(time_calls(fn, steps, warmup, stream)))
        gbs = nbytes[key] / (ms * 1e-3) / 1e9
        r = {"call": label, "ms": round(ms, 5), "bytes": nbytes[key], "GB/s": round(gbs, 1),
             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if key == "proj":
            peak = BF16_PEAK_TFLOPS  # bf16 activations: the projection alone multiplies in bf16
            tf = algorithmic_flops(w) / (ms * 1e-3) / 1e12
            r.update({"TFLOP/s": round(tf, 1), "mfma_peak": peak, "mfma_frac": round(tf / peak, 4)})
        res[key] = r
    return res


def host_facts() -> dict:
    """CPU model and RAM of the host the oracle runs on."""
    model, mem_kib = "unknown", 0
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                mem_kib = int(line.split()[1])
                break
    except OSError:  # pragma: no cover
        pass
    return {"cpu_model": model, "ram_gib": round(mem_kib / 2 ** 20, 1)}


def cpu_baseline(w, n_tokens: int, min_seconds: float = 10.0):
    """The CPU oracle (oracle/engram_oracle.cc: plain C++, IEEE double, threads over tokens), as
    it stands, on the first n_tokens tokens of the same workload (every instance of it in turn,
    each consuming the previous one's output), repeated until at least min_seconds of oracle time
    have accumulated.  Input generation (table rows, wkv) is outside the timed region."""
    import oracle
    import synth
    sel = np.arange(n_tokens)
    mask = w.token_mask().reshape(-1)[sel]
    x0 = w.x_tokens(sel)

    def wkv_of(inst):  # FP8 weights are dequantised once, outside the timed region
        if w.wkv_format == "mxfp8":
            return oracle.wkv_mxfp8_bits(*w.wkv8(inst))
        return w.wkv_f32(inst)

    inputs = []
    for inst in range(w.n_instances):
        ids = w.hash_ids(inst).reshape(w.M, w.n_cols)[sel]
        # the rows these tokens name are generated once, outside the timed region; the oracle
        # asks for exactly those rows (ascending) on every pass
        flat = ids.reshape(-1)
        need = np.unique(flat[(flat >= 0) & (flat < w.n_rows)])
        rows = synth.host_fetch(w, inst)(need)

        def provider(r, need=need, rows=rows):
            assert np.array_equal(r, need)
            return rows
        inputs.append((wkv_of(inst), ids, w.qk(inst), provider))
    dt, reps = 0.0, 0
    while reps == 0 or dt < min_seconds:
        x = x0
        for wkv, ids, (q, k), fetch in inputs:
            t0 = time.perf_counter()
            x = oracle.forward(x, ids, mask, fetch, w.n_rows, w.head_dim, w.scale_block, wkv, q,
                               k, eps=w.eps, clamp=w.clamp, scale_format=w.scale_format,
                               want=("out_bits",))["out_bits"]
            dt += time.perf_counter() - t0
        reps += 1
    return {"value": round(n_tokens * reps / dt, 2), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"first {n_tokens} tokens of {w.name} (full layer dims; C++ oracle, IEEE "
                      f"double, {oracle.threads()} threads over tokens), {reps} passes, {dt:.2f} s",
            **host_facts()}


def layout_of(eg, w):
    return eg.make_layout(w.hc, w.dim, w.n_cols, w.head_dim, w.scale_block, w.n_rows, w.eps, w.clamp,
                          scale_format=eg.SCALE_E8M0 if w.scale_format == "e8m0" else eg.SCALE_FP32,
                          wkv_format=eg.WKV_MXFP8 if w.wkv_format == "mxfp8" else eg.WKV_BF16)


LEAD_IN = 2  # untimed steps in flight when the throughput pass's start event is recorded


def measure(eg, w, steps: int, warmup: int, flush_mib: int = 0, with_standalone: bool = False,
            min_warmup_ms: float = WARMUP_MIN_MS) -> dict:
    """Times `steps` steps of the workload (one step: every instance's engram_forward, the second
    on the first one's output) after `warmup` untimed ones, inputs resident in HBM.

    Two passes of `steps` steps each, events on the stream the kernels run on.  The throughput
    pass records one event before the first step and one after the last, nothing in between
    (an event recorded between two launches adds its own gap on the GPU), with the last warm-up
    steps still running when the first one is recorded; its mean per step is the throughput.  The second pass records a pair around every engram_forward launch: their
    durations give the roofline's time per launch and the step-time percentiles.  With
    flush_mib, that many MiB are written before each step (cold L2s and Infinity Cache) and the
    throughput is the mean of the second pass's step durations."""
    import synth
    insts = []
    for inst in range(w.n_instances):
        d = synth.device_inputs(w, inst=inst)
        if inst:
            del d["x"]  # a later instance reads the previous one's output
        insts.append(d)
    x0 = insts[0]["x"]
    lay = layout_of(eg, w)
    ws = torch.zeros(max(256, eg.engram_forward_workspace_bytes(lay, w.B, w.T)), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty_like(x0) for _ in insts]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    flush = (torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda") if flush_mib else None)
    stream = torch.cuda.current_stream()
    n_launch = steps * len(insts)
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
    ev_run = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    # each instance's call checked once (argument checks in Python per call would leave the GPU
    # idle between launches); instance j > 0 reads instance j - 1's output
    calls = []
    x = x0
    for d, out in zip(insts, outs):
        calls.append(eg.prepare_forward(lay, x, d["hash_ids"], d["token_mask"], d["table"],
                                        d["scales"], d["wkv"], d["q_weight"], d["k_weight"], out,
                                        ws, err))
        x = out

    def step(i=None):
        for j, call in enumerate(calls):
            if i is not None:
                ev_a[i * len(insts) + j].record(stream)
            call()
            if i is not None:
                ev_b[i * len(insts) + j].record(stream)

    # warm-up: `warmup` steps, and more until min_warmup_ms of them have run (on a fresh GPU the
    # first few milliseconds of launches run up to 20% slower while clocks and caches settle)
    n_warm = 0
    tw = time.perf_counter()
    while n_warm < warmup or (time.perf_counter() - tw) * 1e3 < min_warmup_ms:
        step()
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # throughput pass: the timed steps back to back, an event on each side of the region.  The
    # last LEAD_IN warm-up steps are enqueued just before the start event, without waiting for
    # them: the GPU is then busy while the host enqueues the start event and the timed steps, so
    # the region holds the steps back to back and not the host's latency to its first launch
    # after a synchronisation (~30 us, 1.5 us per step at 20 steps).
    wall = None
    if flush is None:
        for _ in range(LEAD_IN):
            step()
        t0 = time.perf_counter()
        ev_run[0].record(stream)
        for i in range(steps):
            step()
        ev_run[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    # per-launch pass: an event pair around every launch
    t1 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))
        step(i)
    torch.cuda.synchronize()
    if wall is None:
        wall = time.perf_counter() - t1
    launch_ms = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    step_ms = [sum(launch_ms[i * len(insts):(i + 1) * len(insts)]) for i in range(steps)]
    if flush is None:
        ms = ev_run[0].elapsed_time(ev_run[1]) / steps   # whole timed region, launch gaps included
        ms_events = ev_a[0].elapsed_time(ev_b[-1]) / steps  # the same with events between launches
    else:
        ms = float(np.mean(step_ms))
        ms_events = ms
    # time per launch: the throughput pass's region over its launches (back to back, nothing
    # recorded between them); with flushing, the mean of the per-launch event pairs
    ms_launch_events = float(np.mean(launch_ms))
    ms_launch = ms * steps / n_launch if flush is None else ms_launch_events
    assert int(err.item()) == 0, "hash ids out of range"
    eg.engram_forward_check(ws)   # raises if a cross-workgroup wait timed out

    mode = "hbm" if w.M <= 512 else "mfma"
    if mode == "hbm":
        ach = algorithmic_bytes(w) / (ms_launch * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w)}
    else:
        ach = algorithmic_flops(w) / (ms_launch * 1e-3) / 1e12
        peak = FP8_PEAK_TFLOPS if fp8_mfma(w) else BF16_PEAK_TFLOPS  # the contraction's own dtype
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": measured_traffic(w)}
    roof["kernel"] = kernel_label(w)
    roof["per_launch_bytes"] = algorithmic_bytes(w)
    roof["per_launch_flops"] = algorithmic_flops(w)
    roof["ms_per_launch"] = round(ms_launch, 5)
    roof["ms_per_launch_events"] = round(ms_launch_events, 5)
    roof["timing"] = ("HIP events on the launches' stream around the timed region of back-to-back "
                      f"launches ({LEAD_IN} untimed steps in flight at its start), divided by the "
                      "launches (ms_per_launch_events: the mean of event pairs around each launch, "
                      "which add their own gaps)" if flush is None else
                      "HIP events around each launch, on its stream")
    res = {
        "warmup_steps_run": n_warm,
        "value": round(w.M / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 5),
        "ms_p10_median_p90": [round(float(v), 5) for v in np.percentile(step_ms, [10, 50, 90])],
        "wall_ms_per_step": round(wall * 1e3 / steps, 5),
        "ms_per_step_with_launch_events": round(ms_events, 5),
        "dtype": "fp8 (e4m3 x E8M0)" if fp8_mfma(w) else "bf16",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "hc": w.hc, "dim": w.dim,
                   "n_cols": w.n_cols, "head_dim": w.head_dim, "scale_block": w.scale_block,
                   "scale_format": w.scale_format, "wkv_format": w.wkv_format,
                   "table_rows": w.n_rows, "hash_ids": w.hash_dist,
                   "instances": w.n_instances, "flush_mib": flush_mib,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if with_standalone:
        res["standalone"] = standalone(eg, lay, w, insts[0] | {"x": x0}, steps, warmup, stream)
    del insts, outs, ws, flush
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


class StandInBackbone:
    """Load on the main stream standing in for the transformer layers around the Engram layers
    (the Engram modules sit at the entries of zero-based layers 1 and 14): per layer two bf16
    GEMMs [M, dim] x [dim, dim], each layer with weights of its own (no cache reuse across
    layers).  Its numbers are not used; it only occupies the GPU as a backbone would."""

    def __init__(self, M: int, dim: int, n_layers: int, device="cuda"):
        g = torch.Generator(device=device).manual_seed(7)
        self.h = torch.randn((M, dim), generator=g, device=device, dtype=torch.bfloat16)
        self.tmp = torch.empty_like(self.h)
        self.w = [(torch.randn((dim, dim), generator=g, device=device, dtype=torch.bfloat16) * 0.01,
                   torch.randn((dim, dim), generator=g, device=device, dtype=torch.bfloat16) * 0.01)
                  for _ in range(n_layers)]

    def layer(self, i: int):
        w1, w2 = self.w[i]
        torch.matmul(self.h, w1, out=self.tmp)
        torch.matmul(self.tmp, w2, out=self.h)


def measure_split_phase(eg, w, steps: int, warmup: int, engram_layers=(1, 14)) -> dict:
    """The split-phase schedule of the pages' serving engine (lookup and projection early, gate at
    the layer's entry) against the fused forward, both inside a stand-in backbone.

    Per step, with the layers 0 .. engram_layers[-1] of the stand-in backbone on the main stream:
      fused:  each Engram layer's entry runs engram_forward on the main stream;
      split:  at step start a side stream runs engram_gather_dequant + engram_kv_proj of every
              instance (their inputs, the hash ids, are known before the first layer); at each
              Engram layer's entry the main stream waits for that instance's kv and runs
              engram_gate_apply;
      alone:  the backbone without Engram.
    The Engram cost a step exposes is its time minus the backbone's alone.  Instance i + 1 reads
    instance i's output, as in the model."""
    import synth
    assert w.n_instances == len(engram_layers)
    insts = []
    for inst in range(w.n_instances):
        d = synth.device_inputs(w, inst=inst)
        if inst:
            del d["x"]
        insts.append(d)
    x0 = insts[0]["x"]
    lay = layout_of(eg, w)
    ws = torch.zeros(max(256, eg.engram_forward_workspace_bytes(lay, w.B, w.T)), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty_like(x0) for _ in insts]
    embs = [torch.empty((w.B, w.T, w.K), dtype=torch.bfloat16, device="cuda") for _ in insts]
    kvs = [torch.empty((w.B, w.T, w.N), dtype=torch.bfloat16, device="cuda") for _ in insts]
    n_layers = engram_layers[-1] + 1
    bb = StandInBackbone(w.M, w.dim, n_layers)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in insts]

    def step(mode: str):
        if mode == "split":
            side.wait_stream(main)
            with torch.cuda.stream(side):
                for j, d in enumerate(insts):
                    eg.engram_gather_dequant(lay, d["table"], d["scales"], d["hash_ids"], emb=embs[j])
                    eg.engram_kv_proj(lay, embs[j], d["wkv"], kv=kvs[j])
                    ready[j].record(side)
        x = x0
        j = 0
        for layer in range(n_layers):
            if mode != "alone" and layer in engram_layers:
                d = insts[j]
                if mode == "fused":
                    eg.engram_forward(lay, x, d["hash_ids"], d["token_mask"], d["table"], d["scales"],
                                      d["wkv"], d["q_weight"], d["k_weight"], out=outs[j], workspace=ws)
                else:
                    main.wait_event(ready[j])
                    eg.engram_gate_apply(lay, x, kvs[j], d["q_weight"], d["k_weight"], d["token_mask"],
                                         out=outs[j])
                x = outs[j]
                j += 1
            bb.layer(layer)
        if mode == "split":
            main.wait_stream(side)  # the side stream's buffers are reused by the next step

    def timed(mode: str) -> float:
        for _ in range(warmup):
            step(mode)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(main)
        for _ in range(steps):
            step(mode)
        b.record(main)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res = {}
    for mode in ("alone", "fused", "split", "alone"):   # the backbone alone before and after
        ms = timed(mode)
        res[mode] = min(ms, res.get(mode, ms))
    check = {}
    step("fused")
    fused = [o.clone() for o in outs]
    step("split")
    torch.cuda.synchronize()
    normal = torch.from_numpy(~w.outlier_tokens()).to(x0.device)
    for j in range(len(insts)):
        a, b = fused[j].reshape(w.M, -1), outs[j].reshape(w.M, -1)
        ulp = (a.view(torch.int16).int() - b.view(torch.int16).int()).abs()
        check[f"instance{j + 1}_vs_fused"] = {
            "max_abs_diff": float((a.float() - b.float()).abs()[normal].max().item()),
            "frac_beyond_1_ulp": float((ulp > 1).float().mean().item())}
    eg.engram_forward_check(ws)
    out = {
        "engram_layers": list(engram_layers), "backbone": f"stand-in: {n_layers} layers x 2 bf16 "
        f"GEMMs [{w.M}, {w.dim}] x [{w.dim}, {w.dim}] on the main stream",
        "ms_backbone_alone": round(res["alone"], 5),
        "ms_fused": round(res["fused"], 5), "ms_split": round(res["split"], 5),
        "ms_exposed_fused": round(res["fused"] - res["alone"], 5),
        "ms_exposed_split": round(res["split"] - res["alone"], 5), **check,
    }
    del insts, outs, embs, kvs, ws, bb
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


METRIC = "Engram forward tokens/sec at T=64 decode and T=8192 prefill; % HBM/MFMA roofline"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_b64")
    ap.add_argument("--prefill-workload", default="prefill_t8192",
                    help="second workload reported in a nested object ('none' to skip); only "
                         "with the default --workload")
    ap.add_argument("--cpu-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-warmup-ms", type=float, default=WARMUP_MIN_MS,
                    help="keep warming up until this much wall time has passed (0: exactly --warmup steps)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write this many MiB between steps and time each step alone")
    ap.add_argument("--standalone", action="store_true",
                    help="also time the split path's three entry points alone")
    ap.add_argument("--split-phase", action="store_true",
                    help="also time the split-phase schedule (gather + projection on a side stream "
                         "ahead of a stand-in backbone, gate at each layer entry) against the fused "
                         "forward (two-instance workloads)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (scales HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the Engram forward is data parallel over tokens and "
              "this build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import hashed_gram_engram_amd as eg
    import synth

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    torch.cuda.set_device(0)
    w = synth.get(args.workload)
    head = measure(eg, w, args.steps, args.warmup, args.flush_mib, args.standalone, args.min_warmup_ms)
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": head["warmup_steps_run"],
        "ms_per_step": head["ms_per_step"],
        "ms_p10_median_p90": head["ms_p10_median_p90"],
        "wall_ms_per_step": head["wall_ms_per_step"],
        "ms_per_step_with_launch_events": head["ms_per_step_with_launch_events"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded counter-based generator; no trained weights)",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    if "standalone" in head:
        res["standalone"] = head["standalone"]
    if args.split_phase:
        res["split_phase"] = measure_split_phase(eg, w, args.steps, args.warmup,
                                                 engram_layers=(1, 14)[:w.n_instances])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens or min(w.M, 64))
    second = args.prefill_workload if args.workload == "decode_b64" else "none"
    if second and second != "none":
        w2 = synth.get(second)
        p = measure(eg, w2, args.steps, args.warmup, args.flush_mib, min_warmup_ms=args.min_warmup_ms)
        p = {"workload": w2.name, "value": p["value"], "unit": "tokens/s",
             **{k: p[k] for k in ("warmup_steps_run", "ms_per_step", "ms_p10_median_p90", "wall_ms_per_step",
                                  "ms_per_step_with_launch_events", "dtype", "config", "roofline")}}
        if not args.no_cpu_baseline:
            p["cpu_baseline"] = cpu_baseline(w2, args.cpu_tokens or 256)
        res["prefill"] = p
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
