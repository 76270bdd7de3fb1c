#!/usr/bin/env python3
"""Benchmark of the Hadamard-rotated ternary-weight path on one MI355X.

Timed step (the value): one decode token through a 64-layer 27B-shaped stack
(d_model 5120, d_ff 17408) at batch 1: for every layer and each fused
projection (QKV 15360x5120, O 5120x5120, gate/up 34816x5120, down
5120x17408) the activations are rotated and encoded as the GEMV operand
(tb_fwht128 with the act8 output), multiplied by the packed ternary weights
(grouped tb_ternary_gemv launches) and the output is rotated back (tb_fwht128
along N); one rotation launch per layer boundary carries the previous
layer's output rotations and this layer's input rotations.  All 6.33 GB of
packed weights are resident in HBM and each is read once per step, far
beyond the 256 MB last-level cache.  The step is captured once in a HIP
graph and replayed.
value = packed weight bytes (codes + scales) streamed per step / step time.

Also measured in the same run, each over its own synthetic input, and
reported under "extra": the same decode step at batch 8, the 2:4 GEMV
(17408x5120, batch 1), the prefill GEMM (M = 2048, both FFN shapes), the
activation FWHT at prefill size, the offline quantiser streamed over a
64-layer stack (absmean rule) and over one layer with the error-minimising
rule.  The CPU oracle is timed on bounded samples of the decode GEMV, the 2:4
GEMV, the GEMM and the quantiser, on one core and on all cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_MFMA_TFLOPS = 2500.0    # dense fp16 / bf16 matrix cores
D, F = 5120, 17408
GEMV_PARTS = None  # K parts per tile of the decode GEMVs (tb_gemv_segment.parts); --gemv-parts


def gemv_parts(batch, k_groups):
    """K parts of one decode product (k_groups: its code groups per row): 8
    for the long-K down projection, 4 for the others, unless --gemv-parts
    fixes it.  Measured on the 64-layer 27B-shaped step with all four
    products in one launch per layer (K = 5120 / 17408 parts): batch 1 1.460
    ms with 4 / 8, 1.467 ms with 4 / 4, 1.478 ms with 2 / 8, 1.535 ms with
    4 / 2; batch 8 2.495 ms with 4 / 8, 2.506 ms with 4 / 4."""
    if GEMV_PARTS is not None:
        return GEMV_PARTS
    return 8 if k_groups > 80 else 4


FUSED = (("qkv", 3 * D, D), ("o", D, D), ("gate_up", 2 * F, D), ("down", D, F))


def auto_grouping(batch, planes=1):
    """All four products of a layer in one GEMV launch ("layer") when each is
    split into K parts (every segment then takes the short K slices), else
    the long-K down projection in a launch of its own ("split"): a shared
    launch would give every segment its long slices."""
    parts = [gemv_parts(batch, planes * k // 128) for _, n, k in FUSED]
    return "layer" if min(parts) > 1 else "split"


GROUP_TEXT = {"layer": "all four products of a layer [QKV 15360x5120, O 5120x5120, gate/up 34816x5120, "
                       "down 5120x17408] in one launch",
              "split": "[QKV 15360x5120, O 5120x5120, gate/up 34816x5120] and [down 5120x17408] per layer",
              "none": "one launch per product"}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


GEMV_SOURCES = ("ternary_weights_hadamard_amd/csrc/gemv_ternary.hip", "ternary_weights_hadamard_amd/csrc/tb_common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode_batch1_hbm_traffic.txt")
CALIB_BYTES = 256 << 20  # plain copy used to calibrate the byte counters


def gemv_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(grouping):
    """HBM bytes per GEMV launch from the committed counter summary, or None when
    it is missing, was taken on other GEMV sources than the current ones or
    with launches grouped otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("gemv_source_hash") != gemv_source_hash() or vals.get("gemv_grouping") != grouping:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gemv_bytes(n, k, b, planes=1):
    """Algorithmic bytes of one GEMV launch: codes + scales (per plane) + activations + output."""
    return planes * (n * k // 4 + n * k // 64) + 2 * b * k + 4 * b * n


def packed_bytes(n, k):
    return n * k // 4 + n * k // 64


class DecodeStack:
    def __init__(self, layers, batch, gen, dev, grouping="auto", planes=1):
        import torch

        from ternary_weights_hadamard_amd import synth

        self.layers, self.batch, self.planes = layers, batch, planes
        self.grouping_arg = grouping
        self.w = []
        # two-plane weights are the dense format of [n, 2k] (the planes' groups interleaved)
        for li in range(layers):
            self.w.append([(synth.torch_code_words(n, planes * k, gen, dev),
                            synth.torch_scales_f16(n, planes * k, gen, dev), n, k) for _, n, k in FUSED])
            if li % 16 == 15:
                log(f"  generated {li + 1}/{layers} layers")
        self.make_acts(batch, gen, dev)

    def make_acts(self, batch, gen, dev):
        import torch

        from ternary_weights_hadamard_amd import synth

        from ternary_weights_hadamard_amd import tb

        self.batch = batch
        # Every product splits its K over several workgroups per tile; the parts
        # are added by the rotation launch that follows (tb_fwht_segment.x_parts),
        # so the split costs no launch of its own
        self.parts = [gemv_parts(batch, self.planes * k // 128) for _, n, k in FUSED]
        self.grouping = self.grouping_arg
        if self.grouping == "auto":
            self.grouping = auto_grouping(batch, self.planes)
        self.x = [synth.torch_gaussian_bf16((batch, k), gen, dev) for _, n, k in FUSED]
        self.act = [torch.empty(tb.tb_act8_bytes(batch, k), dtype=torch.uint8, device=dev) for _, n, k in FUSED]
        self.yr = [torch.empty((p, batch, n) if p > 1 else (batch, n), dtype=torch.float32, device=dev)
                   for p, (_, n, k) in zip(self.parts, FUSED)]
        self.y = [torch.empty((batch, n), dtype=torch.float32, device=dev) for _, n, k in FUSED]

    def gemv_calls(self, layer):
        """The layer's GEMVs as grouped launches: all four in one ("layer"), or
        the three d_model-input projections together and the long-K down
        projection on its own ("split")."""
        from ternary_weights_hadamard_amd import tb

        segs = [(self.act[j], codes, scales, self.batch, self.yr[j], self.planes, self.parts[j])
                for j, (codes, scales, n, k) in enumerate(layer)]
        if self.grouping == "layer":
            tb.tb_ternary_gemv_multi(segs)
        elif self.grouping == "none":
            for sg in segs:
                tb.tb_ternary_gemv_multi([sg])
        else:
            tb.tb_ternary_gemv_multi([s for s, (_, _, _, k) in zip(segs, layer) if k == D])
            tb.tb_ternary_gemv_multi([s for s, (_, _, _, k) in zip(segs, layer) if k != D])

    def step(self, merged=True):
        """One decode step.  Per layer boundary one launch rotates the previous
        layer's four outputs back (fp32) and rotates and encodes this layer's
        four inputs (bf16 -> act8), the place where a model's inter-layer work
        (residual add, norm) sits; then the grouped GEMV launches; after the
        last layer one launch rotates its outputs back.  merged=False makes the
        input and output rotations separate launches (two per layer)."""
        from ternary_weights_hadamard_amd import tb

        rot_in = list(zip(self.x, self.act))
        rot_out = list(zip(self.yr, self.y, self.parts))
        for li, layer in enumerate(self.w):
            if merged:
                tb.tb_fwht128_multi((rot_out if li > 0 else []) + rot_in)
            else:
                tb.tb_fwht128_multi(rot_in)
            self.gemv_calls(layer)
            if not merged:
                tb.tb_fwht128_multi(rot_out)
        if merged:
            tb.tb_fwht128_multi(rot_out)

    def step_sequential(self):
        """The same work in the order a decoder layer imposes: every projection's
        rotation, GEMV and back-rotation one after the other, one launch each."""
        from ternary_weights_hadamard_amd import tb

        for layer in self.w:
            for j, (codes, scales, n, k) in enumerate(layer):
                yr = self.yr[j][0] if self.parts[j] > 1 else self.yr[j]  # one product, no parts
                tb.tb_fwht128(self.x[j], y=self.act[j])
                tb.tb_ternary_gemv(self.act[j], codes, scales, self.batch, y=yr)
                tb.tb_fwht128(yr, y=self.y[j])

    def gemv_only(self):
        for layer in self.w:
            self.gemv_calls(layer)

    def packed_bytes(self):
        return self.planes * sum(packed_bytes(n, k) for layer in self.w for _, _, n, k in layer)

    def gemv_times(self, replays=5):
        """The grouped GEMV launches of one step (one per layer) captured in a
        HIP graph on their own stream and timed with events on that stream over
        `replays` replays; returns (algorithmic bytes per launch, ms per launch,
        launches per step)."""
        ms, _, g = time_graph(self.gemv_only, replays, 1)
        del g
        per_layer = {"layer": 1, "split": 2, "none": 4}[self.grouping]
        nl = per_layer * len(self.w)
        per_launch_bytes = sum(gemv_bytes(n, k, self.batch, self.planes) for _, _, n, k in self.w[0]) / per_layer
        return per_launch_bytes, ms / (replays * nl), nl


class DecodeMidBatch:
    """The decode step of a DecodeStack's weights for a small batch (M <= 16)
    on the mid-batch GEMM: per layer one rotation launch (the previous
    outputs back, fp32; this layer's inputs in, bf16) and one grouped launch
    of the layer's four products (tb_ternary_gemm_multi, fp32 out)."""

    def __init__(self, stack, batch, gen, dev):
        import torch

        from ternary_weights_hadamard_amd import synth

        self.stack, self.batch = stack, batch
        self.x = [synth.torch_gaussian_bf16((batch, k), gen, dev) for _, n, k in FUSED]
        self.xr = [torch.empty((batch, k), dtype=torch.bfloat16, device=dev) for _, n, k in FUSED]
        self.y = [torch.empty((batch, n), dtype=torch.float32, device=dev) for _, n, k in FUSED]
        self.yo = [torch.empty((batch, n), dtype=torch.float32, device=dev) for _, n, k in FUSED]

    def gemm_call(self, layer):
        from ternary_weights_hadamard_amd import tb

        tb.tb_ternary_gemm_multi([(self.xr[j], codes, scales, self.y[j])
                                  for j, (codes, scales, n, k) in enumerate(layer)])

    def step(self):
        from ternary_weights_hadamard_amd import tb

        rot_in = list(zip(self.x, self.xr))
        rot_out = list(zip(self.y, self.yo))
        for li, layer in enumerate(self.stack.w):
            tb.tb_fwht128_multi((rot_out if li > 0 else []) + rot_in)
            self.gemm_call(layer)
        tb.tb_fwht128_multi(rot_out)

    def gemm_only(self):
        for layer in self.stack.w:
            self.gemm_call(layer)

    def gemm_times(self, replays=5):
        """(algorithmic bytes per launch, ms per launch) of the grouped launches."""
        ms, _, g = time_graph(self.gemm_only, replays, 1)
        del g
        per_launch = sum(packed_bytes(n, k) + 2 * self.batch * k + 4 * self.batch * n for *_, n, k in self.stack.w[0])
        return per_launch, ms / (replays * len(self.stack.w))


def gemv24_bytes(n, k, b=1):
    """Algorithmic bytes of one 2:4 GEMV: meta N K/8, signs N K/16, scales N K/64,
    bf16 x and fp32 y."""
    return n * k // 8 + n * k // 16 + n * k // 64 + 2 * b * k + 4 * b * n


class Decode24Stack:
    """The decode step of DecodeStack over 2:4 weights: per layer one launch
    rotates the previous layer's outputs back (fp32) and this layer's inputs
    (bf16), then one grouped 2:4 GEMV launch covers the layer's four
    products."""

    def __init__(self, layers, batch, gen, dev):
        import torch

        from ternary_weights_hadamard_amd import synth

        self.batch = batch
        self.w = []
        for li in range(layers):
            self.w.append([synth.torch_24(n, k, gen, dev) + (synth.torch_scales24_f16(n, k, gen, dev), n, k)
                           for _, n, k in FUSED])
            if li % 16 == 15:
                log(f"  generated {li + 1}/{layers} 2:4 layers")
        self.x = [synth.torch_gaussian_bf16((batch, k), gen, dev) for _, n, k in FUSED]
        self.xr = [torch.empty((batch, k), dtype=torch.bfloat16, device=dev) for _, n, k in FUSED]
        self.y = [torch.empty((batch, n), dtype=torch.float32, device=dev) for _, n, k in FUSED]
        self.yo = [torch.empty((batch, n), dtype=torch.float32, device=dev) for _, n, k in FUSED]

    def gemv_call(self, layer):
        from ternary_weights_hadamard_amd import tb

        tb.tb_ternary24_gemv_multi([(self.xr[j], meta, signs, sc, self.y[j])
                                    for j, (meta, signs, sc, n, k) in enumerate(layer)])

    def step(self):
        from ternary_weights_hadamard_amd import tb

        rot_in = list(zip(self.x, self.xr))
        rot_out = list(zip(self.y, self.yo))
        for li, layer in enumerate(self.w):
            tb.tb_fwht128_multi((rot_out if li > 0 else []) + rot_in)
            self.gemv_call(layer)
        tb.tb_fwht128_multi(rot_out)

    def gemv_only(self):
        for layer in self.w:
            self.gemv_call(layer)

    def packed_bytes(self):
        return sum(gemv24_bytes(n, k, 0) for layer in self.w for *_, n, k in layer)

    def gemv_times(self, replays=5):
        """(algorithmic bytes per launch, ms per launch, launches per step) of
        the grouped 2:4 launches, graph-replayed on their own stream."""
        ms, _, g = time_graph(self.gemv_only, replays, 1)
        del g
        per_launch = sum(gemv24_bytes(n, k, self.batch) for *_, n, k in self.w[0])
        return per_launch, ms / (replays * len(self.w)), len(self.w)


def time_graph(fn, steps, warmup):
    """Capture fn() in a HIP graph, replay `warmup` times untimed, then time
    exactly `steps` replays bracketed by synchronisations; returns ms total."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager pass (first-touch, library load)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3
    return t0.elapsed_time(t1), wall, g


def gpu_state():
    """Clocks and power of the GPU from `rocm-smi --json` (a child process,
    10 s limit): the card's entries whose names mention a clock or power, or
    the error text when the tool is unavailable."""
    import json
    import subprocess

    try:
        r = subprocess.run(["/opt/rocm/bin/rocm-smi", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=10)
        data = json.loads(r.stdout)
    except Exception as e:  # missing tool, timeout, no JSON
        return {"error": str(e)[:200]}
    out = {}
    for card, vals in data.items():
        if isinstance(vals, dict):
            out[card] = {k: v for k, v in vals.items() if "clk" in k.lower() or "power" in k.lower()}
    return out


def time_graph_replays(fn, replays, warmup=2):
    """fn() captured in a HIP graph, replayed `warmup` times untimed, then
    `replays` times with HIP events around each replay; returns the ms of
    every replay."""
    import torch

    _, _, g = time_graph(fn, 1, warmup)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(replays):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    out = [ev[i].elapsed_time(ev[i + 1]) for i in range(replays)]
    del g
    return out


def replay_stats(fn, replays, calls=1):
    """fn() in a HIP graph replayed `replays` times (time_graph_replays):
    (median, p10, p90) ms per call when fn makes `calls` calls."""
    reps = sorted(time_graph_replays(fn, replays))
    pick = lambda f: reps[min(len(reps) - 1, int(f * len(reps)))] / calls
    return pick(0.5), pick(0.1), pick(0.9)


def time_eager(fn, iters, warm_s=0.1):
    """ms per call of fn over `iters` back-to-back calls, after calling it for at
    least warm_s seconds (the first calls of a process run at lower clocks)."""
    import time

    import torch

    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_s:
            break
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def extra_phases(gen, dev, quick):
    """Timings of the other rows of the path, each on its own synthetic input."""
    import torch

    from ternary_weights_hadamard_amd import synth, tb

    out = {}
    # prefill GEMM, M = 2048, both FFN shapes (bf16 out)
    m = 2048
    gemm = {}
    for k, n in ((D, F), (F, D)):
        codes = synth.torch_code_words(n, k, gen, dev)
        scales = synth.torch_scales_f16(n, k, gen, dev)
        x = synth.torch_gaussian_bf16((m, k), gen, dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        reps = 3 if quick else 12
        ms, ms10, ms90 = replay_stats(lambda: [tb.tb_ternary_gemm(x, codes, scales, y=y) for _ in range(8)], reps, 8)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        # the same product through the split-K entry point (the library picks
        # the split count; one pass when splitting does not pay)
        wsb = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
        work = torch.empty(max(wsb // 4, 4), dtype=torch.float32, device=dev)
        ms_k, mk10, mk90 = replay_stats(
            lambda: [tb.tb_ternary_gemm_splitk(x, codes, scales, y=y, workspace=work) for _ in range(8)], reps, 8)
        tf_k = 2.0 * m * n * k / (ms_k * 1e-3) / 1e12
        gemm[f"{k}x{n}"] = {"ms": round(ms, 4), "ms_p10_p90": [round(ms10, 4), round(ms90, 4)],
                            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_MFMA_TFLOPS, 4),
                            "splitk_ms": round(ms_k, 4), "splitk_ms_p10_p90": [round(mk10, 4), round(mk90, 4)],
                            "splitk_splits": wsb // (m * n * 4) if wsb else 1,
                            "splitk_tflops": round(tf_k, 1), "splitk_frac_of_peak": round(tf_k / PEAK_MFMA_TFLOPS, 4)}
        log(f"  prefill GEMM M={m} K={k} N={n}: {ms:.3f} ms, {tf:.1f} TFLOP/s; split-K entry "
            f"({gemm[f'{k}x{n}']['splitk_splits']} splits) {ms_k:.3f} ms, {tf_k:.1f} TFLOP/s")
        del codes, scales, x, y, work
    out["prefill_gemm"] = {"workload": "M=2048, (K,N) = (5120,17408) and (17408,5120), bf16 out; tb_ternary_gemm "
                                       "(one pass) and tb_ternary_gemm_splitk (caller workspace); median (p10, p90) "
                                       "over graph replays of 8 calls back to back",
                           "peak_tflops": PEAK_MFMA_TFLOPS, **gemm}

    # the same GEMMs with the output rotated back in the epilogue, against the
    # product followed by a separate rotation launch
    rot = {}
    for k, n in ((D, F), (F, D)):
        codes = synth.torch_code_words(n, k, gen, dev)
        scales = synth.torch_scales_f16(n, k, gen, dev)
        x = synth.torch_gaussian_bf16((m, k), gen, dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        yf = torch.empty((m, n), dtype=torch.float32, device=dev)
        reps = 3 if quick else 10
        ms_f = replay_stats(lambda: [tb.tb_ternary_gemm_rotated(x, codes, scales, y=y) for _ in range(8)], reps, 8)[0]
        ms_s = replay_stats(lambda: [(tb.tb_ternary_gemm(x, codes, scales, y=yf), tb.tb_fwht128(yf, y=y))
                                     for _ in range(8)], reps, 8)[0]
        rot[f"{k}x{n}"] = {"fused_ms": round(ms_f, 4), "separate_ms": round(ms_s, 4),
                           "fused_tflops": round(2.0 * m * n * k / (ms_f * 1e-3) / 1e12, 1)}
        log(f"  rotated GEMM M={m} K={k} N={n}: fused {ms_f:.3f} ms, product + rotation {ms_s:.3f} ms")
        del codes, scales, x, y, yf
    out["prefill_gemm_rotated"] = {"workload": "M=2048, both shapes, y = R_N y' in bf16: fused (tb_ternary_gemm_rotated) "
                                               "vs tb_ternary_gemm fp32 + tb_fwht128", **rot}

    # mid-batch GEMM, M = 16 (the one-pass kernel for M <= 16) and 256 (split K), the three layer
    # shapes, rotated over weight copies
    mid = {}
    for k, n in ((D, D), (D, F), (F, D)):
        copies = 8
        ws = [(synth.torch_code_words(n, k, gen, dev), synth.torch_scales_f16(n, k, gen, dev)) for _ in range(copies)]
        for m in (16, 256):
            x = synth.torch_gaussian_bf16((m, k), gen, dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wsb = tb.tb_ternary_gemm_splitk_workspace(m, n, k)
            work = torch.empty(max(wsb // 4, 4), dtype=torch.float32, device=dev)

            def runm():
                for c, sc in ws:
                    tb.tb_ternary_gemm_splitk(x, c, sc, y=y, workspace=work)

            us, us10, us90 = (v * 1e3 for v in replay_stats(runm, 8 if quick else 40, copies))
            wbytes = n * k // 4 + n * k // 64
            mid[f"M{m}_{k}x{n}"] = {"us": round(us, 2), "us_p10_p90": [round(us10, 2), round(us90, 2)],
                                    "kernel": "gemm_skinny_kernel" if m <= 16 else "gemm_rw_kernel + splitk_reduce_kernel",
                                    "splits": 1 if m <= 16 else (wsb // (m * n * 4) if wsb else 1),
                                    "tflops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1),
                                    "weight_gbs": round(wbytes / (us * 1e-6) / 1e9, 1),
                                    "weight_frac_of_hbm_peak": round(wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            log(f"  mid-batch GEMM M={m} K={k} N={n}: {us:.1f} us")
            del x, y, work
        del ws
    out["midbatch_gemm"] = {"workload": "tb_ternary_gemm_splitk (M <= 16 runs the one-pass mid-batch kernel), M = 16 "
                                        "and 256, (K, N) = (5120, 5120), (5120, 17408), (17408, 5120), bf16 out, 8 weight "
                                        "copies rotated; median (p10, p90) over graph replays of the 8 launches",
                            **mid}

    # 2:4 GEMV, 17408 x 5120, batch 1, rotated over >= 1 GB of weight copies
    n, k = F, D
    copies = 64
    planes = [synth.torch_24(n, k, gen, dev) + (synth.torch_scales24_f16(n, k, gen, dev),) for _ in range(copies)]
    x = synth.torch_gaussian_bf16((1, k), gen, dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)

    def run24():
        for meta, signs, sc in planes:
            tb.tb_ternary24_gemv(x, meta, signs, sc, y=y)

    # one replay = the 64 launches back to back in a HIP graph; per-launch
    # figures from the median (and p10 / p90) over the replays
    ms, ms10, ms90 = replay_stats(run24, 10 if quick else 60, copies)
    b24 = gemv24_bytes(n, k, 1)
    out["gemv24"] = {"workload": "17408x5120 2:4, batch 1, 64 weight copies (1.16 GB) rotated",
                     "us_per_launch": round(ms * 1e3, 2), "gbs": round(b24 / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(b24 / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "us_per_launch_p10_p90": [round(ms10 * 1e3, 2), round(ms90 * 1e3, 2)],
                     "note": "median over graph replays of the 64 launches"}
    log(f"  2:4 GEMV: {ms * 1e3:.2f} us/launch (p10 {ms10 * 1e3:.2f}, p90 {ms90 * 1e3:.2f}), "
        f"{out['gemv24']['gbs']} GB/s")
    del planes

    # activation FWHT at prefill size: 2048 x 17408 bf16 -> bf16
    xa = synth.torch_gaussian_bf16((2048, F), gen, dev)
    ya = torch.empty_like(xa)
    # eager back-to-back calls: graph replays of this one-kernel call read 8 %
    # slower (25.3-26.2 against 23.6 us), the GEMM's agree with eager within 2 %
    ms = time_eager(lambda: tb.tb_fwht128(xa, y=ya), 5 if quick else 20)
    fb = 2 * 2 * 2048 * F
    out["fwht128"] = {"workload": "2048x17408 bf16 -> bf16", "us": round(ms * 1e3, 2),
                      "gbs": round(fb / (ms * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(fb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"  FWHT 2048x17408: {ms * 1e3:.1f} us, {out['fwht128']['gbs']} GB/s")
    del xa, ya

    out["ceilings"] = ceilings(dev)

    # offline quantiser streamed over the 64-layer stack (its own function)
    out["quantize_stack"] = quantize_stack(dev, 64)

    # the error-minimising rule on layer 0 of the same stack recipe
    mats = synth.LAYER_MATRICES
    g0 = torch.Generator(device=dev)
    g0.manual_seed(5000)
    ws = [synth.torch_stack_weights(n, k, g0, dev) for _, n, k in mats]
    outs = [(torch.empty((n // 16, k // 128, 128), dtype=torch.int32, device=dev),
             torch.empty((n // 16, k // 128, 16), dtype=torch.float16, device=dev)) for _, n, k in mats]

    def runq_minerr():
        for w, (c, sc) in zip(ws, outs):
            tb.tb_quantize_pack(w, fmt=tb.TB_FMT_DENSE_MINERR, codes=c, scales=sc)

    ms = time_eager(runq_minerr, 1 if quick else 2)
    nw = sum(n * k for _, n, k in mats)
    qb = nw * 4 + nw // 4 + nw // 64
    out["quantize_minerr"] = {"workload": "layer 0 of the stack recipe (7 matrices, 372,244,480 weights), "
                                          "error-minimising threshold and scale per group",
                              "ms_per_layer": round(ms, 3), "gbs": round(qb / (ms * 1e-3) / 1e9, 1),
                              "note": "every group magnitude tried as the threshold (128 x 128 compares per group)"}
    log(f"  quantise one layer, min-error rule: {ms:.3f} ms")
    del ws, outs
    return out


QUANT_BYTES_PER_WEIGHT = 4 + 1 / 4 + 1 / 64  # fp32 read, 2-bit codes and fp16 scales written


def quantize_stack(dev, layers):
    """The offline quantiser streamed over a 27B-shaped stack, layer by layer.
    Each layer's 7 fp32 matrices (Q, K, V, O 5120x5120, up and gate
    17408x5120, down 5120x17408) are drawn on the device with the stack recipe
    (N(0, 0.02^2) with 1 % of the input columns 0.02 * Student-t(3); the
    generator seeded 5000 + 8 * layer), quantised with the absmean rule and
    packed (tb_quantize_pack), and the codes and scales copied to pinned host
    memory.  The quantiser launches and the copies are timed apart with events
    on the stream; drawing the weights is outside both."""
    import torch

    from ternary_weights_hadamard_amd import synth, tb

    mats = synth.LAYER_MATRICES
    codes = [torch.empty((n // 16, k // 128, 128), dtype=torch.int32, device=dev) for _, n, k in mats]
    scales = [torch.empty((n // 16, k // 128, 16), dtype=torch.float16, device=dev) for _, n, k in mats]
    codes_h = [torch.empty(c.shape, dtype=c.dtype, pin_memory=True) for c in codes]
    scales_h = [torch.empty(x.shape, dtype=x.dtype, pin_memory=True) for x in scales]
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    q_ms, c_ms = [], []
    w0 = time.perf_counter()
    for layer in range(layers):
        gen.manual_seed(5000 + 8 * layer)
        ws = [synth.torch_stack_weights(n, k, gen, dev) for _, n, k in mats]
        if layer == 0:  # first-touch and clocks: one untimed pass over layer 0
            for w, c, sc in zip(ws, codes, scales):
                tb.tb_quantize_pack(w, codes=c, scales=sc)
        ev[0].record()
        for w, c, sc in zip(ws, codes, scales):
            tb.tb_quantize_pack(w, codes=c, scales=sc, err_flag=flag)
        ev[1].record()
        for j in range(len(mats)):
            codes_h[j].copy_(codes[j], non_blocking=True)
            scales_h[j].copy_(scales[j], non_blocking=True)
        ev[2].record()
        ev[2].synchronize()
        q_ms.append(ev[0].elapsed_time(ev[1]))
        c_ms.append(ev[1].elapsed_time(ev[2]))
        del ws
        if layer % 16 == 15:
            log(f"  quantised {layer + 1}/{layers} layers")
    wall = time.perf_counter() - w0
    nw = layers * sum(n * k for _, n, k in mats)
    packed = layers * sum(n * k // 4 + n * k // 64 for _, n, k in mats)
    tq = sum(q_ms)
    gbs = nw * QUANT_BYTES_PER_WEIGHT / (tq * 1e-3) / 1e9
    qs = sorted(q_ms)
    pct = lambda p: round(qs[min(len(qs) - 1, int(p * len(qs)))], 4)
    res = {"workload": f"{layers}-layer 27B-shaped stack (7 matrices per layer), fp32 N(0, 0.02^2) with 1 % "
                       "Student-t(3) outlier input columns drawn on the device per layer; absmean rule, 2-bit pack; "
                       "codes and scales copied to pinned host memory",
           "layers": layers, "weights": nw, "bytes_per_weight": QUANT_BYTES_PER_WEIGHT,
           "quantize_ms_total": round(tq, 3), "ms_per_layer_median": pct(0.5), "ms_per_layer_p10": pct(0.1),
           "ms_per_layer_p90": pct(0.9), "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "d2h_ms_total": round(sum(c_ms), 3), "d2h_gbs": round(packed / (sum(c_ms) * 1e-3) / 1e9, 1),
           "wall_s_with_generation": round(wall, 2), "error_flag": int(flag.item())}
    log(f"  quantise stack: {layers} layers, {tq:.2f} ms of quantiser kernels ({gbs:.1f} GB/s, "
        f"{gbs / PEAK_HBM_GBS:.3f} of HBM), D2H {sum(c_ms):.1f} ms, wall {wall:.1f} s")
    return res


PROBE_LIB = os.path.join(ROOT, "ternary_weights_hadamard_amd", "libtb_probe.so")


def probe_lib():
    """The measurement probes of include/tb_probe.h (libtb_probe.so)."""
    import ctypes

    lib = ctypes.CDLL(PROBE_LIB)
    lib.tbp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.tbp_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def _cur_stream():
    import torch

    return torch.cuda.current_stream().cuda_stream


def ceilings(dev):
    """What this device achieves with the simplest kernels (tb_probe.h): a
    streaming read of 1 GiB; reads of the byte counts of a layer's grouped
    GEMV launch (all four products) and of its two parts when split (QKV + O +
    gate/up, down), each over its own buffer, rotated over >= 1 GB of buffers
    and replayed in a HIP graph as the step is; and a register-only loop of
    bf16 matrix instructions."""
    import torch

    lib = probe_lib()
    sink = torch.empty(16384 * 256, dtype=torch.int32, device=dev)
    out = {}
    big = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(7)
    best = 0.0
    for grid in (2048, 4096, 8192):
        ms, _, g = time_graph(lambda: lib.tbp_stream_read(big.data_ptr(), big.numel() * 4, sink.data_ptr(), grid,
                                                         _cur_stream()), 10, 2)
        del g
        best = max(best, big.numel() * 4 * 10 / (ms * 1e-3) / 1e9)
    out["read_1gib_gbs"] = round(best, 1)
    del big
    first = sum(gemv_bytes(n, k, 1) for _, n, k in FUSED[:3])
    down = gemv_bytes(FUSED[3][1], FUSED[3][2], 1)
    for label, nbytes in (("read_layer_launch", first + down), ("read_first_launch", first),
                          ("read_down_launch", down)):
        nbytes = nbytes // 4096 * 4096
        copies = -(-(1 << 30) // nbytes)
        bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(7) for _ in range(copies)]
        res = {}
        for grid in (512, 2048):
            def fn():
                for b in bufs:
                    lib.tbp_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), grid, _cur_stream())
            ms, _, g = time_graph(fn, 5, 2)
            del g
            us = ms * 1e3 / (5 * copies)
            res[grid] = us
        us = min(res.values())
        out[label] = {"bytes": nbytes, "us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del bufs
    fs = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    grid, iters = 2048, 4000
    lib.tbp_mfma_bf16(fs.data_ptr(), 100, grid, _cur_stream())
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    lib.tbp_mfma_bf16(fs.data_ptr(), iters, grid, _cur_stream())
    b.record()
    torch.cuda.synchronize()
    flops = grid * 4 * iters * 4 * 2.0 * 16 * 16 * 32
    out["mfma_bf16_tflops"] = round(flops / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    log(f"  ceilings: read 1 GiB {out['read_1gib_gbs']} GB/s; layer-launch bytes {out['read_layer_launch']['us']} us, "
        f"first-launch bytes {out['read_first_launch']['us']} us, "
        f"down-launch bytes {out['read_down_launch']['us']} us; bf16 MFMA {out['mfma_bf16_tflops']} TFLOP/s")
    return out


def _calibration_copy(dev):
    """A plain device copy of CALIB_BYTES, three times: the byte counters of
    the same run are scaled by what they read for it."""
    import torch

    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


PROFILE_KINDS = ("gemv", "gemv8", "gemm", "gemv24", "quant", "midbatch", "ceiling")


def profile_pass(dev, kind):
    """Short runs for rocprofv3 counter passes, one workload each, then the
    calibration copy:
      gemv      the decode step's grouped GEMV launches over a 4-layer stack
                (weights beyond the 256 MB last-level cache), 3 times;
      gemv8     the same at batch 8;
      gemm      the prefill GEMM, M = 2048, both FFN shapes, twice each;
      gemv24    the 2:4 GEMV, 17408 x 5120, batch 1, over 16 weight copies, then
                the grouped 2:4 launches of a 4-layer 2:4 stack, 3 times;
      quant     the quantiser on one layer of the stack recipe, twice;
      midbatch  the mid-batch GEMM (M = 16) on the three layer shapes, 4 copies,
                then the grouped M = 16 launches of a 4-layer stack, 3 times;
      ceiling   the streaming-read probe over 256 MiB, 3 times."""
    import torch

    from ternary_weights_hadamard_amd import synth, tb

    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    info = {"profile_pass": kind}
    if kind in ("gemv", "gemv8"):
        stack = DecodeStack(4, 8 if kind == "gemv8" else 1, gen, dev)
        stack.step()
        torch.cuda.synchronize()
        for _ in range(3):
            stack.gemv_only()
        per_layer = {"layer": 1, "split": 2, "none": 4}[stack.grouping]
        info["grouping"] = stack.grouping
        info["algorithmic_bytes_per_launch"] = sum(gemv_bytes(n, k, stack.batch) for _, _, n, k in stack.w[0]) / per_layer
    elif kind == "gemm":
        for k, n in ((D, F), (F, D)):
            codes = synth.torch_code_words(n, k, gen, dev)
            scales = synth.torch_scales_f16(n, k, gen, dev)
            x = synth.torch_gaussian_bf16((2048, k), gen, dev)
            y = torch.empty((2048, n), dtype=torch.bfloat16, device=dev)
            for _ in range(2):
                tb.tb_ternary_gemm(x, codes, scales, y=y)
            torch.cuda.synchronize()
    elif kind == "gemv24":
        n, k = F, D
        planes = [synth.torch_24(n, k, gen, dev) + (synth.torch_scales24_f16(n, k, gen, dev),) for _ in range(16)]
        x = synth.torch_gaussian_bf16((1, k), gen, dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        for meta, signs, sc in planes:
            tb.tb_ternary24_gemv(x, meta, signs, sc, y=y)
        torch.cuda.synchronize()
        info["algorithmic_bytes_per_launch"] = gemv24_bytes(n, k, 1)
        del planes
        stack24 = Decode24Stack(4, 1, gen, dev)
        for _ in range(3):
            stack24.gemv_only()
        torch.cuda.synchronize()
        info["grouped_algorithmic_bytes_per_launch"] = sum(gemv24_bytes(n, k, 1) for *_, n, k in stack24.w[0])
    elif kind == "quant":
        g0 = torch.Generator(device=dev)
        g0.manual_seed(5000)
        for _ in range(2):
            for _, n, k in synth.LAYER_MATRICES:
                w = synth.torch_stack_weights(n, k, g0, dev)
                tb.tb_quantize_pack(w)
                torch.cuda.synchronize()
                del w
        info["algorithmic_bytes_per_weight"] = QUANT_BYTES_PER_WEIGHT
    elif kind == "midbatch":
        for k, n in ((D, D), (D, F), (F, D)):
            ws = [(synth.torch_code_words(n, k, gen, dev), synth.torch_scales_f16(n, k, gen, dev)) for _ in range(4)]
            x = synth.torch_gaussian_bf16((16, k), gen, dev)
            y = torch.empty((16, n), dtype=torch.bfloat16, device=dev)
            for c, sc in ws:
                tb.tb_ternary_gemm(x, c, sc, y=y)
            torch.cuda.synchronize()
            del ws
        # then a 4-layer stack's grouped M = 16 launches (one per layer), 3 times
        stack = DecodeStack(4, 1, gen, dev)
        mid = DecodeMidBatch(stack, 16, gen, dev)
        for _ in range(3):
            mid.gemm_only()
        torch.cuda.synchronize()
        info["grouped_algorithmic_bytes_per_launch"] = sum(packed_bytes(n, k) + 2 * 16 * k + 4 * 16 * n
                                                           for *_, n, k in stack.w[0])
    elif kind == "ceiling":
        lib = probe_lib()
        buf = torch.empty(CALIB_BYTES // 4, dtype=torch.int32, device=dev).fill_(7)
        sink = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
        for _ in range(3):
            lib.tbp_stream_read(buf.data_ptr(), CALIB_BYTES, sink.data_ptr(), 4096, _cur_stream())
        info["read_bytes_per_launch"] = CALIB_BYTES
    else:
        raise SystemExit(f"unknown profile pass {kind}; one of {PROFILE_KINDS}")
    torch.cuda.synchronize()
    _calibration_copy(dev)
    info["calibration_copy_bytes"] = CALIB_BYTES
    print(json.dumps(info), flush=True)


def summarize_pmc(out_path, dirs, command_lines, title):
    """Per-kernel means per dispatch of every counter found in the rocprofv3
    --pmc output folders `dirs` (libtb and probe kernels; FETCH_SIZE and
    WRITE_SIZE also as bytes, scaled by what each reads for the calibration
    copy of the same run)."""
    import csv
    import glob

    per = {}  # (kernel, counter) -> [values]
    calib = {}  # counter -> [values of the calibration copies]
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows = list(csv.DictReader(open(f)))
            by = {}
            for r in rows:
                key = (r.get("Dispatch_Id"), r.get("Kernel_Name", ""), r.get("Counter_Name"))
                by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
            for (_, name, counter), v in by.items():
                if "tb::" in name or "stream_read_kernel" in name or "mfma_bf16_kernel" in name:
                    short = name.replace("void ", "").replace("tb::(anonymous namespace)::", "")
                    short = short.replace("(anonymous namespace)::", "").split("(")[0]
                    per.setdefault((short, counter), []).append(v)
                elif "copy" in name.lower():
                    calib.setdefault(counter, []).append(v)
    kib = 1024.0
    scale = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = sorted(calib.get(counter, []))[-3:]
        if vals:
            scale[counter] = CALIB_BYTES / (sum(vals) / len(vals) * kib)
    lines = [f"# {title}", "# rocprofv3 counter passes on one MI355X; commands (run from the repository root):"]
    lines += [f"#   {c}" for c in command_lines]
    lines += ["# Per kernel: the mean per dispatch.  FETCH_SIZE / WRITE_SIZE are KiB per dispatch; the bytes",
              f"# column scales them by what the same counter reads for a {CALIB_BYTES >> 20} MiB device copy",
              "# (read once, written once) in the same run.", ""]
    for c, f in sorted(scale.items()):
        lines.append(f"calibration {c}: x {f:.4f}")
    lines.append("")
    lines.append("kernel | counter | dispatches | mean per dispatch | bytes per dispatch")
    for (kern, counter) in sorted(per):
        v = per[(kern, counter)]
        mean = sum(v) / len(v)
        b = f"{mean * kib * scale[counter]:.0f}" if counter in scale else ""
        lines.append(f"{kern} | {counter} | {len(v)} | {mean:.6g} | {b}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(fetch_dir, write_dir, out_path, commands):
    """Turn the FETCH_SIZE and WRITE_SIZE passes of profile_pass into HBM bytes
    per GEMV launch: each counter is scaled by what it reads for the copy of
    CALIB_BYTES (copy read = CALIB_BYTES, copy write = CALIB_BYTES)."""
    import csv
    import glob

    def load(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        per = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") != counter:
                    continue
                key = (r.get("Dispatch_Id"), r.get("Kernel_Name", ""))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        return per

    def split(per):
        gemv = [v for (_, name), v in per.items() if "gemv_staged_kernel" in name]
        copy = [v for (_, name), v in per.items() if "copy" in name.lower() and "tb::" not in name]
        copy = sorted(copy)[-3:]  # the three calibration copies are the largest copy dispatches
        return gemv, copy

    fg, fc = split(load(fetch_dir, "FETCH_SIZE"))
    wg, wc = split(load(write_dir, "WRITE_SIZE"))
    kib = 1024.0
    f_scale = CALIB_BYTES / (sum(fc) / len(fc) * kib)
    w_scale = CALIB_BYTES / (sum(wc) / len(wc) * kib)
    fetch = sum(fg) / len(fg) * kib * f_scale
    write = sum(wg) / len(wg) * kib * w_scale
    grouping = auto_grouping(1)  # what the profile pass runs
    lines = ["# HBM traffic of the grouped decode GEMV (batch 1, 27B-shaped layers,",
             f"# {GROUP_TEXT[grouping]}, K parts per tile "
             f"{'/'.join(str(gemv_parts(1, k // 128)) for _, n, k in FUSED)})",
             "# from two rocprofv3 counter passes over `python3 bench.py --profile-pass`:"]
    lines += [f"#   {c}" for c in commands]
    lines += ["# Counters are KiB per dispatch; each is scaled by what it reads for a plain",
              f"# {CALIB_BYTES >> 20} MiB device copy (torch copy_, read and written once).",
              f"gemv_dispatches_fetch = {len(fg)}", f"gemv_dispatches_write = {len(wg)}",
              f"fetch_calibration_factor = {f_scale:.4f}", f"write_calibration_factor = {w_scale:.4f}",
              f"fetch_bytes_per_launch = {fetch:.0f}", f"write_bytes_per_launch = {write:.0f}",
              f"hbm_bytes_per_launch = {fetch + write:.0f}",
              f"gemv_grouping = {grouping}",
              f"gemv_source_hash = {gemv_source_hash()}"]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_kernel_stats(stats_csv, out_path, command):
    """Short text summary of a rocprofv3 --stats kernel table: the library's
    kernels with calls, average and total duration."""
    import csv

    rows = [r for r in csv.DictReader(open(stats_csv)) if "tb::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["# rocprofv3 kernel statistics of a bench.py run on one MI355X (libtb kernels only;",
             "# the input generation outside the timed regions is left out)", f"#   {command}",
             "# kernel | calls | average us | total us | share of libtb kernel time", ""]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        short = r["Name"].replace("void ", "").replace("tb::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"{short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / total * 100:.1f}%")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---------------------------------------------------------------- CPU oracle baseline
# The oracle (plain float64 numpy, oracle/) timed on this host's cores on
# bounded samples of the workloads.  A task runs one oracle call and returns
# its elapsed seconds (and, for the quantiser, its near-threshold count); the
# all-cores runs hand the row chunks of a sample to one spawned worker process
# per core, each with one BLAS thread.

BLAS_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def _one_blas_thread():
    # the workers inherit BLAS_THREAD_VARS = 1 from the parent; numpy is loaded
    # here, before any task, and its pools are held at one thread as well
    import numpy  # noqa: F401

    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass


def _oracle_task(task):
    import numpy as np

    import oracle

    kind, args = task
    t0 = time.perf_counter()
    near = 0
    if kind == "gemv":
        oracle.matvec.gemv(*args)
    elif kind == "gemv24":
        oracle.matvec.gemv24(*args)
    elif kind == "quant":
        for blk in args:
            r = oracle.quant.quantize_dense(blk.astype(np.float64))
            near += int(oracle.quant.near_threshold(r["wr"], r["s"]).sum())
    else:
        raise ValueError(kind)
    return time.perf_counter() - t0, near


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _chunks(n_rows, parts, align=16):
    """[lo, hi) row ranges, multiples of `align`, splitting n_rows into about `parts` pieces."""
    step = max(align, (n_rows // parts + align - 1) // align * align)
    return [(lo, min(n_rows, lo + step)) for lo in range(0, n_rows, step)]


def cpu_baseline(stack, dev, max_seconds=20.0):
    """The CPU oracle on bounded samples of the decode GEMV (the headline,
    value), the 2:4 GEMV, the prefill GEMM and the quantiser, each on one
    core and on all of this host's cores (the worker count is what the
    process may use, at most 16, the CPU share of one GPU here)."""
    import multiprocessing as mp

    import numpy as np
    import torch

    from ternary_weights_hadamard_amd import synth
    import oracle

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    saved = {v: os.environ.get(v) for v in BLAS_THREAD_VARS}
    os.environ.update({v: "1" for v in BLAS_THREAD_VARS})  # inherited by the spawned workers
    try:
        pool = ctx.Pool(workers, initializer=_one_blas_thread)
    finally:
        for v, old in saved.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old
    pool.map(_oracle_task, [("quant", [])] * workers)  # workers up and importing before any timing

    def one_core(tasks):
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            return [_oracle_task(t) for t in tasks]

    def all_cores(tasks):
        t0 = time.perf_counter()
        res = pool.map(_oracle_task, tasks, chunksize=1)
        return time.perf_counter() - t0, res

    out = {}
    # decode GEMV, batch 1, layer 0's fused matrices of the stack (the same bits the GPU used),
    # x rotated by the oracle first (not timed); one core until max_seconds, all cores on the same matrices
    t1, done, names, mats = 0.0, 0, [], []
    for j, (codes, scales, n, k) in enumerate(stack.w[0]):
        c = codes.cpu().numpy().view(np.uint32)
        sc = scales.cpu().view(torch.int16).numpy().view(np.uint16)
        xb = stack.x[j][:1].cpu().view(torch.int16).numpy().view(np.uint16)
        xr = oracle.numerics.f64_to_bf16_bits(oracle.hadamard.fwht_dense(oracle.numerics.bf16_bits_to_f64(xb)))
        dt, _ = one_core([("gemv", (xr, c, sc, k))])[0]
        t1 += dt
        done += packed_bytes(n, k)
        names.append(FUSED[j][0])
        mats.append((xr, c, sc, n, k))
        log(f"  oracle GEMV {FUSED[j][0]} {n}x{k}, one core: {dt:.2f} s")
        if t1 > max_seconds:
            break
    tasks = [("gemv", (xr, c[lo // 16:hi // 16], sc[lo // 16:hi // 16], k)) for xr, c, sc, n, k in mats for lo, hi in
             _chunks(n, workers)]
    ta, _ = all_cores(tasks)
    log(f"  oracle GEMV, {workers} cores: {ta:.2f} s (one core {t1:.2f} s)")
    gemv_sample = (f"float64 numpy oracle GEMV (dequantise + matmul), batch 1, layer 0's fused matrices "
                   f"{'/'.join(names)} ({done / 1e6:.1f} MB packed)")

    # 2:4 GEMV, 17408 x 5120, batch 1: a 2048-row slice
    n24, k24 = 2048, D
    meta, signs = synth.random_24(n24, k24, seed=30)
    sc24 = synth.random_scales24_f16(n24, k24, seed=31)
    x24 = synth.gaussian_bf16((1, k24), seed=32)
    b24 = n24 * k24 // 8 + n24 * k24 // 16 + n24 * k24 // 64
    d1, _ = one_core([("gemv24", (x24, meta, signs, sc24, k24))])[0]
    da, _ = all_cores([("gemv24", (x24, meta[lo // 16:hi // 16], signs[lo // 16:hi // 16], sc24[lo // 16:hi // 16],
                                   k24)) for lo, hi in _chunks(n24, workers)])
    out["gemv24"] = {"sample": "2:4 GEMV 2048 x 5120 rows of the 17408 x 5120 shape, batch 1", "unit": "GB/s",
                     "one_core": round(b24 / d1 / 1e9, 4), "all_cores": round(b24 / da / 1e9, 4)}

    # prefill GEMM, M = 2048, K = 5120: a 512-column slice of N (the dequantised fp64 matmul)
    m, kg, ng = 2048, D, 512
    cg = synth.random_code_words(ng, kg, seed=40)
    sg = synth.random_scales_f16(ng, kg, seed=41)
    xg = synth.gaussian_bf16((m, kg), seed=42)
    fl = 2.0 * m * ng * kg
    d1, _ = one_core([("gemv", (xg, cg, sg, kg))])[0]
    da, _ = all_cores([("gemv", (xg[lo:hi], cg, sg, kg)) for lo, hi in _chunks(m, workers)])
    out["gemm"] = {"sample": "prefill GEMM M = 2048, K = 5120, a 512-wide slice of N (dequantise + float64 matmul)",
                   "unit": "GFLOP/s", "one_core": round(fl / d1 / 1e9, 2), "all_cores": round(fl / da / 1e9, 2)}

    # quantiser: 1 % of the 128 x 128 blocks of layer 0 of the stack recipe, drawn on the
    # device as the stack phase draws them; near-threshold elements counted on the way
    gen = torch.Generator(device=dev)
    gen.manual_seed(5000)
    rng = np.random.default_rng(7000)
    blocks, total_blocks = [], 0
    for _, n, k in synth.LAYER_MATRICES:
        w = synth.torch_stack_weights(n, k, gen, dev)
        nb = (n // 128) * (k // 128)
        total_blocks += nb
        for b in rng.choice(nb, max(1, nb // 100), replace=False):
            a, c = divmod(int(b), k // 128)
            blocks.append(w[128 * a:128 * (a + 1), 128 * c:128 * (c + 1)].cpu().numpy())
        del w
    per = (len(blocks) + workers - 1) // workers
    d1, near1 = one_core([("quant", blocks)])[0]
    da, res = all_cores([("quant", blocks[i:i + per]) for i in range(0, len(blocks), per)])
    qw = len(blocks) * 128 * 128
    stack_weights = 64 * sum(n * k for _, n, k in synth.LAYER_MATRICES)
    frac = len(blocks) / total_blocks
    out["quantize"] = {"sample": f"{len(blocks)} random 128 x 128 blocks ({frac:.4f} of layer 0) of the stack recipe",
                       "unit": "GB/s", "bytes_per_weight": QUANT_BYTES_PER_WEIGHT,
                       "one_core": round(qw * QUANT_BYTES_PER_WEIGHT / d1 / 1e9, 5),
                       "all_cores": round(qw * QUANT_BYTES_PER_WEIGHT / da / 1e9, 5),
                       "near_threshold_in_sample": near1,
                       "near_threshold_per_weight": near1 / qw,
                       "near_threshold_projected_64_layers": round(near1 / qw * stack_weights)}
    pool.close()
    pool.join()
    return {"value": round(done / ta / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": gemv_sample + f", {workers} worker processes with one BLAS thread each, {ta:.2f} s",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)),
            "one_core": {"value": round(done / t1 / 1e9, 4), "unit": "GB/s", "seconds": round(t1, 2)},
            "other_configs": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--gemv-parts", type=int, default=None, choices=(1, 2, 4, 8),
                    help="K parts per tile of the decode GEMVs, added by the output rotation "
                         "(default: 8 for the down projection, 4 for the others)")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-extra", action="store_true", help="skip the extra phases")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="fewer iterations in the extra phases")
    ap.add_argument("--grouping", choices=("auto", "layer", "split", "none"), default="auto",
                    help="GEMV launches per layer: one over all four matrices, two (d_model-input ones, then down), "
                         "or one per matrix; auto: one when every product is split into K parts, else two")
    ap.add_argument("--profile-pass", nargs="?", const="gemv", choices=PROFILE_KINDS,
                    help="short run of one workload for rocprofv3 counter passes (default: gemv)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar=("OUT", "DIR"),
                    help="write a per-kernel summary of rocprofv3 --pmc output folders: OUT DIR [DIR ...]")
    ap.add_argument("--pmc-title", default="counter summary", help="title line of --summarize-pmc")
    ap.add_argument("--pmc-command", action="append", default=[], help="a command to record in --summarize-pmc")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc output folders")
    ap.add_argument("--summarize-kernel-stats", nargs=2, metavar=("STATS_CSV", "OUT"),
                    help="write a text summary of a rocprofv3 --stats kernel table")
    ap.add_argument("--stats-command", default=None,
                    help="the profiled command to record in the kernel-stats summary (default: the decode-step trace)")
    args = ap.parse_args()
    globals()["GEMV_PARTS"] = args.gemv_parts

    if args.summarize_kernel_stats:
        cmd = args.stats_command or ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                                     "python3 bench.py --steps 5 --warmup 1 --no-extra --no-cpu-baseline")
        summarize_kernel_stats(args.summarize_kernel_stats[0], args.summarize_kernel_stats[1], cmd)
        return

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1:], args.pmc_command, args.pmc_title)
        return

    if args.summarize_counters:
        cmds = ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -- python3 bench.py --profile-pass",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -- python3 bench.py --profile-pass",
                "python3 bench.py --summarize-counters <fetch_dir> <write_dir>"]
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], TRAFFIC_FILE, cmds)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the products would shard "
              "by output rows, or by K with one all-reduce of the partial outputs); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from ternary_weights_hadamard_amd import tb

    tb.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_pass:
        profile_pass(dev, args.profile_pass)
        return
    gen = torch.Generator(device=dev)
    gen.manual_seed(29)

    log(f"building {args.layers}-layer stack (batch {args.batch}) on {torch.cuda.get_device_name(0)}")
    stack = DecodeStack(args.layers, args.batch, gen, dev, args.grouping)
    step_bytes = stack.packed_bytes()
    log(f"packed weights per step: {step_bytes / 1e9:.3f} GB")

    torch.cuda.synchronize()
    state_before = gpu_state()
    ms_total, wall_ms, graph = time_graph(stack.step, args.steps, args.warmup)
    state_after = gpu_state()
    ms_step = ms_total / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"decode step: {ms_step:.4f} ms ({value:.1f} GB/s packed); wall {wall_ms / args.steps:.4f} ms/step")
    del graph

    # dominant kernel: the grouped GEMV (one launch per layer), timed with
    # events on the stream its graph replays on
    gb, gms, nl = stack.gemv_times()
    achieved = gb / (gms * 1e-3) / 1e9
    log(f"GEMV: {nl} launches per step, avg {gms * 1e3:.2f} us per launch, {achieved:.1f} GB/s algorithmic")

    extra = {"step_wall_ms": round(wall_ms / args.steps, 4),
             "gemv_avg_launch_us": round(gms * 1e3, 3), "gemv_launches_per_step": nl,
             "gpu_state": {"note": "rocm-smi clocks and power just before and after the timed decode steps",
                           "before": state_before, "after": state_after}}
    # the same step with the input and output rotations as separate launches
    if not args.no_extra:
        ms_apart, _, ga = time_graph(lambda: stack.step(merged=False), max(3, args.steps // 2), 2)
        del ga
        ms_apart /= max(3, args.steps // 2)
        extra["decode_rotations_apart"] = {"ms_per_step": round(ms_apart, 4),
                                           "gbs_packed": round(step_bytes / (ms_apart * 1e-3) / 1e9, 1),
                                           "note": "input and output rotations as two launches per layer"}
        log(f"decode step, rotations apart: {ms_apart:.4f} ms")
    # the same step with a decoder layer's ordering (no grouping across projections)
    if not args.no_extra:
        ms_seq, _, gs = time_graph(stack.step_sequential, max(3, args.steps // 2), 2)
        del gs
        ms_seq /= max(3, args.steps // 2)
        extra["decode_sequential"] = {"ms_per_step": round(ms_seq, 4),
                                      "gbs_packed": round(step_bytes / (ms_seq * 1e-3) / 1e9, 1),
                                      "note": "each projection rotated, multiplied and rotated back in order, "
                                              "12 launches per layer"}
        log(f"decode step, sequential order: {ms_seq:.4f} ms ({step_bytes / (ms_seq * 1e-3) / 1e9:.1f} GB/s)")
    # batch 8 decode
    if not args.no_extra:
        stack.make_acts(8, gen, dev)
        ms8, _, g8 = time_graph(stack.step, max(3, args.steps // 2), 2)
        del g8
        ms8 /= max(3, args.steps // 2)
        gb8, gms8, nl8 = stack.gemv_times()
        extra["decode_batch8"] = {"ms_per_step": round(ms8, 4), "gbs_packed": round(step_bytes / (ms8 * 1e-3) / 1e9, 1),
                                  "gemv_gbs_algorithmic": round(gb8 / (gms8 * 1e-3) / 1e9, 1),
                                  "gemv_frac_of_hbm_peak": round(gb8 / (gms8 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"decode batch 8: {ms8:.4f} ms/step, GEMV {extra['decode_batch8']['gemv_gbs_algorithmic']} GB/s")
        # batch 16: sixteen activation rows (the mid-batch M = 16 case) through the
        # same layer-grouped decode step
        stack.make_acts(16, gen, dev)
        ms16, _, g16 = time_graph(stack.step, max(3, args.steps // 2), 2)
        del g16
        ms16 /= max(3, args.steps // 2)
        gb16, gms16, _ = stack.gemv_times()
        extra["decode_batch16"] = {"ms_per_step": round(ms16, 4),
                                   "gbs_packed": round(step_bytes / (ms16 * 1e-3) / 1e9, 1),
                                   "gemv_gbs_algorithmic": round(gb16 / (gms16 * 1e-3) / 1e9, 1),
                                   "gemv_frac_of_hbm_peak": round(gb16 / (gms16 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "note": "16 rows per step: the M = 16 products of a layer in one grouped launch"}
        log(f"decode batch 16: {ms16:.4f} ms/step, GEMV {extra['decode_batch16']['gemv_gbs_algorithmic']} GB/s")
        stack.make_acts(args.batch, gen, dev)
        # the same batch-16 step on the mid-batch GEMM, one grouped launch per layer
        mid = DecodeMidBatch(stack, 16, gen, dev)
        msm, _, gm = time_graph(mid.step, max(3, args.steps // 2), 2)
        del gm
        msm /= max(3, args.steps // 2)
        gbm, gmsm = mid.gemm_times()
        extra["decode_batch16_midbatch_gemm"] = {
            "ms_per_step": round(msm, 4), "gbs_packed": round(step_bytes / (msm * 1e-3) / 1e9, 1),
            "gemm_us_per_layer_launch": round(gmsm * 1e3, 2),
            "gemm_gbs_algorithmic": round(gbm / (gmsm * 1e-3) / 1e9, 1),
            "gemm_frac_of_hbm_peak": round(gbm / (gmsm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "note": "16 rows per step on the mid-batch kernel (tb_ternary_gemm_multi), bf16 activations"}
        log(f"decode batch 16, mid-batch GEMM: {msm:.4f} ms/step, {gmsm * 1e3:.2f} us per layer launch, "
            f"{extra['decode_batch16_midbatch_gemm']['gemm_gbs_algorithmic']} GB/s")
        del mid
        # the same decode step over two-plane weights (residual second plane)
        two = DecodeStack(args.layers, args.batch, gen, dev, args.grouping, planes=2)
        ms2, _, g2 = time_graph(two.step, max(3, args.steps // 2), 2)
        del g2
        ms2 /= max(3, args.steps // 2)
        gb2, gms2, _ = two.gemv_times()
        tb2 = two.packed_bytes()
        extra["decode_two_plane"] = {"ms_per_step": round(ms2, 4), "packed_bytes_per_step": tb2,
                                     "gbs_packed": round(tb2 / (ms2 * 1e-3) / 1e9, 1),
                                     "gemv_gbs_algorithmic": round(gb2 / (gms2 * 1e-3) / 1e9, 1),
                                     "gemv_frac_of_hbm_peak": round(gb2 / (gms2 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     "gemv_avg_launch_us": round(gms2 * 1e3, 3)}
        log(f"decode two-plane: {ms2:.4f} ms/step, GEMV {extra['decode_two_plane']['gemv_gbs_algorithmic']} GB/s")
        del two
        torch.cuda.empty_cache()
        # the same decode step over 2:4 weights (one grouped 2:4 launch per layer)
        d24 = Decode24Stack(args.layers, args.batch, gen, dev)
        ms24, _, g24 = time_graph(d24.step, max(3, args.steps // 2), 2)
        del g24
        ms24 /= max(3, args.steps // 2)
        gb24, gms24, _ = d24.gemv_times()
        tb24 = d24.packed_bytes()
        extra["decode_24"] = {"ms_per_step": round(ms24, 4), "packed_bytes_per_step": tb24,
                              "gbs_packed": round(tb24 / (ms24 * 1e-3) / 1e9, 1),
                              "gemv_bytes_per_launch": gb24,
                              "gemv_gbs_algorithmic": round(gb24 / (gms24 * 1e-3) / 1e9, 1),
                              "gemv_frac_of_hbm_peak": round(gb24 / (gms24 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "gemv_avg_launch_us": round(gms24 * 1e3, 3),
                              "note": "2:4 weights (1.625 bit), one grouped 2:4 GEMV launch per layer"}
        log(f"decode 2:4: {ms24:.4f} ms/step, GEMV {gms24 * 1e3:.2f} us per layer launch, "
            f"{extra['decode_24']['gemv_gbs_algorithmic']} GB/s")
        del d24
        torch.cuda.empty_cache()
        extra.update(extra_phases(gen, dev, args.quick))

    traffic = recorded_traffic(stack.grouping)
    result = {
        "metric": "ternary GEMV packed-weight GB/s (% HBM peak); prefill GEMM TFLOP/s (% MFMA)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4,f32acc",
        "data": "synthetic",
        "config": {"workload": f"decode GEMV, {args.layers}-layer 27B-shaped stack (d_model 5120, d_ff 17408; fused QKV, O, "
                               f"gate/up, down), batch {args.batch}, FWHT128 in and out, HIP graph",
                   "layers": args.layers, "batch": args.batch, "packed_bytes_per_step": step_bytes,
                   "gemv_k_parts": [gemv_parts(args.batch, k // 128) for _, n, k in FUSED],
                   "gemv_grouping": GROUP_TEXT[stack.grouping],
                   "code_distribution": "P(-1,0,+1) = (0.35, 0.30, 0.35)", "scales": "U(0.005, 0.05) fp16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None or args.batch != 1 else round(traffic),
                     "kernel": f"{'gemv_staged_kernel' if args.batch == 1 else 'gemv_wide_kernel'} "
                               f"({GROUP_TEXT[stack.grouping]}; each product's K split into parts per tile, "
                               "added by the next rotation launch)",
                     "bytes_per_launch": "sum over the launch's matrices of N*K/4 + N*K/64 + 2*B*K + 4*B*N"},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(stack, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
