#!/usr/bin/env python3
"""Benchmark: MoE layer forward tokens/s on one MI355X, with roofline fractions.

One step = one moe_layer_forward (route, dispatch/permute, wave-scheduled
linear1 + SwiGLU + linear2, combine) over one batch of synthetic inputs that
are already resident in HBM.  The headline workload is the long-tail decode
batch (T=128, H=4096, I=2048, E=256, top-8); the prefill batch (T=8192) is
reported alongside.  Weights are random FP4 E2M1 with power-of-two sub-block
scales and fp32 128x128 block scales (seed 0).

Roofline of the dominant kernel (the expert-FFN kernel), timed with HIP events
that the library records around it on its own stream, in an instrumented pass
of the same number of steps right after the contract loop (recording events
between kernels adds a few microseconds per step, so the contract loop runs
bare steps):
  decode:  algorithmic bytes = active experts x (FP4 codes + E8M0 sub-block
           scales + fp32 block scales) = 13,375,488 B each, against 8 TB/s;
  prefill: algorithmic FLOP = 2*T*k*3*H*I against the dense FP8 peak 5.0 PFLOP/s.
HBM traffic of the FFN (roofline.traffic) comes from the committed rocprofv3
TCC counter summary (FETCH_SIZE + WRITE_SIZE per FFN, scaled by
the same counters' reading for a plain copy kernel of known size); it is
reported only while the kernel sources hash to the value recorded with it.
Every workload record carries both roofline fractions of its FFN (HBM GB/s
on the weight bytes, FP8 TFLOP/s on the algorithmic FLOP), a cold-cache
protocol run (512 MiB of scratch written between steps, outside the per-step
HIP events, so nothing is left in the 256 MB last-level cache) and a
determinism flag (the first and the last timed step's outputs bit-identical).
Records: the headline decode batch, prefill (T=8192), the skewed batch with a
Zipf router bias (T=4096), hash routing (T=4096), the ragged batch of 64
requests and the tiny layer (T=64, H=256, I=128, E=8, k=2).
The CPU baseline is the C oracle (test infrastructure) timed on the host
cores: the whole decode batch for the headline, and a bounded sample of 16
tokens (all tokens routed) for each side record.  Its outputs are also
compared with the GPU's on the same inputs; the result is the record's
`parity` (ids and offsets bit-exact, weights, output rel-L2 and max|d|).
The weight quantiser (FP32 master -> MXFP4, one layer's experts), the layer
backward (decode and prefill) and the gate-less squared-ReLU layer at the same
parameter count (I=3072) are reported as side records.  Each workload record also carries the
per-step device time (median, p10, p90 of HIP events around each step), the
device time of each step of the layer through the separate entry points
(route, permute, expert_ffn, combine), and board power and shader clock
sampled from the amdgpu sysfs files during about a second of back-to-back
steps outside the timed region.  The weights of the large workloads (3.4 GB)
are 13x the 256 MB last-level cache, so every step streams them from HBM.

`--copy-bytes N` runs only a plain device copy of N bytes (the calibration
kernel for those counters) and prints what it did.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "MoE layer tokens/s; %HBM peak at T=128, %FP8 MFMA peak at T=8192"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 matrix


def weight_bytes_per_expert(H: int, I: int, mats: int = 3) -> int:
    """FP4 codes + E8M0 sub-block scales + fp32 block scales of gate (SwiGLU
    only), up and down."""
    return mats * (H * I // 2 + H * I // 32 + (H // 128) * (I // 128) * 4)


def ffn_flops(T: int, k: int, H: int, I: int, mats: int = 3) -> int:
    """Two grouped GEMMs: gate (SwiGLU only) and up (2*H*I each) plus down
    (2*H*I) per token-expert pair."""
    return 2 * T * k * mats * H * I


def kernel_source_hash() -> str:
    """sha256 over the sources the layer forward is built from (every file of
    the library's csrc/ except the backward kernels, v4moe_bwd.hip), in
    file-name order."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "fp4_weight_grouped_amd", "csrc", "*"))):
        if os.path.basename(f) == "v4moe_bwd.hip":
            continue
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the FFN kernel for `workload` from the committed
    counter summary, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "expert_ffn_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    row = fields.get(workload)
    if not row:
        return None
    kv = dict(x.split("=", 1) for x in row.split() if "=" in x)
    return float(kv["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in kv else None


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of nbytes (int32 elements), reps times: reads and
    writes nbytes per launch.  Used to scale the TCC byte counters."""
    import torch
    n = nbytes // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    print(json.dumps({"copy_bytes": n * 4, "launches": reps, "kernel": "torch copy_ int32"}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pct(v, q):
    return float(np.percentile(np.asarray(v, np.float64), q))


def attribution(layer, x, bias, mode, tid, reps=10):
    """Device time of each step of the layer, through the separate entry
    points (moe_route, moe_permute = x quantisation + permutation,
    moe_expert_ffn, moe_combine) with events between them; medians in ms."""
    import torch
    from fp4_weight_grouped_amd import v4moe
    T = x.shape[0]
    d = layer.dims(T)
    dev = layer.device
    P = T * layer.topk
    ids = torch.empty((T, layer.topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, layer.topk), dtype=torch.float32, device=dev)
    off = torch.empty(layer.E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(P, dtype=torch.int32, device=dev)
    pp = torch.empty(P, dtype=torch.int32, device=dev)
    xq = torch.empty((T, layer.H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, layer.H // 128), dtype=torch.float32, device=dev)
    y = torch.empty((P, layer.H), dtype=torch.int16, device=dev)
    out = torch.empty((T, layer.H), dtype=torch.int16, device=dev)
    ws = layer.workspace(T)
    steps = [
        ("route", lambda: v4moe.moe_route(d, x, layer.w_router, bias, mode, tid, ids, w, ws)),
        ("permute", lambda: v4moe.moe_permute(d, x, ids, off, sp, pp, xq, xs, ws)),
        ("expert_ffn", lambda: v4moe.moe_expert_ffn(d, xq, xs, off, sp, layer.experts, y, ws)),
        ("combine", lambda: v4moe.moe_combine(d, y, w, out)),
    ]
    times = {k: [] for k, _ in steps}
    for rep in range(reps + 2):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)]
        evs[0].record()
        for i, (_, f) in enumerate(steps):
            f()
            evs[i + 1].record()
        torch.cuda.synchronize()
        if rep >= 2:
            for i, (k, _) in enumerate(steps):
                times[k].append(evs[i].elapsed_time(evs[i + 1]))
    return {k: float(np.median(v)) for k, v in times.items()}


def read_sysfs_power_clock():
    """Best effort: average board power (W) and current shader clock (MHz) from
    the amdgpu sysfs files of the first card that has them."""
    pw = clk = None
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            f = glob.glob(dev + "/hwmon/hwmon*/power1_average") + glob.glob(dev + "/hwmon/hwmon*/power1_input")
            if f and pw is None:
                pw = int(open(f[0]).read()) / 1e6
            if clk is None and os.path.exists(dev + "/pp_dpm_sclk"):
                for line in open(dev + "/pp_dpm_sclk"):
                    if line.strip().endswith("*"):
                        clk = float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            continue
    return pw, clk


def sustained_power_clock(fn, seconds=1.0):
    """Run fn back to back for about `seconds` (not timed for the metric) and
    sample power and clock every 20 ms on a host thread."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append(read_sysfs_power_clock())
            time.sleep(0.02)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    pw = [p for p, _ in samples if p is not None]
    ck = [c for _, c in samples if c is not None]
    return dict(power_w_mean=float(np.mean(pw)) if pw else None, power_w_max=float(np.max(pw)) if pw else None,
                sclk_mhz_mean=float(np.mean(ck)) if ck else None, samples=len(samples),
                source="amdgpu sysfs (hwmon power1_average, pp_dpm_sclk), sampled every 20 ms")


SCRATCH_BYTES = 512 << 20      # written between protocol steps: 2x the 256 MB last-level cache


def run_gpu(name, steps, warmup, layer_cache, extras=True, scratch=None):
    """Time one workload.  The contract loop: `steps` back-to-back layer
    forwards, bracketed by synchronisations (ms_per_step, tokens/s).  The
    instrumented pass: the same steps with HIP events around each step and
    around each FFN launch (the roofline's kernel time).  The cold-cache
    protocol loop: the same number of steps, each preceded by a write of
    SCRATCH_BYTES (outside its HIP events), so weights and activations come
    from HBM; per-step device times from those events.  Determinism: the
    output of every pass must equal that of a step run before them, bit for
    bit."""
    import torch
    from fp4_weight_grouped_amd import inputs, v4moe

    inp = inputs.make(name)
    d = inp.dims
    dev = "cuda:0"
    key = (d.H, d.I, d.E, d.topk, d.act)
    if key not in layer_cache:
        layer_cache.clear()
        torch.cuda.empty_cache()
        t0 = time.time()
        dims = v4moe.dims(d.T, d.H, d.I, d.E, d.topk, d.act)
        ex = v4moe.upload_experts(inp.experts, dims, dev)
        layer_cache[key] = v4moe.MoELayer(d.H, d.I, d.E, d.topk, ex,
                                          torch.from_numpy(inp.w_router).to(dev), dev, act=d.act)
        log(f"[bench] uploaded + prepacked weights in {time.time() - t0:.1f}s")
    layer = layer_cache[key]
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    tid = None if inp.token_ids is None else torch.from_numpy(inp.token_ids).to(dev)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)

    def new_events(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:    # torch creates the HIP event on first record
            a.record()
            b.record()
        return evs

    for _ in range(warmup):
        layer.forward(x, bias, inp.mode, tid, out=out)
    torch.cuda.synchronize()
    first = layer.forward(x, bias, inp.mode, tid)[0]
    # the contract loop: `steps` bare layer forwards back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        _, ids, w, off = layer.forward(x, bias, inp.mode, tid, out=out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    deterministic = bool(torch.equal(first, out))
    ms_step = (t1 - t0) * 1e3 / steps
    # the instrumented pass right after it: HIP events around each step and,
    # recorded by the library on its launch stream, around each FFN launch
    # (recording them adds a few microseconds between kernels, so they are
    # kept out of the contract loop)
    ev, sev = new_events(steps), new_events(steps)
    torch.cuda.synchronize()
    for i in range(steps):
        sev[i][0].record()
        v4moe.moe_time_next_ffn(*ev[i])
        layer.forward(x, bias, inp.mode, tid, out=out)
        sev[i][1].record()
    torch.cuda.synchronize()
    deterministic = deterministic and bool(torch.equal(first, out))
    ffn_all = [a.elapsed_time(b) for a, b in ev]
    step_all = [a.elapsed_time(b) for a, b in sev]
    ffn_ms = float(np.mean(ffn_all))

    # cold-cache protocol: SCRATCH_BYTES written between steps, outside the events
    cold = None
    if scratch is not None:
        cev, csev = new_events(steps), new_events(steps)
        torch.cuda.synchronize()
        for i in range(steps):
            scratch.fill_(i & 0xFF)
            csev[i][0].record()
            v4moe.moe_time_next_ffn(*cev[i])
            layer.forward(x, bias, inp.mode, tid, out=out)
            csev[i][1].record()
        torch.cuda.synchronize()
        deterministic = deterministic and bool(torch.equal(first, out))
        cs = [a.elapsed_time(b) for a, b in csev]
        cf = [a.elapsed_time(b) for a, b in cev]
        cold = dict(scratch_bytes=scratch.numel(), step_device_ms=dict(median=float(np.median(cs)), p10=pct(cs, 10),
                                                                       p90=pct(cs, 90)),
                    ffn_device_ms=dict(median=float(np.median(cf)), p10=pct(cf, 10), p90=pct(cf, 90)),
                    tokens_per_s=d.T / (float(np.median(cs)) / 1e3))
    attr = attribution(layer, x, bias, inp.mode, tid) if extras else None
    pc = sustained_power_clock(lambda: layer.forward(x, bias, inp.mode, tid, out=out)) if extras else None
    counts = np.diff(off.cpu().numpy())
    n_active = int((counts > 0).sum())
    mats = 3 if d.act == inputs.ACT_SWIGLU else 2
    wbytes = n_active * weight_bytes_per_expert(d.H, d.I, mats)
    flops = ffn_flops(d.T, d.topk, d.H, d.I, mats)
    act = {inputs.ACT_SWIGLU: "swiglu", inputs.ACT_RELU2: "relu2 (gate-less)", inputs.ACT_RELU: "relu (gate-less)"}
    hbm = wbytes / (ffn_ms / 1e3) / 1e9
    tfl = flops / (ffn_ms / 1e3) / 1e12
    r = dict(workload=name, T=d.T, H=d.H, I=d.I, E=d.E, topk=d.topk, activation=act[d.act],
             routing="hash" if inp.mode == inputs.ROUTE_HASH else ("learned + zipf bias" if inp.bias is not None
                                                                    else "learned"),
             ms_per_step=ms_step, tokens_per_s=d.T / (ms_step / 1e3), ffn_ms=ffn_ms, active_experts=n_active,
             load_max_over_mean=float(counts.max() / counts.mean()), idle_experts=int((counts == 0).sum()),
             weight_bytes=wbytes, ffn_flop=flops, ffn_hbm_gbs=hbm, ffn_tflops=tfl,
             roofline_hbm=dict(achieved=hbm, peak=HBM_PEAK_GBS, unit="GB/s", frac=hbm / HBM_PEAK_GBS,
                               work="FP4 codes + E8M0 + fp32 block scales of the active experts"),
             roofline_mfma=dict(achieved=tfl, peak=FP8_DENSE_PEAK_TFLOPS, unit="TFLOP/s",
                                frac=tfl / FP8_DENSE_PEAK_TFLOPS, work=f"2*T*k*{mats}*H*I FLOP"),
             deterministic=deterministic,
             step_device_ms=dict(median=float(np.median(step_all)), p10=pct(step_all, 10), p90=pct(step_all, 90)),
             ffn_device_ms=dict(median=float(np.median(ffn_all)), p10=pct(ffn_all, 10), p90=pct(ffn_all, 90)),
             cold_cache=cold, attribution_ms=attr, power_clock=pc)
    r["_gpu"] = dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), offsets=off.cpu().numpy(), out=out.cpu().numpy())
    log(f"[bench] {name}: {ms_step:.3f} ms/step, ffn {ffn_ms:.3f} ms, "
        f"{hbm:.0f} GB/s, {tfl:.0f} TFLOP/s, active {n_active}, deterministic {deterministic}")
    log(f"[bench] {name}: step device ms median {r['step_device_ms']['median']:.3f} "
        f"(p10 {r['step_device_ms']['p10']:.3f}, p90 {r['step_device_ms']['p90']:.3f})"
        + (f"; cold-cache median {cold['step_device_ms']['median']:.3f}" if cold else ""))
    if extras:
        log(f"[bench] {name}: attribution {', '.join(f'{k} {v:.3f}' for k, v in attr.items())}; power/clock {pc}")
    return r, inp


def run_quantizer(E, H, I, reps):
    """FP32 master -> MXFP4 quantisation of every expert's gate, up and down
    matrices of one layer straight into the packed layout the layer reads
    (moe_quantize_weights, one launch per matrix: the QAT forward's weight
    step).  Algorithmic bytes per weight: 4 read + 1/2 + 1/32 written (+ 4 per
    128x128 block)."""
    import torch
    from fp4_weight_grouped_amd import v4moe

    dev = "cuda:0"
    shapes = [(E, I, H), (E, I, H), (E, H, I)]
    ws = [torch.randn(sh, device=dev) * 0.02 for sh in shapes]
    outs = [v4moe.quantize_weights(w, packed=True) for w in ws]
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for w, o in zip(ws, outs):
            v4moe.moe_quantize_weights(w, o, packed=True)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    n = sum(int(np.prod(sh)) for sh in shapes)
    nbytes = n * 4 + n // 2 + n // 32 + (n // (128 * 128)) * 4
    del ws, outs
    torch.cuda.empty_cache()
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"[bench] weight quantiser: {ms:.3f} ms for {n / 1e9:.2f} G weights, {gbs:.0f} GB/s")
    return dict(E=E, H=H, I=I, weights=n, ms=ms, algorithmic_bytes=nbytes, bound="hbm", achieved=gbs,
                peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                kernel="k_quantize_weights (fp32 master -> packed fp4 e2m1 + e8m0 + fp32 block scale)")


BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix


def run_backward(name, steps, warmup, layer_cache):
    """One backward step = moe_layer_backward (forward recompute, combine
    backward, dgrad, activation derivative, un-permute, weight gradients) on
    the workload's layer, inputs and dout resident in HBM.  Two rooflines:
    HBM bytes = the packed weights of the active experts read twice (the
    forward recompute and the data gradients; the E4M3 transposed copy the
    kernels read instead is an implementation choice and not counted), the
    fp32 weight gradients of all experts written once, x and dout read (bf16),
    dx (fp32) and dw written; and the dense bf16 matrix peak over 4 *
    T*k*mats*H*I FLOP (data and weight gradients).  The record's bound is the
    roofline whose ideal time is the longer; both fractions are kept."""
    import torch
    from fp4_weight_grouped_amd import inputs, v4moe
    inp = inputs.make(name)
    d = inp.dims
    dev = "cuda:0"
    key = (d.H, d.I, d.E, d.topk, d.act)
    if key not in layer_cache:
        layer_cache.clear()
        torch.cuda.empty_cache()
        dims = v4moe.dims(d.T, d.H, d.I, d.E, d.topk, d.act)
        ex = v4moe.upload_experts(inp.experts, dims, dev)
        layer_cache[key] = v4moe.MoELayer(d.H, d.I, d.E, d.topk, ex,
                                          torch.from_numpy(inp.w_router).to(dev), dev, act=d.act)
    layer = layer_cache[key]
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    r = np.random.default_rng(9)
    dout = torch.from_numpy(inputs.to_bf16_bits(r.standard_normal((d.T, d.H)).astype(np.float32)).view(np.int16)).to(dev)
    grads = layer.backward(x, dout)
    for _ in range(warmup):
        layer.backward(x, dout, grads=grads)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        layer.backward(x, dout, grads=grads)
        b.record()
    torch.cuda.synchronize()
    ms_all = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.median(ms_all))
    off = torch.diff(layer.forward(x)[3]).cpu().numpy()
    n_active = int((off > 0).sum())
    mats = 3 if d.act == inputs.ACT_SWIGLU else 2
    hi = d.H * d.I
    nbytes = (2 * n_active * weight_bytes_per_expert(d.H, d.I, mats) + d.E * mats * hi * 4
              + d.T * d.H * (2 + 2 + 4) + d.T * d.topk * 4)
    flops = 4 * d.T * d.topk * mats * hi
    gbs = nbytes / (ms / 1e3) / 1e9
    tfs = flops / (ms / 1e3) / 1e12
    rec = dict(workload=name, T=d.T, ms=ms, p10=pct(ms_all, 10), p90=pct(ms_all, 90), tokens_per_s=d.T / (ms / 1e3),
               algorithmic_bytes=nbytes, bf16_flops=flops,
               hbm_frac=gbs / HBM_PEAK_GBS, bf16_mfma_frac=tfs / BF16_DENSE_PEAK_TFLOPS,
               ideal_ms_hbm=nbytes / (HBM_PEAK_GBS * 1e9) * 1e3,
               ideal_ms_bf16_mfma=flops / (BF16_DENSE_PEAK_TFLOPS * 1e12) * 1e3)
    if rec["ideal_ms_hbm"] >= rec["ideal_ms_bf16_mfma"]:
        rec.update(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS)
    else:
        rec.update(bound="mfma (bf16)", achieved=tfs, peak=BF16_DENSE_PEAK_TFLOPS, unit="TFLOP/s",
                   frac=tfs / BF16_DENSE_PEAK_TFLOPS)
    log(f"[bench] backward {name}: {ms:.3f} ms (p10 {rec['p10']:.3f}, p90 {rec['p90']:.3f}), "
        f"{rec['achieved']:.0f} {rec['unit']} = {rec['frac']:.3f} of peak")
    return rec


def cpu_baseline(inp, gpu=None, max_tokens=128, min_seconds=10.0, max_reps=8):
    """The oracle's layer forward on the same inputs (test infrastructure: it
    shares no code with the library), repeated until about min_seconds of CPU
    work have been timed: routing, quantisation and permutation of all T
    tokens, the expert FFN and combine of a bounded sample of tokens.  With
    `gpu` (the GPU record's outputs of the same inputs) the oracle's results
    are also compared with them: ids and offsets bit for bit, the output of the
    sampled tokens at the stated bars."""
    import oracle
    T = inp.dims.T
    if T <= max_tokens:
        sub = None
    else:   # evenly spread tokens, always the first and the last
        sub = np.unique(np.linspace(0, T - 1, max_tokens).round().astype(np.int32))
    n = T if sub is None else len(sub)
    reps, dt, ref = 0, 0.0, None
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        ref = oracle.layer_forward(inp, subset=sub)
        dt += time.perf_counter() - t0
        reps += 1
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rec = dict(value=reps * n / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
               seconds=dt, repetitions=reps, cpu_model=cpu_model,
               sample=(f"whole layer forward of all {T} tokens of the workload, {reps} times" if sub is None else
                       f"routing/quantisation/permutation of all {T} tokens, expert FFN + combine "
                       f"of {n} evenly spaced tokens, {reps} times; rate = those tokens / wall time"))
    if gpu is not None:
        toks = np.arange(T) if sub is None else sub

        def f64(bits):
            return (np.asarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        g, r = f64(gpu["out"][toks]), f64(ref["out"][toks])
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
        mx = float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))
        wrel = float(np.max(np.abs(gpu["w"].astype(np.float64) - ref["w"]) / np.abs(ref["w"])))
        rec["parity"] = dict(ids_bit_exact=bool(np.array_equal(gpu["ids"], ref["ids"])),
                             offsets_bit_exact=bool(np.array_equal(gpu["offsets"], ref["offsets"])),
                             weights_max_rel=wrel, out_rel_l2=rel, out_max_rel=mx, tokens_compared=int(len(toks)),
                             within_bar=bool(rel <= 2e-3 and mx <= 1e-2 and wrel <= 1e-6),
                             bar="ids/offsets bit-exact; weights 1e-6 relative; out rel-L2 <= 2e-3, "
                                 "max|d| <= 1e-2 max|ref|")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill side report")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true", help="skip the weight-quantiser side report")
    ap.add_argument("--no-backward", action="store_true", help="skip the layer-backward side report")
    ap.add_argument("--no-gateless", action="store_true", help="skip the gate-less (squared ReLU) side report")
    ap.add_argument("--only-backward", default=None, metavar="WORKLOAD",
                    help="only time the layer backward on this workload and print its record")
    ap.add_argument("--copy-bytes", type=int, default=0, help="only run the counter-calibration copy")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-entry-point attribution and the power/clock sampling")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the tiny, zipf, hash and ragged side records")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache protocol loop (scratch writes between steps)")
    ap.add_argument("--only-quantizer", action="store_true",
                    help="only time the weight quantiser on the workload's layer shape and print its record")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: libv4moe has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return
    if args.only_backward:
        print(json.dumps({"backward": [run_backward(args.only_backward, args.steps, args.warmup, {})]}), flush=True)
        return
    if args.only_quantizer:
        from fp4_weight_grouped_amd import inputs
        d = inputs.WORKLOADS[args.workload].dims
        print(json.dumps({"weight_quantizer": run_quantizer(d.E, d.H, d.I, args.steps)}), flush=True)
        return
    cache = {}
    scratch = None if args.no_cold else torch.empty(SCRATCH_BYTES, dtype=torch.uint8, device="cuda:0")
    head, inp = run_gpu(args.workload, args.steps, args.warmup, cache, not args.no_extras, scratch)
    side = side_inp = None
    side_steps, side_warm = max(5, min(20, args.steps)), max(2, args.warmup // 2)
    if not args.no_prefill and args.workload != "prefill":
        side, side_inp = run_gpu("prefill", side_steps, side_warm, cache, not args.no_extras, scratch)

    # the other configurations of the method: skewed (Zipf bias), hash routing,
    # the ragged batch of 64 requests (same layer as decode/prefill), and the
    # tiny layer (run last: it replaces the cached layer)
    others = []
    if not args.no_workloads:
        for w in ("zipf", "hash", "ragged"):
            if w != args.workload:
                others.append(run_gpu(w, side_steps, side_warm, cache, False, scratch))

    bwd = None
    if not args.no_backward:
        bwd = [run_backward(w, max(3, min(10, args.steps // 4)), 2, cache) for w in ("decode", "prefill")]

    quant = None
    if not args.no_quantizer:
        quant = run_quantizer(head["E"], head["H"], head["I"], max(3, min(10, args.steps // 4)))

    def roofline(r):
        if r["T"] <= 1024:
            roof = dict(bound="hbm", achieved=r["ffn_hbm_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=r["ffn_hbm_gbs"] / HBM_PEAK_GBS)
        else:
            roof = dict(bound="mfma", achieved=r["ffn_tflops"], peak=FP8_DENSE_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=r["ffn_tflops"] / FP8_DENSE_PEAK_TFLOPS)
        roof["traffic"] = measured_traffic(r["workload"])
        roof["traffic_unit"] = "HBM bytes per FFN (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        roof["algorithmic_bytes"] = r["weight_bytes"]
        roof["kernel"] = ("k_ffn_persistent (expert FFN: both grouped GEMMs, SwiGLU, requant, scatter)"
                          if r["T"] <= 1024 else
                          "k_ffn<1,...> + k_ffn<2,...> (expert FFN: linear1+SwiGLU+requant, linear2+scatter)")
        roof["kernel_ms"] = r["ffn_ms"]
        return roof

    roof = roofline(head)

    gateless = None
    if not args.no_gateless and args.workload in ("decode", "prefill"):
        gateless = []
        for w in ("decode_relu2", "prefill_relu2"):
            r, _ = run_gpu(w, side_steps, side_warm, cache, False, scratch)
            r.pop("_gpu")
            gateless.append(dict(r, roofline=roofline(r)))
    if not args.no_workloads and args.workload != "tiny":
        others.append(run_gpu("tiny", side_steps, side_warm, cache, False, scratch))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(inp, head["_gpu"])
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads; parity {cpu['parity']}")
        # a bounded oracle leg per side record: its time, and the parity of that record
        for r, winp in ([(side, side_inp)] if side is not None else []) + others:
            r["cpu_baseline"] = cpu_baseline(winp, r["_gpu"], max_tokens=16, min_seconds=0.0, max_reps=1)
            log(f"[bench] {r['workload']}: oracle parity {r['cpu_baseline']['parity']}")
    head.pop("_gpu")

    rec = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": head["workload"], "T": head["T"], "H": head["H"], "I": head["I"],
                   "E": head["E"], "topk": head["topk"], "activation": head["activation"],
                   "weights": "fp4-e2m1/e8m0-32/fp32-128x128",
                   "parallelism": "none (one GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": cpu["parity"] if cpu else None,
        "deterministic": head["deterministic"],
        "detail": head,
    }
    if side is not None:
        side.pop("_gpu")
        rec["prefill"] = dict(side, roofline=roofline(side))
    for r, _ in others:
        r.pop("_gpu")
        rec[r["workload"]] = dict(r, roofline=roofline(r))
    if quant is not None:
        rec["weight_quantizer"] = quant
    if bwd is not None:
        rec["backward"] = bwd
    if gateless is not None:
        rec["gateless"] = gateless
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
