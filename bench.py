#!/usr/bin/env python3
"""Throughput of the latent-MoE layer forward on one MI355X.

Headline (the JSON line's ``value``): the 145B-shaped layer at decode /
speculative-verify size, T = 4 tokens per call (hidden 2560, latent 1792,
512 experts of SwiGLU width 640 in 4-bit e2m1 + E4M3/16 scales, top-10 + one
shared expert), in tokens/s. One step is one full layer forward. The weights
rotate over ``--copies`` copies at distinct HBM addresses (and each copy has
its own input tokens) so successive steps cannot be served by the 256 MB
Infinity Cache: one layer call touches ~97 MB.

Secondary objects:
``prefill``: the same layer on a 16K-token prefill with a Zipf(1.1) router
bias, in tokens/s and matrix-core utilisation; ``prefill120``: the
120B-shaped layer (latent 1280) on a 4096-token prefill; ``mixed_record``:
the same layer with the mixed 3/4-bit expert record (3-bit E1M1 gate/up,
4-bit down), at decode T = 4 and per stage at the 16K prefill; ``grouped``:
the layer with 8 routing groups, each with its own (D_g, U_g), at decode
T = 4 and a 4096-token prefill; ``stack``:
48 residual blocks of 145B shapes, all resident, one decode step at T = 8
(bytes, GB/s and fraction of the HBM peak).

``value`` comes from K back-to-back steps with no events inside the timed
region. A second pass over the same K steps records HIP events on the launch
stream around the dominant kernel (``roofline``) and at every step boundary
(per-step p10 / p50 / p90); events cost a few microseconds each, which is why
they stay out of the headline pass. ``roofline.traffic`` is read from the
committed rocprofv3 counter summary of that kernel when the kernel source is
unchanged since the counters were taken, else null. ``cpu_baseline`` is the
float64 oracle on the host cores (median whole-layer call time of the same
decode workload, all cores and one thread, each in a child process with its
BLAS thread count set).

Profiling helpers: ``--only copy`` runs a plain 1 GiB device copy (the
calibration kernel for the HBM byte counters), ``--only decode`` /
``--only prefill`` run one workload, and ``--summarize-pmc CSV`` prints the
per-kernel average of a rocprofv3 counter-collection file.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix cores

def rec_bytes(L, I, gateup_bits=4):
    """One expert's codes + E4M3 block scales (gate/up codes of gateup_bits,
    4-bit down codes), without the three fp32 matrix scales."""
    return 2 * L * I * gateup_bits // 8 + L * I // 2 + 3 * L * I // 16


# the kernels that run each stage, by the base name of the kernel template
# (the first one present in the stored counter run is used)
DECODE_STAGE_KERNELS = {"dproj": ("k_dec_front",), "router": ("k_dec_router",),
                        "gateup": ("k_dec_gateup",), "down": ("k_dec_down",),
                        "uproj": ("k_dec_uproj",)}
GROUPED_STAGE_KERNELS = {"gateup": ("k_expert_gateup_p", "k_expert_gateup"),
                         "down": ("k_expert_down_p", "k_expert_down")}
# workloads whose counter runs traffic.json holds (bench.py --only argument)
TRAFFIC_WORKLOADS = {"decode145": "decode", "prefill145": "prefill", "prefill120": "prefill120"}


def kernel_bytes(d, T, n_routed, decode=True, folded=True):
    """Algorithmic HBM bytes of each kernel of one layer call: every weight
    byte it must read once (4-bit codes, or 3-bit E1M1 gate/up codes in the
    mixed record, + E4M3 block scales + fp32 matrix scales for experts, bf16
    for D / R / U, the folded router W = R D as bf16 hi + lo) plus its
    activation inputs and outputs. Decode path: front (D and, folded, the
    logits from x), router (only when not folded), gate/up (routed experts
    and the shared one, slot 0), down (writes z as 64-bit fixed point),
    U (reads it)."""
    L, H, E, I, k = d.latent, d.hidden, d.n_experts, d.inter, d.top_k
    G = getattr(d, "n_groups", 1)
    GL = G * L
    fp4 = lambda n_, k_, b=4: n_ * k_ * b // 8 + n_ * k_ // 16
    gu = 2 * fp4(I, L, d.gateup_bits) + 8   # gate + up of one expert
    dn = fp4(L, I) + 4               # down of one expert
    sh = d.n_shared
    x = out = T * H * 2
    h2 = T * GL * 2 * 2              # latent as bf16 hi + lo
    if decode:
        return {
            "dproj": GL * H * 2 + x + h2 + (2 * E * H * 2 + 2 * T * E * 4 if folded else 0),
            "router": 0 if folded else E * L * 2 + E * 4 + h2 + T * E * 4,
            "gateup": (n_routed + sh) * (gu + T * I * 2) + T * GL * 2 + 2 * T * E * 4,
            "down": (n_routed + sh) * (dn + T * I * 2) + T * GL * 8,
            "uproj": H * GL * 2 + T * GL * 8 + out,
        }
    rows = T * k + T * sh
    return {
        "dproj": GL * H * 2 + x + h2,
        "router": E * L * 2 + h2 + T * E * 4,
        "gateup": (n_routed + sh) * gu + rows * (L * 2 + I * 2),
        "down": (n_routed + sh) * dn + rows * (I * 2 + L * 2),
        "uproj": H * GL * 2 + T * GL * 2 + out,
    }


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=8, help="rotating weight copies (decode)")
    p.add_argument("--path", choices=["auto", "grouped", "decode"], default="auto")
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--prefill-warmup", type=int, default=3)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="oracle time per CPU measurement (all cores; half of it at one thread)")
    p.add_argument("--only", choices=["decode", "prefill", "prefill120", "copy", "stack", "mixed",
                                      "grouped"],
                   default=None, help="run one workload and print its object (profiling)")
    p.add_argument("--no-mixed", action="store_true",
                   help="skip the mixed 3/4-bit expert record")
    p.add_argument("--no-family", action="store_true",
                   help="skip the decode shape family (T = 1, 2, 3, 5, 8), e.g. under a profiler")
    p.add_argument("--no-grouped", action="store_true",
                   help="skip the routing-groups layer (8 D/U pairs)")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the 48-block stack (its 48 layers take about 2 minutes to generate)")
    p.add_argument("--stack-steps", type=int, default=20)
    p.add_argument("--stack-warmup", type=int, default=3)
    p.add_argument("--summarize-pmc", metavar="CSV", default=None,
                   help="print per-kernel averages of a rocprofv3 counter_collection.csv")
    p.add_argument("--write-traffic", metavar="DIR", default=None,
                   help="print traffic.json from DIR/{copy,decode,prefill}_{fetch,write}.csv "
                        "(rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter_collection files)")
    return p.parse_args()


def source_digest():
    """Hash of the HIP sources; counter summaries record it so that a changed
    kernel invalidates its stored traffic figure."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "latent_sparse_moe_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernels, workload):
    """HBM bytes per launch of a stage's kernel on one workload, from
    profiles/traffic.json (two rocprofv3 --pmc runs of that workload,
    FETCH_SIZE and WRITE_SIZE, each divided by the factor the same counter
    reads on the copy kernel). kernels: base names of the kernel templates
    that can run the stage; the first one the counter run saw is used. None
    when the file is absent, lacks the workload or the kernel, or was taken
    on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    seen = t.get("workloads", {}).get(workload, {})
    for base in kernels:
        for name, k in sorted(seen.items()):
            if name.split("<")[0] == base:
                return k.get("hbm_bytes_per_launch")
    return None


def kernel_key(name):
    """'void moe::k_dec_gateup<7>(moe::DecodeArgs)' -> 'k_dec_gateup<7>'."""
    short = name.split("(")[0].strip()
    for p in ("void ", "moe::"):
        short = short.replace(p, "")
    return short.strip()


def pmc_averages(path):
    """{(kernel, counter): (dispatches, average value)} of a counter_collection.csv."""
    acc = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            key = (kernel_key(row.get("Kernel_Name", "")), row.get("Counter_Name", ""))
            v = float(row.get("Counter_Value", 0) or 0)
            n, tot = acc.get(key, (0, 0.0))
            acc[key] = (n + 1, tot + v)
    return {k: (n, tot / n) for k, (n, tot) in acc.items()}


def summarize_pmc(path):
    for (k, c), (n, avg) in sorted(pmc_averages(path).items()):
        print(f"{k}\t{c}\tdispatches={n}\tavg={avg:.1f}")


def write_traffic(d):
    """HBM bytes per launch of each kernel of each workload: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) from DIR/{workload}_{fetch,write}.csv, each
    divided by what the same counter reads per byte on the 1 GiB copy kernel
    (DIR/copy_{fetch,write}.csv)."""
    gib_kib = (1 << 30) / 1024.0
    copy_f = pmc_averages(os.path.join(d, "copy_fetch.csv"))
    copy_w = pmc_averages(os.path.join(d, "copy_write.csv"))
    cf = max(v for (k, c), (n, v) in copy_f.items() if "copyBuffer" in k) / gib_kib
    cw = max(v for (k, c), (n, v) in copy_w.items() if "copyBuffer" in k) / gib_kib
    workloads = {}
    for wl in TRAFFIC_WORKLOADS:
        fp, wp = os.path.join(d, f"{wl}_fetch.csv"), os.path.join(d, f"{wl}_write.csv")
        if not (os.path.exists(fp) and os.path.exists(wp)):
            continue
        f, w = pmc_averages(fp), pmc_averages(wp)
        kernels = {}
        for (k, c), (n, v) in f.items():
            if not k.startswith("k_"):
                continue
            wv = w.get((k, "WRITE_SIZE"), (0, 0.0))[1]
            kernels[k] = {"dispatches": n, "fetch_kib": round(v, 1), "write_kib": round(wv, 1),
                          "hbm_bytes_per_launch": round((v / cf + wv / cw) * 1024.0)}
        workloads[wl] = kernels
    out = {"source_digest": source_digest(),
           "calibration": {"copy_bytes": 1 << 30, "fetch_counter_per_byte": cf,
                           "write_counter_per_byte": cw},
           "workloads": workloads}
    print(json.dumps(out, indent=1))


def copy_probe(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size: each dispatch reads and
    writes exactly nbytes (the calibration for FETCH_SIZE / WRITE_SIZE)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return {"bytes_read_per_dispatch": nbytes, "bytes_written_per_dispatch": nbytes,
            "dispatches": reps, "ms": ms, "GBps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}


def percentiles(xs):
    xs = sorted(xs)
    q = lambda f: xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]
    return {"p10": q(0.1), "p50": statistics.median(xs), "p90": q(0.9)}


def clone_layer(lsm, dl):
    import dataclasses

    def c(v):
        if v is None:
            return None
        if dataclasses.is_dataclass(v) and not isinstance(v, type):
            return type(v)(**{f.name: (c(getattr(v, f.name)) if f.name != "dims" else getattr(v, f.name))
                              for f in dataclasses.fields(v)})
        return v.clone() if hasattr(v, "clone") else v   # tensors; ints (bits) as they are
    return c(dl)


def event_pair(torch):
    """Two timing events whose HIP handles exist (torch creates them lazily
    on first record), so the library can record them on its stream."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    return a, b


def stage_times(lsm, torch, run, stages, n=5):
    """Average duration (ms) of each stage over n untimed calls."""
    acc = {s: 0.0 for s in stages}
    for _ in range(n):
        ev = {s: event_pair(torch) for s in stages}
        torch.cuda.synchronize()
        run(ev)
        torch.cuda.synchronize()
        for s, (a, b) in ev.items():
            acc[s] += a.elapsed_time(b) / n  # ~0 for stages this path does not run
    return acc


def bench_decode(args, torch, lsm, synth, dev):
    cfg = synth.CONFIGS["decode145"]
    d, T = cfg.dims, cfg.T
    t0 = time.time()
    host = synth.make_layer(d, cfg.seed, cfg.bias, cfg.zipf_s)
    log(f"[decode] generated layer in {time.time() - t0:.1f}s")
    # weights also in the decode-packed layout the decode kernels load from
    # (a one-time reorder at load time, outside the timed region); each
    # rotating copy has its own
    base = lsm.DeviceLayer.from_host(host, dev).pack(grouped=False)
    layers = [base] + [clone_layer(lsm, base) for _ in range(args.copies - 1)]
    xs_host = [synth.make_x(T, d.hidden, cfg.seed + i) for i in range(args.copies)]
    xs = [torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev) for x in xs_host]
    outs = [torch.empty_like(x) for x in xs]
    ws = lsm.alloc_workspace(d, T, dev)
    path = {"auto": lsm.PATH_AUTO, "grouped": lsm.PATH_GROUPED, "decode": lsm.PATH_DECODE}[args.path]

    # routing of each copy's tokens (untimed) -> experts touched -> algorithmic bytes
    n_touched = []
    for i in range(args.copies):
        dbg = lsm.RouteDebug.alloc(d, T, dev)
        lsm.forward(xs[i], layers[i], out=outs[i], workspace=ws, debug=dbg, path=path)
        torch.cuda.synchronize()
        n_touched.append(int((dbg.counts > 0).sum().item()))
    rec = rec_bytes(d.latent, d.inter, d.gateup_bits)
    dense = 2 * d.latent * d.hidden * 2 + d.n_experts * d.latent * 2 + 2 * T * d.hidden * 2
    layer_bytes = [(n + d.n_shared) * (rec + 12) + dense for n in n_touched]
    use_decode = path == lsm.PATH_DECODE or (path == lsm.PATH_AUTO and T <= lsm.DECODE_MAX_T)
    stage_bytes = [kernel_bytes(d, T, n, decode=use_decode) for n in n_touched]

    def step(i, ev=None):
        c = i % args.copies
        lsm.forward(xs[c], layers[c], out=outs[c], workspace=ws, path=path, stage_events=ev)

    # which kernel dominates (untimed pass over the stages this path runs)
    names = (["dproj", "router", "gateup", "down", "uproj"] if use_decode
             else ["dproj", "router", "topk", "route", "gateup", "down", "combine", "uproj"])
    st = stage_times(lsm, torch, lambda ev: step(0, ev), names)
    ran = dict(st)
    dom = max(ran, key=ran.get)
    log(f"[decode] stage ms: " + ", ".join(f"{s}={v * 1e3:.1f}us" for s, v in ran.items()))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # pass A: the headline, no events inside the timed region
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    # pass B: the same steps with events around the dominant kernel and at
    # every step boundary
    evs = [event_pair(torch) for _ in range(args.steps)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(args.steps):
        step(i, {dom: evs[i]})
        marks[i + 1].record()
    torch.cuda.synchronize()
    dom_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    step_us = [marks[i].elapsed_time(marks[i + 1]) * 1e3 for i in range(args.steps)]
    mean_bytes = sum(layer_bytes[i % args.copies] for i in range(args.steps)) / args.steps
    dom_bytes = sum(stage_bytes[i % args.copies].get(dom, 0) for i in range(args.steps)) / args.steps
    dom_bytes = dom_bytes or None
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9 if dom_bytes else None
    res = {
        "tok_s": T * args.steps / (total_ms * 1e-3),
        "ms_per_step": ms_step,
        "dominant": dom,
        "dominant_ms": dom_ms,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS if achieved else None,
            "traffic": (stored_traffic(DECODE_STAGE_KERNELS.get(dom, ("k_dec_" + dom,)),
                                       "decode145") if use_decode else None),
            "kernel": dom, "algorithmic_bytes_per_launch": dom_bytes,
            "kernel_us": dom_ms * 1e3,
        },
        "detail": {
            "layer_bytes_per_step": mean_bytes,
            "layer_GBps": mean_bytes / (ms_step * 1e-3) / 1e9,
            "layer_frac_of_hbm_peak": mean_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "experts_touched_per_copy": n_touched,
            "stage_us_untimed_pass": {s: round(v * 1e3, 2) for s, v in ran.items()},
            "stage_GBps_untimed_pass": {s: round(stage_bytes[0].get(s, 0) / (v * 1e-3) / 1e9, 1)
                                        for s, v in ran.items() if stage_bytes[0].get(s)},
            "path": "decode" if use_decode else "grouped",
            "copies": args.copies,
            "step_us_with_events": {k: round(v, 2) for k, v in percentiles(step_us).items()},
            "shape_family": (None if args.no_family else
                             decode_family(args, torch, lsm, synth, d, layers, path, dev)),
        },
    }
    return res


def decode_family(args, torch, lsm, synth, d, layers, path, dev, Ts=(1, 2, 3, 5, 8)):
    """Step time of the same layer copies at other token counts: T = 1 (chat
    decode) to T = 5 (a verify window of 4 drafted tokens + 1), and T = 8
    (the decode kernels' limit). Same rotation and timing as the headline
    pass, without events inside the timed region."""
    out = {}
    for T in Ts:
        xs = [torch.from_numpy(synth.make_x(T, d.hidden, 1000 + T + i).view("int16"))
              .view(torch.bfloat16).to(dev) for i in range(args.copies)]
        outs = [torch.empty_like(x) for x in xs]
        ws = lsm.alloc_workspace(d, T, dev)

        def step(i):
            c = i % args.copies
            lsm.forward(xs[c], layers[c], out=outs[c], workspace=ws, path=path)
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            step(i)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.steps
        out[f"T={T}"] = {"us_per_step": round(us, 2), "tok_s": round(T / (us * 1e-6), 1)}
    log("[decode] shape family: " + ", ".join(f"{k} {v['us_per_step']:.1f}us" for k, v in out.items()))
    return out


def bench_prefill(args, torch, lsm, synth, dev, name="prefill145"):
    """A prefill workload on the grouped path: ``prefill145`` (16K tokens,
    145B shapes, Zipf(1.1) router bias) or ``prefill120`` (4096 tokens,
    latent 1280, no bias)."""
    cfg = synth.CONFIGS[name]
    d, T = cfg.dims, cfg.T
    t0 = time.time()
    host = synth.make_layer(d, cfg.seed, cfg.bias, cfg.zipf_s)
    log(f"[{name}] generated layer in {time.time() - t0:.1f}s")
    # experts also in the packed layout the grouped kernels load from (a
    # one-time reorder at load time, outside the timed region)
    dl = lsm.DeviceLayer.from_host(host, dev).pack(decode=False)
    torch.cuda.synchronize()
    del host
    x = torch.from_numpy(synth.make_x(T, d.hidden, cfg.seed).view("int16")).view(torch.bfloat16).to(dev)
    out = torch.empty_like(x)
    ws = lsm.alloc_workspace(d, T, dev)
    P = T * d.top_k
    rows = P + T * d.n_shared
    fl = {
        "dproj": 2.0 * T * d.hidden * d.latent,
        "router": 2.0 * T * d.latent * d.n_experts,
        "gateup": 2.0 * rows * d.latent * 2 * d.inter,
        "down": 2.0 * rows * d.inter * d.latent,
        "uproj": 2.0 * T * d.latent * d.hidden,
    }
    total_flop = sum(fl.values())

    def step(ev=None):
        lsm.forward(x, dl, out=out, workspace=ws, path=lsm.PATH_GROUPED, stage_events=ev)

    names = ["dproj", "router", "topk", "route", "gateup", "down", "combine", "uproj"]
    step()  # first launches of each kernel (code-object loading) stay out of the stage times
    torch.cuda.synchronize()
    st = stage_times(lsm, torch, step, names, n=3)
    dom = max(st, key=st.get)
    log(f"[{name}] stage ms: " + ", ".join(f"{s}={v:.3f}" for s, v in st.items()))
    for _ in range(args.prefill_warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.prefill_steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.prefill_steps
    evs = [event_pair(torch) for _ in range(args.prefill_steps)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.prefill_steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(args.prefill_steps):
        step({dom: evs[i]})
        marks[i + 1].record()
    torch.cuda.synchronize()
    dom_ms = sum(a.elapsed_time(b) for a, b in evs) / args.prefill_steps
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.prefill_steps)]
    dom_tf = fl[dom] / (dom_ms * 1e-3) / 1e12 if dom in fl else None
    layer_tf = total_flop / (ms * 1e-3) / 1e12
    what = ("16K prefill tokens/s (145B-shaped layer, Zipf router bias)" if name == "prefill145"
            else f"{T}-token prefill tokens/s (120B-shaped layer, latent {d.latent})")
    return {
        "metric": what,
        "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
        "steps": args.prefill_steps, "warmup": args.prefill_warmup,
        "layer_tflops": layer_tf, "layer_frac_of_bf16_peak": layer_tf / BF16_PEAK_TFLOPS,
        "algorithmic_tflop_per_step": total_flop / 1e12,
        "roofline": {"bound": "mfma", "achieved": dom_tf, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": dom_tf / BF16_PEAK_TFLOPS if dom_tf else None,
                     "traffic": stored_traffic(GROUPED_STAGE_KERNELS.get(dom, ()), name),
                     "kernel": dom,
                     "kernel_ms": dom_ms},
        "step_ms_with_events": {k: round(v, 4) for k, v in percentiles(step_ms).items()},
        "stage_ms_untimed_pass": {s: round(v, 4) for s, v in st.items()},
        "config": {"workload": name, "T": T, "hidden": d.hidden, "latent": d.latent,
                   "experts": d.n_experts, "inter": d.inter, "top_k": d.top_k,
                   "shared": d.n_shared,
                   "router_bias": "zipf(1.1)" if cfg.bias == "zipf" else "none"},
    }


def bench_mixed(args, torch, lsm, synth, dev):
    """The mixed 3/4-bit expert record (E1M1 gate/up, e2m1 down) on the
    145B-shaped layer: decode T = 4 over rotating decode-packed copies, timed
    as the headline pass, and the 16K prefill's per-stage times on
    grouped-packed weights (3 untimed calls with stage events)."""
    cfg = synth.CONFIGS["decode145"]
    d, T = synth.replace(cfg.dims, gateup_bits=3), cfg.T
    t0 = time.time()
    host = synth.make_layer(d, cfg.seed, cfg.bias, cfg.zipf_s)
    log(f"[mixed] generated layer in {time.time() - t0:.1f}s")
    base = lsm.DeviceLayer.from_host(host, dev)
    del host
    dec = lsm.DeviceLayer(**{**base.__dict__}).pack(grouped=False).drop_plain()
    layers = [dec] + [clone_layer(lsm, dec) for _ in range(args.copies - 1)]
    xs = [torch.from_numpy(synth.make_x(T, d.hidden, cfg.seed + i).view("int16"))
          .view(torch.bfloat16).to(dev) for i in range(args.copies)]
    outs = [torch.empty_like(x) for x in xs]
    ws = lsm.alloc_workspace(d, T, dev)
    n_touched = []
    for i in range(args.copies):
        dbg = lsm.RouteDebug.alloc(d, T, dev)
        lsm.forward(xs[i], layers[i], out=outs[i], workspace=ws, debug=dbg)
        torch.cuda.synchronize()
        n_touched.append(int((dbg.counts > 0).sum().item()))
    rec = rec_bytes(d.latent, d.inter, 3)
    dense = 2 * d.latent * d.hidden * 2 + d.n_experts * d.latent * 2 + 2 * T * d.hidden * 2
    layer_bytes = sum((n + d.n_shared) * (rec + 12) + dense for n in n_touched) / len(n_touched)
    gu_bytes = kernel_bytes(d, T, n_touched[0])["gateup"]

    def step(i, ev=None):
        c = i % args.copies
        lsm.forward(xs[c], layers[c], out=outs[c], workspace=ws, stage_events=ev)
    names = ["dproj", "router", "gateup", "down", "uproj"]
    st = stage_times(lsm, torch, lambda ev: step(0, ev), names)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    log(f"[mixed] decode T={T}: {us:.1f} us/step; stage us: "
        + ", ".join(f"{s}={v * 1e3:.1f}" for s, v in st.items()))
    res = {
        "record": "E1M1 gate/up + e2m1 down, E4M3 per-16 block scales, fp32 per matrix",
        "expert_record_bytes": rec + 12,
        "decode": {
            "T": T, "us_per_step": round(us, 2), "tok_s": round(T / (us * 1e-6), 1),
            "layer_bytes_per_step": layer_bytes,
            "layer_GBps": round(layer_bytes / (us * 1e-6) / 1e9, 1),
            "stage_us_untimed_pass": {s: round(v * 1e3, 2) for s, v in st.items()},
            "gateup_GBps_untimed_pass": round(gu_bytes / (st["gateup"] * 1e-3) / 1e9, 1),
            "experts_touched_per_copy": n_touched, "copies": args.copies,
        },
    }
    del layers, dec, xs, outs, ws
    if not args.no_prefill:
        pcfg = synth.CONFIGS["prefill145"]
        Tp = pcfg.T
        pre = base.pack(decode=False)
        # routing bias as in the prefill workload (the layer above has none)
        pre.bias = torch.from_numpy(synth.zipf_bias(d.n_experts, pcfg.zipf_s)).to(dev)
        x = torch.from_numpy(synth.make_x(Tp, d.hidden, pcfg.seed).view("int16")).view(
            torch.bfloat16).to(dev)
        out = torch.empty_like(x)
        ws = lsm.alloc_workspace(d, Tp, dev)
        pn = ["dproj", "router", "topk", "route", "gateup", "down", "combine", "uproj"]
        lsm.forward(x, pre, out=out, workspace=ws, path=lsm.PATH_GROUPED)  # warm the kernels
        torch.cuda.synchronize()
        pst = stage_times(lsm, torch, lambda ev: lsm.forward(
            x, pre, out=out, workspace=ws, path=lsm.PATH_GROUPED, stage_events=ev), pn, n=3)
        rows = Tp * d.top_k + Tp * d.n_shared
        gu_fl = 2.0 * rows * d.latent * 2 * d.inter
        res["prefill_untimed"] = {
            "T": Tp, "ms_per_call": round(sum(pst.values()), 4),
            "stage_ms": {s: round(v, 4) for s, v in pst.items()},
            "gateup_tflops": round(gu_fl / (pst["gateup"] * 1e-3) / 1e12, 1),
        }
        log(f"[mixed] prefill T={Tp}: " + ", ".join(f"{s}={v:.3f}" for s, v in pst.items()))
    return res


def bench_grouped(args, torch, lsm, synth, dev):
    """Routing groups of D/U: the 145B-shaped layer with 8 groups of 64
    experts, each group with its own (D_g, U_g). Decode T = 4 over rotating
    decode-packed copies (folded router), timed as the headline pass; and a
    4096-token prefill on the grouped path with grouped-packed weights."""
    cfg = synth.CONFIGS["grouped145"]
    d, T, G = cfg.dims, cfg.T, cfg.dims.n_groups
    t0 = time.time()
    host = synth.make_layer(d, cfg.seed, cfg.bias, cfg.zipf_s)
    log(f"[grouped] generated layer in {time.time() - t0:.1f}s")
    plain = lsm.DeviceLayer.from_host(host, dev)
    del host
    dec = lsm.DeviceLayer(**{**plain.__dict__}).pack(grouped=False).drop_plain()
    copies = max(2, args.copies // 2)   # each copy is ~1.3 GB: 4 copies pass the Infinity Cache
    layers = [dec] + [clone_layer(lsm, dec) for _ in range(copies - 1)]
    xs = [torch.from_numpy(synth.make_x(T, d.hidden, cfg.seed + i).view("int16"))
          .view(torch.bfloat16).to(dev) for i in range(copies)]
    outs = [torch.empty_like(x) for x in xs]
    ws = lsm.alloc_workspace(d, T, dev)
    n_touched = []
    for i in range(copies):
        dbg = lsm.RouteDebug.alloc(d, T, dev)
        lsm.forward(xs[i], layers[i], out=outs[i], workspace=ws, debug=dbg)
        torch.cuda.synchronize()
        n_touched.append(int((dbg.counts > 0).sum().item()))
    rec = rec_bytes(d.latent, d.inter, d.gateup_bits)
    dense = (2 * G * d.latent * d.hidden * 2 + 2 * d.n_experts * d.hidden * 2
             + 2 * T * d.hidden * 2)   # D_g and U_g of every group, the folded router (hi + lo)
    layer_bytes = sum((n + d.n_shared) * (rec + 12) + dense for n in n_touched) / copies

    def step(i):
        c = i % copies
        lsm.forward(xs[c], layers[c], out=outs[c], workspace=ws)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    log(f"[grouped] decode T={T}: {us:.1f} us/step, {layer_bytes / 1e6:.1f} MB/step")
    res = {"config": {"workload": "grouped145", "groups": G, "experts_per_group": d.n_experts // G,
                      "hidden": d.hidden, "latent": d.latent, "experts": d.n_experts,
                      "inter": d.inter, "top_k": d.top_k, "shared": d.n_shared},
           "decode": {"T": T, "us_per_step": round(us, 2), "tok_s": round(T / (us * 1e-6), 1),
                      "layer_bytes_per_step": layer_bytes,
                      "layer_GBps": round(layer_bytes / (us * 1e-6) / 1e9, 1),
                      "frac_of_hbm_peak": round(layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                      "experts_touched_per_copy": n_touched, "copies": copies}}
    del layers, dec, xs, outs, ws
    torch.cuda.empty_cache()
    if not args.no_prefill:
        Tp = 4096
        pre = plain.pack(decode=False)
        x = torch.from_numpy(synth.make_x(Tp, d.hidden, cfg.seed).view("int16")).view(
            torch.bfloat16).to(dev)
        out = torch.empty_like(x)
        ws = lsm.alloc_workspace(d, Tp, dev)
        rows = Tp * d.top_k + Tp * d.n_shared
        flop = (2.0 * Tp * d.hidden * G * d.latent + 2.0 * Tp * d.latent * d.n_experts
                + 2.0 * rows * d.latent * 3 * d.inter + 2.0 * Tp * G * d.latent * d.hidden)

        def pstep():
            lsm.forward(x, pre, out=out, workspace=ws, path=lsm.PATH_GROUPED)
        pstep()
        torch.cuda.synchronize()
        for _ in range(args.prefill_warmup):
            pstep()
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.prefill_steps):
            pstep()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.prefill_steps
        log(f"[grouped] prefill T={Tp}: {ms:.3f} ms/call")
        res["prefill"] = {"T": Tp, "ms_per_step": round(ms, 4), "tok_s": round(Tp / (ms * 1e-3), 1),
                          "algorithmic_tflop_per_step": flop / 1e12,
                          "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                          "frac_of_bf16_peak": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return res


def bench_stack(args, torch, lsm, synth, dev):
    """48 residual blocks (RMSNorm + latent MoE) of 145B shapes, all resident
    (~48 GB of decode-packed weights, far beyond the Infinity Cache), T = 8
    with Zipf routing bias;
    one step runs the blocks in order, each block's output feeding the next."""
    cfg = synth.CONFIGS["stack145"]
    d, T, nl = cfg.dims, cfg.T, cfg.n_layers
    t0 = time.time()
    dls = []
    for l in range(nl):
        h = synth.make_layer(d, cfg.seed + l, cfg.bias, cfg.zipf_s)
        # decode-packed copies only: the plain weights are freed once packed
        dls.append(lsm.DeviceLayer.from_host(h, dev).pack(grouped=False).drop_plain())
        del h
        if (l + 1) % 8 == 0:
            log(f"[stack] {l + 1}/{nl} blocks resident ({time.time() - t0:.0f}s)")
    log(f"[stack] generated and uploaded {nl} blocks in {time.time() - t0:.1f}s")
    x = torch.from_numpy(synth.make_x(T, d.hidden, cfg.seed).view("int16")).view(torch.bfloat16).to(dev)
    bufs = [torch.empty_like(x), torch.empty_like(x)]
    ws = lsm.alloc_workspace(d, T, dev)

    # experts touched by each block on this input (untimed pass, debug copies)
    n_touched, cur = [], x
    for l in range(nl):
        dbg = lsm.RouteDebug.alloc(d, T, dev)
        out = bufs[l % 2]
        lsm.forward(cur, dls[l], out=out, workspace=ws, debug=dbg, residual=True)
        torch.cuda.synchronize()
        n_touched.append(int((dbg.counts > 0).sum().item()))
        cur = out
    rec = rec_bytes(d.latent, d.inter, d.gateup_bits)
    per_block_dense = (2 * d.latent * d.hidden * 2 + d.n_experts * d.latent * 2 + d.n_experts * 4
                       + d.hidden * 4 + 2 * T * d.hidden * 2)
    step_bytes = sum((n + d.n_shared) * (rec + 12) + per_block_dense for n in n_touched)

    def step():
        cur = x
        for l in range(nl):
            out = bufs[l % 2]
            lsm.forward(cur, dls[l], out=out, workspace=ws, residual=True)
            cur = out

    for _ in range(args.stack_warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.stack_steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.stack_steps
    gbps = step_bytes / (ms * 1e-3) / 1e9
    # the same step captured once in a HIP graph and replayed (kernel
    # launches only: the path records no memset, copy or host sync)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.stack_warmup):
        graph.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.stack_steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / args.stack_steps
    return {"metric": "48-block stack decode step (T = 8), tokens/s", "value": T / (ms * 1e-3),
            "unit": "tokens/s", "ms_per_step": ms, "steps": args.stack_steps,
            "warmup": args.stack_warmup, "bytes_per_step": step_bytes, "GBps": gbps,
            "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS, "us_per_block": ms * 1e3 / nl,
            "graph_replay": {"ms_per_step": graph_ms, "us_per_block": graph_ms * 1e3 / nl},
            "experts_touched_per_block": n_touched,
            "config": {"workload": "stack145", "blocks": nl, "T": T, "hidden": d.hidden,
                       "latent": d.latent, "experts": d.n_experts, "inter": d.inter,
                       "top_k": d.top_k, "shared": d.n_shared, "router_bias": "zipf(1.1)",
                       "resident_weight_GB": sum(
                           sum(t.numel() * t.element_size() for t in _tensors(dl)) for dl in dls) / 1e9}}


def _tensors(v):
    import dataclasses
    import torch
    if v is None:
        return
    if dataclasses.is_dataclass(v) and not isinstance(v, type):
        for f in dataclasses.fields(v):
            yield from _tensors(getattr(v, f.name))
    elif isinstance(v, torch.Tensor):
        yield v


def cpu_child(threads, seconds, min_calls):
    """Runs in a child process started with OMP_NUM_THREADS and
    OPENBLAS_NUM_THREADS = threads (set before numpy loads its BLAS): the
    float64 oracle on the decode workload (145B layer, T = 4, seed 0), whole
    layer calls back to back for about ``seconds`` (at least ``min_calls``);
    prints one JSON object."""
    import numpy as np
    import oracle
    import synth
    cfg = synth.CONFIGS["decode145"]
    host = synth.make_layer(cfg.dims, cfg.seed, cfg.bias, cfg.zipf_s)
    x0 = synth.make_x(cfg.T, cfg.dims.hidden, cfg.seed)
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = None
    ts, t0 = [], time.perf_counter()
    while len(ts) < min_calls or time.perf_counter() - t0 < seconds:
        a = time.perf_counter()
        oracle.forward(host, x0)
        ts.append(time.perf_counter() - a)
        if len(ts) >= 20:
            break
    print(json.dumps({"threads": threads, "blas_threads": blas, "calls": len(ts),
                      "median_s": statistics.median(ts), "T": int(x0.shape[0])}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(args):
    """The float64 oracle, untuned, on the host cores: median time of whole
    decode-layer calls (T = 4) with every host core, and with one, each in
    a child process whose OMP_NUM_THREADS / OPENBLAS_NUM_THREADS are set."""
    import subprocess
    n = min(os.cpu_count() or 1, 64)
    runs = {}
    for threads, secs, mn in ((n, args.cpu_seconds, 5), (1, args.cpu_seconds / 2, 3)):
        env = dict(os.environ, OMP_NUM_THREADS=str(threads), OPENBLAS_NUM_THREADS=str(threads),
                   MKL_NUM_THREADS=str(threads))
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child",
                              str(threads), str(secs), str(mn)], env=env, capture_output=True,
                             text=True, timeout=600)
        if res.returncode != 0:
            raise RuntimeError(f"cpu baseline child failed: {res.stderr[-2000:]}")
        runs[threads] = json.loads(res.stdout.strip().splitlines()[-1])
        log(f"[cpu] {threads} threads: median {runs[threads]['median_s']:.2f} s per call over "
            f"{runs[threads]['calls']} calls")
    full, one = runs[n], runs[1]
    T = full["T"]
    return {"value": T / full["median_s"], "unit": "tokens/s", "cores": n, "kind": "oracle",
            "impl": "float64 oracle (numpy)",
            "sample": f"median of {full['calls']} whole decode-layer calls (145B shapes, T={T}) "
                      f"with OMP_NUM_THREADS=OPENBLAS_NUM_THREADS={n}",
            "median_s_per_call": full["median_s"], "blas_threads": full["blas_threads"],
            "one_thread": {"value": T / one["median_s"], "unit": "tokens/s",
                           "median_s_per_call": one["median_s"], "calls": one["calls"]},
            "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    if len(sys.argv) == 5 and sys.argv[1] == "--cpu-child":
        cpu_child(int(sys.argv[2]), float(sys.argv[3]), int(sys.argv[4]))
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    import torch
    import latent_sparse_moe_amd as lsm
    import synth

    lsm.load_library()
    dev = torch.device("cuda:0")
    if args.only == "copy":
        print(json.dumps(copy_probe(torch, dev)), flush=True)
        return
    if args.only in ("prefill", "prefill120"):
        print(json.dumps(bench_prefill(args, torch, lsm, synth, dev, args.only.replace(
            "prefill", "prefill145") if args.only == "prefill" else args.only)), flush=True)
        return
    if args.only == "stack":
        print(json.dumps(bench_stack(args, torch, lsm, synth, dev)), flush=True)
        return
    if args.only == "mixed":
        print(json.dumps(bench_mixed(args, torch, lsm, synth, dev)), flush=True)
        return
    if args.only == "grouped":
        print(json.dumps(bench_grouped(args, torch, lsm, synth, dev)), flush=True)
        return
    dec = bench_decode(args, torch, lsm, synth, dev)
    if args.only == "decode":
        print(json.dumps(dec), flush=True)
        return
    torch.cuda.empty_cache()
    line = {
        "metric": "latent-MoE layer tokens/sec: decode T=4 (HBM GB/s) and 16K prefill (MFMA %)",
        "value": dec["tok_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dec["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode145", "T": 4, "hidden": 2560, "latent": 1792,
                   "experts": 512, "inter": 640, "top_k": 10, "shared": 1,
                   "weights": "e2m1 + E4M3/16 + fp32 per matrix",
                   "rotating_copies": args.copies, "path": args.path},
        "roofline": dec["roofline"],
        "decode_detail": dec["detail"],
    }
    if not args.no_prefill:
        line["prefill"] = bench_prefill(args, torch, lsm, synth, dev)
        torch.cuda.empty_cache()
        line["prefill120"] = bench_prefill(args, torch, lsm, synth, dev, "prefill120")
        torch.cuda.empty_cache()
    if not args.no_mixed:
        line["mixed_record"] = bench_mixed(args, torch, lsm, synth, dev)
        torch.cuda.empty_cache()
    if not args.no_grouped:
        line["grouped"] = bench_grouped(args, torch, lsm, synth, dev)
        torch.cuda.empty_cache()
    if not args.no_stack:
        line["stack"] = bench_stack(args, torch, lsm, synth, dev)
        torch.cuda.empty_cache()
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
