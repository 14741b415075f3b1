#!/usr/bin/env python3
"""Benchmark of the batch-1 speculative-decode verify loop on one MI355X.

Default workload: the 32-layer stack of fp8-expert MoE layers (384 routed
experts top-8 + 1 shared, hidden 4096, T = 6 verify rows, KV cache from 4096
positions, vocab 129280), run as a device-resident verify loop: every step is
the embedding gather, 32 layer launches and one LM-head/argmax/accept launch,
with the KV length kept on the device.  Weights and inputs are synthetic and
seeded (the trained model is not used); with random weights almost no draft is
accepted, so a step commits ~1 token, and tokens/s is also given for the
acceptance lengths the pages report.

Printed: one JSON line with the step time (and its per-step median, p10, p90),
tokens/s per stream, per-layer microseconds, algorithmic HBM bytes and
bandwidth, the roofline of the layer kernel (live HIP-event timing of its
launches), the share of the layer kernel's time spent in grid barriers (from
its in-kernel trace, on an untimed step), launches per step, the spread over
several process starts, and the CPU oracle timed on a bounded sample as a
baseline.  --workload C2|C3|C4|C3X times a single layer instead (three rotating
weight copies so the 256 MB last-level cache cannot serve repeats); C5X is the
stack with MXFP4 experts (each of the 32 layers with routed experts of its own).
"""
import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode step µs/layer & tok/s/stream at T=6; achieved HBM GB/s vs peak"
PEAK_GBPS = 8000.0      # MI355X HBM3E peak
TAUS = (3.3, 4.0, 5.17)
EXPERT_DESC = {"fp8": "fp8 e4m3 experts (128x128 fp32 scales)",
               "mxfp4": "mxfp4 experts (e2m1, an e8m0 scale per 32 elements)",
               "bf16": "bf16 experts", "f32": "fp32 experts"}  # tokens per verify step the pages report (bench, live traffic, single-GB300 lane)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_bytes(s):
    e = 2 if s.attn_fmt == "bf16" else 4
    # the query projection: W_Q, or W_DQ and W_UQ (+ the q-norm gain) with a low-rank query
    q = s.q_lora * s.d + s.n_h * s.qw * s.q_lora + 2 * s.q_lora if s.q_lora else s.n_h * s.qw * s.d
    # sparse attention: the indexer's rows [W_IQ; W_IW; W_IK] of the first projection
    idx = (s.idx_heads * s.idx_dim + s.idx_heads + s.idx_dim) * s.d if s.idx_topk else 0
    return e * (q + idx + s.kvw * s.d + 2 * s.n_h * s.d_h * s.d_c + s.d * s.n_h * s.d_h) + \
        (4 * s.d_c if s.kv_norm else 0)


def router_bytes(s):
    return (2 if s.attn_fmt == "bf16" else 4) * s.E * s.d + (4 * s.E if s.routing == "skew" else 0)


def expert_bytes(s):
    if s.exp_fmt == "mxfp4":
        return 3 * s.f * s.d // 2 + 3 * s.f * s.d // 32      # half a byte per weight + a byte per 32
    if s.exp_fmt == "fp8":
        nsc = ((s.f + 127) // 128) * ((s.d + 127) // 128)
        return 3 * s.f * s.d + 3 * nsc * 4
    return 3 * s.f * s.d * (2 if s.exp_fmt == "bf16" else 4)


def head_bytes(s):
    """LM-head table bytes read per step (bf16, or E4M3 codes + fp32 128x128 block scales)."""
    if s.head_fmt == "fp8":
        return s.V * s.d + ((s.V + 127) // 128) * ((s.d + 127) // 128) * 4
    return s.V * s.d * 2


def layer_bytes(s, L, slots, kept_rows=None):
    """Algorithmic bytes of one layer step: touched weights, KV read/write, activations in/out.
    Sparse attention reads every row's index key and, of the latent and RoPE key,
    only the rows some verify row keeps (kept_rows: the size of that union)."""
    from synth import recipe
    rb = recipe.kv_row_bytes(s)          # one cache row (fp8 rows: codes, scale, padding)
    if s.idx_topk and kept_rows is None:
        raise ValueError("sparse attention: the kept-row count is needed")
    if s.idx_topk:
        # per row read: its index key, and for a kept row its latent and RoPE key
        # (fp8 rows: the codes, and the row's scale with each)
        ib, kb = (s.idx_dim + 4, s.kvw + 4) if s.kv_fmt == "fp8row" else (2 * s.idx_dim, 2 * s.kvw)
        kv = (L + s.T) * ib + kept_rows * kb + s.T * rb
    else:
        kv = (L + s.T) * rb + s.T * rb
    act = 2 * s.T * s.d * 4 + 2 * s.d * 4
    return attn_bytes(s) + router_bytes(s) + slots * expert_bytes(s) + kv + act


# The sources that make up the layer kernel and its launch configuration
# (the head, pack and embedding units do not change it).
LAYER_SOURCES = ("mk_common.h", "mk_device.h", "mk_layer_kernel.h", "mk_layer.hip", "mk_layer_kv8.hip",
                 "mk_layer_lr.hip", "mk_layer_lr_spec.hip", "mk_layer_sparse.hip", "mk_layer_sparse_kv8.hip",
                 "mk_api.cpp")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decoder_megakernel_amd", "csrc")
    for name in LAYER_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch from the committed counter profile, or None when the
    kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec["hbm_bytes_per_launch"]


def read_i32(dev_ptr):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    out = ctypes.c_int32(0)
    if hip.hipMemcpy(ctypes.byref(out), ctypes.c_void_p(dev_ptr), ctypes.c_size_t(4), ctypes.c_int(2)) != 0:
        raise RuntimeError("hipMemcpy failed")
    return out.value


def cores_used():
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(omp)) if omp and omp.isdigit() else n


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pct(xs):
    xs = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(xs)), 4), "p10": round(float(np.percentile(xs, 10)), 4),
            "p90": round(float(np.percentile(xs, 90)), 4)}


# ---------------------------------------------------------------- in-kernel trace: barrier share
# the phase that ends at each barrier slot of a layer launch, then the last phase
PHASE_NAMES = {0: "P0 Q/KV proj", 8: "P0b W_UQ", 1: "P1 RoPE+absorb", 9: "P1b index scores", 10: "P1c top-k",
               2: "P2 attention", 3: "P3 merge+W_UV", 4: "P4 W_O", 5: "P5 norm+router", 6: "P6 gate/up",
               7: "P6/7 experts", 11: "P8 combine"}
def trace_summary(layers, run_once):
    """Runs one untimed step with the layers' in-kernel trace on and returns the
    mean over the traced launches of: time in grid barriers (from the last
    arrival to the release), the critical path of each phase, and the launch's
    in-kernel total.  Timestamps: 100 MHz, per workgroup."""
    for dl in layers:
        dl.layer.set_trace(True)
    run_once()
    totals, bars, phases = [], [], []
    for dl in layers:
        st = dl.layer.stats()
        nb = st.barriers_per_step
        stride = 2 + 2 * nb + 16
        tr = np.zeros((st.grid_wgs, stride), np.int64)
        dl.layer.read_trace(tr)
        start, end = tr[:, 0], tr[:, 1 + 2 * nb]
        # the barrier slots a launch used, in the order it reached them
        used = [k for k in range(nb) if (tr[:, 1 + 2 * k] != 0).any()]
        used.sort(key=lambda k: np.median(tr[:, 2 + 2 * k]))
        prev = start
        bsum, ph = 0.0, {}
        for k in used:
            arr, rel = tr[:, 1 + 2 * k], tr[:, 2 + 2 * k]
            ph[PHASE_NAMES[k]] = (arr.max() - prev.min()) / 100.0
            bsum += (np.median(rel) - arr.max()) / 100.0
            prev = rel
        ph[PHASE_NAMES[nb]] = (end.max() - prev.min()) / 100.0
        totals.append((end.max() - start.min()) / 100.0)
        bars.append(bsum)
        phases.append(ph)
    for dl in layers:
        dl.layer.set_trace(False)
    names = [k for k in phases[0] if all(k in p for p in phases)]
    return {"barrier_share": round(float(np.mean(bars) / np.mean(totals)), 4),
            "barrier_us_per_launch": round(float(np.mean(bars)), 2),
            "in_kernel_us_per_launch": round(float(np.mean(totals)), 2),
            "phase_critical_path_us": {k: round(float(np.mean([p[k] for p in phases])), 2) for k in names},
            "launches_traced": len(layers)}


# ---------------------------------------------------------------- CPU baseline
def _omp_threads(n):
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def _time_layer(s, wx, H, kv, reps):
    import oracle
    ts = []
    for _ in range(reps):
        k = kv.copy()
        t0 = time.perf_counter()
        oracle.layer_step(s, wx, H, k, s.L)
        ts.append(time.perf_counter() - t0)
    return ts


def cpu_layer_sample(s):
    """The oracle (untuned) on one layer step of the workload: all cores, three
    repeats, and once on one thread; the routed experts the step needs are drawn
    beforehand (outside the timing)."""
    import oracle
    from synth import recipe
    w = recipe.layer_weights_host(s, 0, 0, experts=[])
    H = recipe.hidden_host(s, 0, 0)
    kv = recipe.kv_prefill_host(s, 0, 0)
    _, _, wx = oracle.layer_step_lazy(s, 0, 0, H, kv.copy(), s.L, base_weights=w)
    n = cores_used()
    _omp_threads(n)
    multi = _time_layer(s, wx, H, kv, 3)
    _omp_threads(1)
    single = _time_layer(s, wx, H, kv, 1)[0]
    _omp_threads(n)
    return multi, single


def cpu_baseline_stack(s, tokens_per_step):
    """A stack step is extrapolated as n_layers layer steps + one LM-head step."""
    import oracle
    from synth import recipe
    multi, single = cpu_layer_sample(s)
    emb, head, gf = recipe.stack_tables_host(s, 0)
    h = oracle.embed(emb, recipe.tokens_host(s, 0, 0))
    t0 = time.perf_counter()
    if s.head_fmt == "fp8":
        oracle.head_fp8(head[0], head[1], gf, h, s.eps)
    else:
        oracle.head(head, gf, h, s.eps, want_logits=False)
    t_head = time.perf_counter() - t0
    t_layer = float(np.median(multi))
    t_step = s.n_layers * t_layer + t_head
    return {"value": tokens_per_step / t_step, "unit": "tok/s/stream", "cores": cores_used(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "layer_step_s_all_cores": [round(x, 3) for x in multi],
            "layer_step_s_one_thread": round(single, 3),
            "head_step_s_all_cores": round(t_head, 3),
            "sample": "one layer step (layer 0, T=%d, L=%d, experts drawn beforehand) timed 3 times on %d threads "
                      "(median %.3f s) and once on 1 thread (%.2f s), one LM-head step %.2f s; stack step = %d x "
                      "layer + head = %.1f s; tokens/step as realized on the GPU"
                      % (s.T, s.L, cores_used(), t_layer, single, t_head, s.n_layers, t_step)}


def cpu_baseline_layer(s):
    multi, single = cpu_layer_sample(s)
    t = float(np.median(multi))
    return {"value": t * 1e6, "unit": "us/layer", "cores": cores_used(), "kind": "oracle", "cpu_model": cpu_model(),
            "layer_step_s_all_cores": [round(x, 3) for x in multi], "layer_step_s_one_thread": round(single, 3),
            "sample": "one layer step (T=%d, L=%d), experts drawn beforehand, 3 times on %d threads, once on 1"
                      % (s.T, s.L, cores_used())}


# ---------------------------------------------------------------- stack
def run_stack(s, args):
    import torch
    from decoder_megakernel_amd import harness
    from synth import recipe
    dev = torch.device("cuda", 0)
    n_layers = args.layers or s.n_layers
    s = s.with_(n_layers=n_layers)
    t0 = time.perf_counter()
    st = harness.DeviceStack(s, seed=0)
    log("[bench] stack of %d layers built in %.1f s" % (n_layers, time.perf_counter() - t0))
    if args.temperature > 0:
        st.model.set_sampling(args.temperature, 0)
    K, W = args.steps, args.warmup
    drafts = np.stack([recipe.tokens_host(s, 0, i + 1)[1:] for i in range(W + K + 2)]).astype(np.int32)
    drafts_d = torch.from_numpy(drafts).to(dev)
    tokens = torch.from_numpy(recipe.tokens_host(s, 0, 0)).to(dev)
    am = torch.empty(s.T, dtype=torch.int32, device=dev)
    com = torch.zeros(s.T + 1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step(i):
        st.model.step(tokens.data_ptr(), s.T, drafts_d[i].data_ptr(), am.data_ptr(), com.data_ptr(), None, sh)

    for i in range(W):
        step(i)
    torch.cuda.synchronize(dev)
    len0 = read_i32(st.model.length_ptr())
    stats0 = [dl.layer.stats() for dl in st.layers]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize(dev)
    evs[0].record(stream)
    for i in range(K):
        step(W + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    if st.model.sync_status() != 0:
        raise RuntimeError("device fault during the timed steps")
    ms = evs[0].elapsed_time(evs[K])
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
    len1 = read_i32(st.model.length_ptr())
    stats1 = [dl.layer.stats() for dl in st.layers]
    committed = len1 - len0
    slots = [(b.expert_blocks_sum - a.expert_blocks_sum) / max(1, b.device_launches - a.device_launches)
             for a, b in zip(stats0, stats1)]
    layer_launches = sum(b.launches - a.launches for a, b in zip(stats0, stats1))
    Lavg = 0.5 * (len0 + len1)
    step_bytes = sum(layer_bytes(s, Lavg, sl) for sl in slots) + head_bytes(s) + s.T * s.d * 2 + s.d * 4
    ms_step = ms / K
    tok_s = committed / (ms / 1e3)

    # dominant kernel: the layer launches of a step, timed alone (HIP events on the launch stream)
    reps = args.layer_reps
    h = torch.from_numpy(recipe.hidden_host(s, 0, 0)).to(dev)
    buf = [h.clone(), torch.empty_like(h)]
    Lnow = len1
    stats2 = [dl.layer.stats() for dl in st.layers]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for r in range(reps):
        for l, dl in enumerate(st.layers):
            dl.layer.decode_step(buf[l & 1].data_ptr(), s.T, st.kv[l].data_ptr(), st.capacity, Lnow,
                                 buf[(l + 1) & 1].data_ptr(), sh)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    launches = reps * n_layers
    us_layer = e0.elapsed_time(e1) * 1e3 / launches
    stats3 = [dl.layer.stats() for dl in st.layers]
    slots_l = [(b.expert_blocks_sum - a.expert_blocks_sum) / max(1, b.device_launches - a.device_launches)
               for a, b in zip(stats2, stats3)]
    lb = sum(layer_bytes(s, Lnow, sl) for sl in slots_l) / n_layers
    achieved = lb / (us_layer * 1e-6) / 1e9

    def traced_step():
        step(W + K)
        torch.cuda.synchronize(dev)

    tsum = trace_summary(st.layers, traced_step) if args.layer_trace else None
    res = {
        "metric": METRIC, "value": round(tok_s, 3), "unit": "tok/s/stream", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name, "layers": n_layers, "T": s.T, "kv_len_start": len0, "kv_len_end": len1,
                   "experts": s.E, "top_k": s.top_k, "shared": s.n_shared, "d_model": s.d, "d_ff": s.f,
                   "vocab": s.V, "expert_pools": s.n_pools or n_layers, "weights": EXPERT_DESC[s.exp_fmt] +
                   ", bf16 attention/router/embedding, %s head" % s.head_fmt, "kv": s.kv_fmt,
                   "verification": ("sampled, temperature %g" % args.temperature) if args.temperature > 0
                   else "greedy",
                   "compute": "bf16 MFMA operands, fp32 accumulation"},
        "tokens_per_step": round(committed / K, 4),
        "ms_per_step_dist": pct(per_step),
        "tok_s_at_tokens_per_step": {str(t): round(t / (ms_step * 1e-3), 1) for t in TAUS},
        "launches_per_step": round(layer_launches / K + 2, 2),
        "us_per_layer_step": round(ms_step * 1e3 / n_layers, 2),
        "us_per_layer_kernel": round(us_layer, 2),
        "step_bytes": int(step_bytes),
        "hbm_gbps_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "experts_streamed_per_layer": round(float(np.mean(slots)), 2),
        "barrier_share": tsum["barrier_share"] if tsum else None,
        "layer_trace": tsum,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": measured_traffic("layer_kernel_stack32_%s_T6_hbm_counters.json"
                                                 % (s.exp_fmt + ("" if s.kv_fmt == "bf16" else "_kv" + s.kv_fmt))),
                     "kernel": "layer_kernel<bf16, %s, %s>" % (s.exp_fmt, s.kv_fmt), "bytes_per_launch": int(lb),
                     "avg_launch_us": round(us_layer, 2), "launches_timed": launches},
    }
    if args.cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        res["cpu_baseline"] = cpu_baseline_stack(s, committed / K)
    return res


# ---------------------------------------------------------------- single layer
def run_layer(s, args):
    import torch
    from decoder_megakernel_amd import harness
    dev = torch.device("cuda", 0)
    copies = []
    ws = None
    for seed in range(3):
        dl = harness.DeviceLayer(s, seed, 0, workspace=ws)
        ws = dl.workspace
        copies.append((dl, harness.kv_cache(s, seed), [harness.hidden(s, seed, 0, j) for j in range(4)]))
    log("[bench] 3 weight copies of %s built" % s.name)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    out = torch.empty((s.T, s.d), dtype=torch.float32, device=dev)
    seq = [(c, j) for j in range(4) for c in range(3)]

    def launch(i):
        c, j = seq[i % len(seq)]
        dl, kv, hs = copies[c]
        dl.layer.decode_step(hs[j].data_ptr(), s.T, kv.data_ptr(), kv.shape[0], s.L, out.data_ptr(), sh)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize(dev)
    st0 = [c[0].layer.stats() for c in copies]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        launch(args.warmup + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    for c in copies:
        if c[0].layer.sync_status() != 0:
            raise RuntimeError("device fault during the timed steps")
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / args.steps
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]
    st1 = [c[0].layer.stats() for c in copies]
    slots = sum(b.expert_blocks_sum - a.expert_blocks_sum for a, b in zip(st0, st1)) / args.steps
    kept = None
    if s.idx_topk:
        # rows of the cache some verify row keeps, per launch (the mean over the weight copies)
        sizes = []
        for i in range(len(copies)):
            launch(i)
            torch.cuda.synchronize(dev)
            sel = np.empty((s.T, s.idx_topk), np.int32)
            copies[i][0].layer.debug_tap(8, sel)
            n_t = [min(s.idx_topk, s.L + t + 1) for t in range(s.T)]
            sizes.append(len(set(np.concatenate([sel[t, :n_t[t]] for t in range(s.T)]).tolist())))
        kept = float(np.mean(sizes))
    lb = layer_bytes(s, s.L, slots, kept)
    achieved = lb / (us * 1e-6) / 1e9

    def traced():
        launch(0)
        torch.cuda.synchronize(dev)

    tsum = trace_summary([copies[0][0]], traced) if args.layer_trace else None
    res = {
        "metric": METRIC, "value": round(us, 2), "unit": "us/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name, "T": s.T, "L": s.L, "experts": s.E, "top_k": s.top_k, "d_model": s.d,
                   "d_ff": s.f, "expert_format": s.exp_fmt, "routing": s.routing, "weight_copies": 3},
        "us_per_launch_dist": pct(per),
        "experts_streamed_per_step": round(slots, 2), "step_bytes": int(lb),
        "kept_rows_union": kept,
        "barrier_share": tsum["barrier_share"] if tsum else None,
        "layer_trace": tsum,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": None, "bytes_per_launch": int(lb),
                     "avg_launch_us": round(us, 2)},
    }
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_layer(s)
    return res


def process_starts(args, n):
    """Runs the same measurement in n separate processes (one after another,
    before this process touches the GPU) and returns their values."""
    vals = []
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", args.workload, "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--no-cpu-baseline", "--starts", "1", "--head-fmt", args.head_fmt,
           "--temperature", repr(args.temperature)]
    if args.kv_len is not None:
        cmd += ["--kv-len", str(args.kv_len)]
    for i in range(n):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("bench child process failed (%d): %s" % (r.returncode, r.stderr[-2000:]))
        v = json.loads(r.stdout.strip().splitlines()[-1])["value"]
        log("[bench] process start %d: %s" % (i + 1, v))
        vals.append(v)
    return vals


def main():
    from synth.configs import BY_KEY
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="C5", choices=[k for k in BY_KEY if k not in ("C0", "C1")])
    ap.add_argument("--layers", type=int, default=None, help="stack depth override (diagnostics only)")
    ap.add_argument("--kv-len", type=int, default=None,
                    help="cached positions before the step, for a single-layer workload (context sweeps)")
    ap.add_argument("--head-fmt", default="bf16", choices=["bf16", "fp8"],
                    help="LM-head table format (the stack workload names bf16)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="0: greedy verification; > 0: sampled verification at this temperature")
    ap.add_argument("--layer-reps", type=int, default=4)
    ap.add_argument("--starts", type=int, default=5,
                    help="process starts measured (this one and starts-1 child processes run before it)")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-layer-trace", dest="layer_trace", action="store_false",
                    help="skip the traced (untimed) step that measures the barrier share")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one elementwise kernel reading and writing this many MiB (a "
                         "known-size kernel for scaling hardware byte counters in a profile)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    s = BY_KEY[args.workload].with_(head_fmt=args.head_fmt)
    if args.kv_len is not None:
        if s.n_layers > 1 or args.kv_len < 0:
            print("--kv-len applies to single-layer workloads, with a length >= 0", file=sys.stderr)
            sys.exit(2)
        s = s.with_(name="%s@L%d" % (s.name, args.kv_len), L=args.kv_len, kv_capacity=0)
    if s.n_layers > 1:
        args.steps = args.steps or 256
        args.warmup = args.warmup if args.warmup is not None else 8
    else:
        args.steps = args.steps or 60
        args.warmup = args.warmup if args.warmup is not None else 12
    others = process_starts(args, args.starts - 1) if args.starts > 1 and args.layers is None else []
    res = run_stack(s, args) if s.n_layers > 1 else run_layer(s, args)
    if others:
        allv = others + [res["value"]]
        res["process_starts"] = {"values": allv, "median": round(float(np.median(allv)), 3),
                                 "min": min(allv), "max": max(allv),
                                 "spread": round((max(allv) - min(allv)) / float(np.median(allv)), 4)}
    if args.calib_copy_mib:
        import torch
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 2.0, out=dst)      # reads and writes exactly n bytes each
        torch.cuda.synchronize()
        log("[bench] calibration copy of %d MiB done" % args.calib_copy_mib)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
