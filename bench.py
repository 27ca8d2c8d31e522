#!/usr/bin/env python3
"""Benchmark of the static-cache additive-bias GQA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--secondary | --no-secondary] [--eager] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of seeded synthetic
input: TensorScatter of K and V (skipped by the KV-shared variant), the bias
build and the attention. A decode step is one launch (attn_bias_gqa_decode_step:
the scatters, the bias and the attention in the split-KV kernel); a prefill
step is two, the scatters and the bias fused (kv_scatter_and_bias), then the
attention. --separate-calls times a decode step as those two launches too. The
default workload is the sliding-window decode layer (B8 Hq16 Hkv8 D256,
max_seq 4096, window 1024, S_q 1); the secondary lines are the other four
workload shapes, the two sliding layers over a circular (window-sized) cache,
and the main decode workload as separate calls.

Timing. Inputs are resident in HBM before the timed region. R copies of every
input rotate through the steps (step i uses copy i % R), R chosen so that the
bytes the R copies' steps read cover three times the 256 MB Infinity Cache: no
step finds its data left warm by the steps before it. The K timed steps are
captured into one HIP graph (torch.cuda.CUDAGraph over the library's launches
on the capture stream), which is replayed once in the timed region: exactly K
steps. Its output is compared bit for bit with the eager result first. A second
graph holds the same K attention launches alone: its replay time per launch is
the dominant kernel's average duration (HIP events on the stream the kernels
run on). --eager times launch by launch instead (used under rocprofv3 counter
runs).

Output: one JSON line. value = algorithmic bytes of a step / step time (GB/s).
roofline = the dominant kernel's algorithmic bytes (decode: the fused step
kernel, or the attention kernel of separate calls) or flops (prefill) per
launch / its average duration, against the MI355X peak (HBM 8 TB/s; bf16 dense
matrix cores 2.5 PFLOP/s). cpu_baseline = the fp64 oracle timed on the
host cores on a bounded sample of the same workload (every secondary workload
carries its own).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
CACHE_BYTES = 256 << 20  # Infinity Cache

WORKLOADS = ["decode_sliding", "decode_full", "decode_full_kvshared", "prefill_vision",
             "prefill_long", "decode_sliding_circular", "prefill_vision_circular"]
DECODE = {"decode_sliding", "decode_full", "decode_full_kvshared", "decode_sliding_circular"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


V_HEAD = None      # --v-head-size: V head size of the KV-shared decode or of a prefill


def make_workload(name):
    from additive_bias_gqa_amd import workloads as wl
    return {
        "decode_sliding": wl.decode_sliding,
        "decode_full": wl.decode_full,
        "decode_full_kvshared": lambda: wl.decode_full(kv_shared=True, Dv=V_HEAD),
        "prefill_vision": lambda: wl.prefill_vision(Dv=V_HEAD),
        "prefill_long": lambda: wl.prefill_long(Dv=V_HEAD),
        # the sliding layers over a circular (window-sized) cache
        "decode_sliding_circular": wl.decode_sliding_circular,
        "prefill_vision_circular": wl.prefill_vision_circular,
    }[name]()


class InputSet:
    """One resident copy of every input and output of a step."""

    def __init__(self, w, step, torch):
        d = "cuda"
        self.k = w.k_cache.to(d)
        self.v = w.v_cache.to(d)
        self.q = step.q.to(d)
        self.k_new = None if step.k_new is None else step.k_new.to(d)
        self.v_new = None if step.v_new is None else step.v_new.to(d)
        self.wi = None if step.write_indices is None else step.write_indices.to(d)
        self.nonpad = step.nonpad.to(d)
        self.q_start = step.q_start.to(d)
        self.kind = None if step.slot_kind is None else step.slot_kind.to(d)
        self.bias = torch.empty((w.B, 1, step.S_q, w.max_seq), dtype=w.dtype, device=d)
        self.out = torch.empty((w.B, w.Hq, step.S_q, w.Dv), dtype=w.dtype, device=d)


VARIANT = "bias"   # "bias": materialised bias tensor; "rules": rules evaluated in-kernel
SOFTCAP = 0.0      # > 0: softcap * tanh(score / softcap) before the bias


def run_scatter_bias(ab, w, step, s):
    """TensorScatter of K and V and the bias build, as one fused launch
    (kv_scatter_and_bias; bit-identical to the three separate calls). The
    KV-shared workload has nothing to scatter; the rules variant builds no bias;
    a circular cache takes the circular calls."""
    if w.circular:
        ab.kv_scatter_and_bias_circular(s.k, s.v, s.k_new, s.v_new, s.wi, s.nonpad, s.q_start, s.kind,
                                        step.S_q, w.window, bias=s.bias if VARIANT == "bias" else None)
        return
    if s.k_new is None or s.v.shape[-1] != s.k.shape[-1]:
        # KV-shared: nothing to scatter; V of another head size: the two
        # scatters apart (the fused launch takes one row size)
        if s.k_new is not None:
            ab.kv_tensor_scatter(s.k, s.k_new, s.wi)
            ab.kv_tensor_scatter(s.v, s.v_new, s.wi)
        if VARIANT == "bias":
            ab.build_static_cache_bias(s.nonpad, s.q_start, s.kind, step.S_q, w.max_seq, w.window,
                                       out=s.bias)
        return
    ab.kv_scatter_and_bias(s.k, s.v, s.k_new, s.v_new, s.wi, s.nonpad, s.q_start, s.kind, step.S_q,
                           w.window, bias=s.bias if VARIANT == "bias" else None)


def fused_step(w, step, fused):
    """Whether this step runs as one launch (bf16 decode: rows of the split-KV kernel)."""
    return fused and w.dtype.is_floating_point and w.dtype.itemsize == 2 and \
        step.S_q * (w.Hq // w.Hkv) <= 16


def run_step(ab, w, step, s, ws, fused):
    """One whole step: the fused decode step, or the separate launches."""
    if fused:
        fn = ab.attn_bias_gqa_decode_step_circular if w.circular else ab.attn_bias_gqa_decode_step
        fn(s.q, s.k, s.v, s.k_new, s.v_new, s.wi, s.nonpad, w.scale, q_start=s.q_start,
           slot_kind=s.kind, window=w.window, bias=s.bias if VARIANT == "bias" else None, out=s.out,
           workspace=ws, softcap=SOFTCAP)
        return
    run_scatter_bias(ab, w, step, s)
    run_attention(ab, w, s, ws)


def run_attention(ab, w, s, ws):
    fwd = ab.attn_bias_gqa_fwd_circular if w.circular else ab.attn_bias_gqa_fwd
    if VARIANT == "bias":
        fwd(s.q, s.k, s.v, s.bias, s.nonpad, w.scale, out=s.out, workspace=ws, softcap=SOFTCAP)
    else:
        fwd(s.q, s.k, s.v, None, s.nonpad, w.scale, q_start=s.q_start, slot_kind=s.kind,
            window=w.window, out=s.out, workspace=ws, softcap=SOFTCAP)


def work_counts(w, step, s, torch):
    """Algorithmic work of one step, counted from the bias the step builds:
    live keys (allowed for some query row, below nonpad) and allowed pairs."""
    T = w.max_seq
    allowed = (s.bias[:, 0] == 0)                                  # [B, S_q, T]
    valid = torch.arange(T, device="cuda")[None, None, :] < s.nonpad[:, None, None]
    allowed &= valid
    pairs = int(allowed.sum().item())
    live_keys = int(allowed.any(dim=1).sum().item())              # sum over b of live slots
    nonpad_sum = int(s.nonpad.clamp(0, T).sum().item())
    e = 2 if w.dtype == torch.bfloat16 else 4
    B, Hq, Hkv, D, Dv, S_q = w.B, w.Hq, w.Hkv, w.D, w.Dv, step.S_q
    kv = live_keys * Hkv * (D + Dv) * e                            # K and V rows read once
    bias_read = S_q * nonpad_sum * e                               # bias rows below nonpad
    qo = B * Hq * S_q * (D + Dv) * e                               # Q read + out written
    attn_bytes = kv + bias_read + qo
    attn_flops = 2.0 * (D + Dv) * Hq * pairs                       # QK^T and PV, 2 flop/MAC
    S_new = 0 if step.k_new is None else step.k_new.shape[2]
    scatter_bytes = 2 * B * Hkv * S_new * (D + Dv) * e             # K and V: read + write
    kind_bytes = 0 if step.slot_kind is None else B * T * 4
    bias_bytes = B * S_q * T * e + kind_bytes                      # written once, kinds read
    return dict(pairs=pairs, live_keys=live_keys, attn_bytes=attn_bytes, attn_flops=attn_flops,
                step_bytes=attn_bytes + scatter_bytes + bias_bytes,
                scatter_bytes=scatter_bytes, bias_bytes=bias_bytes, bias_read=bias_read)


def time_graph(torch, g, reps):
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)  # ms


def bench_workload(name, steps, warmup, eager, torch, ab, fused=True):
    w = make_workload(name)
    step = w.steps[0]
    fused = fused_step(w, step, fused)
    log(f"{name}: {w.describe()}, {'one fused launch' if fused else 'separate launches'} per step")
    probe = InputSet(w, step, torch)
    per_set = sum(t.numel() * t.element_size() for t in
                  (probe.k, probe.v, probe.q, probe.bias, probe.out))
    need = ab.attn_bias_gqa_workspace_bytes(w.B, w.Hq, w.Hkv, step.S_q, w.max_seq, w.D, w.Dv)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda") if need else None

    # the work of a step, counted from the bias it builds (the rules variant
    # materialises the same rules once for the count)
    run_scatter_bias(ab, w, step, probe)
    if VARIANT == "rules":
        ab.build_static_cache_bias(probe.nonpad, probe.q_start, probe.kind, step.S_q, w.max_seq,
                                   w.window, dtype=w.dtype, out=probe.bias)
    counts = work_counts(w, step, probe, torch)
    if VARIANT == "rules":   # no bias tensor is read or written in this variant
        counts["attn_bytes"] -= counts["bias_read"]
        counts["step_bytes"] = counts["attn_bytes"] + counts["scatter_bytes"]
    elif fused:              # the fused step writes the bias but never reads it
        counts["step_bytes"] -= counts["bias_read"]
    # bytes of the dominant kernel: the fused step's whole step, or the attention
    counts["kernel_bytes"] = counts["step_bytes"] if fused else counts["attn_bytes"]

    # Copies of the inputs rotate so that a step never finds the data it reads
    # in the 256 MB Infinity Cache: the sets' live bytes (what a step actually
    # reads) cover at least three times the cache.
    n_sets = max(2, min(32, math.ceil(3 * CACHE_BYTES / max(counts["attn_bytes"], 1))))
    sets = [probe] + [InputSet(w, step, torch) for _ in range(n_sets - 1)]
    log(f"{name}: {n_sets} rotating input sets ({counts['attn_bytes'] / 2**20:.0f} MiB read by a step, "
        f"{per_set / 2**20:.0f} MiB allocated per set), workspace {need} B")

    # eager warm-up (every set at least once) and reference outputs
    for i in range(max(warmup, n_sets)):
        run_step(ab, w, step, sets[i % n_sets], ws, fused)
    torch.cuda.synchronize()
    ref_out = [s.out.clone() for s in sets]
    for s in sets:
        assert torch.isfinite(s.out.float()).all(), "non-finite output"

    K = steps   # exactly the steps asked for; step i uses set i % n_sets
    ibits = torch.int16 if w.dtype == torch.bfloat16 else torch.int32
    if eager:
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for i in range(K):
            s = sets[i % n_sets]
            if not fused:
                run_scatter_bias(ab, w, step, s)
            ev[i][0].record(st)
            if fused:
                run_step(ab, w, step, s, ws, True)
            else:
                run_attention(ab, w, s, ws)
            ev[i][1].record(st)
        e1.record(st)
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / K
        attn_ms = sum(a.elapsed_time(b) for a, b in ev) / K
        mode = "eager"
    else:
        # one graph of the K steps, and one of their K attention launches alone
        g_step, g_attn = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g_step):
                for i in range(K):
                    run_step(ab, w, step, sets[i % n_sets], ws, fused)
            with torch.cuda.graph(g_attn):
                for i in range(K):
                    if fused:   # the one kernel of the step
                        run_step(ab, w, step, sets[i % n_sets], ws, True)
                    else:
                        run_attention(ab, w, sets[i % n_sets], ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        # the graphs must reproduce the eager outputs bit for bit, replay after replay
        for g in (g_step, g_attn, g_step):
            for s in sets:
                s.out.view(ibits).fill_(0x7FC1)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for s, r in zip(sets[:K], ref_out):
                assert torch.equal(s.out.view(ibits), r.view(ibits)), "graph replay differs from eager"
        step_ms = time_graph(torch, g_step, 1) / K
        attn_ms = time_graph(torch, g_attn, 1) / K
        mode = "graph"

    res = dict(workload=name, mode=mode, steps=K, ms_per_step=step_ms, attn_ms=attn_ms,
               counts=counts, desc=w.describe(), n_sets=n_sets, fused=fused)
    if name in DECODE:
        res["attn_rate"] = counts["kernel_bytes"] / (attn_ms * 1e-3) / 1e9     # GB/s
        res["roofline"] = dict(bound="hbm", achieved=round(res["attn_rate"], 1),
                               peak=HBM_PEAK_GBS, unit="GB/s",
                               frac=round(res["attn_rate"] / HBM_PEAK_GBS, 4))
    else:
        res["attn_rate"] = counts["attn_flops"] / (attn_ms * 1e-3) / 1e12      # TFLOP/s
        res["roofline"] = dict(bound="mfma", achieved=round(res["attn_rate"], 1),
                               peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                               frac=round(res["attn_rate"] / BF16_PEAK_TFLOPS, 4))
        # the same call against HBM (a prefill chunk of few rows per key sits
        # near the ridge point): its algorithmic bytes over the same time
        hbm = counts["attn_bytes"] / (attn_ms * 1e-3) / 1e9
        res["hbm_side"] = dict(achieved=round(hbm, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                               frac=round(hbm / HBM_PEAK_GBS, 4))
    res["step_gbs"] = counts["step_bytes"] / (step_ms * 1e-3) / 1e9
    side = f", HBM side {100 * res['hbm_side']['frac']:.1f}%" if "hbm_side" in res else ""
    log(f"{name}: {mode} step {step_ms * 1e3:.1f} us, {'fused kernel' if fused else 'attention'} "
        f"{attn_ms * 1e3:.1f} us, "
        f"{res['roofline']['achieved']} {res['roofline']['unit']} "
        f"({100 * res['roofline']['frac']:.1f}% of peak{side})")
    del sets, probe, ws
    torch.cuda.empty_cache()
    return res, w


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy (torch copy_ kernel) of nbytes: the
    practical HBM ceiling on this device, read + write bytes per second."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(st)
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


KERNEL_SOURCES_DIR = os.path.join("additive_bias_gqa_amd", "csrc")


def fused_default(name):
    """The step form a default run takes (traffic records are taken on it):
    one fused launch for the decode workloads."""
    return name in DECODE


def kernel_sources(name):
    """The sources that build the dominant kernel of a workload's step: the ABI
    dispatch, the phase's kernel files and the headers they include."""
    common = ["abi.hip", "common.h", "kernels.h", "mask_rules.h"]
    if name.startswith("decode"):
        files = common + ["attn_decode_step.hip", "decode_kernel.h"]
    else:
        files = common + ["attn_prefill_dma.hip", "attn_prefill_dma_wide.hip", "prefill_dma.h",
                          "prefill_common.h"]
    return sorted(os.path.join(KERNEL_SOURCES_DIR, f) for f in files)


def sources_sha256(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_for(name):
    """HBM bytes per attention call from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; else None."""
    path = os.path.join(HERE, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    try:
        if sources_sha256(rec.get("sources", [])) != rec.get("source_sha256") or \
                rec.get("sources") != kernel_sources(name):
            return None
    except OSError:
        return None
    return rec.get("hbm_bytes_per_launch")


def write_traffic(name, fetch_csv, write_csv, copy_bytes=1 << 30):
    """Turn two rocprofv3 --pmc runs of `bench.py --eager` (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into HBM bytes per attention call.

    Each counter is scaled by what it reads for the plain 1 GiB device copy
    that bench.py runs first (the largest __amd_rocclr_copyBuffer dispatch):
    scale = copy bytes / (counter KiB * 1024). The attention call is every
    kernel it launches (abgqa::attn_*, and the prefill's live-tile map pass),
    averaged per dispatch and summed."""
    import csv
    import collections

    def read(path):
        per = collections.defaultdict(list)
        copy_max = 0.0
        with open(path) as f:
            for r in csv.DictReader(f):
                k, v = r["Kernel_Name"], float(r["Counter_Value"])
                if k == "__amd_rocclr_copyBuffer":
                    copy_max = max(copy_max, v)
                elif k.startswith("void abgqa::attn_") or "tilemap_kernel" in k:
                    per[k].append(v)
        if not per or copy_max <= 0:
            raise SystemExit(f"{path}: no attention or copy dispatches found")
        return per, copy_bytes / (copy_max * 1024.0)

    fetch, fs = read(fetch_csv)
    write, ws = read(write_csv)
    kernels = {}
    total = 0.0
    for k in sorted(fetch):
        fk = sum(fetch[k]) / len(fetch[k]) * 1024.0 * fs
        wk = sum(write[k]) / len(write[k]) * 1024.0 * ws if k in write else 0.0
        kernels[k] = dict(dispatches=len(fetch[k]), fetch_bytes=round(fk), write_bytes=round(wk))
        total += fk + wk
    rels = kernel_sources(name)
    rec = dict(workload=name, fetch_scale=round(fs, 5), write_scale=round(ws, 5),
               copy_bytes=copy_bytes, kernels=kernels, hbm_bytes_per_launch=round(total),
               sources=rels, source_sha256=sources_sha256(rels))
    path = os.path.join(HERE, "profiles", f"traffic_{name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def cpu_baseline(name, w, counts, budget_s=12.0):
    """The oracle (scatter + bias + attention, fp64, OpenMP) on the workload's
    batch entries, one after another and round again, until ~budget_s of host
    work. value: algorithmic step bytes per second (the unit of the step rate);
    attn_rate: the attention's algorithmic work per second in the unit of the
    workload's roofline (GB/s for decode, TFLOP/s for prefill)."""
    import oracle
    step = w.steps[0]
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    oracle.build(force=False)
    t0 = time.perf_counter()
    done = 0
    while True:
        b = done % w.B
        sl = slice(b, b + 1)
        k, v = w.k_cache[sl], w.v_cache[sl]
        scatter = oracle.scatter_circular if w.circular else oracle.scatter
        if step.k_new is not None:
            k = scatter(k, step.k_new[sl], step.write_indices[sl])
            v = scatter(v, step.v_new[sl], step.write_indices[sl])
        kind = None if step.slot_kind is None else step.slot_kind[sl]
        build = oracle.bias_circular if w.circular else oracle.bias
        bias = build(step.nonpad[sl], step.q_start[sl], kind, step.S_q, w.max_seq, w.window)
        oracle.attention(step.q[sl], k, v, bias, step.nonpad[sl].clamp(0, w.max_seq), w.scale)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    frac_steps = done / w.B
    rate = counts["step_bytes"] * frac_steps / dt / 1e9
    if name in DECODE:
        attn_rate, attn_unit = counts["attn_bytes"] * frac_steps / dt / 1e9, "GB/s"
    else:
        attn_rate, attn_unit = counts["attn_flops"] * frac_steps / dt / 1e12, "TFLOP/s"
    return dict(value=round(rate, 4), unit="GB/s", cores=cores, kind="oracle",
                attn_rate=round(attn_rate, 6), attn_unit=attn_unit,
                sample=f"{done} batch-entry passes ({frac_steps:.2f} steps of B={w.B}; "
                       f"scatter + bias + attention of one batch entry each) in {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_sliding", choices=WORKLOADS)
    ap.add_argument("--secondary", dest="secondary", action="store_true", default=True)
    ap.add_argument("--no-secondary", dest="secondary", action="store_false")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", default="bias", choices=["bias", "rules"],
                    help="bias: build and read the bias tensor; rules: evaluate the mask "
                         "rules inside the attention kernel (no bias tensor)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="softcap of the attention scores (0 = none, the workloads' setting)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time a decode step as kv_scatter_and_bias + attn_bias_gqa_fwd (two "
                         "launches) instead of the fused step")
    ap.add_argument("--v-head-size", type=int, default=None,
                    help="head size of V for decode_full_kvshared, prefill_vision or prefill_long (V "
                         "may have another head size than Q and K; default: the query's)")
    args = ap.parse_args()
    if args.v_head_size is not None and args.workload not in ("decode_full_kvshared", "prefill_vision",
                                                               "prefill_long"):
        ap.error("--v-head-size applies to --workload decode_full_kvshared, prefill_vision or prefill_long")
    if args.traffic_from:
        write_traffic(args.workload, *args.traffic_from)
        return
    global VARIANT, SOFTCAP, V_HEAD
    VARIANT = args.variant
    SOFTCAP = args.softcap
    V_HEAD = args.v_head_size

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported: the "
              f"hot path is measured on one GPU's share of the work (the kernels need no exchange "
              f"when batch rows or KV heads are split across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import additive_bias_gqa_amd as ab
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ab.load()
    log(f"device {torch.cuda.get_device_name(0)}, library {ab.library_path()}")

    t_start = time.perf_counter()
    copy_gbs = copy_bandwidth(torch)
    log(f"device copy bandwidth {copy_gbs:.0f} GB/s (read + write)")
    fused = not args.separate_calls
    main_res, w = bench_workload(args.workload, args.steps, args.warmup, args.eager, torch, ab, fused)
    secondary = {}
    if args.secondary:
        runs = [(n, fused) for n in WORKLOADS if n != args.workload]
        if main_res["fused"]:   # the main decode workload as separate calls, for comparison
            runs.append((args.workload, False))
        for name, fz in runs:
            r, w2 = bench_workload(name, max(8, args.steps // 10), 2, args.eager, torch, ab, fz)
            key = name if fz or not main_res["fused"] or name != args.workload else f"{name}_separate_calls"
            secondary[key] = dict(
                attn_us=round(r["attn_ms"] * 1e3, 2), step_us=round(r["ms_per_step"] * 1e3, 2),
                steps=r["steps"], rotating_input_sets=r["n_sets"],
                step_form="fused" if r["fused"] else "separate",
                roofline=dict(r["roofline"], traffic=traffic_for(name) if r["fused"] == fused_default(name) else None),
                step_gbs=round(r["step_gbs"], 1), config=r["desc"])
            if "hbm_side" in r:
                secondary[key]["hbm_side"] = r["hbm_side"]
            if not args.no_cpu_baseline and key == name:
                log(f"{name}: cpu baseline (oracle) ...")
                secondary[key]["cpu_baseline"] = cpu_baseline(name, w2, r["counts"], budget_s=8.0)
            del w2

    rl = dict(main_res["roofline"])
    rl["traffic"] = traffic_for(args.workload) if main_res["fused"] == fused_default(args.workload) else None
    counts = main_res["counts"]
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(args.workload, w, counts)
    cfg = dict(main_res["desc"])
    cfg.update({"kernel_timing": main_res["mode"], "rotating_input_sets": main_res["n_sets"],
                "device_copy_gbs": round(copy_gbs, 1), "variant": VARIANT, "softcap": SOFTCAP,
                "step_form": ("one launch (attn_bias_gqa_decode_step: scatters, bias, attention)"
                              if main_res["fused"] else "separate launches"),
                "kernel_us": round(main_res["attn_ms"] * 1e3, 2),
                "kernel_bytes": counts["kernel_bytes"], "step_bytes": counts["step_bytes"],
                **({"hbm_side": main_res["hbm_side"]} if "hbm_side" in main_res else {}),
                "live_keys": counts["live_keys"]})
    line = {
        "metric": "decode KV GB/s (% of HBM peak) + prefill attention TFLOP/s (% of MFMA peak)",
        "value": round(main_res["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64; N(0,1) bf16 values, random bits beyond nonpad)",
        "config": cfg,
        "roofline": rl,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "wall_s": round(time.perf_counter() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
