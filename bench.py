"""Benchmark of the fused power pass on one MI355X.

Workload: the 10M-event design (100,000 gates with 1-4 inputs, 7x7 fp64
LUTs, 10,000 cycles of 1 ns, uniform activity scaled to 10M events; seeded
synthetic data of that shape).  A step is one pa_run: the fused pass over
all events and gates plus the finalize kernel.

Timing: W untimed warm-up passes plus >= 2 s of passes to reach steady
clocks; then K passes, each preceded by a 1 GiB write that evicts the L2s
and the 256 MB Infinity Cache (so the events come from HBM), all bracketed
by torch.cuda.synchronize().  ms_per_step is the median device time of the
pass (HIP events recorded by the library on its stream before the first
kernel and after the last); wall_ms_per_step is the bracket divided by K
(includes the flushes and the host side of each call).  The fused kernel's
algorithmic bytes per launch (12 B per event, 9 B per pin, 12 B per gate,
the tables once) over its own device time (HIP events attached to its
dispatch, which time the kernel's execution as the profiler's kernel trace
does) give roofline.achieved.

"per_event_and_per_gate" times the headline workload's pass with per-event
outputs and its per-gate pass (pa_run_gates), whole passes and the walk
kernel alone.

"configs" repeats the measurement for the other workloads (Tiny, Skewed,
Glitch-heavy and the 200M-event one), each loaded, warmed up and timed the
same way; the headline value stays the 10M-event workload's.

The CPU baseline is the C oracle timed on this host on the same workload:
whole passes on one core, then on all the cores this process may use (at
most 16), the gates cut into contiguous ranges, one per thread; the line
gives both, the thread count and the CPU model.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def clocks():
    """Current shader and memory clock levels read from the amdgpu sysfs files
    (no child process: the GPU is already initialised when this runs)."""
    import glob

    found = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [ln.strip() for ln in f if ln.rstrip().endswith("*")]
            except OSError:
                continue
            if cur:
                found.append(f"{os.path.basename(os.path.dirname(dev))} {name}: {cur[0]}")
    return found[:4]


def kernel_text(src):
    """Source text without comments and blank space: edits to comments do not
    change the kernel the counters were taken on."""
    import re

    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def profiled_traffic(workload):
    """HBM bytes per launch of the pass kernel (k_walk) from the committed
    rocprofv3 counter summary, or None when the kernel or the layout code
    changed since."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"k_walk_{workload}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    h = hashlib.sha256()
    # the kernel and the layout code (the stream's slots are the traffic)
    for f in ("pa_pass.hip", "pa_common.h", "pa_api.hip", "pa_load.hip"):
        with open(os.path.join(ROOT, "eda_gate_level_amd", "csrc", f)) as fh:
            h.update(kernel_text(fh.read()).encode())
    m_sha = re.search(r"fused_source_sha256: ([0-9a-f]{64})", text)
    m_tr = re.search(r"fused_traffic_bytes: ([0-9]+)", text)
    if not (m_sha and m_tr) or m_sha.group(1) != h.hexdigest():
        return None
    return int(m_tr.group(1))


def window_ablation(args, w, dev):
    """The paper's fixed-window comparison on this layout: the same pass with
    density-aware windows and with every gate's windows fixed at n cycles."""
    import torch

    import eda_gate_level_amd as pa

    d, tr = w.design, w.trace
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for n_fix in (0, 1, 2, 4, 8, 16, 32):
        an = pa.PowerAnalysis(0, torch.cuda.current_stream(dev), chunk_cycles=args.chunk_cycles,
                              grid_blocks=args.grid_blocks, time_kernels=1, fixed_window_cycles=n_fix)
        an.load(d, tr)
        outs = an.alloc_outputs()
        for _ in range(max(3, args.warmup // 4)):
            an.run(outs)
        fused = []
        for _ in range(max(5, args.steps // 2)):
            flush.fill_(1.0)
            an.run(outs)
            fused.append(an.info()["kernel_ms"][0])
        st = an.window_stats()
        print(json.dumps({"workload": w.name, "windows": "density-aware" if n_fix == 0 else f"fixed {n_fix} cycles",
                          "fused_ms": statistics.median(fused), "events_per_window": st}), flush=True)
        an.close()


def atomic_ablation(args, dev):
    """The paper's waveform-bin atomic stress test: 32 two-input gates, 100,000
    cycles, every pin toggling m = 1, 2, 4, 8 times per cycle (every event of
    a cycle lands in one bin), the pass with its LDS bin atomics against the
    same pass with plain loads, adds and stores and with plain stores alone
    (plain_bins 1 and 2: timing only, their bins are wrong)."""
    import torch

    import eda_gate_level_amd as pa
    from workloads import synth

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for m in (1, 2, 4, 8):
        w = synth.contention(m)
        row = {"workload": w.name, "events": w.trace.n_events, "toggles_per_cycle": m}
        for plain in (0, 1, 2):
            an = pa.PowerAnalysis(0, torch.cuda.current_stream(dev), time_kernels=1, plain_bins=plain)
            an.load(w.design, w.trace)
            outs = an.alloc_outputs()
            for _ in range(max(3, args.warmup // 4)):
                an.run(outs)
            fused = []
            for _ in range(max(5, args.steps // 2)):
                flush.fill_(1.0)
                an.run(outs)
                fused.append(an.info()["kernel_ms"][0])
            row[("atomic_fused_ms", "plain_add_fused_ms", "plain_store_fused_ms")[plain]] = statistics.median(fused)
            an.close()
        for k in ("plain_add", "plain_store"):
            row[f"atomic_overhead_vs_{k}_pct"] = round(100.0 * (row["atomic_fused_ms"] / row[f"{k}_fused_ms"] - 1.0), 2)
        print(json.dumps(row), flush=True)


def text_pipeline(args, w, dev):
    """Activity text through the host packer: the whole text packed on host
    threads alone, then the text's power analysis with packing and GPU work
    one after the other and overlapped (the paper's CPU-side event packing
    hidden behind the GPU), beside loading the same events from arrays."""
    import numpy as np
    import torch

    import eda_gate_level_amd as pa
    from workloads import vcd_text

    d, tr = w.design, w.trace
    t0 = time.time()
    text = vcd_text.write(tr)
    print(f"[bench] text of {w.name}: {len(text)} bytes, written in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    pack = []
    for _ in range(5):
        t0 = time.time()
        r = pa.pa_pack_text(text, tr.n_pins, args.text_threads)
        pack.append(time.time() - t0)
    same = all(np.array_equal(r[k], getattr(tr, k)) for k in ("pin_ptr", "pin_init", "evt_t", "evt_val", "evt_slew"))
    del r
    an = pa.PowerAnalysis(0, torch.cuda.current_stream(dev))
    an.load_design(d)
    t0 = time.time()
    an.load_events(tr)
    ref = an.run()
    torch.cuda.synchronize()
    arrays_s = time.time() - t0
    ref_tot = ref["totals"]
    ref_wave = ref["wave_J"].cpu().numpy()
    runs = {}
    for serial in (True, False):
        walls, st, tot = [], None, None
        for i in range(6):
            r = an.run_text(text, tr.t_clk, tr.t_max, tr.tick_s, segment_cycles=args.segment_cycles,
                            n_threads=args.text_threads, serial=serial)
            if i:
                walls.append(r["stats"]["wall_s"])
                st, tot = r["stats"], r["totals"]
        wave = r["wave_J"].cpu().numpy()
        err = max(abs(tot[k] - ref_tot[k]) / max(abs(ref_tot[k]), 1e-300) for k in ("e_int_J", "e_sw_J", "e_gl_J",
                                                                                        "e_leak_J"))
        werr = float(np.max(np.abs(wave - ref_wave) / np.maximum(np.abs(ref_wave), 1e-300)))
        runs[serial] = dict(wall_s=statistics.median(walls), stats=st, rel_err_totals=err, rel_err_bins=werr)
    an.close()
    E = tr.n_events
    ser, ovl = runs[True], runs[False]
    print(json.dumps({
        "workload": w.name, "mode": "activity text", "events": E, "text_bytes": len(text),
        "segment_cycles": args.segment_cycles or 1024, "threads": args.text_threads or "default",
        "pack_only_s": statistics.median(pack), "pack_only_GBps": len(text) / statistics.median(pack) / 1e9,
        "pack_only_matches_trace": bool(same),
        "serial_wall_s": ser["wall_s"], "overlapped_wall_s": ovl["wall_s"],
        "overlapped_events_per_s": E / ovl["wall_s"],
        "overlapped_parse_s": ovl["stats"]["parse_s"], "overlapped_gpu_s": ovl["stats"]["gpu_s"],
        "index_s": ovl["stats"]["index_s"], "header_s": ovl["stats"]["header_s"],
        "overlap_saving": 1.0 - ovl["wall_s"] / ser["wall_s"],
        "arrays_load_and_pass_s": arrays_s,
        "rel_err_totals": max(ser["rel_err_totals"], ovl["rel_err_totals"]),
        "rel_err_bins": max(ser["rel_err_bins"], ovl["rel_err_bins"])}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="medium")
    ap.add_argument("--chunk-cycles", type=int, default=0)
    ap.add_argument("--grid-blocks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="no 2 s clock warm-up, no CPU baseline and no other configurations (profiling runs)")
    ap.add_argument("--no-configs", action="store_true", help="time the chosen workload only")
    ap.add_argument("--window-ablation", action="store_true",
                    help="time the pass with density-aware windows and with fixed windows of 1..32 cycles "
                         "(one JSON line each, with the events-per-window distribution)")
    ap.add_argument("--atomic-ablation", action="store_true",
                    help="the waveform-bin stress workloads (m = 1, 2, 4, 8 toggles per pin and cycle), bin "
                         "atomics against plain loads and stores, one JSON line each")
    ap.add_argument("--text", action="store_true",
                    help="write the workload as activity text and time its host packing and the overlapped "
                         "text pipeline (one JSON line)")
    ap.add_argument("--segment-cycles", type=int, default=0, help="clock cycles per text segment (0 = 1024)")
    ap.add_argument("--text-threads", type=int, default=0, help="host packing threads (0 = min(16, cores))")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch

        n = args.copy_calibration << 18  # float32 elements
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 5}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the multi-GPU sharding is a design note "
                                   "(one all-reduce of the per-cycle bins), not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import eda_gate_level_amd as pa
    from workloads import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.atomic_ablation:
        atomic_ablation(args, dev)
        return
    t0 = time.time()
    w = synth.make(args.workload)
    if args.window_ablation:
        window_ablation(args, w, dev)
        return
    if args.text:
        text_pipeline(args, w, dev)
        return
    gen_s = time.time() - t0
    head = measure(args, w, dev, gen_s, flush_gib=1)
    info, tot = head.pop("_info"), head.pop("_totals")
    d, tr = w.design, w.trace
    E, G, P, C = tr.n_events, d.n_gates, tr.n_pins, tr.n_cycles

    # plain device copy in the same session: the HBM rate a streaming kernel reaches here
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    copy_ms = []
    for i in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flush.copy_(src)
        e1.record()
        e1.synchronize()
        if i >= 2:
            copy_ms.append(e0.elapsed_time(e1))
    copy_gbs = 2 * src.numel() * 4 / (statistics.median(copy_ms) * 1e-3) / 1e9
    del src, flush

    cpu = None
    if not (args.no_cpu_baseline or args.quick):
        cpu = cpu_baseline(w, tot)
    diag = None if args.quick else diag_passes(w, dev)

    # every other configuration: the same measurement, one line each in "configs"
    configs = {w.name: {k: head[k] for k in ("events", "fused_ms", "pass_ms", "events_per_s", "frac", "traffic")}}
    if not (args.quick or args.no_configs):
        del w, d, tr
        for name in ("tiny", "skewed", "glitch_heavy", "large"):
            if name in configs:
                continue
            t0 = time.time()
            wc = synth.make(name)
            r = measure(args, wc, dev, time.time() - t0, flush_gib=1, steps=max(10, args.steps // 3))
            configs[name] = {k: r[k] for k in ("events", "fused_ms", "pass_ms", "events_per_s", "frac", "traffic")}
            del wc, r
            torch.cuda.empty_cache()

    ms_step, ms_fused = head["pass_ms"], head["fused_ms"]
    line = {
        "metric": "events/sec and gate-cycles/sec (fused power pass), % of HBM roofline",
        "value": E / (ms_step * 1e-3),
        "unit": "events/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": head["workload"], "gates": G, "pins": P, "events": E, "cycles": C,
                   "chunk_cycles": info["chunk_cycles"], "grid_blocks": info["grid_blocks"],
                   "block_threads": info["block_threads"], "windows": info["n_windows"],
                   "stream_slots": info["n_slots"], "wave_steps_max": info["wave_steps_max"],
                   "wave_steps_mean": round(info["wave_steps_mean"], 2)},
        "gate_cycles_per_s": G * C / (ms_step * 1e-3),
        "fused_ms": ms_fused,
        "pass_ms_p10_p90": head["pass_ms_p10_p90"],
        "warm_pass_ms_median": head["warm_pass_ms"],
        "wall_ms_per_step": head["wall_ms_per_step"],
        "load_s": head["load_s"],
        "load_plus_pass_events_per_s": E / (head["load_s"] + ms_step * 1e-3),
        "roofline": {"bound": "hbm", "achieved": head["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["frac"], "traffic": head["traffic"], "alg_bytes_per_launch": head["alg_bytes"],
                     "copy_GBs": copy_gbs, "frac_of_copy": head["achieved"] / copy_gbs},
        "configs": configs,
        "per_event_and_per_gate": diag,
        "cpu_baseline": cpu,
        "clocks": head["clocks"],
        "device_bytes": info["device_bytes"],
    }
    print(json.dumps(line), flush=True)


def diag_passes(w, dev, steps=10):
    """The headline workload's pass with per-event outputs (glitch flags and
    states in the caller's order) and its per-gate pass (pa_run_gates): the
    median device time of each over cold passes, and of the walk kernel alone."""
    import torch

    import eda_gate_level_amd as pa

    out = {}
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    an = pa.PowerAnalysis(0, torch.cuda.current_stream(dev), time_kernels=1)
    try:
        an.load(w.design, w.trace)
        for name, outs in (("per_event", an.alloc_outputs(per_event=True)), ("per_gate", an.alloc_outputs(per_gate=True))):
            for _ in range(3):
                an.run(outs)
            kern, whole = [], []
            for mode in (1, 2):
                an.set_timing(mode)
                for _ in range(steps):
                    flush.fill_(1.0)
                    an.run(outs)
                    (kern if mode == 1 else whole).append(an.info()["kernel_ms"][0 if mode == 1 else 3])
            an.set_timing(1)
            out[name] = {"walk_kernel_ms": statistics.median(kern), "pass_ms": statistics.median(whole)}
            del outs
    finally:
        an.close()
    del flush
    return out


def measure(args, w, dev, gen_s, flush_gib=1, steps=None):
    """Load one workload and time its pass: W warm-up passes plus >= 2 s of
    passes for steady clocks, then K cold passes (a 1 GiB write before each
    evicts the L2s and the Infinity Cache), timed by the library's HIP events
    on its stream: the fused kernel alone, then the whole pass."""
    import numpy as np
    import torch

    import eda_gate_level_amd as pa

    steps = steps or args.steps
    d, tr = w.design, w.trace
    E, G, P, C = tr.n_events, d.n_gates, tr.n_pins, tr.n_cycles
    print(f"[bench] workload {w.name}: {G} gates, {P} pins, {E} events, {C} cycles (gen {gen_s:.1f}s)",
          file=sys.stderr, flush=True)
    an = pa.PowerAnalysis(0, torch.cuda.current_stream(dev), chunk_cycles=args.chunk_cycles,
                          grid_blocks=args.grid_blocks, time_kernels=True)
    t0 = time.time()
    an.load(d, tr)
    torch.cuda.synchronize()
    load_s = time.time() - t0
    outs = an.alloc_outputs(per_event=False)
    flush = torch.empty(flush_gib << 28, dtype=torch.float32, device=dev)

    clk_before = clocks()
    for _ in range(args.warmup):
        an.run(outs)
    t_end = time.time() + (0.0 if args.quick else 2.0)
    while time.time() < t_end:
        an.run(outs)
    warm = []
    an.set_timing(2)
    for _ in range(10):
        an.run(outs)
        warm.append(an.info()["kernel_ms"])
    an.set_timing(1)
    fused_ms, pass_ms = [], []
    for _ in range(steps):
        if not args.no_flush:
            flush.fill_(1.0)
        an.run(outs)
        fused_ms.append(an.info()["kernel_ms"][0])
    an.set_timing(2)
    torch.cuda.synchronize()
    tb0 = time.perf_counter()
    for _ in range(steps):
        if not args.no_flush:
            flush.fill_(1.0)
        tot = an.run(outs)["totals"]
        pass_ms.append(an.info()["kernel_ms"][3])
    torch.cuda.synchronize()
    tb1 = time.perf_counter()
    an.set_timing(1)
    clk_after = clocks()
    info = an.info()
    an.close()
    del flush, outs
    ms_step = statistics.median(pass_ms)
    ms_fused = statistics.median(fused_ms)
    tables = d.lut_J.nbytes + d.leak_W.nbytes + d.slew_axis.nbytes + d.cap_axis.nbytes
    alg_bytes = 12 * E + 9 * P + 12 * G + tables
    achieved = alg_bytes / (ms_fused * 1e-3) / 1e9
    return {
        "workload": f"{w.name}: {G} gates (inputs {int(d.cell_n_in.min())}-{int(d.cell_n_in.max())}, "
                    f"{d.n_slew}x{d.n_cap} fp64 LUTs), {C} cycles of {tr.t_clk} fs, {E} events, seed 0",
        "events": E, "fused_ms": ms_fused, "pass_ms": ms_step, "events_per_s": E / (ms_step * 1e-3),
        "achieved": achieved, "frac": achieved / HBM_PEAK_GBS, "alg_bytes": alg_bytes,
        "traffic": profiled_traffic(w.name),
        "pass_ms_p10_p90": [float(np.percentile(pass_ms, 10)), float(np.percentile(pass_ms, 90))],
        "warm_pass_ms": statistics.median(x[3] for x in warm),
        "wall_ms_per_step": (tb1 - tb0) * 1e3 / steps, "load_s": load_s,
        "clocks": {"before": clk_before, "after": clk_after}, "_info": info, "_totals": tot,
    }


def cpu_baseline(w, tot):
    """The oracle as it stands, on this host: whole passes of the workload on
    one core until about 10 s have run, then on all the host cores this
    process may use (at most 16, the CPU share of one GPU) until about 5 s
    have run; the medians per pass."""
    import oracle

    oracle.build()
    d, tr = w.design, w.trace
    E = tr.n_events
    one = []
    while sum(one) < 10.0 and len(one) < 20:
        t0 = time.perf_counter()
        o = oracle.run(d, tr, per_event=False)
        one.append(time.perf_counter() - t0)
    n = oracle.host_threads()
    many = []
    while sum(many) < 5.0 and len(many) < 40:
        t0 = time.perf_counter()
        om = oracle.run(d, tr, per_event=False, threads=n)
        many.append(time.perf_counter() - t0)
    s1, sn = statistics.median(one), statistics.median(many)
    rel = max(abs(o["e_int_J"] - tot["e_int_J"]) / abs(o["e_int_J"]),
              abs(om["e_leak_J"] - tot["e_leak_J"]) / abs(om["e_leak_J"]))
    return {"value": E / sn, "unit": "events/s", "cores": n, "kind": "oracle",
            "cpu_model": oracle.cpu_model(),
            "single_core": {"value": E / s1, "unit": "events/s", "cores": 1, "s_per_pass": s1, "passes": len(one)},
            "all_core": {"s_per_pass": sn, "passes": len(many), "threads": n},
            "sample": f"whole passes of the {w.name} workload ({E} events each) by the C oracle: {len(one)} on one "
                      f"core (median {s1:.2f} s), then {len(many)} on {n} threads (gate ranges, median "
                      f"{sn:.3f} s); its e_int and e_leak agree with the GPU to {rel:.1e}"}


if __name__ == "__main__":
    main()
