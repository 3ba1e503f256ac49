#!/usr/bin/env python3
"""Benchmark of the latent mixture-of-experts decode layer on one MI355X.

A step is one forward of the whole layer (gate gemv, route, fc1_latent_proj, routed 4-bit
experts, combine, fc2_latent_proj, shared expert, residual) over one batch of rows, with
inputs already resident in HBM. Consecutive steps rotate through `--instances` distinct
copies of the layer's weights (independent seeded draws), so that each step streams its
weights from HBM instead of the 256 MB Infinity Cache: 8 copies of the 107 MB Bolt-like
layer are 0.86 GB. The steps are replayed from a captured HIP graph.

Prints one JSON line: layer-tokens/s (rows x steps / seconds), the whole layer's achieved
HBM bandwidth from its algorithmic bytes, the dominant kernel's roofline (algorithmic
bytes of one launch / its average duration inside full forwards, the duration taken from
HIP events that the launch's own kernel dispatch records on the launch stream), and the
CPU oracle timed on this host. Each launch group is also timed alone (graph replays of that
launch over all instances, "us_alone"): a launch runs 0.2-1.7 us faster after itself than
after the previous launch of a forward.
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

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
# stages of the work-item table, in the library's order (include/moe_latent.h,
# moe_latent_group_stages), and the keys of stage_bytes
STAGE_KEYS = ["gate", "fc1", "shup", "route", "shdn_a", "up", "shdn_b", "down", "fc2"]
KERNEL_SOURCES = ["latent_mixture_experts_bf16_amd/csrc/layer_kernels.hip",
                  "latent_mixture_experts_bf16_amd/csrc/layer_items.h",
                  "latent_mixture_experts_bf16_amd/csrc/layer_plan.h",
                  "latent_mixture_experts_bf16_amd/csrc/moe_latent_api.hip"]
COPY_MIB = 512   # size of the calibration copy (int32 negation: reads and writes COPY_MIB MiB)


def plan_groups(B, handle, dims, rows):
    """The launch groups of a pass, from the library's plan: index, name, stages (stage_bytes
    keys), side stream, workgroups, kernel name."""
    out = []
    for g in range(16):
        n, f, l, side = B.moe_latent_group_stages(handle, rows, g)
        if n <= 0:
            break
        stages = STAGE_KEYS[f:l + 1]
        name = "+".join(stages) + (" [side stream]" if side else "")
        out.append({"group": g, "name": name, "stages": stages, "side": side, "items": n,
                    "kernel": B.moe_latent_group_kernel(handle, rows, g), "first": f, "last": l})
    # the route items end the gate launch (the library's logit hand-off): the route stage of
    # any later launch range holds no items
    if out:
        for o in out:
            if "route" in o["stages"]:
                o["stages"] = [st for st in o["stages"] if st != "route"]
                o["name"] = "+".join(o["stages"]) + (" [side stream]" if o["side"] else "")
        out[0]["stages"] = out[0]["stages"] + ["route"]
        out[0]["name"] = out[0]["name"] + "+route"
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400)
    ap.add_argument("--warmup", type=int, default=240)
    ap.add_argument("--config", type=int, default=1, help="workload id (0..3 single layer)")
    ap.add_argument("--instances", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many forwards eagerly, then one calibration copy, and exit "
                         "(the workload of the rocprofv3 --pmc runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) into "
                         "the traffic summary --pmc-out")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="turn a rocprofv3 --kernel-trace --stats output folder into a text summary "
                         "written to --stats-out")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="turn a rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 output folder into "
                         "the MFMA summary --mfma-out")
    ap.add_argument("--mfma-out")
    ap.add_argument("--mfma-workload", default="")
    ap.add_argument("--pmc-out")
    ap.add_argument("--stats-out")
    ap.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--no-rows-sweep", action="store_true",
                    help="skip the 16-row and 64-row passes reported beside the one-row line")
    ap.add_argument("--formats", default="",
                    help="also time the Bolt-like layer with routed experts in these affine formats, "
                         "e.g. 2:64,3:64,4:64,4:128,5:64,6:64,8:64 (bits:group_size)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the fused prefill timing")
    ap.add_argument("--only-prefill", action="store_true", help="time the fused prefill only")
    ap.add_argument("--no-lm-head", action="store_true",
                    help="skip the lm_head gemv (K 4096, N 131072, 1 and 16 rows) reported beside it")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.json")


def _csv_rows(folder, name):
    import csv
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", f"*{name}"), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{name} under {folder}")
    return rows


def _layer_kernel(kernel_name):
    """A layer kernel's name as the library reports it (moe_latent_group_kernel), or None."""
    if "moe_stage_kernel<" in kernel_name:
        return "moe_stage_kernel<" + kernel_name.split("moe_stage_kernel<")[1].split(">")[0] + ">"
    return "moe_front_kernel" if "moe_front_kernel" in kernel_name else None


def _short(kernel_name):
    k = _layer_kernel(kernel_name)
    if k is not None:
        return k
    return "copy" if "elementwise" in kernel_name else None


def summarize_pmc(args):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each layer kernel, scaled by the
    same counters of the calibration copy of known size."""
    import numpy as np
    out = {}
    for counter, folder in (("FETCH_SIZE", args.summarize_pmc[0]), ("WRITE_SIZE", args.summarize_pmc[1])):
        per = {}
        for r in _csv_rows(folder, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            k = _short(r.get("Kernel_Name", ""))
            if k is None:
                continue
            per.setdefault(k, []).append(float(r["Counter_Value"]))
        if "copy" not in per:
            raise SystemExit(f"{counter}: the calibration copy kernel is missing")
        copy_kib = float(np.max(per["copy"]))   # the big copy is the largest elementwise dispatch
        factor = copy_kib / (COPY_MIB * 1024.0)
        out[counter] = {"copy_kib": copy_kib, "factor": factor,
                        "kernels": {k: {"dispatches": len(v), "kib_mean": float(np.mean(v)),
                                        "bytes_scaled": float(np.mean(v)) * 1024.0 / factor}
                                    for k, v in per.items() if k != "copy"}}
    summary = {"workload": "bolt-latent-E240-rows1", "kernel_source_sha256": source_hash(),
               "command": args.command, "copy_mib_read_and_written": COPY_MIB, "counters": out}
    with open(args.pmc_out, "w") as fh:
        json.dump(summary, fh, indent=1)
    print(json.dumps(summary, indent=1))
    return 0


def summarize_stats(args):
    rows = _csv_rows(args.summarize_stats, "kernel_stats.csv")
    lines = [f"rocprofv3 kernel statistics ({args.command})", "",
             f"{'kernel':70s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{r['Name'][:70]:70s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.3f} "
                     f"{float(r['MinNs']) / 1e3:9.3f} {float(r['MaxNs']) / 1e3:9.3f} {float(r['Percentage']):6.2f}")
    # the same dispatches split by what ran just before: another kernel (inside a forward) or
    # the same one (the replays of one launch group alone)
    trace = _csv_rows(args.summarize_stats, "kernel_trace.csv")
    disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in trace)
    split = {}
    for i in range(1, len(disp)):
        st, en, name = disp[i]
        if _layer_kernel(name) is None:
            continue
        key = (name, "inside forwards" if disp[i - 1][2] != name else "after itself")
        split.setdefault(key, []).append((en - st) / 1e3)
    if split:
        lines += ["", "by the dispatch before (layer kernels only)",
                  f"{'kernel':70s} {'context':>16s} {'calls':>7s} {'avg_us':>9s}"]
    for (name, ctx), v in sorted(split.items()):
        lines.append(f"{name[:70]:70s} {ctx:>16s} {len(v):7d} {sum(v) / len(v):9.3f}")
    # prefill kernels by grid size (each row count of a prefill pass launches its own grids)
    grids = {}
    for r in trace:
        if "pf_" in r["Kernel_Name"]:
            key = (r["Kernel_Name"].split("(")[0].replace("void ", ""), int(r["Grid_Size_X"]))
            grids.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if grids:
        lines += ["", "prefill kernels by grid size (threads)", f"{'kernel':60s} {'grid':>9s} {'calls':>7s} {'median_us':>10s}"]
        for (name, grid), v in sorted(grids.items()):
            v = sorted(v)
            lines.append(f"{name[:60]:60s} {grid:9d} {len(v):7d} {v[len(v) // 2]:10.1f}")
    txt = "\n".join(lines) + "\n"
    with open(args.stats_out, "w") as fh:
        fh.write(txt)
    print(txt)
    return 0


def stage_bytes(dims, rows, n_distinct):
    """Algorithmic bytes of each stage of one pass: every weight byte read once (routed
    experts: only the distinct experts the pass picked), activations in and out."""
    H, L, E, I, SI, K = dims.hidden, dims.latent, dims.n_experts, dims.expert_inter, dims.shared_inter, dims.top_k
    D = L or H
    a = 2  # activation bytes
    expert = D * I * dims.quant_bits // 8 + (D * I // dims.group_size) * 4   # codes + bf16 scale, bias per group
    half = (H // 16 // 2) * 16
    lg = 4 if dims.router_dtype == 3 else 2   # logit bytes (fp32 router: fp32 logits)
    return {
        "gate": E * H * lg + rows * H * a + rows * E * lg,
        "fc1": L * H * 2 + rows * L * a,
        "shup": SI * H * 2 + rows * SI * a,
        "route": (E * 4 if dims.has_bias else 0) + rows * E * lg + rows * K * 8,
        "shdn_a": half * SI * 2 + rows * SI * a + rows * half * a if SI else 0,
        "up": n_distinct * expert + rows * D * a + rows * K * I * a,
        "shdn_b": (H - half) * SI * 2 + rows * SI * a + rows * (H - half) * a if SI else 0,
        "down": n_distinct * expert + rows * K * I * a + rows * K * D * a + rows * K * 4 + rows * D * a
                + (2 * rows * H * a if not L else 0),
        "fc2": (H * L * 2 + rows * D * a + 3 * rows * H * a) if L else 0,
    }


def main():
    args = parse()
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_mfma:
        return summarize_mfma(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from latent_mixture_experts_bf16_amd import binding as B
    from latent_mixture_experts_bf16_amd import layer as LY
    from latent_mixture_experts_bf16_amd import synth

    if args.only_prefill:
        print(json.dumps({"prefill": prefill_bench(B, LY, synth)}), flush=True)
        return 0
    wl = synth.WORKLOADS[args.config]
    if len(wl.layers) != 1 and args.profile_steps:
        return profile_stack(args, B, LY, synth)
    if len(wl.layers) != 1:
        print("bench.py times single-layer workloads (configs 0-3); the stack is timed by the rows "
              "sweep", file=sys.stderr)
        return 2
    dims = wl.layers[0]
    rows = wl.rows
    inst = args.instances or (8 if args.config == 1 else (4 if args.config in (2, 3) else 2))
    print(f"[bench] workload {wl.name}: generating {inst} weight instances", file=sys.stderr, flush=True)
    t0 = time.time()
    layers, xs, outs, host0 = [], [], [], None
    for i in range(inst):
        d, arrays = next(synth.workload_layers(args.config, instance=i))
        layers.append(LY.DeviceLayer(d, arrays, max_rows=rows))
        xs.append(LY.to_device(arrays["x"]))
        outs.append(torch.empty_like(xs[-1]))
        if i == 0:
            host0 = arrays
        del arrays
    torch.cuda.synchronize()
    print(f"[bench] generated and uploaded in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    s = torch.cuda.Stream()
    for lay in layers:
        B.moe_latent_set_stream(lay.handle, s.cuda_stream)
    if args.profile_steps:
        # the workload of the counter runs: eager forwards, then a copy of known size
        with torch.cuda.stream(s):
            for i in range(args.profile_steps):
                layers[i % inst].forward(xs[i % inst], outs[i % inst], rows)
            src = torch.ones(COPY_MIB << 18, dtype=torch.int32, device="cuda")
            dst = torch.empty_like(src)
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        for lay in layers:
            lay.status()
            lay.close()
        print(f"[bench] profile workload done: {args.profile_steps} forwards, one {COPY_MIB} MiB copy",
              file=sys.stderr, flush=True)
        return 0
    with torch.cuda.stream(s):
        for lay, x, o in zip(layers, xs, outs):
            lay.forward(x, o, rows)
    s.synchronize()
    for lay in layers:
        lay.status()

    # distinct experts each instance's pass picks (for its algorithmic bytes)
    distinct = []
    for lay in layers:
        idx, _ = lay.routing(rows)
        distinct.append(len(np.unique(idx)))
    sb = [stage_bytes(dims, rows, u) for u in distinct]
    step_bytes = float(np.mean([sum(g.values()) for g in sb]))
    groups = plan_groups(B, layers[0].handle, dims, rows)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        return g

    # Steps are replayed from graphs of consecutive forwards that rotate through the
    # instances: chunks of CH forwards, and one graph for a remainder, so that every block of
    # timed steps is whole graph replays and a step's time does not depend on --steps.
    CH = inst * max(1, 64 // inst)
    graphs = {}

    def graph_of(n):
        if n not in graphs:
            with torch.cuda.stream(s):
                graphs[n] = capture(lambda: [layers[i % inst].forward(xs[i % inst], outs[i % inst], rows)
                                             for i in range(n)])
        return graphs[n]

    def run_steps(n):
        for _ in range(n // CH):
            graph_of(CH).replay()
        if n % CH:
            graph_of(n % CH).replay()

    # the timed steps in NBLOCK blocks, each bracketed by events: the whole span gives the
    # value, the blocks its spread (one block unless every block holds whole chunks)
    nblock = 5 if args.steps >= 5 * CH else 1
    bsteps = [args.steps // nblock + (1 if b < args.steps % nblock else 0) for b in range(nblock)]
    with torch.cuda.stream(s):
        run_steps(args.warmup)
        for n in sorted({CH, *(b % CH for b in bsteps)} - {0}):   # every graph the blocks replay, twice
            for _ in range(2):
                graph_of(n).replay()
    s.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nblock + 1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        evs[0].record(s)
        for b in range(nblock):
            run_steps(bsteps[b])
            evs[b + 1].record(s)
    torch.cuda.synchronize()
    ms_total = evs[0].elapsed_time(evs[nblock])
    block_us = sorted(evs[b].elapsed_time(evs[b + 1]) * 1e3 / bsteps[b] for b in range(nblock))
    for lay in layers:
        lay.status()
    ms_step = ms_total / args.steps
    tok_s = rows * args.steps / (ms_total / 1e3)
    layer_gbps = step_bytes / (ms_step * 1e-3) / 1e9

    # each launch group on its own: replay graphs of that group over all instances
    group_stats = {}
    reps = max(20, args.steps // (4 * inst))
    for grp in groups:
        gid, gname, stages = grp["group"], grp["name"], grp["stages"]
        with torch.cuda.stream(s):
            gg = capture(lambda gid=gid: [B.moe_latent_launch_group(lay.handle, rows, x.data_ptr(), o.data_ptr(), gid)
                                          for lay, x, o in zip(layers, xs, outs)])
            for _ in range(3):
                gg.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(reps):
                gg.replay()
            b.record(s)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * inst)
        gbytes = float(np.mean([sum(g[st] for st in stages) for g in sb]))
        group_stats[gid] = {"name": gname, "us": round(us, 3), "bytes": int(gbytes),
                            "gbps": round(gbytes / (us * 1e-6) / 1e9, 1), "kernel": grp["kernel"],
                            "side_stream": bool(grp["side"]), "workgroups": grp["items"]}
        del gg
    for lay in layers:
        lay.status()
    # each launch inside full forwards, as the roofline's duration: its kernel's start and end
    # recorded by the kernel's own dispatch (no marker packets between the launches)
    inside = in_forward_launches(B, layers, xs, outs, rows, s, len(groups))
    for gid, v in group_stats.items():
        v["us_alone"] = v["us"]
        v["us"] = round(float(inside[gid]), 3)
        v["gbps"] = round(v["bytes"] / (v["us"] * 1e-6) / 1e9, 1)
    for lay in layers:
        lay.status()
    dom = max(group_stats, key=lambda k: group_stats[k]["us"])
    d = group_stats[dom]
    traffic, traffic_note = None, "no counter summary for this workload"
    tf = traffic_file(wl.name)
    if rows == 1 and os.path.exists(tf):
        with open(tf) as fh:
            pmc = json.load(fh)
        if pmc.get("kernel_source_sha256") != source_hash():
            traffic_note = "counter summary predates the current kernel source"
        else:
            kname = d["kernel"]
            try:
                traffic = int(pmc["counters"]["FETCH_SIZE"]["kernels"][kname]["bytes_scaled"] +
                              pmc["counters"]["WRITE_SIZE"]["kernels"][kname]["bytes_scaled"])
                traffic_note = f"FETCH_SIZE + WRITE_SIZE of {kname}, scaled by the calibration copy"
            except KeyError:
                traffic_note = f"{kname} missing from the counter summary"
    print(f"[bench] groups: {json.dumps(group_stats)}", file=sys.stderr, flush=True)

    # a plain read-only stream over 1 GiB on the same box: the measured reference beside the
    # 8 TB/s peak (never instead of it)
    stream_ref = None
    if rows == 1:
        buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        nb = buf.numel() * 4
        with torch.cuda.stream(s):
            for _ in range(3):
                B.moe_latent_stream_read(buf.data_ptr(), nb, sink.data_ptr(), s.cuda_stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(20):
                B.moe_latent_stream_read(buf.data_ptr(), nb, sink.data_ptr(), s.cuda_stream)
            b.record(s)
        torch.cuda.synchronize()
        gbps_ref = nb * 20 / (a.elapsed_time(b) * 1e-3) / 1e9
        stream_ref = {"gbps": round(gbps_ref, 1), "frac_of_peak": round(gbps_ref / HBM_PEAK_GBPS, 4),
                      "bytes": nb, "kernel": "moe_stream_read_kernel (read-only, 16-byte nontemporal loads, one workgroup "
                                "per compute unit, 8 loads in flight per thread)"}
        del buf, sink

    # parity of instance 0 against the oracle, and the oracle timed on this host
    cpu = None
    cpu_single = None
    parity = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        out0 = outs[0].cpu().numpy().view(np.uint16)
        idx0, w0 = layers[0].routing(rows)
        n, t_start = 0, time.time()
        ref = None
        while True:
            r = O.forward(dims, host0)
            ref = ref or r
            n += 1
            if time.time() - t_start >= args.cpu_seconds:
                break
        el = time.time() - t_start
        got = O.act_to_f32(dims, out0).astype(np.float64)
        refv = ref["out_f32"].astype(np.float64)
        rms = float(np.sqrt((refv ** 2).mean()))
        dd = np.abs(got - refv)
        rel_rms = float(np.sqrt((dd ** 2).mean())) / rms
        rel_max = float((dd / np.maximum(rms, np.abs(refv))).max())
        big = np.abs(refv) >= rms
        if dims.act_dtype == 1:
            ulp = np.spacing(np.abs(refv[big]).astype(np.float32)).astype(np.float64) * 65536.0
        else:
            ulp = np.spacing(np.abs(refv[big]).astype(np.float16)).astype(np.float64)
        parity = {"routing_bitwise": bool(np.array_equal(idx0, ref["idx"]) and
                                          np.array_equal(w0.view(np.uint32), ref["w"].view(np.uint32))),
                  "rel_rms": rel_rms, "max_rel": rel_max, "max_abs_over_rms": float(dd.max()) / rms,
                  "max_abs": float(dd.max()), "max_ulp_where_abs_ge_rms": float((dd[big] / ulp).max()),
                  "bar": "rel_rms <= 5e-3 and max |err| / max(RMS(oracle), |oracle|) <= 2e-2",
                  "ok": bool(rel_rms <= 5e-3 and rel_max <= 2e-2)}
        cpu_single = {"value": round(rows * n / el, 3), "unit": "layer-tokens/s", "cores": 1, "kind": "oracle",
                      "sample": f"{n} forwards of instance 0 ({rows} row(s) each), single-threaded plain C, "
                                f"{el:.1f} s"}
        cpu = cpu_parallel(args.config, args.cpu_seconds) or cpu_single

    line = {
        "metric": "MoE-layer decode tokens/s and achieved HBM GB/s (% of roofline) at 1/16/64 rows",
        "value": round(tok_s, 1),
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dims.act_dtype == 1 else "f16",
        "data": "synthetic (seeded; random-init weights of the workload's shapes)",
        "config": {"workload": wl.name, "rows": rows, "hidden": dims.hidden, "latent": dims.latent,
                   "n_experts": dims.n_experts, "top_k": dims.top_k, "expert_inter": dims.expert_inter,
                   "shared_inter": dims.shared_inter, "weight_instances": inst},
        "layer_hbm": {"bytes_per_step": int(step_bytes), "achieved_gbps": round(layer_gbps, 1),
                      "frac": round(layer_gbps / HBM_PEAK_GBPS, 4)},
        "roofline": {"bound": "hbm", "kernel": f"launch {dom}: {d['kernel']} ({d['name']})",
                     "achieved": d["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(d["gbps"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_note": traffic_note,
                     "bytes_per_launch": d["bytes"], "us_per_launch": d["us"]},
        "launches": {v["name"]: {"us": v["us"], "us_alone": v["us_alone"], "bytes": v["bytes"], "gbps": v["gbps"],
                                 "kernel": v["kernel"], "workgroups": v["workgroups"]}
                     for v in group_stats.values()},
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu_single,
        "host_cpu": host_cpu(),
        "blocks": {"n": nblock, "us_per_step_median": round(float(np.median(block_us)), 3),
                   "us_per_step_min": round(block_us[0], 3), "us_per_step_max": round(block_us[-1], 3)},
        "stream_read_reference": stream_ref,
        "parity": parity,
    }
    for lay in layers:
        lay.close()
    del layers, xs, outs
    torch.cuda.empty_cache()
    if not args.no_rows_sweep and rows == 1:
        line["rows_sweep"] = [rows_sweep(2, 2, B, LY, synth), rows_sweep(3, 4, B, LY, synth),
                              rows_sweep(4, 1, B, LY, synth)]
    if not args.no_lm_head and rows == 1:
        line["lm_head"] = lm_head_bench(B, LY, synth)
    if not args.no_prefill and rows == 1:
        line["prefill"] = prefill_bench(B, LY, synth)
    if args.formats and rows == 1:
        fmts = [tuple(int(v) for v in f.split(":")) for f in args.formats.split(",")]
        line["formats"] = formats_sweep(B, LY, synth, fmts)
    print(json.dumps(line), flush=True)
    return 0


def prefill_flops(d, rows):
    """Algorithmic flops of one prefill pass: the MFMA GEMMs (fc1, shared up and down, fc2,
    routed up and down over rows * top_k picks) and, apart, the gate (vector fp32 FMAs)."""
    D = d.latent or d.hidden
    gemm = 2 * rows * (d.latent * d.hidden * 2 + d.shared_inter * d.hidden * 2 +
                       d.top_k * d.expert_inter * D * 2)
    gate = 2 * rows * d.n_experts * d.hidden
    return gemm, gate


def prefill_bench(B, LY, synth, rows_list=(512, 4096), reps=10):
    """The fused prefill of the Bolt-like layer (240 experts) at 512 and 4096 rows: one pass
    captured in a graph and replayed; rows/s and the MFMA GEMMs' flops per second against the
    dense bf16 peak."""
    import numpy as np
    import torch
    out = {"workload": "bolt-latent-E240 prefill", "peak_tflops_bf16": MFMA_PEAK_TFLOPS}
    for rows in rows_list:
        d, arrays = next(synth.workload_layers(1, rows=rows))
        lay = LY.DeviceLayer(d, arrays, max_rows=rows)
        x = LY.to_device(arrays["x"])
        o = torch.empty_like(x)
        del arrays
        s = torch.cuda.Stream()
        B.moe_latent_set_stream(lay.handle, s.cuda_stream)
        with torch.cuda.stream(s):
            lay.prefill(x, o, rows)
        s.synchronize()
        lay.status()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                lay.prefill(x, o, rows)
            for _ in range(3):
                g.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(reps):
                g.replay()
            b.record(s)
        torch.cuda.synchronize()
        lay.status()
        us = a.elapsed_time(b) * 1e3 / reps
        gemm, gate = prefill_flops(d, rows)
        tf = gemm / (us * 1e-6) / 1e12
        out[f"rows{rows}"] = {"us": round(us, 1), "tokens_per_s": round(rows / (us * 1e-6), 1),
                              "gemm_tflops": round(tf, 1), "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                              "gemm_flops": gemm, "gate_flops": gate}
        print(f"[bench] prefill rows {rows}: {json.dumps(out[f'rows{rows}'])}", file=sys.stderr, flush=True)
        lay.close()
        del lay, x, o, g
        torch.cuda.empty_cache()
    return out


def lm_head_bench(B, LY, synth, K=4096, N=131072, reps=40):
    """The bf16 lm_head gemv beside the layer (K = 4096, N = 131072: 1 GiB of weights, four
    times the 256 MB cache, so every replay streams from HBM), at 1 and 16 rows, bf16 output:
    graph replays timed with events; algorithmic bytes = weights + input rows + outputs."""
    import torch
    d = synth.make_lm_head(K, N, 16, seed=2718)
    wd = LY.to_device(d["w"])
    xd = LY.to_device(d["x"])
    del d
    desc = B.make_tensor(wd.data_ptr(), B.MOE_DT_BF16, [N, K])
    s = torch.cuda.Stream()
    res = {"K": K, "N": N, "weight_bytes": N * K * 2, "kernel": "moe_lm_head_kernel"}
    for rows in (1, 16):
        out = torch.empty((rows, N), dtype=torch.int16, device="cuda")
        with torch.cuda.stream(s):
            B.moe_lm_head_gemv(desc, rows, xd.data_ptr(), out.data_ptr(), B.MOE_DT_BF16, s.cuda_stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(4):
                    B.moe_lm_head_gemv(desc, rows, xd.data_ptr(), out.data_ptr(), B.MOE_DT_BF16, s.cuda_stream)
            for _ in range(3):
                g.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(reps // 4):
                g.replay()
            b.record(s)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        nbytes = N * K * 2 + rows * K * 2 + rows * N * 2
        gbps = nbytes / (us * 1e-6) / 1e9
        res[f"rows{rows}"] = {"us": round(us, 2), "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                              "tokens_per_s": round(rows / (us * 1e-6), 1)}
        del g, out
    print(f"[bench] lm_head: {json.dumps(res)}", file=sys.stderr, flush=True)
    del wd, xd
    torch.cuda.empty_cache()
    return res


def profile_stack(args, B, LY, synth):
    """The counter runs' workload for a multi-layer configuration: every layer of the stack
    forwarded --profile-steps times, eagerly."""
    import torch
    wl = synth.WORKLOADS[args.config]
    layers, xs, outs = [], [], []
    for d, arrays in synth.workload_layers(args.config):
        layers.append(LY.DeviceLayer(d, arrays, max_rows=wl.rows))
        xs.append(LY.to_device(arrays["x"]))
        outs.append(torch.empty_like(xs[-1]))
        del arrays
    for _ in range(args.profile_steps):
        for lay, x, o in zip(layers, xs, outs):
            lay.forward(x, o, wl.rows)
    torch.cuda.synchronize()
    for lay in layers:
        lay.status()
        lay.close()
    print(f"[bench] profile workload done: {args.profile_steps} passes over {len(layers)} layers",
          file=sys.stderr, flush=True)
    return 0


def summarize_mfma(args):
    """MFMA utilisation (percent of SIMD cycles with the matrix core busy) and bf16 MFMA flops
    of each layer kernel, from one rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 run."""
    import numpy as np
    rows = _csv_rows(args.summarize_mfma, "counter_collection.csv")
    per = {}
    for r in rows:
        k = _layer_kernel(r.get("Kernel_Name", ""))
        if k is None:
            continue
        per.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    out = {}
    for (k, c), v in sorted(per.items()):
        out.setdefault(k, {"dispatches": len(v)})[c + "_mean"] = float(np.mean(v))
    for k, v in out.items():
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16_mean" in v:
            v["mfma_bf16_flops_per_dispatch"] = v["SQ_INSTS_VALU_MFMA_MOPS_BF16_mean"] * 512
    summary = {"workload": args.mfma_workload, "kernel_source_sha256": source_hash(), "command": args.command,
               "kernels": out}
    with open(args.mfma_out, "w") as fh:
        json.dump(summary, fh, indent=1)
    print(json.dumps(summary, indent=1))
    return 0


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cores_available": len(os.sched_getaffinity(0))}


_CPU_WORKER = r"""
import sys, time
sys.path.insert(0, sys.argv[1])
from latent_mixture_experts_bf16_amd import synth
from oracle import oracle as O
d, arrays = next(synth.workload_layers(int(sys.argv[2])))
seconds = float(sys.argv[3])
n, t0 = 0, time.time()
while True:
    O.forward(d, arrays)
    n += 1
    if time.time() - t0 >= seconds:
        break
print(n, time.time() - t0, flush=True)
"""


def cpu_parallel(cfg, seconds, max_workers=16):
    """The oracle as it stands, one copy per host core (at most 16): each child process draws
    instance 0 and runs whole forwards for `seconds`; the children are separate programs
    (nothing in them touches the GPU)."""
    import subprocess
    nw = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, "-c", _CPU_WORKER, ROOT, str(cfg), str(seconds)],
                              stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, env=env)
             for _ in range(nw)]
    tok_s, n_tot = 0.0, 0
    rows = None
    for p in procs:
        try:
            out, _ = p.communicate(timeout=seconds * 4 + 120)
            n, el = out.split()
            tok_s += int(n) / float(el)
            n_tot += int(n)
        except Exception:   # a worker that failed or timed out leaves the parallel figure out
            p.kill()
            return None
    from latent_mixture_experts_bf16_amd import synth
    rows = synth.WORKLOADS[cfg].rows
    return {"value": round(rows * tok_s, 3), "unit": "layer-tokens/s", "cores": nw, "kind": "oracle",
            "sample": f"{nw} processes, each whole forwards of instance 0 ({rows} row(s)) for {seconds:.0f} s: "
                      f"{n_tot} forwards in all, plain C, one thread each"}


def in_forward_launches(B, layers, xs, outs, rows, s, ng, sweeps=4, rounds=30):
    """Mean duration (us) of each launch group inside full forwards: forwards enqueued eagerly,
    `sweeps` sweeps over the instances between synchronizations, each launch's kernel start and
    end recorded by its own dispatch; the first forward after each synchronization and the
    first two rounds are left out. Each round first queues about 1.5 ms of streaming reads, so
    that the host has enqueued every forward before the first one starts and they run back to
    back, as in a replayed graph, whatever the host's launch rate."""
    import numpy as np
    import torch
    busy = torch.ones(1 << 26, dtype=torch.int32, device="cuda")   # 256 MiB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nf = sweeps * len(layers)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * ng)] for _ in range(nf)]
    with torch.cuda.stream(s):
        for lst in evs:
            for e in lst:
                e.record(s)
    s.synchronize()
    handles = [[e.cuda_event for e in lst] for lst in evs]
    acc, n = np.zeros(ng), 0
    with torch.cuda.stream(s):
        for r in range(rounds + 2):
            for _ in range(40):
                B.moe_latent_stream_read(busy.data_ptr(), busy.numel() * 4, sink.data_ptr(), s.cuda_stream)
            for f in range(nf):
                i = f % len(layers)
                B.moe_latent_forward_timed(layers[i].handle, rows, xs[i].data_ptr(), outs[i].data_ptr(), handles[f])
            s.synchronize()
            if r < 2:
                continue
            for f in range(1, nf):
                for g in range(ng):
                    acc[g] += evs[f][2 * g].elapsed_time(evs[f][2 * g + 1]) * 1e3
                n += 1
    del busy, sink
    return acc / n


def rows_sweep(cfg, instances, B, LY, synth, sweeps=200, warmup=20):
    """Multi-row passes: the 16-row pass, the 4-row pass of the non-latent fp16 layer with the
    fp32 router (distinct weight instances rotated through HBM), or the 8-layer 64-row stack
    (each layer with its own input), timed as graph replays of one sweep over all layers and
    instances; algorithmic bytes as for the one-row line."""
    wl = synth.WORKLOADS[cfg]
    t0 = time.time()
    sets = [(d, arrays) for i in range(instances) for d, arrays in synth.workload_layers(cfg, instance=i)]
    out = time_layer_set(B, LY, sets, wl.rows, sweeps, warmup)
    out = {"workload": wl.name, **out}
    print(f"[bench] rows sweep ({time.time() - t0:.1f} s): {json.dumps(out)}", file=sys.stderr, flush=True)
    return out


def formats_sweep(B, LY, synth, formats, rows_list=(1, 16), instances=4, sweeps=200, warmup=20):
    """The Bolt-like layer (240 experts) with its routed experts in other affine formats
    (code width, group size), at 1 and 16 rows: weight instances rotated through HBM as for
    the one-row line; algorithmic bytes count each format's own codes, scales and biases."""
    import dataclasses
    base = synth.WORKLOADS[1].layers[0]
    res = []
    for bits, gs in formats:
        dims = dataclasses.replace(base, quant_bits=bits, group_size=gs)
        for rows in rows_list:
            t0 = time.time()
            sets = [(dims, synth.make_layer(dims, rows, weight_seed=8000 + 100 * i + bits, input_seed=8050 + i))
                    for i in range(instances)]
            out = {"bits": bits, "group_size": gs, **time_layer_set(B, LY, sets, rows, sweeps, warmup)}
            del sets
            print(f"[bench] format {bits}-bit g{gs} rows {rows} ({time.time() - t0:.1f} s): {json.dumps(out)}",
                  file=sys.stderr, flush=True)
            res.append(out)
    return res


def time_layer_set(B, LY, sets, rows, sweeps, warmup):
    """One sweep over the layers of `sets` ((dims, arrays) pairs, each with its own input),
    captured in a graph and replayed: time per layer pass and achieved algorithmic GB/s."""
    import numpy as np
    import torch
    layers, xs, outs, nbytes = [], [], [], 0.0
    for d, arrays in sets:
        lay = LY.DeviceLayer(d, arrays, max_rows=rows)
        layers.append(lay)
        xs.append(LY.to_device(arrays["x"]))
        outs.append(torch.empty_like(xs[-1]))
    s = torch.cuda.Stream()
    for lay in layers:
        B.moe_latent_set_stream(lay.handle, s.cuda_stream)
    with torch.cuda.stream(s):
        for lay, x, o in zip(layers, xs, outs):
            lay.forward(x, o, rows)
    s.synchronize()
    for lay in layers:
        lay.status()
        idx, _ = lay.routing(rows)
        nbytes += sum(stage_bytes(lay.dims, rows, len(np.unique(idx))).values())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for lay, x, o in zip(layers, xs, outs):
                lay.forward(x, o, rows)
        for _ in range(warmup):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(sweeps):
            g.replay()
        b.record(s)
    torch.cuda.synchronize()
    for lay in layers:
        lay.status()
    us_sweep = a.elapsed_time(b) * 1e3 / sweeps
    n_layers = len(layers)
    gbps = nbytes / (us_sweep * 1e-6) / 1e9
    out = {"rows": rows, "layers_per_sweep": n_layers,
           "us_per_layer_pass": round(us_sweep / n_layers, 2),
           "layer_tokens_per_s": round(rows * n_layers / (us_sweep * 1e-6), 1),
           "hbm_gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
           "bytes_per_sweep": int(nbytes)}
    for lay in layers:
        lay.close()
    del layers, xs, outs, g
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    sys.exit(main())
