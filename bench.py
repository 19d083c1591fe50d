"""Benchmark: packet-hops/s of the batched simulator on one MI355X.

A step is one pass of the whole hot path over one batch: every experiment of the
batch simulated from tick 0 to completion by one msim_run launch (the state is
restored to tick 0 with msim_reset before each step).  The default workload is
the k=8 fat-tree batch of 4096 experiments (16 data-parallel ring all-reduces of
256 MiB plus 16 tensor-parallel ring all-gathers of 56 MiB per experiment, 4 KiB
packets, 0-4 failed cables).  Inputs are synthetic and seeded, and resident in
HBM before the timed region starts.

Prints one JSON line (rank 0): throughput, the roofline of the megakernel
(algorithmic bytes: 8 B per packet-hop + 8 B per delivered packet, over the
kernel's average launch time measured with HIP events on its stream; when
every experiment keeps its state in LDS, also against the chip's LDS read
bandwidth as the library's probe kernel measures it) and the CPU oracle timed on a bounded sample of the same batch on the host's cores,
with its results compared to the GPU's for those experiments.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
ALG_BYTES_PER_HOP = 8
ALG_BYTES_PER_DELIVERY = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu():
    """Logical CPUs this process may run on, the machine's count, and the model name."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return usable, os.cpu_count() or usable, model


def cpu_baseline(batch, gpu_res, sample_ids, threads):
    """The oracle, untouched, on a sample of experiments, in parallel threads.
    Returns its packet-hop rate, wall time, packet-hops, experiment-ticks and
    how many sampled experiments the GPU matched exactly."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as O
    import threading
    ob = O.OracleBatch(batch.pack())
    t0 = time.perf_counter()
    lock, finished = threading.Lock(), [0]

    def one(e):
        r = O.run(ob, e)
        with lock:
            finished[0] += 1
            log(f"[bench] CPU oracle: {finished[0]}/{len(sample_ids)} experiments done "
                f"({time.perf_counter() - t0:.0f}s)")
        return r
    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, sample_ids))
    dt = time.perf_counter() - t0
    hops = sum(r["pkt_hops"] for r in res)
    ticks = sum(r["t_end"] + 1 for r in res)
    ok = 0
    for e, r in zip(sample_ids, res):
        same = (r["rc"] == 0 and r["status"] == int(gpu_res["status"][e]) and r["t_end"] == int(gpu_res["tick"][e])
                and r["pkt_hops"] == int(gpu_res["pkt_hops"][e]) and r["digest"] == int(gpu_res["digest"][e])
                and r["delivered"] == int(gpu_res["delivered"][e]))
        ok += same
    return hops / dt, dt, hops, ok, ticks


def cpu_record(rate, dt, chops, ok, ticks, threads, n_sample, n, gpu_rate):
    usable, machine, model = host_cpu()
    return {"value": rate, "unit": "packet-hops/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_sample} of {n} experiments (every {n / n_sample:.0f}th index), run to completion in "
                      f"{dt:.1f}s ({chops} packet-hops, {ticks} experiment-ticks); GPU results identical on "
                      f"{ok}/{n_sample}",
            "per_core": rate / threads, "experiment_ticks_per_s": ticks / dt,
            "host_cpus_usable": usable, "host_cpus": machine, "host_cpu_model": model,
            "gpu_over_oracle": gpu_rate / rate if rate else None,
            "parity_ok": ok, "parity_n": n_sample}


def copy_bandwidth(nbytes: int = 1 << 31, reps: int = 5) -> float:
    """GB/s of a plain device-to-device copy (bytes read + bytes written per
    second), the best of a few timed copies on the current stream."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (best / 1e3) / 1e9


def lds_bandwidth(reps: int = 5) -> dict:
    """LDS read bandwidth of the whole chip, measured by the library's probe
    kernel (conflict-free 16-byte reads, two 64 KiB workgroups per CU): the
    best of a few timed launches on the current stream."""
    import torch
    from experiment_network_simulation_amd.sim import lds_probe
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = n_cu * 16
    out = torch.empty(blocks * 1024, dtype=torch.int32, device="cuda:0")
    lds_probe(out, blocks, 16)
    best, nbytes = None, 0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        nbytes = lds_probe(out, blocks, 1024)
        b.record()
        b.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    gbs = nbytes / (best / 1e3) / 1e9
    return {"gbs": gbs, "cus": n_cu, "bytes_per_clk_per_cu_at_2p4ghz": gbs * 1e9 / (n_cu * 2.4e9)}


def measured_traffic(kernel: str, workload_cfg: int, n: int):
    """HBM bytes per launch (for a chunked run: over all its launches) from the
    committed rocprofv3 counter runs in profiles/traffic.json, if one was
    taken on this kernel source, this kernel and this workload; else None."""
    rec = traffic_record(kernel, workload_cfg, n)
    return rec["traffic_bytes_per_launch"] if rec is not None else None


def traffic_source(kernel: str, workload_cfg: int, n: int, chunked: bool = False) -> str:
    """Where the bench line's roofline.traffic comes from, with the record's
    note on the source its counters were taken on, if it has one."""
    rec = traffic_record(kernel, workload_cfg, n)
    if rec is None:
        return "not measured for this kernel source and workload"
    src = ("rocprofv3 FETCH_SIZE + WRITE_SIZE " + ("over all launches " if chunked else "") +
           "of this kernel source on this workload, taken in a separate profiled run and stored in "
           "profiles/traffic.json, each scaled by a plain copy's calibration")
    if rec.get("source_note"):
        src += "; " + rec["source_note"] + " (" + rec.get("counters_taken_on_sha256", "")[:8] + ")"
    return src


def traffic_record(kernel: str, workload_cfg: int, n: int):
    """The profiles/traffic.json record for this kernel source, kernel and
    workload, or None."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        recs = json.load(open(os.path.join(here, "profiles", "traffic.json")))
    except (OSError, ValueError):
        return None
    csrc = os.path.join(here, "experiment_network_simulation_amd", "csrc")
    h = hashlib.sha256()
    for f in ("msim_kernel.hip", "msim_layout.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    for rec in recs if isinstance(recs, list) else [recs]:
        if (rec.get("kernel") == kernel and rec.get("kernel_source_sha256") == h.hexdigest()
                and rec.get("config") == workload_cfg and rec.get("experiments") == n):
            return rec
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4, help="workload 1..5 (default 4: k=8 fat-tree, E=4096)")
    ap.add_argument("--n-exp", type=int, default=0, help="first n experiments only (default: the full batch)")
    ap.add_argument("--exp-ids", type=str, default="",
                    help="comma-separated experiment indices of the config to run instead (e.g. 21: one C3 A=16, K=1 broadcast)")
    ap.add_argument("--cpu-sample", type=int, default=32,
                    help="experiments in the CPU-oracle sample, evenly strided over the batch (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--force-global", action="store_true")
    ap.add_argument("--no-ring-path", action="store_true",
                    help="run ring-only experiments on the general compact kernels instead of the ring kernel")
    ap.add_argument("--max-ticks", type=int, default=0xFFFFFFF0,
                    help="tick budget of each run (default: to completion); a run that ends incomplete fails")
    ap.add_argument("--chunk", type=int, default=0,
                    help="run the batch in chunks of this many experiments, compiling the next chunk while the "
                         "current one runs (default: whole batch; C5 beyond 2048 experiments: 2048)")
    ap.add_argument("--dse", choices=["tune", "reshard"], default=None,
                    help="time a design-space-exploration driver instead: AutoCCL tuning or AlpaComm schedules")
    ap.add_argument("--dse-n", type=int, default=0, help="tuning tasks / resharding instances (default 256 / 64)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); experiments are "
              "independent, so N GPUs would each run their own share of the batch.", file=sys.stderr)
        sys.exit(2)

    if args.dse:
        return dse_bench(args)

    import numpy as np
    import torch
    from experiment_network_simulation_amd import inputs as I
    from experiment_network_simulation_amd.sim import KERNEL_NAMES, Sim

    cid = args.config
    ids = [int(v) for v in args.exp_ids.split(",") if v.strip()] if args.exp_ids else None
    n = len(ids) if ids else (args.n_exp or I.FULL_E[cid])
    chunk = 0 if ids else (args.chunk or (2048 if cid == 5 and n > 2048 else 0))
    if chunk and chunk < n:
        return chunked_bench(args, cid, n, chunk)
    log(f"[bench] generating config C{cid} with {n} experiments")
    t = time.perf_counter()
    batch = I.make_config(cid, exp_ids=ids) if ids else I.make_config(cid, n_exp=n)
    log(f"[bench] generated in {time.perf_counter() - t:.1f}s; compiling")
    t = time.perf_counter()
    sim = Sim(batch, force_global=args.force_global, no_ring_path=args.no_ring_path)
    info = sim.info()
    log(f"[bench] compiled in {time.perf_counter() - t:.1f}s: {info}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t = time.perf_counter()
    sim.bind(device="cuda:0", stream=stream)
    log(f"[bench] bind (upload + reset) {time.perf_counter() - t:.2f}s")
    info = sim.info()
    log(f"[bench] bound: grid {info['grid_blocks']} x {info['block_threads']} threads, lds {info['lds_bytes']} B "
        f"({info['n_lds_exp']} experiments in LDS), workspace {info['workspace_bytes'] / 2**20:.0f} MiB")

    kernel_ms = []

    def step(timed):
        sim.reset(stream)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        sim.run(max_ticks=args.max_ticks, stream=stream)
        ev1.record(stream)
        if timed:
            kernel_ms.append((ev0, ev1))

    for i in range(args.warmup):
        t = time.perf_counter()
        step(False)
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i} {time.perf_counter() - t:.2f}s")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        log(f"[bench] step {i} done at {time.perf_counter() - t0:.2f}s")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res = sim.results(stream)
    if res["rc"] != 0:
        raise SystemExit(f"bench: simulation did not complete (rc={res['rc']})")
    hops = int(res["pkt_hops"].sum())
    delivered = int(res["delivered"].sum())
    exp_ticks = int((res["tick"].astype(np.int64) + 1).sum())
    k_ms = [a.elapsed_time(b) for a, b in kernel_ms]
    k_avg_s = sum(k_ms) / len(k_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = hops * args.steps / wall
    alg_bytes = ALG_BYTES_PER_HOP * hops + ALG_BYTES_PER_DELIVERY * delivered
    achieved = alg_bytes / k_avg_s / 1e9
    log(f"[bench] kernel {k_ms} ms; packet-hops {hops}, delivered {delivered}, experiment-ticks {exp_ticks}")

    copy_gbs = copy_bandwidth()
    log(f"[bench] device copy {copy_gbs:.0f} GB/s (read + write)")
    lds = None
    if info["n_lds_exp"] == n:
        lb = lds_bandwidth()
        log(f"[bench] LDS read {lb['gbs']:.0f} GB/s ({lb['bytes_per_clk_per_cu_at_2p4ghz']:.0f} B/clk/CU at 2.4 GHz)")
        lds = {"peak": lb["gbs"], "achieved": achieved, "unit": "GB/s", "frac": achieved / lb["gbs"],
               "peak_bytes_per_clk_per_cu_at_2p4ghz": lb["bytes_per_clk_per_cu_at_2p4ghz"],
               "peak_source": "msim_lds_probe (measured, conflict-free 16-byte LDS reads)"}

    cpu = None
    if args.cpu_sample and n > 0:
        k = min(args.cpu_sample, n)
        sample = sorted(set(int(round(i * n / k)) for i in range(k)) - {n})
        threads = args.cpu_threads or min(16, os.cpu_count() or 1, len(sample))
        log(f"[bench] CPU oracle on {len(sample)} experiments with {threads} threads")
        rate, dt, chops, ok, oticks = cpu_baseline(batch, res, sample, threads)
        cpu = cpu_record(rate, dt, chops, ok, oticks, threads, len(sample), n, value)
        log(f"[bench] CPU oracle {rate:.3e} packet-hops/s; parity {ok}/{len(sample)}")

    traffic = measured_traffic(KERNEL_NAMES[info["main_kernel"]], cid, n)
    traffic_src = traffic_source(KERNEL_NAMES[info["main_kernel"]], cid, n)
    out = {
        "metric": "packet-hops/sec (batched, 1 GPU) + % of HBM roofline at E=4096",
        "value": value,
        "unit": "packet-hops/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": I.CONFIG_NAMES[cid],
            "experiments": n,
            **({"exp_ids": ids} if ids else {}),
            "pkt_bytes": I.PKT_BYTES,
            "experiment_ticks_per_s": exp_ticks * args.steps / wall,
            "packet_hops_per_step": hops,
            "delivered_per_step": delivered,
            "experiment_ticks_per_step": exp_ticks,
            "grid": info["grid_blocks"],
            "block_threads": info["block_threads"],
            "lds_bytes": info["lds_bytes"],
            "state_in_lds": info["n_lds_exp"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_source": traffic_src,
            "kernel": KERNEL_NAMES[info["main_kernel"]],
            "kernel_ms_avg": k_avg_s * 1e3,
            "alg_bytes_per_launch": alg_bytes,
            "copy_gbs": copy_gbs,
            "frac_of_copy": achieved / copy_gbs,
            "lds": lds,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def chunked_bench(args, cid, n, chunk):
    """The batch in chunks: each chunk is compiled (on a host thread, while the
    previous chunk runs), bound, and simulated by one msim_run whose kernel
    time is taken with HIP events on its stream.  value = packet-hops of the
    whole batch / summed kernel time (each chunk's inputs are resident in HBM
    when its launch starts); the wall-clock rate with compile and upload is
    reported in config."""
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from experiment_network_simulation_amd import inputs as I
    from experiment_network_simulation_amd.sim import KERNEL_NAMES, Sim

    if args.warmup or args.steps != 1:
        log("[bench] chunked runs time one pass over the batch (steps 1, warmup 0)")
    ids = [list(range(i, min(n, i + chunk))) for i in range(0, n, chunk)]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def compile_chunk(k):
        b = I.make_config(cid, exp_ids=ids[k])
        return b, Sim(b, force_global=args.force_global, no_ring_path=args.no_ring_path)

    res_all = {k: [] for k in ("status", "tick", "pkt_hops", "delivered", "digest")}
    k_ms, kernels = [], set()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(1) as ex:
        nxt = ex.submit(compile_chunk, 0)
        for k in range(len(ids)):
            b, sim = nxt.result()
            if k + 1 < len(ids):
                nxt = ex.submit(compile_chunk, k + 1)
            sim.bind(device="cuda:0", stream=stream)
            info = sim.info()
            kernels.add(KERNEL_NAMES[info["main_kernel"]])
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            sim.run(stream=stream)
            ev1.record(stream)
            r = sim.results(stream)
            if r["rc"] != 0:
                raise SystemExit(f"bench: chunk {k} did not complete (rc={r['rc']})")
            k_ms.append(ev0.elapsed_time(ev1))
            for key in res_all:
                res_all[key].append(r[key])
            log(f"[bench] chunk {k + 1}/{len(ids)}: {len(ids[k])} experiments, kernel {k_ms[-1]:.0f} ms, "
                f"wall {time.perf_counter() - t0:.1f}s")
            sim.close()
            del sim, b
    wall = time.perf_counter() - t0
    res = {key: np.concatenate(v) for key, v in res_all.items()}
    hops = int(res["pkt_hops"].sum())
    delivered = int(res["delivered"].sum())
    exp_ticks = int((res["tick"].astype(np.int64) + 1).sum())
    k_s = sum(k_ms) / 1e3
    alg_bytes = ALG_BYTES_PER_HOP * hops + ALG_BYTES_PER_DELIVERY * delivered
    cpu = None
    if args.cpu_sample:
        kk = min(args.cpu_sample, n)
        sample = sorted(set(int(round(i * n / kk)) for i in range(kk)) - {n})
        threads = args.cpu_threads or min(16, os.cpu_count() or 1, len(sample))
        sb = I.make_config(cid, exp_ids=sample)
        sres = {key: v[sample] for key, v in res.items()}
        rate, dt, chops, ok, oticks = cpu_baseline(sb, sres, list(range(len(sample))), threads)
        cpu = cpu_record(rate, dt, chops, ok, oticks, threads, len(sample), n, hops / k_s)
        log(f"[bench] CPU oracle {rate:.3e} packet-hops/s; parity {ok}/{len(sample)}")
    copy_gbs = copy_bandwidth()
    log(f"[bench] device copy {copy_gbs:.0f} GB/s (read + write)")
    out = {
        "metric": "packet-hops/sec (batched, 1 GPU) + % of HBM roofline at E=4096",
        "value": hops / k_s,
        "unit": "packet-hops/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 0,
        "ms_per_step": k_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": I.CONFIG_NAMES[cid], "experiments": n, "chunks": len(ids), "chunk": chunk,
                   "pkt_bytes": I.PKT_BYTES, "experiment_ticks_per_s": exp_ticks / k_s,
                   "packet_hops_per_step": hops, "delivered_per_step": delivered,
                   "experiment_ticks_per_step": exp_ticks, "wall_s": wall,
                   "wall_rate_incl_compile_upload": hops / wall, "chunk_kernel_ms": k_ms},
        "roofline": {
            "bound": "hbm",
            "achieved": alg_bytes / k_s / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": alg_bytes / k_s / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic("+".join(sorted(kernels)), cid, n),
            "traffic_source": traffic_source("+".join(sorted(kernels)), cid, n, chunked=True),
            "kernel": "+".join(sorted(kernels)),
            "kernel_ms_avg": k_s * 1e3 / len(ids),
            "alg_bytes_per_launch": alg_bytes / len(ids),
            "copy_gbs": copy_gbs,
            "frac_of_copy": alg_bytes / k_s / 1e9 / copy_gbs,
            "lds": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def dse_bench(args):
    """One driver run: every candidate of every search scored on the GPU, one
    batch per lockstep step.  value = candidates scored per second of wall time
    (host compile of each batch included); the roofline is over the simulation
    kernels of all batches (HIP events around each msim_run)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from experiment_network_simulation_amd import dse as P
    from experiment_network_simulation_amd import inputs as I

    ev = P.GpuEvaluator()
    threads = args.cpu_threads or min(16, os.cpu_count() or 1)
    if args.dse == "tune":
        n = args.dse_n or 256
        tasks = I.tune_tasks_c2(n)
        starts = I.tune_starts(0xA7C5, n)
        workload = (f"AutoCCL coordinate descent over (algorithm ring/tree, NC 1..16, C 32..512 KiB) for {n} "
                    "64 MiB all-reduces over 32 hosts of C2's leaf-spine (seeded ring order and ECMP seed each)")
        t0 = time.perf_counter()
        res = P.tune(tasks, starts, ev, log=log)
        wall = time.perf_counter() - t0
        detail = {"tasks": n, "tree_chosen": sum(r.algo == I.COLL_TREE_AR for r in res),
                  "mean_best_ticks": float(np.mean([r.ticks for r in res]))}
        unit = "probes/s"
        cpu = None
        if args.cpu_sample:
            from oracle import dse as D
            ids = sorted(set(int(round(i * n / min(args.cpu_sample, n))) for i in range(min(args.cpu_sample, n))) - {n})
            t1 = time.perf_counter()
            with ThreadPoolExecutor(min(threads, len(ids))) as ex:
                refs = list(ex.map(lambda t: D.tune(tasks[t], starts[t]), ids))
            dt = time.perf_counter() - t1
            probes = sum(len(r["profiled"]) for ref in refs for r in ref["runs"])
            ok = sum(ref["ticks"] == res[t].ticks and ref["algo"] == res[t].algo for t, ref in zip(ids, refs))
            cpu = {"value": probes / dt, "unit": unit, "cores": min(threads, len(ids)), "kind": "oracle",
                   "sample": f"{len(ids)} of {n} tuning tasks, {probes} probes in {dt:.1f}s; same result on "
                             f"{ok}/{len(ids)}", "parity_ok": ok, "parity_n": len(ids)}
    else:
        n = args.dse_n or 64
        topo = I.fat_tree(8)
        K, G = 16, 32
        insts = [(topo, I.resharding_tasks(0x5C00 + i, 48, range(64), range(64, 128))) for i in range(n)]
        keys = [I.greedy_keys(0x6E00 + g, 48, 8) for g in range(G)]
        workload = (f"AlpaComm schedulers on {n} cross-mesh resharding instances of 48 unit tasks (mesh A: hosts "
                    f"0-63, mesh B: 64-127 of a k=8 fat-tree; 1-3 holders, 1-4 receivers, 256 KiB-2 MiB slices; "
                    f"broadcast K = {K}): naive, load balance and {G} randomised greedy schedules each, "
                    "scored by simulation")
        t0 = time.perf_counter()
        res = P.reshard(insts, K, keys, ev)
        wall = time.perf_counter() - t0
        gain = [float(r.simulated[0]) / float(r.simulated.min()) for r in res]
        detail = {"instances": n, "schedules_per_instance": len(res[0].names),
                  "mean_naive_over_best": float(np.mean(gain)),
                  "best_is_greedy": sum(r.names[r.best].startswith("greedy") for r in res)}
        unit = "schedules/s"
        cpu = None
        if args.cpu_sample:
            from oracle import dse as D
            flat = [(i, k) for i in range(n) for k in range(len(res[i].names))]
            m = min(args.cpu_sample, len(flat))
            ids = [flat[int(round(j * len(flat) / m))] for j in range(m) if int(round(j * len(flat) / m)) < len(flat)]
            t1 = time.perf_counter()
            with ThreadPoolExecutor(min(threads, len(ids))) as ex:
                refs = list(ex.map(lambda ik: D.simulate_schedule(
                    topo, insts[ik[0]][1], res[ik[0]].schedules[ik[1]].sender,
                    res[ik[0]].schedules[ik[1]].order, K), ids))
            dt = time.perf_counter() - t1
            ok = sum(r["t_end"] == int(res[i].simulated[k]) for (i, k), r in zip(ids, refs))
            cpu = {"value": len(ids) / dt, "unit": unit, "cores": min(threads, len(ids)), "kind": "oracle",
                   "sample": f"{len(ids)} of {len(flat)} schedules simulated in {dt:.1f}s; same completion tick "
                             f"on {ok}/{len(ids)}", "parity_ok": ok, "parity_n": len(ids)}
    st = ev.stats
    alg_bytes = ALG_BYTES_PER_HOP * st.pkt_hops + ALG_BYTES_PER_DELIVERY * st.delivered
    achieved = alg_bytes / (st.kernel_ms / 1e3) / 1e9
    out = {
        "metric": f"{unit} (design-space exploration scored by the batched simulator, 1 GPU)",
        "value": st.experiments / wall,
        "unit": unit,
        "n_gpus": 1,
        "steps": st.batches,
        "warmup": 0,
        "ms_per_step": wall / max(st.batches, 1) * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": workload, "batches": st.batches, "experiments": st.experiments,
                   "packet_hops": st.pkt_hops, "kernel_ms_total": st.kernel_ms, "host_s": st.host_s,
                   "wall_s": wall, **detail},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "kernel": "all simulation launches of the run (ring probes compact, tree probes and task graphs general)",
            "kernel_ms_avg": st.kernel_ms / max(st.batches, 1),
            "alg_bytes_total": alg_bytes,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
