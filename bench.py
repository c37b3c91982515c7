"""Throughput of the KDA decode step on one MI355X.

One step = one launch of the whole hot path (slot resolution, convolution,
gate projection, decay, L2 norm, recurrence, state write-back, window update,
gated RMSNorm) over one batch: the decode workload B=256 requests x H=32
heads (8192 items), T=1, d=128, a pool of 512 state slots (1 GiB FP32), with
seeded synthetic inputs resident in HBM before the timed region.

Prints one JSON line.  `value` is (request, head) items per second over the
timed region.  `roofline` relates the kernel's algorithmic bytes per launch
to its duration.  The headline (`achieved`, `frac`, `kernel_us`) is the
cold-clean median: launches each preceded by a 1 GiB read, so that no
operand is cached.  Secondary figures:
  * `roofline.warm`: the span of one pair of HIP events on the launch
    stream around the K back-to-back launches of the timed region, / K;
  * `roofline.cold_dirty`: launches each after a 1 GiB write (dirty lines
    written back during the launch);
  * `single_launch_us`: launches timed one by one;
  * `roofline.copy_ceiling`: what a plain 1 GiB device copy reaches.
`cpu_baseline` times the CPU oracle on the same workload, pinned to one core
(the median over whole passes), and split over host threads.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                    [--cold-launches C]
    python bench.py --mode copy      # 1 GiB device copies (counter calibration)
    python bench.py --mode sweep     # small batches, unsplit vs split (graph replay)
    python bench.py --mode pagecopy [--workload W]   # the page traffic alone (its ceiling)

Workloads: tiny_decode, decode_b64, decode_b256 (default), verify_t4,
verify_record_t8 (the step), and replay_t8 (the RecoverSSM replay of
recorded tokens onto checkpoint pages).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_decode_03_amd", "csrc")
# The sources a workload's kernel is built from: a counter summary taken on
# other source text does not describe the current kernel.
KERNEL_SOURCES = {
    "step": ("kda_device.hpp", "kda_stages.hpp", "kda_step.hip"),
    "replay": ("kda_device.hpp", "kda_replay.hip"),
}


def kernel_source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()
D = 128


def algorithmic_bytes(p) -> int:
    """Bytes the method must move for one launch (each operand once):
    per live item: the 64 KiB state page read, 64 KiB written per stored
    token (1 for decode, T for verify, 0 for record), records T KiB, the
    3 read taps and T+2 written columns of its 384 convolution channels
    (2 bytes each, 4 with an FP32 pool),
    x (768 B), gate (256 B), beta (2 B) and out (256 B) per token; per padded
    item its 256 B of zeros per token; per live request f_a (256 B per
    token); the slot tables; once per launch the weights (F_B, conv weights,
    dt_bias, A_log, norm weight)."""
    import numpy as np

    from linear_attention_decode_03_amd.inputs import live_items

    B, H, T = p["B"], p["H"], p["T"]
    live = len(live_items(p))
    live_req = live // H
    pad = B * H - live
    stored = 0 if p["record"] else (1 if T == 1 else T)
    ce = 4 if p.get("conv_f32") else 2  # bytes per convolution-pool entry
    per_live = (65536 * (1 + stored) + (1024 * T if p["record"] else 0)
                + 3 * D * 3 * ce + 3 * D * (T + 2) * ce + T * (768 + 256 + 2 + 256))
    total = live * per_live + pad * 256 * T + live_req * 256 * T
    total += int(np.asarray(p["slots"]).nbytes) + (B * 4 if T > 1 else 0)
    total += H * (3 * 4 * D * 2 + D * D * 2 + D * 4 + 4) + D * 2
    return int(total)


def replay_algorithmic_bytes(r) -> int:
    """Bytes one replay launch must move: per valid (request, head) the 64 KiB
    checkpoint page read and the 64 KiB page written, and per applied token
    its records (512 B of u, 512 B of k | raw_g); the three slot tables;
    A_log and dt_bias once."""
    B, H, T, N = r["B"], r["H"], r["T"], r["N"]
    total = 0
    for b in range(B):
        src, dst, n = int(r["src"][b]), int(r["dst"][b]), int(r["n"][b])
        if 0 < src < N and 0 < dst < N and 0 <= n <= T:
            total += H * (2 * 65536 + n * 1024)
    return int(total + 3 * B * 4 + H * 4 + H * D * 4)


def measured_traffic(workload):
    """HBM bytes per launch from the committed counter summary of this
    workload, if it was taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"kda_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src_hash = kernel_source_hash("replay" if workload.startswith("replay") else "step")
    if fields.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(p, replay=False, min_seconds=10.0, min_passes=3):
    """The oracle as it is (single-threaded C) on the same workload, with this
    process pinned to one core while it runs: whole passes over all items
    (the step, or the replay), at least `min_passes` and until `min_seconds`
    have elapsed; the rate is the median over the passes."""
    import oracle
    from linear_attention_decode_03_amd.inputs import copy_problem

    oracle.build(force=False)
    q = copy_problem(p)
    n_items = p["B"] * p["H"]
    cores = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {cores[0]})
    try:
        rates, t0 = [], time.perf_counter()
        while len(rates) < min_passes or time.perf_counter() - t0 < min_seconds:
            ts = time.perf_counter()
            if replay:
                oracle.replay(q)
            else:
                oracle.run(q)
            rates.append(n_items / (time.perf_counter() - ts))
        el = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, set(cores))
    rates.sort()
    res = {"value": rates[len(rates) // 2], "unit": "items/s", "cores": 1, "kind": "oracle",
           "sample": f"median of {len(rates)} full passes over the {n_items} items of the same "
                     f"workload, single-threaded, pinned to core {cores[0]}, {el:.1f} s",
           "cpu_model": cpu_model()}
    if not replay:
        res["threaded"] = cpu_baseline_threaded(q, min_seconds=min_seconds / 2)
    return res


def cpu_model():
    """The host CPU as /proc/cpuinfo names it (model name, family, model and
    the number of logical CPUs)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                fields.setdefault(k, v)
    except OSError:
        return None
    name = fields.get("model name")
    if not name:
        return None
    return (f"{name} (family {fields.get('cpu family', '?')}, model {fields.get('model', '?')}; "
            f"{os.cpu_count()} logical CPUs, {len(os.sched_getaffinity(0))} usable)")


def cpu_baseline_threaded(q, min_seconds=5.0, max_threads=16):
    """The same oracle on the same problem with its items split statically
    over host threads: one contiguous block of item ids per thread, each a
    plain oracle call on that block (the C code holds an item's state on its
    own stack and items touch disjoint memory; ctypes releases the GIL for
    the call).  Threads: the cores this process may run on, at most
    `max_threads`."""
    import threading

    import numpy as np

    import oracle

    n_items = q["B"] * q["H"]
    n = max(1, min(max_threads, len(os.sched_getaffinity(0)), n_items))
    blocks = np.array_split(np.arange(n_items, dtype=np.int32), n)
    done, t0 = 0, time.perf_counter()
    while True:
        ts = [threading.Thread(target=oracle.run, args=(q,), kwargs={"items": blk})
              for blk in blocks]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        done += n_items
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": done / el, "unit": "items/s", "cores": n,
            "sample": f"{done // n_items} full pass(es) over the {n_items} items, "
                      f"static split over {n} threads, {el:.1f} s"}


def copy_ceiling(torch, reps=10):
    """What a plain device copy moves on this GPU: 1 GiB copied `reps` times
    between one pair of events (read + write bytes / time), after one
    untimed copy."""
    n = 1 << 28  # 1 GiB of float32
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return {"gbps": 2 * n * 4 / sec / 1e9, "bytes": 2 * n * 4,
            "what": "1 GiB device-to-device copy (torch copy_), read + write bytes / time"}


def run_copy(args):
    import torch

    n = 1 << 28  # 1 GiB of float32
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"mode": "copy", "bytes_per_copy": 2 * n * 4, "steps": args.steps,
                      "gbps": 2 * n * 4 * args.steps / el / 1e9}))


def run_sweep(args):
    """Small batches: per-launch time of decode (T=1) and verify (T=2, 4, 8)
    at H=32 and B*H in {32 .. 2048} items, unsplit and split over 2 and 4
    workgroups per item.  Each configuration captures 20 launches in one HIP
    graph (so host launch overhead is out of the figure) and replays it;
    the median over 15 timed replays, divided by 20, is printed per
    configuration as one JSON line."""
    import torch

    from linear_attention_decode_03_amd import inputs, kda
    from linear_attention_decode_03_amd import device as dev

    kda.load_library()
    H = 32
    for T in (1, 2, 4, 8):
        for items in (32, 64, 128, 256, 512, 1024, 2048):
            B = items // H
            cfg = dict(B=B, H=H, T=T, seed=11, N=(2 * B + 2) if T == 1 else B * T + 1,
                       W=3 if T == 1 else T + 2)
            p = inputs.make_problem(cfg)
            row = {"mode": "sweep", "T": T, "items": items}
            for split in (1, 2, 4):
                if split > 1 and items * split > 2048:
                    continue
                d = dev.to_device(p)
                ws = kda.split_workspace(B, H, T, d["state"].device)

                def step():
                    if split == 1:
                        dev.run(d)
                    else:
                        dev.run_split(d, ws, split=split)

                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    for _ in range(3):
                        step()
                torch.cuda.current_stream().wait_stream(s)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(20):
                        step()
                g.replay()
                torch.cuda.synchronize()
                times = []
                for _ in range(15):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1) * 1e3 / 20)
                row[f"split{split}_us"] = sorted(times)[len(times) // 2]
                del g, d, ws
            print(json.dumps(row), flush=True)


def run_pagecopy(args):
    """The ceiling of the step's page traffic: kda_page_copy on the workload's
    own slot tables (each item reads its 64 KiB page and writes it to its
    stored-token targets: in place for decode, T pages for verify, none for
    record), in the step kernels' access shape and with no compute.  Times K
    back-to-back launches between one event pair, and cold-clean launches
    (each after a 1 GiB read); prints one JSON line."""
    import numpy as np
    import torch

    from linear_attention_decode_03_amd import device as dev
    from linear_attention_decode_03_amd import inputs, kda

    kda.load_library()
    p = inputs.make_problem(args.workload)
    B, T = p["B"], p["T"]
    if T == 1:
        src = p["slots"].astype(np.int32)
        dst = src.reshape(B, 1).copy()
    else:
        src = p["slots"][np.arange(B), p["accepted"] - 1].astype(np.int32)
        dst = p["slots"][:, :T].copy() if not p["record"] else np.zeros((B, 0), np.int32)
    n_dst = dst.shape[1]
    d = dev.to_device(p)
    src_t = torch.from_numpy(np.ascontiguousarray(src)).cuda()
    dst_t = torch.from_numpy(np.ascontiguousarray(dst)).cuda() if n_dst else None

    def step():
        kda.kda_page_copy(d["state"], src_t, dst_t, n_dst)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / K
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    flush.fill_(1.0)
    clean = []
    for _ in range(max(1, args.cold_launches)):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        clean.append(a.elapsed_time(b) * 1e3)
    clean.sort()
    live = int((src > 0).sum()) * p["H"]
    writes = int((dst > 0).sum()) * p["H"]
    page_bytes = (live + writes) * 65536
    print(json.dumps({"mode": "pagecopy", "workload": args.workload, "items": B * p["H"],
                      "pages_read": live, "pages_written": writes, "bytes": page_bytes,
                      "warm_us": warm_us, "warm_gbps": page_bytes / warm_us / 1e3,
                      "clean_us": clean[len(clean) // 2],
                      "clean_gbps": page_bytes / clean[len(clean) // 2] / 1e3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_b256")
    ap.add_argument("--ahead", type=int, default=-1)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cold-launches", type=int, default=20)
    ap.add_argument("--conv-f32", action="store_true",
                    help="keep the convolution pool in FP32 (kda_*_f32conv)")
    ap.add_argument("--mode", choices=["kda", "copy", "sweep", "pagecopy"], default="kda")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA step has no cross-GPU exchange "
              "(each GPU would run its own share of heads); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.mode == "copy":
        return run_copy(args)
    if args.mode == "sweep":
        return run_sweep(args)
    if args.mode == "pagecopy":
        return run_pagecopy(args)

    from linear_attention_decode_03_amd import device as _gpu
    from linear_attention_decode_03_amd import inputs, kda

    kda.load_library()
    replay = args.workload in inputs.REPLAY_CONFIGS
    if replay:
        p = inputs.make_replay_problem(args.workload)
    else:
        p = inputs.make_problem(args.workload, conv_f32=int(args.conv_f32))
    print(f"[bench] workload {args.workload}: inputs ready", file=sys.stderr, flush=True)
    d = _gpu.to_device(p)

    def step():
        if replay:
            _gpu.run_replay(d)
        else:
            _gpu.run(d, ahead=args.ahead)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region: exactly K back-to-back steps between one pair of
    # events on the launch stream (nothing else is enqueued between the
    # launches), bracketed by device synchronisations.  The events' span / K
    # is the average launch duration, gaps between launches included.
    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(K):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    kernel_ms = ev0.elapsed_time(ev1) / K
    print(f"[bench] {K} steps, {ms_per_step * 1e3:.1f} us/step, kernel {kernel_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    # Spread of single launches: a second pass (outside the timed region)
    # with an event pair around every launch.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    single = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))

    # Cold launches: before each one (outside the launch's own events) a
    # 1 GiB pass over a scratch buffer evicts the L2s and the memory-side
    # cache.  "cold": the pass writes, so the caches are full of dirty lines
    # that are written back while the launch runs; "clean": the pass only
    # reads, so nothing of the launch is cached and nothing else is dirty.
    k_cold = max(0, args.cold_launches)
    cold, clean = [], []
    if k_cold:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        flush.fill_(1.0)
        for mode, out_list in (("write", cold), ("read", clean)):
            ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(k_cold)]
            ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(k_cold)]
            for i in range(k_cold):
                if mode == "write":
                    flush.fill_(float(i))
                else:
                    flush.sum()
                ev_s[i].record()
                step()
                ev_e[i].record()
            torch.cuda.synchronize()
            out_list.extend(sorted(s_.elapsed_time(e_) for s_, e_ in zip(ev_s, ev_e)))
        del flush

    copy = copy_ceiling(torch) if k_cold else None

    items = p["B"] * p["H"]
    abytes = replay_algorithmic_bytes(p) if replay else algorithmic_bytes(p)
    traffic = measured_traffic(args.workload)

    def rate(us):
        gbps = abytes / (us * 1e-6) / 1e9
        return {"kernel_us": us, "achieved": gbps, "frac": gbps / HBM_PEAK_GBPS}

    warm = dict(rate(kernel_ms * 1e3), method=f"span of the {K} back-to-back launches of the "
                "timed region between one event pair on the launch stream, / K")
    cold_dirty = None if not cold else dict(
        rate(cold[k_cold // 2] * 1e3), launches=k_cold,
        method="median of launches each preceded by a 1 GiB write outside its events "
               "(the caches hold dirty lines written back during the launch)")
    cold_clean = None if not clean else dict(
        rate(clean[k_cold // 2] * 1e3), launches=k_cold,
        method="median of launches each preceded by a 1 GiB read outside its events "
               "(nothing of the launch is cached, nothing else dirty)")
    # The headline: cold-clean (no operand cached), else the warm figure.
    head = cold_clean or warm
    roofline = {"bound": "hbm", "achieved": head["achieved"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": head["frac"], "kernel_us": head["kernel_us"],
                "method": "cold_clean" if cold_clean else "warm",
                "traffic": traffic, "algorithmic_bytes_per_launch": abytes,
                "warm": warm, "cold_clean": cold_clean, "cold_dirty": cold_dirty,
                "single_launch_us": {"p10": single[K // 10] * 1e3,
                                     "median": single[K // 2] * 1e3,
                                     "p90": single[(9 * K) // 10] * 1e3},
                "copy_ceiling": copy}
    if not replay:
        extra = {"record": p["record"], "gate_mode": p["gate_mode"],
                 "conv_pool": "f32" if p["conv_f32"] else "bf16"}
    else:
        extra = {"tokens_applied": int(p["n"].sum())}
    result = {
        "metric": "KDA decode (request,head)-steps/sec and achieved HBM GB/s (% of peak)",
        "value": items / (ms_per_step * 1e-3),
        "unit": "items/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: KDA {'replay' if replay else 'step'} "
                               f"T={p['T']}, B={p['B']} requests, H={p['H']} heads, d=128, "
                               f"{p['N']}-slot FP32 state pool",
                   "B": p["B"], "H": p["H"], "T": p["T"], "N": p["N"], "items": items},
        "roofline": roofline,
    }
    result["config"].update(extra)
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(p, replay=replay)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
