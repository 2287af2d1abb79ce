"""Benchmark: paged decode steps on one MI355X.

A step is one pass of the whole hot path over one synthetic batch:
copy-on-write of diverging blocks (when the workload has any), the
new tokens' slot scatter, then paged decode attention. The default workload
is the Llama-3-8B-shaped grouped-query decode layer: 256 sequences, 32 query
and 8 KV heads, head size 128, 16-token blocks, context lengths lognormal
(median 1024, sigma 0.5, clipped to [16, 4096]), a shuffled pool of 65536
blocks.

Prints one JSON line. After ``--warmup`` untimed steps and at least 200 ms
more of untimed steps, exactly ``--steps`` steps are timed: ``value`` is
algorithmic bytes per step / time per step (GB/s). ``roofline`` covers the
decode call (the decode kernel and the merge of cut pieces that follows it
on the same stream), timed over at least 100 more steps and 200 ms with HIP
events around the call on the launch stream: its algorithmic bytes / its
mean time, against 8 TB/s, with the median, p10 and p90 beside the mean; ``traffic`` is the call's HBM bytes from rocprofv3 counters
(profiles/decode_traffic.json) when they were taken on the current kernel;
``mean_launch_us_mall_evicted`` repeats the call with the 256 MB memory-side
cache evicted before each launch (a 2 GiB read scan outside the events), and
``stream_read_same_bytes`` is a streaming read of as many contiguous bytes
timed the same way (``frac_of_stream_read`` = achieved / that).
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on this host, on one worker process per core and on one thread.

    python bench.py [--gpus 1] [--steps 500] [--warmup 20] [--config NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak) and seq-steps/sec"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak
# Timing protocol: an untimed warm-up of at least WARMUP_S seconds of steps
# before anything is timed; the decode call's roofline time over at least
# ROOF_MIN_LAUNCHES launches and ROOF_MIN_S seconds (mean, median, p10, p90).
WARMUP_S = 0.2
ROOF_MIN_LAUNCHES = 100
ROOF_MIN_S = 0.2
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_433_amd", "csrc", "decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
CACHE_NOTES = {
    "tiny_mha": "warm: the whole cache fits in L2",
    "beam_cow": "warm in part: the 4 beams of a prompt read its shared blocks, so some logical bytes come from cache",
    "beam_cow_shared": "cold in part: a prompt's blocks are read once per group of beams, beams forked from the same "
                       "parent read its history each (about 0.38 GB; the MALL is 256 MB)",
    "beam_cow_tree": "cold in part: every distinct block is read once per call (about 0.35 GB; the MALL is 256 MB)",
    "beam_cow_shared_planned": "cold in part: as beam_cow_shared, the plan built once before the timed calls",
    "beam_cow_tree_planned": "cold in part: as beam_cow_tree, the plan built once before the timed calls",
}


def source_digest(path=DECODE_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """Per-launch HBM bytes of the decode kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("decode_hip_sha256_16") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def _counter_means(path: str, counter: str) -> dict:
    """Mean value of `counter` per kernel name in a rocprofv3 counter CSV."""
    import csv

    sums, counts = {}, {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            sums[name] = sums.get(name, 0.0) + float(row["Counter_Value"])
            counts[name] = counts.get(name, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def _one(means: dict, fragment: str) -> float:
    hits = [v for k, v in means.items() if fragment in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {fragment!r}, found {len(hits)}")
    return hits[0]


def record_traffic(prefix: str, workload: str, copy_bytes: int, copy_prefix: str | None = None) -> int:
    """Write the decode call's per-launch HBM bytes into profiles/decode_traffic.json.

    Reads four rocprofv3 --pmc runs: {prefix}_fetch_decode and
    {prefix}_write_decode (this bench on `workload`, counters FETCH_SIZE and
    WRITE_SIZE), {prefix}_fetch_copy and {prefix}_write_copy (--probe-copy of
    `copy_bytes` bytes). The call's kernels are the decode and merge kernels,
    the plan kernel when the call is sharing-aware, and the scatter kernel
    when the decode step runs as two launches. Each counter is scaled by what it reads for the copy,
    which moves exactly `copy_bytes` each way, so the units need not be known.
    """
    def means(kind, counter, pre=None):
        return _counter_means(f"{pre or prefix}_{kind}/run_counter_collection.csv", counter)

    fetch_copy = _one(means("fetch_copy", "FETCH_SIZE", copy_prefix), "probe_copy")
    write_copy = _one(means("write_copy", "WRITE_SIZE", copy_prefix), "probe_copy")
    fd, wd = means("fetch_decode", "FETCH_SIZE"), means("write_decode", "WRITE_SIZE")
    f_scale, w_scale = copy_bytes / fetch_copy, copy_bytes / write_copy
    per = {}
    frags = ["decode_kernel", "merge_kernel"]
    if any("share_plan_kernel" in k for k in fd):  # the sharing-aware call's plan
        frags.insert(0, "share_plan_kernel")
    if any("step_scatter_kernel" in k for k in fd):  # the decode step in two launches
        frags.insert(0, "step_scatter_kernel")
    for frag in frags:
        per[frag] = {"fetch_bytes": int(_one(fd, frag) * f_scale), "write_bytes": int(_one(wd, frag) * w_scale)}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in per.values())
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[workload] = {
        "decode_hip_sha256_16": source_digest(),
        "bytes_per_launch": total,
        "kernels": per,
        "calibration": {"copy_bytes": copy_bytes, "fetch_size_per_copy": fetch_copy,
                        "write_size_per_copy": write_copy},
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[workload]))
    return 0


def _oracle_worker(task):
    """One process of the CPU baseline: run the oracle on whole units of its
    share of the seeded order, cycling, for `seconds` with BLAS on one
    thread. A unit is a sequence, or (sharing-aware decode) a group or a run
    of sequences that share leading blocks. The cache arrays are
    memory-mapped read-only from files the parent wrote, so the workers
    share one copy. Returns (units done, seconds)."""
    from threadpoolctl import threadpool_limits

    import numpy as np

    import oracle

    (paths, shape, q, tables, lens, scale, q_len, kind, units, order, seconds) = task
    kc = np.memmap(paths[0], dtype=np.uint16, mode="r", shape=shape)
    vc = np.memmap(paths[1], dtype=np.uint16, mode="r", shape=shape)
    done = []
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for u in order:
                lo, hi, shared = units[u]
                if kind == "groups":
                    oracle.decode_shared(q[lo:hi], kc, vc, tables[lo:hi], lens[lo:hi], [0, hi - lo], [shared],
                                         scale)
                elif kind == "tree":  # true declarations: the plain decode of the run
                    oracle.decode(q[lo:hi], kc, vc, tables[lo:hi], lens[lo:hi], scale)
                elif q_len > 1:
                    oracle.decode_multi(q[lo:hi], kc, vc, tables[lo:hi], lens[lo:hi], scale)
                else:
                    oracle.decode_sequence(q[lo], kc, vc, tables[lo], lens[lo], scale)
                done.append(int(u))
                if time.perf_counter() - t0 >= seconds:
                    break
        dt = time.perf_counter() - t0
    return done, dt


def _time_oracle(batch, paths, order, seconds: float, procs: int, kind, units):
    """The oracle on `procs` worker processes (each a slice of `order`), or
    in this process when procs == 1; returns (units done, seconds)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    shape = batch.k_cache.shape
    tasks = [(paths, shape, batch.q, batch.block_tables, batch.context_lens, batch.scale, batch.q_len, kind, units,
              order[i::procs], seconds) for i in range(procs)]
    if procs == 1:
        res = [_oracle_worker(tasks[0])]
    else:
        # Fresh interpreters (spawn), not forks of this process: they never
        # touch the GPU and hold no copy of its state.
        ex = ProcessPoolExecutor(procs, mp_context=mp.get_context("spawn"))
        try:
            res = list(ex.map(_oracle_worker, tasks, timeout=seconds + 300))
        finally:
            ex.shutdown(wait=False, cancel_futures=True)
    done = [s for r in res for s in r[0]]
    return done, max(r[1] for r in res)


def cpu_baseline(batch, seconds: float, sharing=None):
    """Time the float64 oracle on whole units of the batch in a seeded order
    (cycling through it), for `seconds`: once on one worker process per
    core this process may use (the oracle is serial numpy, so the host's
    cores work through separate units), and once on a single thread; rate
    in the metric's unit (algorithmic GB/s). A unit is a sequence, or with
    `sharing` ("groups", starts, shared) a group, or with ("tree", sprev) a
    run of sequences each sharing leading blocks with the one before. The
    all-cores run is the reported value."""
    import shutil
    import tempfile

    import numpy as np

    import oracle
    from paged_kv_cache_433_amd import workloads as W

    kc, vc = batch.k_cache, batch.v_cache  # updated in place; the device copies exist already
    if len(batch.cow_pairs):
        oracle.copy_blocks(kc, vc, batch.cow_pairs)
    oracle.reshape_and_cache(kc, vc, batch.new_k, batch.new_v, batch.slot_mapping)
    S, mb = batch.num_seqs, batch.max_blocks_per_seq
    kind = sharing[0] if sharing else "plain"
    if kind == "groups":
        starts, shared = sharing[1], sharing[2]
        units = [(int(starts[g]), int(starts[g + 1]), int(shared[g])) for g in range(len(shared))]
    elif kind == "tree":
        sprev = sharing[1]
        cuts = list(np.flatnonzero(W.chain_sharing(batch.context_lens, sprev, mb) == 0)) + [S]
        units = [(int(cuts[i]), int(cuts[i + 1]), 0) for i in range(len(cuts) - 1)]
    else:
        units = [(s, s + 1, 0) for s in range(S)]

    def unit_bytes(u):
        lo, hi, shared = units[u]
        n = batch.context_lens[lo:hi]
        if kind == "groups":
            return W.shared_algorithmic_bytes(n, [0, hi - lo], [shared], mb, batch.num_q_heads,
                                              batch.num_kv_heads, batch.head_size)
        if kind == "tree":
            return W.tree_algorithmic_bytes(n, sprev[lo:hi], mb, batch.num_q_heads, batch.num_kv_heads,
                                            batch.head_size)
        return W.algorithmic_bytes(n, batch.num_q_heads, batch.num_kv_heads, batch.head_size, q_len=batch.q_len)

    order = np.random.default_rng(0).permutation(len(units))
    # The host share this process may use: its CPU affinity, capped by the
    # thread count the environment sets for OpenMP/BLAS.
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    tmp = tempfile.mkdtemp(prefix="pa_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    paths = (os.path.join(tmp, "k_cache"), os.path.join(tmp, "v_cache"))
    res = {}
    try:
        kc.tofile(paths[0])
        vc.tofile(paths[1])
        for procs in (cores, 1):
            done, dt = _time_oracle(batch, paths, order, seconds, procs, kind, units)
            nbytes = sum(unit_bytes(u) for u in done)
            seqs = sum(units[u][1] - units[u][0] for u in done)
            tokens = sum(int(batch.context_lens[units[u][0]:units[u][1]].sum()) for u in done)
            res[procs] = (seqs, tokens, dt, nbytes / dt / 1e9, seqs / dt)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    n, tokens, dt, gbps, sps = res[cores]
    what = {"plain": "", "groups": " of whole groups (decode_shared)",
            "tree": " of whole runs of sequences sharing prefixes (decode_shared_tree)"}[kind]
    return {
        "value": round(gbps, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{n} sequence-steps of the {batch.num_seqs}-sequence batch, taken in a seeded "
                   f"order{what} ({tokens} tokens), "
                   f"float64 numpy oracle on {cores} worker processes (one per core, BLAS on one thread "
                   f"each, cache arrays shared read-only), {dt:.1f} s"),
        "seq_steps_per_s": round(sps, 3),
        "single_thread": {"value": round(res[1][3], 4), "unit": "GB/s", "seq_steps_per_s": round(res[1][4], 3),
                          "sample": f"{res[1][0]} sequence-steps on one thread, {res[1][2]:.1f} s"},
    }


def probe_copy(nbytes: int, steps: int, warmup: int, dev) -> int:
    """Time pa_probe_copy over `nbytes` bytes (read once, written once)."""
    import numpy as np
    import torch

    import paged_kv_cache_433_amd as pa

    nbytes = (nbytes + 15) // 16 * 16
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        pa.probe_copy(dst, src)
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        pa.probe_copy(dst, src)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs]) * 1e3)
    print(json.dumps({"probe": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": warmup + steps,
                      "median_us": round(us, 2), "read_plus_write_GBps": round(2 * nbytes / us / 1e3, 1)}),
          flush=True)
    return 0


def swap_probe(num_blocks: int, steps: int, dev) -> int:
    """Time pa_swap_blocks of `num_blocks` scattered blocks of the GQA layer's
    shape (8 KV heads of 128: 64 KiB of K and V per block) out to pinned host
    memory and back in, against a DMA copy of the same bytes (torch's pinned
    host <-> device copy of one contiguous buffer) as the link's reference."""
    import numpy as np
    import torch

    import paged_kv_cache_433_amd as pa

    shape = (65536, 16, 8, 128)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    hk = torch.empty((num_blocks,) + shape[1:], dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    rng = np.random.default_rng(7)
    out_pairs = torch.from_numpy(np.stack([rng.permutation(shape[0])[:num_blocks], np.arange(num_blocks)],
                                          axis=1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(num_blocks), rng.permutation(shape[0])[:num_blocks]],
                                         axis=1).astype(np.int64)).to(dev)
    nbytes = 2 * hk.numel() * hk.element_size()
    stream = torch.cuda.current_stream(dev)
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, z in evs:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(z) for a, z in evs])) * 1e3

    t_out = timed(lambda: pa.swap_blocks(kc, vc, hk, hv, out_pairs, "out"))
    t_in = timed(lambda: pa.swap_blocks(kc, vc, hk, hv, in_pairs, "in"))
    t_d2h = timed(lambda: hbuf.copy_(dbuf, non_blocking=True))
    t_h2d = timed(lambda: dbuf.copy_(hbuf, non_blocking=True))
    print(json.dumps({"probe": "swap_blocks", "blocks": num_blocks, "bytes_per_direction": nbytes,
                      "out_us": round(t_out, 1), "out_GBps": round(nbytes / t_out / 1e3, 2),
                      "in_us": round(t_in, 1), "in_GBps": round(nbytes / t_in / 1e3, 2),
                      "dma_d2h_GBps": round(nbytes / t_d2h / 1e3, 2),
                      "dma_h2d_GBps": round(nbytes / t_h2d / 1e3, 2)}), flush=True)
    return 0


def workload_name(args) -> str:
    """Key of a workload and call kind in the traffic record."""
    return (args.config + {None: "", "groups": "_shared", "tree": "_tree"}[args.shared]
            + ("_planned" if args.plan_once else "") + ("_unfused" if args.unfused else "")
            + (f"_bs{args.block_size}" if args.block_size != 16 else "") + (f"_q{args.q_len}" if args.q_len > 1 else ""))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama3_8b_gqa")
    ap.add_argument("--q-len", type=int, default=1,
                    help="new tokens per sequence (speculative-decode verification): the step scatters them "
                         "and runs pa_decode_multi")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="tokens per cache block for the named single-step configs (same pool capacity in "
                         "tokens)")
    ap.add_argument("--unfused", action="store_true",
                    help="single new token: scatter with pa_reshape_and_cache, then pa_decode (two launches), "
                         "instead of the fused step (pa_decode_step: the new token is attended from its K/V "
                         "row and written to its slot in the decode launch)")
    ap.add_argument("--shared", nargs="?", const="groups", choices=("groups", "tree"), default=None,
                    help="beam_cow only: sharing-aware decode with the sharing read back from the block tables. "
                         "groups (the default): pa_decode_shared, a prompt's shared blocks read once for its "
                         "beams; tree: pa_decode_shared_tree over the beams in depth-first order, so beams "
                         "that forked from the same parent also read its history once")
    ap.add_argument("--plan-once", action="store_true",
                    help="with --shared: build the sharing plan once (pa_share_plan, as a model does once per step "
                         "for all its layers) and time the per-layer call pa_decode_shared_planned")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of oracle work per CPU-baseline run (two runs: all cores, one thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-launches", type=int, default=100,
                    help="extra decode calls timed with the MALL evicted before each (0: skip)")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="BYTES",
                    help="instead of the decode step: time a plain 16-byte copy of BYTES bytes "
                         "(the reference kernel that calibrates rocprofv3 byte counters)")
    ap.add_argument("--swap-blocks", type=int, default=0, metavar="N",
                    help="instead of the decode step: time swapping N blocks out to pinned host memory and in")
    ap.add_argument("--record-traffic", metavar="PREFIX",
                    help="no GPU work: turn the rocprofv3 --pmc runs PREFIX_{fetch,write}_decode and "
                         "COPY_{fetch,write}_copy (COPY from --copy-prefix, default PREFIX) into the traffic "
                         "record for the workload --config and the other flags name (copy size from --probe-copy)")
    ap.add_argument("--copy-prefix", default=None,
                    help="with --record-traffic: prefix of the copy probe's counter runs")
    args = ap.parse_args(argv)
    if args.record_traffic:
        return record_traffic(args.record_traffic, workload_name(args), args.probe_copy or (1 << 30),
                              args.copy_prefix)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_433_amd as pa
    from paged_kv_cache_433_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.probe_copy:
        return probe_copy(args.probe_copy, args.steps, args.warmup, dev)
    if args.swap_blocks:
        return swap_probe(args.swap_blocks, min(args.steps, 50), dev)
    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    # The beam-search workload's first step: its copy-on-write pairs, its
    # scatter and its decode are repeated every step (both are idempotent).
    if args.config == "beam_cow":
        if args.q_len != 1:
            raise SystemExit("--q-len applies to the named single-step configs")
        wl = W.BeamSearchWorkload()
        b = wl.step()
        if args.shared == "tree":
            # the scheduler lists the beams depth first in their prefix tree
            b = W.permuted(b, W.tree_order(b.block_tables, b.context_lens))
    else:
        if args.shared:
            raise SystemExit("--shared applies to the beam_cow workload")
        b = W.make_config(args.config, q_len=args.q_len, block_size=args.block_size)
    if args.plan_once and not args.shared:
        raise SystemExit("--plan-once applies to --shared")
    multi = args.q_len > 1
    fused = not (multi or args.shared or args.unfused)
    if fused:
        # The fused step derives each new token's slot from its table: the
        # batch's slots must be position n - 1 of each sequence.
        pos = b.context_lens.astype(np.int64) - 1
        want = b.block_tables[np.arange(b.num_seqs), pos // b.block_size].astype(np.int64) * b.block_size + \
            pos % b.block_size
        assert np.array_equal(want, b.slot_mapping), "new tokens are not at position n - 1 of their sequences"
    if args.config == "beam_cow" and args.block_size != 16:
        raise SystemExit("--block-size applies to the named single-step configs")
    workload = workload_name(args)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    kc, vc = bf16(b.k_cache), bf16(b.v_cache)
    q = bf16(b.q)
    new_k, new_v = bf16(b.new_k), bf16(b.new_v)
    tables = torch.from_numpy(b.block_tables).to(dev)
    lens = torch.from_numpy(b.context_lens).to(dev)
    slots = torch.from_numpy(b.slot_mapping).to(dev)
    pairs = torch.from_numpy(b.cow_pairs).to(dev) if len(b.cow_pairs) else None
    out = torch.empty_like(q)
    scale = float(b.scale)

    logical_bytes = W.algorithmic_bytes(b.context_lens, b.num_q_heads, b.num_kv_heads, b.head_size,
                                        block_size=b.block_size, q_len=args.q_len)
    decode_bytes = logical_bytes
    sharing = None
    if args.shared == "tree":
        sprev = W.declared_chain(b.block_tables, b.context_lens)
        sprev_t = torch.from_numpy(sprev).to(dev)
        decode_bytes = W.tree_algorithmic_bytes(b.context_lens, sprev, b.max_blocks_per_seq, b.num_q_heads,
                                                b.num_kv_heads, b.head_size)
        sharing = ("tree", sprev)
    elif args.shared:
        gstarts = W.consecutive_groups(b.num_seqs, wl.beams)
        gshared = W.declared_sharing(b.block_tables, b.context_lens, gstarts)
        gstarts_t = torch.from_numpy(gstarts).to(dev)
        gshared_t = torch.from_numpy(gshared).to(dev)
        decode_bytes = W.shared_algorithmic_bytes(b.context_lens, gstarts, gshared, b.max_blocks_per_seq,
                                                  b.num_q_heads, b.num_kv_heads, b.head_size)
        sharing = ("groups", gstarts, gshared)
    if fused:
        decode_bytes += W.step_write_bytes(b.context_lens, b.num_kv_heads, b.head_size)
        step_bytes = decode_bytes
    else:
        step_bytes = decode_bytes + W.scatter_bytes(len(b.slot_mapping), b.num_kv_heads, b.head_size)
    if pairs is not None:
        step_bytes += W.copy_bytes(len(b.cow_pairs), b.block_size, b.num_kv_heads, b.head_size)

    plan = None
    if args.plan_once:
        plan = (pa.share_plan(kc, lens, b.num_q_heads, b.max_blocks_per_seq, shared_prev=sprev_t)
                if args.shared == "tree" else
                pa.share_plan(kc, lens, b.num_q_heads, b.max_blocks_per_seq, gstarts_t, gshared_t))

    def run_decode():
        if plan is not None:
            pa.decode_shared_planned(q, kc, vc, tables, plan, scale, out=out)
        elif fused:
            pa.decode_step(q, new_k, new_v, kc, vc, tables, lens, scale, out=out)
        elif args.shared == "tree":
            pa.decode_shared_tree(q, kc, vc, tables, lens, sprev_t, scale, out=out)
        elif args.shared:
            pa.decode_shared(q, kc, vc, tables, lens, gstarts_t, gshared_t, scale, out=out)
        elif multi:
            pa.decode_multi(q, kc, vc, tables, lens, scale, out=out)
        else:
            pa.decode(q, kc, vc, tables, lens, scale, out=out)

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if pairs is not None:
            pa.copy_blocks(kc, vc, pairs)
        if not fused:
            pa.reshape_and_cache(new_k, new_v, kc, vc, slots)
        if ev is not None:
            ev[0].record(stream)
        run_decode()
        if ev is not None:
            ev[1].record(stream)

    def events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    print(f"[bench] warmup {args.warmup} steps + at least {WARMUP_S * 1e3:.0f} ms", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Untimed warm-up of at least WARMUP_S of steps, whatever --warmup says,
    # so that clocks and caches have settled before any event is recorded.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < WARMUP_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()

    # Exactly `steps` timed steps (the step time), back to back between two
    # events: no marker inside the timed region.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps

    # The decode call's time for the roofline: at least ROOF_MIN_LAUNCHES
    # launches and ROOF_MIN_S of them, each inside a whole step as above,
    # with events around the call.
    n_roof = max(ROOF_MIN_LAUNCHES, args.steps, int(np.ceil(ROOF_MIN_S / (ms * 1e-3))))
    ev_roof = events(n_roof)
    for i in range(n_roof):
        step(ev_roof[i])
    torch.cuda.synchronize()
    dec_us = np.array([a.elapsed_time(z) for a, z in ev_roof]) * 1e3
    dec_mean_us = float(np.mean(dec_us))
    dec_pct = {p: float(np.percentile(dec_us, p)) for p in (10, 50, 90)}
    print(f"[bench] {args.steps} steps: {ms * 1e3:.1f} us/step; "
          f"{n_roof} decode calls: mean {dec_mean_us:.1f} us, median {dec_pct[50]:.1f}, p10 {dec_pct[10]:.1f}, "
          f"p90 {dec_pct[90]:.1f}", file=sys.stderr, flush=True)

    # The same decode call again with the 256 MB MALL (memory-side cache)
    # evicted before each launch by reading a 2 GiB buffer, outside the
    # events: shows whether repeated calls on the same cache are served from
    # it. A read scan leaves no dirty lines behind to be written back later.
    cold_us = stream_read_gbps = None
    if args.cold_launches:
        scratch = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
        sink = torch.empty(pa.probe_read_sink_bytes(), dtype=torch.uint8, device=dev)
        cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.cold_launches)]
        for a, z in cold:
            pa.probe_read(scratch, sink)
            a.record(stream)
            run_decode()
            z.record(stream)
        torch.cuda.synchronize()
        cold_us = float(np.mean([a.elapsed_time(z) for a, z in cold])) * 1e3
        # A streaming read (pa_probe_read) of as many bytes as the call's
        # algorithmic bytes, with the MALL evicted the same way: what one pass
        # over contiguous memory achieves at this size.
        span = torch.ones(int(decode_bytes) // 16 * 16, dtype=torch.uint8, device=dev)
        reads = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        pa.probe_read(span, sink)
        for a, z in reads:
            pa.probe_read(scratch, sink)
            a.record(stream)
            pa.probe_read(span, sink)
            z.record(stream)
        torch.cuda.synchronize()
        read_us = float(np.median([a.elapsed_time(z) for a, z in reads])) * 1e3
        stream_read_gbps = span.numel() / read_us / 1e3
        del scratch, sink, span

    value = step_bytes / (ms * 1e-3) / 1e9
    achieved = decode_bytes / (dec_mean_us * 1e-6) / 1e9
    # Which peak binds the call: the time its bytes need at peak HBM
    # bandwidth against the time its flops need at the bf16 matrix-core peak.
    flops = W.algorithmic_flops(b.context_lens, b.num_q_heads, b.head_size, q_len=args.q_len)
    achieved_tflops = flops / (dec_mean_us * 1e-6) / 1e12
    mfma_bound = flops / (PEAK_BF16_TFLOPS * 1e12) > decode_bytes / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(workload)
    if args.plan_once:
        kernel = "decode_shared_planned call (plan built once per step): decode_kernel + merge_kernel"
    elif args.shared == "tree":
        kernel = "decode_shared_tree call: share_plan_kernel + decode_kernel + merge_kernel"
    elif args.shared:
        kernel = "decode_shared call: share_plan_kernel + decode_kernel + merge_kernel"
    elif fused:
        kernel = ("decode_step call (new tokens attended and written in the decode launch; with more sequences "
                  "per workgroup than it can stage, a scatter launch first): [step_scatter_kernel +] "
                  "decode_kernel + merge_kernel")
    else:
        kernel = "decode call: decode_kernel + merge_kernel"
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.config,
            "num_seqs": b.num_seqs,
            "num_q_heads": b.num_q_heads,
            "num_kv_heads": b.num_kv_heads,
            "head_size": b.head_size,
            "block_size": b.block_size,
            "kv_pool_blocks": b.num_blocks,
            "kv_memory_utilization": round(W.memory_utilization(b.context_lens, b.block_size), 5),
            "sum_context_tokens": int(b.context_lens.sum()),
            "seed": b.seed,
            "q_len": args.q_len,
            "step": ("copy_blocks + " if pairs is not None else "")
                    + ("reshape_and_cache + decode_multi" if multi else
                       "reshape_and_cache + decode_shared_planned (plan built once)" if args.plan_once else
                       "reshape_and_cache + decode_shared_tree" if args.shared == "tree" else
                       "reshape_and_cache + decode_shared" if args.shared else
                       "decode_step (scatter and decode in one launch, or two with many sequences per workgroup)" if fused
                       else "reshape_and_cache + decode"),
            "parallelism": "single GPU",
            "cache": CACHE_NOTES.get(workload, "cold: the K/V of a call is several times the 256 MB MALL"),
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "seq_steps_per_s": round(b.num_seqs / (ms * 1e-3), 1),
        "bytes_per_step": int(step_bytes),
        "roofline": {
            "kernel": kernel,
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(achieved_tflops, 2) if mfma_bound else round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round((achieved_tflops / PEAK_BF16_TFLOPS) if mfma_bound else (achieved / PEAK_HBM_GBS), 4),
            "hbm_achieved_GBps": round(achieved, 2),
            "hbm_frac": round(achieved / PEAK_HBM_GBS, 4),
            "flops_per_launch": int(flops),
            "mfma_achieved_TFLOPs": round(achieved_tflops, 2),
            "mfma_frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(decode_bytes),
            "logical_bytes_per_launch": int(logical_bytes),
            "mean_launch_us": round(dec_mean_us, 2),
            "median_launch_us": round(dec_pct[50], 2),
            "p10_launch_us": round(dec_pct[10], 2),
            "p90_launch_us": round(dec_pct[90], 2),
            "launches_timed": int(n_roof),
            "mean_launch_us_mall_evicted": round(cold_us, 2) if cold_us else None,
            "achieved_mall_evicted": round(decode_bytes / cold_us / 1e3, 2) if cold_us else None,
            "stream_read_same_bytes": round(stream_read_gbps, 1) if stream_read_gbps else None,
            "frac_of_stream_read": round(achieved / stream_read_gbps, 4) if stream_read_gbps else None,
        },
        "cpu_baseline": None,
    }
    if args.config == "beam_cow":
        # Copy-on-write pairs of the step, and the K/V bytes of the distinct
        # blocks the step's tables use (every block read by the step, once).
        used = np.unique(np.concatenate([b.block_tables[s, :(int(n) + b.block_size - 1) // b.block_size]
                                         for s, n in enumerate(b.context_lens)]))
        rec["config"]["cow_pairs"] = int(len(b.cow_pairs))
        rec["config"]["distinct_blocks"] = int(len(used))
        rec["config"]["distinct_block_kv_bytes"] = int(len(used)) * 2 * b.block_size * b.num_kv_heads * b.head_size * 2
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (~{2 * args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds, sharing)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
