#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = one ``paged_attention_decode`` call over the whole batch (for the
split path: the partition kernel plus the log-sum-exp reduce), with the
inputs already resident in HBM.  Prints ONE JSON line:

  value        KV GB/s = (bytes of K and V of the valid tokens) / (wall time per step)
  ms_per_step  wall time per step: K steps back to back between two device
               synchronisations
  us_per_step_flushed
               the same step timed alone, N times: before each, an untimed
               512 MiB write evicts the caches (L2 and MALL), then one pair of
               HIP events on the launch stream brackets the step; p10/p50/p90
  roofline     the decode launches: algorithmic KV bytes / their mean duration
               (one pair of HIP events around the K back-to-back steps on the
               launch stream), against 8000 GB/s HBM3E peak; the flushed
               median gives ``frac_flushed_p50``; ``traffic`` is the HBM bytes
               per step from committed counter runs on the same kernel
               sources (``frac_traffic`` prices the step on them)
  cpu_baseline the float64 oracle on the host cores: a process pool over the
               batch's sequences (one BLAS thread per process), run before the
               GPU is touched; a one-core walk of the same batch beside it

Workload (default): 8B-shaped GQA decode batch, 256 sequences, 32 query / 8
kv heads, head_size 128, bf16, block_size 16, lognormal lengths (median 1024,
sigma 1, clipped to [16, 4096]), shuffled block pool.  Synthetic N(0, 1) data.

Other lines (``--op``): ``copy_blocks`` times the copy-on-write block copies on
the same pool layout (HBM roofline); ``prefill`` the multi-token rows
(speculative verification or a chunked prefill); ``block_manager`` times the
host block manager building one decode step of a 256-sequence batch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention: KV GB/s and % of HBM peak; us per decode step"
# partition size the timed launch uses per workload (0 = the library's balanced split)
DEFAULT_PARTITION = {1: 0, 2: 0, 3: 0, 4: 0, 5: 0}
# the shared-prefix workload names the same blocks from many sequences
DEFAULT_FLAGS = {5: 1}
KERNEL_SRC_DIR = os.path.join(ROOT, "paged_kv_cache_291_amd", "csrc")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--op", default="decode", choices=["decode", "copy_blocks", "block_manager", "prefill"])
    ap.add_argument("--prefill-case", default="verify", choices=["verify", "chunk"],
                    help="prefill: verify = the 8B batch with --query-tokens query tokens per sequence "
                         "(speculative verification); chunk = 8 sequences, 3584 cached + 512 new tokens")
    ap.add_argument("--query-tokens", type=int, default=4,
                    help="prefill verify: query tokens per sequence (the speculative draft length)")
    ap.add_argument("--kv", default="native", choices=["native", "fp8"],
                    help="fp8: the same workload over OCP e4m3 pools (random finite codes, scales 1/128 and 1/96)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--partition", type=int, default=-1, help="tokens per partition; -1 = workload default")
    ap.add_argument("--flags", type=int, default=-1, help="decode flags (1 = shared blocks); -1 = workload default")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of each oracle leg (the process pool and the one-core walk)")
    ap.add_argument("--cpu-cores", type=int, default=0,
                    help="oracle processes; 0 = the cores this process may run on, at most 16")
    ap.add_argument("--flush-iters", type=int, default=100,
                    help="steps timed one by one after a 512 MiB cache-evicting write (p10/p50/p90)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="capture the decode step in a HIP graph and time replays")
    ap.add_argument("--graph-calls", type=int, default=1, metavar="N",
                    help="with --graph: decode calls per captured graph (e.g. one per model layer); "
                         "times are per call")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--traffic-from", default="", metavar="FETCH_DIR,WRITE_DIR",
                    help="no GPU run: turn two rocprofv3 --pmc result folders of this benchmark into "
                         "profiles/traffic.json (pass the same --config/--partition/--copy-calibration)")
    return ap.parse_args()


def code_only(text: str) -> str:
    """C/C++ source without comments and with runs of white space collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the code of every kernel source file (comments and layout
    excluded): counter results are tied to it."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SRC_DIR)):
        h.update(name.encode())
        h.update(code_only(open(os.path.join(KERNEL_SRC_DIR, name)).read()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel_name: str, workload: str):
    """HBM bytes per decode step from committed counter runs, if they were
    taken on the current kernel sources (else None)."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        rec = json.load(open(TRAFFIC_JSON)).get(f"{kernel_name}|{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def traffic_from_counters(fetch_dir: str, write_dir: str, cfg: int, partition: int, flags: int):
    """Turn two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then
    WRITE_SIZE, each with --copy-calibration) into HBM bytes per decode step.

    Each counter is scaled by what it reads for the calibration copy (the last
    plain copy dispatch, of known size): the ratio of known bytes to counted
    bytes.  The result is stored in profiles/traffic.json under the step's
    kernel names and the workload, with the hash of the kernel sources.
    """
    import csv
    import glob

    def rows(d, counter):
        f = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
        return [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]

    out = {}
    known = None
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rs = rows(d, counter)
        copies = [r for r in rs if "copyBuffer" in r["Kernel_Name"]]
        calib_kib = float(copies[-1]["Counter_Value"])
        step = {}
        for r in rs:
            name = r["Kernel_Name"]
            if "pa::" not in name or "scatter" in name:
                continue
            short = name.replace("(anonymous namespace)::", "").split("<")[0].split("(")[0].split("::")[-1]
            step.setdefault(short, []).append(float(r["Counter_Value"]))
        out[counter] = (calib_kib, {k: sum(v) / len(v) for k, v in step.items()})
    return out


def write_traffic(args):
    fetch_dir, write_dir = args.traffic_from.split(",")
    cfg = args.config
    ps = DEFAULT_PARTITION[cfg] if args.partition < 0 else args.partition
    flags = DEFAULT_FLAGS.get(cfg, 0) if args.flags < 0 else args.flags
    res = traffic_from_counters(fetch_dir, write_dir, cfg, ps, flags)
    calib_bytes = args.copy_calibration << 20
    f_calib, f_kern = res["FETCH_SIZE"]
    w_calib, w_kern = res["WRITE_SIZE"]
    f_scale = calib_bytes / (f_calib * 1024.0)
    w_scale = calib_bytes / (w_calib * 1024.0)
    names = sorted(f_kern, key=lambda k: -f_kern[k])
    fetch = sum(f_kern[k] for k in names) * 1024.0 * f_scale
    write = sum(w_kern.get(k, 0.0) for k in names) * 1024.0 * w_scale
    key = "+".join(names) + f"|cfg{cfg}"
    db = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    db[key] = {
        "source_hash": source_hash(),
        "bytes_per_launch": int(round(fetch + write)),
        "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write)),
        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
        "per_kernel_fetch_bytes": {k: int(round(f_kern[k] * 1024.0 * f_scale)) for k in names},
        "per_kernel_write_bytes": {k: int(round(w_kern.get(k, 0.0) * 1024.0 * w_scale)) for k in names},
        "partition_size": ps, "flags": flags,
    }
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    print(json.dumps({key: db[key]}))


FLUSH_BYTES = 512 << 20
_ORACLE = {}                                     # inputs the oracle processes inherit (fork, no GPU yet)


def host_cores(requested: int = 0) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = min(n, 16)
    return max(1, min(requested, n) if requested > 0 else n)


def _oracle_init():
    from threadpoolctl import threadpool_limits
    _ORACLE["limits"] = threadpool_limits(1)      # one BLAS thread per process


def _oracle_seq(s: int):
    import oracle
    st = _ORACLE
    t0 = time.perf_counter()
    ref = oracle.paged_decode_ref(st["q"], st["kc"], st["vc"], st["bt"], st["sl"], st["scale"], st["dtype"],
                                  seqs=[s], **st["extra"])
    return s, ref[0], time.perf_counter() - t0


def cpu_baseline(wl, seconds: float, cores: int, fp8_pools=None):
    """The float64 oracle over the workload's sequences, on the host cores.

    Must run before this process touches the GPU: the pool forks it.
    * pool leg: ``cores`` processes (one BLAS thread each) walk the batch's
      sequences, whole passes, until ``seconds`` of wall time are spent;
    * one-core leg: the same walk in this process, one thread, for
      ``seconds``;
    * the tiny MHA batch (4 sequences, fp32) once on one core.
    Returns (record, {sequence: oracle output}) for the sequences walked.
    """
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from paged_kv_cache_291_amd import workloads as W

    q, kc, vc = W.raw_numpy(wl.query), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache)
    extra = {}
    if fp8_pools is not None:
        kc, vc = fp8_pools[0].numpy(), fp8_pools[1].numpy()
        extra = dict(kv_dtype="e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    if wl.slot_mapping is not None:                 # the new tokens' rows, as the GPU step scatters them
        nk, nv = W.raw_numpy(wl.new_key), W.raw_numpy(wl.new_value)
        if fp8_pools is not None:
            kc, vc = oracle.reshape_and_cache_fp8_ref(nk, nv, kc, vc, wl.slot_mapping, wl.dtype, FP8_K_SCALE,
                                                      FP8_V_SCALE)
        else:
            kc, vc = oracle.reshape_and_cache_ref(nk, nv, kc, vc, wl.slot_mapping)
    _ORACLE.update(q=q, kc=kc, vc=vc, bt=wl.block_tables, sl=wl.seq_lens, scale=wl.scale, dtype=wl.dtype,
                   extra=extra)
    S = wl.num_seqs
    e = 1 if fp8_pools is not None else W.ELEM_BYTES[wl.dtype]
    seq_bytes = wl.seq_lens.astype(np.int64) * wl.num_kv_heads * wl.head_size * 2 * e
    refs = {}

    # pool leg: whole passes over the batch (sequences longest first, so the pass ends evenly)
    order = [int(s) for s in np.argsort(-wl.seq_lens, kind="stable")]
    passes, t0 = 0, time.perf_counter()
    with mp.get_context("fork").Pool(cores, initializer=_oracle_init) as pool:
        while passes == 0 or (time.perf_counter() - t0 < seconds and passes < 64):
            for s, ref, _ in pool.imap_unordered(_oracle_seq, order, chunksize=1):
                refs.setdefault(s, ref)
            passes += 1
    pool_s = time.perf_counter() - t0
    pool_bytes = passes * int(seq_bytes.sum())

    # one-core leg: sequences in order, in this process
    done, el = 0, 0.0
    with threadpool_limits(1):
        while el < seconds and done < 64 * S:
            _, _, dt = _oracle_seq(done % S)
            el += dt
            done += 1
    one_bytes = int(sum(int(seq_bytes[i % S]) for i in range(done)))

    # the tiny MHA batch, whole, on one core
    tiny = W.make_config(1, 0, poison=False)
    with threadpool_limits(1):
        t1 = time.perf_counter()
        oracle.paged_decode_ref(W.raw_numpy(tiny.query), W.raw_numpy(tiny.k_cache), W.raw_numpy(tiny.v_cache),
                                tiny.block_tables, tiny.seq_lens, tiny.scale, tiny.dtype)
        tiny_s = time.perf_counter() - t1
    rec = {
        "value": round(pool_bytes / pool_s / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{passes} whole passes over all {S} sequences of the same workload ({pool_bytes} KV bytes), "
                  f"float64 NumPy, {cores} processes x 1 BLAS thread, {pool_s:.2f} s wall",
        "one_core": {"value": round(one_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                     "sample": f"{done} sequences walked in order ({one_bytes} KV bytes), one thread, {el:.2f} s"},
        "tiny_mha_one_core_us": round(tiny_s * 1e6, 1),
    }
    return rec, refs


def timed_steps(step, stream, K: int, warmup: int, flush_iters: int, device):
    """W untimed steps; K steps back to back between two synchronisations
    (wall clock, and one pair of HIP events on ``stream`` for the mean launch
    time); then ``flush_iters`` steps each after an untimed 512 MiB write,
    each bracketed by its own pair of events on ``stream``."""
    import numpy as np
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(K):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = ev0.elapsed_time(ev1) / K
    flushed = []
    if flush_iters > 0:
        scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=device)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(flush_iters)]
        with torch.cuda.stream(stream):
            for i, (a, b) in enumerate(evs):
                scratch.fill_(i & 255)
                a.record(stream)
                step()
                b.record(stream)
        torch.cuda.synchronize()
        flushed = [a.elapsed_time(b) for a, b in evs]
        del scratch
    dist = None
    if flushed:
        p10, p50, p90 = (float(x) * 1e3 for x in np.percentile(flushed, [10, 50, 90]))
        dist = {"p10": round(p10, 2), "p50": round(p50, 2), "p90": round(p90, 2), "n": len(flushed),
                "flush_bytes": FLUSH_BYTES}
    return wall, mean_ms, dist


COPY_PAIRS, COPY_POOL = 4096, 25000
FP8_K_SCALE, FP8_V_SCALE = 1.0 / 128, 1.0 / 96


def bench_copy_blocks(args):
    """copy_blocks on the 8B workload's pool layout: 4096 (shared, fresh)
    pairs of bf16 blocks (16 tokens x 8 kv heads x 128 = 32 KiB per cache)."""
    import numpy as np
    import torch

    import paged_kv_cache_291_amd as P

    NB, BS, Hkv, D = COPY_POOL, 16, 8, 128
    dev = torch.device("cuda:0")
    kc = torch.zeros((NB, BS, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    ids = np.random.default_rng(np.random.SeedSequence([291, 300, args.seed])).permutation(NB)
    src = torch.from_numpy(ids[:COPY_PAIRS].astype(np.int32)).to(dev)
    dst = torch.from_numpy(ids[COPY_PAIRS:2 * COPY_PAIRS].astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        P.copy_blocks(kc, vc, src, dst, stream=stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    K = args.steps
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(K):
        P.copy_blocks(kc, vc, src, dst, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = ev0.elapsed_time(ev1) / K / 1e3
    block_bytes = BS * Hkv * D * 2
    moved = COPY_PAIRS * 2 * 2 * block_bytes          # K and V blocks, read and written
    rec = {
        "metric": "copy_blocks: GB/s moved (read + write) per call",
        "value": round(moved / (wall / K) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"copy-on-write copies: {COPY_PAIRS} block pairs of a {NB}-block pool, "
                               "16 tokens x 8 kv heads x 128 bf16 per block and cache",
                   "pairs": COPY_PAIRS, "block_bytes_per_cache": block_bytes},
        "roofline": {"bound": "hbm", "achieved": round(moved / launch_s / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(moved / launch_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_copy_blocks_kernel", "bytes_per_launch": moved},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from paged_kv_cache_291_amd import workloads as W
        nb, pairs = 1200, 512
        k = W.raw_numpy(torch.zeros((nb, BS, Hkv, D), dtype=torch.bfloat16))
        v = k.copy()
        sample_ids = np.random.default_rng(1).permutation(nb)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or reps == 0:
            oracle.copy_blocks_ref(k, v, sample_ids[:pairs], sample_ids[pairs:2 * pairs])
            reps += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(reps * pairs * 2 * 2 * block_bytes / el / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} calls of {pairs} pairs on a {nb}-block pool of the same block "
                                         f"shape, NumPy, {el:.2f} s"}
    return rec


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(args):
    """Multi-token causal queries: speculative verification (memory-bound) or
    a chunked prefill (matrix-core bound)."""
    import numpy as np
    import torch

    import paged_kv_cache_291_amd as P
    from paged_kv_cache_291_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.prefill_case == "verify":
        wl = W.make_config(3, args.seed, poison=False)
        nq = np.full(wl.num_seqs, args.query_tokens, dtype=np.int32)
        desc = (f"speculative verification on the 8B-shaped GQA batch: 256 seqs, {args.query_tokens} query tokens each "
                "(32/8 heads, D=128, bf16)")
    else:
        S, L, n = 8, 4096, 512
        wl = W.make_random(args.seed, S, 32, 8, 128, "bf16", [L] * S, poison=False)
        nq = np.full(S, n, dtype=np.int32)
        desc = "chunked prefill: 8 seqs x (3584 cached + 512 new tokens), 32/8 heads, D=128, bf16"
    starts = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T = int(starts[-1])
    q = W.random_rows(args.seed, 500, (T, wl.num_heads, wl.head_size), wl.dtype).to(dev)
    kc, vc = wl.k_cache.to(dev), wl.v_cache.to(dev)
    bt, sl = torch.from_numpy(wl.block_tables).to(dev), torch.from_numpy(wl.seq_lens).to(dev)
    qs = torch.from_numpy(starts).to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    mq = int(nq.max())
    # the library's path: the balanced split for one 16-row tile per kv head, and
    # for two while the batch has fewer than 32 sequences or 1024 (sequence, kv
    # head) pairs; else the many-tile LDS kernel (longest first from 32 sequences)
    rows = mq * (wl.num_heads // wl.num_kv_heads)
    split = rows <= 16 or (rows <= 32 and not (wl.num_seqs >= 32 and wl.num_seqs * wl.num_kv_heads >= 1024))

    def step():
        P.paged_attention_prefill(out, q, kc, vc, bt, sl, qs, wl.scale, max_query_len=mq, stream=stream)

    K = args.steps
    wall, mean_ms, dist = timed_steps(step, stream, K, args.warmup, args.flush_iters, dev)
    wall /= K
    launch = mean_ms / 1e3
    D, Hq = wl.head_size, wl.num_heads
    # (query row, visible key) pairs: row i of n sees L - n + i + 1 keys
    pairs = int(sum(int(n) * (int(L) - int(n)) + int(n) * (int(n) + 1) // 2 for n, L in zip(nq, wl.seq_lens)))
    flops = 4.0 * D * Hq * pairs
    kv = wl.kv_bytes()
    rec = {
        "metric": "paged multi-token causal attention: " + ("KV GB/s" if args.prefill_case == "verify" else "TFLOP/s"),
        "value": round(kv / wall / 1e9, 2) if args.prefill_case == "verify" else round(flops / wall / 1e12, 2),
        "unit": "GB/s" if args.prefill_case == "verify" else "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": desc, "query_tokens": T, "kv_bytes": kv, "flops": flops},
        "us_per_step": round(wall * 1e6, 2), "us_per_step_flushed": dist, "launch_us": round(launch * 1e6, 2),
        "roofline": ({"bound": "hbm", "achieved": round(kv / launch / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(kv / launch / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                      "kernel": ("pa_decode_sk_kernel(multi-token rows)+pa_sk_merge_mq_kernel" if split else
                                 "pa_prefill_lds_kernel" + ("+pa_order_by_length_kernel" if wl.num_seqs >= 32 else "")),
                      "bytes_per_launch": kv}
                     if args.prefill_case == "verify" else
                     {"bound": "mfma", "achieved": round(flops / launch / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(flops / launch / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                      "traffic": None, "kernel": "pa_prefill_lds_kernel", "flops_per_launch": flops}),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        qr, kr, vr = W.raw_numpy(q.cpu()), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache)
        done, el, work = 0, 0.0, 0.0
        with threadpool_limits(1):
            while done < wl.num_seqs and (el < min(args.cpu_seconds, 20.0) or done == 0):
                t1 = time.perf_counter()
                oracle.paged_prefill_ref(qr, kr, vr, wl.block_tables, wl.seq_lens, starts, wl.scale, wl.dtype,
                                         seqs=[done])
                el += time.perf_counter() - t1
                n_, L_ = int(nq[done]), int(wl.seq_lens[done])
                work += (L_ * wl.num_kv_heads * D * 2 * 2 if args.prefill_case == "verify"
                         else 4.0 * D * Hq * (n_ * (L_ - n_) + n_ * (n_ + 1) // 2))
                done += 1
        rec["cpu_baseline"] = {"value": round(work / el / (1e9 if args.prefill_case == "verify" else 1e12), 5),
                               "unit": rec["unit"], "cores": 1, "kind": "oracle",
                               "sample": f"first {done} of {wl.num_seqs} sequences, float64 NumPy, {el:.2f} s"}
    return rec


def bench_block_manager(args):
    """Host block manager building decode steps of a 256-sequence batch."""
    import numpy as np

    import paged_kv_cache_291_amd as P

    S, NB, BS, MB = 256, 40000, 16, 512
    rng = np.random.default_rng(np.random.SeedSequence([291, 301, args.seed]))

    def prompt_len():
        return int(np.clip(np.round(1024 * np.exp(rng.standard_normal())), 16, 4096))

    # the same trace for the native manager and the oracle: a list of steps
    K = args.steps
    trace = []
    next_id = S
    live = list(range(S))
    init = [(s, prompt_len()) for s in live]
    for k in range(K):
        ev = []
        if k % 16 == 15:                                   # 8 finish, 4 new prompts and 4 beams
            for _ in range(8):
                ev.append(("free", live.pop(int(rng.integers(len(live))))))
            for j in range(8):
                if j < 4:
                    ev.append(("allocate", next_id, prompt_len()))
                else:
                    ev.append(("fork", live[int(rng.integers(len(live)))], next_id))
                live.append(next_id)
                next_id = (next_id + 1) % 2048
                while next_id in live:
                    next_id = (next_id + 1) % 2048
        trace.append((ev, list(live)))

    def run(mgr_new, allocate, append, fork, free, take, tables, steps):
        m = mgr_new()
        for s, n in init:
            allocate(m, s, n)
        t0 = time.perf_counter()
        for ev, batch in trace[:steps]:
            for e in ev:
                if e[0] == "free":
                    free(m, e[1])
                elif e[0] == "allocate":
                    allocate(m, e[1], e[2])
                else:
                    fork(m, e[1], e[2])
            append(m, batch)
            take(m)
            tables(m, batch)
        return time.perf_counter() - t0

    el = run(lambda: P.BlockManager(NB, BS, 2048, MB), lambda m, s, n: m.allocate(s, n),
             lambda m, b: m.append_batch(b), lambda m, p, c: m.fork(p, c), lambda m, s: m.free(s),
             lambda m: m.take_copies(), lambda m, b: m.block_tables(b), K)
    us = el / K * 1e6
    rec = {
        "metric": "block manager: host us to build one decode step (appends, copy queue, tables)",
        "value": round(us, 2), "unit": "us/step", "n_gpus": 0, "steps": K, "warmup": 0,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": "serving trace at the 8B batch's scale: 256 live sequences with lognormal "
                               "prompts (median 1024), one token appended to each per step, every 16 steps "
                               "8 finish and 4 new prompts + 4 forks arrive; 40000-block pool"},
        "roofline": None,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        n = min(K, 64)
        el_ref = run(lambda: oracle.BlockManagerRef(NB, BS, 2048, MB), lambda m, s, n_: m.allocate(s, n_),
                     lambda m, b: m.append_batch(b), lambda m, p, c: m.fork(p, c), lambda m, s: m.free_seq(s),
                     lambda m: m.take_copies(), lambda m, b: m.block_tables(b), n)
        rec["cpu_baseline"] = {"value": round(el_ref / n * 1e6, 2), "unit": "us/step", "cores": 1,
                               "kind": "oracle", "sample": f"first {n} steps of the same trace, pure Python"}
    return rec


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, ROOT)
    import paged_kv_cache_291_amd as P

    if args.op == "block_manager":
        print(json.dumps(bench_block_manager(args)))
        return
    if args.op == "decode":
        print(json.dumps(bench_decode(args)), flush=True)
        return
    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    P.load_library()
    if args.op == "copy_blocks":
        print(json.dumps(bench_copy_blocks(args)))
        return
    if args.op == "prefill":
        print(json.dumps(bench_prefill(args)))
        return


WORKLOADS = {1: "tiny MHA paged decode (4 seqs, 8/8 heads, D=64, fp32)",
             2: "13B-shaped MHA paged decode (64 seqs, 40/40 heads, D=128, fp16)",
             3: "8B-shaped GQA paged decode (256 seqs, 32/8 heads, D=128, bf16)",
             4: "long-context GQA paged decode (8 seqs x 32768, 64/8 heads, D=128, bf16)",
             5: "shared-prefix GQA paged decode (128 seqs, 1024-token shared prefix, 32/8 heads, bf16)"}


def bench_decode(args):
    import numpy as np
    import torch

    import paged_kv_cache_291_amd as P
    from paged_kv_cache_291_amd import workloads as W

    cfg = args.config
    ps = DEFAULT_PARTITION[cfg] if args.partition < 0 else args.partition
    flags = DEFAULT_FLAGS.get(cfg, 0) if args.flags < 0 else args.flags
    fp8 = args.kv == "fp8"
    t0 = time.time()
    wl = W.make_config(cfg, args.seed, poison=False)
    if fp8 and wl.dtype == "f32":
        print("fp8 pools need a bf16 or fp16 query", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] workload cfg{cfg} generated in {time.time() - t0:.1f}s: S={wl.num_seqs} "
          f"tokens={int(wl.seq_lens.sum())} kv_bytes={wl.kv_bytes()}", file=sys.stderr, flush=True)
    kc_host, vc_host = wl.k_cache, wl.v_cache
    if fp8:
        kc_host = W.random_fp8_codes(1000 + args.seed, tuple(wl.k_cache.shape))
        vc_host = W.random_fp8_codes(1001 + args.seed, tuple(wl.v_cache.shape))

    # the oracle legs run first: the pool forks this process, which must not have touched the GPU yet
    cb, refs = None, {}
    if not args.no_cpu_baseline:
        cores = host_cores(args.cpu_cores)
        print(f"[bench] oracle on {cores} host cores ({args.cpu_seconds:.0f} s per leg)", file=sys.stderr,
              flush=True)
        cb, refs = cpu_baseline(wl, args.cpu_seconds, cores, (kc_host, vc_host) if fp8 else None)

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    P.load_library()
    dev = torch.device("cuda:0")
    q = wl.query.to(dev)
    kc, vc = kc_host.to(dev), vc_host.to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    out = torch.empty_like(q)
    ws = None
    need = P.decode_workspace_bytes(q, bt, wl.block_size, ps, wl.max_seq_len)
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    scatter_us = None
    if wl.slot_mapping is not None:
        nk, nv = wl.new_key.to(dev), wl.new_value.to(dev)
        sm = torch.from_numpy(wl.slot_mapping).to(dev)
        scatter = (lambda: P.reshape_and_cache_fp8(nk, nv, kc, vc, sm, FP8_K_SCALE, FP8_V_SCALE, stream=stream)
                   ) if fp8 else (lambda: P.reshape_and_cache(nk, nv, kc, vc, sm, stream=stream))
        _, sc_ms, _ = timed_steps(scatter, stream, 100, 10, 0, dev)   # idempotent: the same rows each time
        scatter_us = round(sc_ms * 1e3, 2)

    def decode(stream_):
        if fp8:
            P.paged_attention_decode_fp8(out, q, kc, vc, bt, sl, wl.scale, FP8_K_SCALE, FP8_V_SCALE,
                                         partition_size=ps, max_seq_len=wl.max_seq_len, workspace=ws, flags=flags,
                                         stream=stream_)
        else:
            P.paged_attention_decode(out, q, kc, vc, bt, sl, wl.scale, partition_size=ps,
                                     max_seq_len=wl.max_seq_len, workspace=ws, flags=flags, stream=stream_)

    step = lambda: decode(stream)                      # noqa: E731
    calls = 1
    if args.graph:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):                  # launches go to the capturing stream
            for _ in range(args.graph_calls):
                decode(None)
        stream = torch.cuda.current_stream()
        step = graph.replay
        calls = args.graph_calls                       # decode calls per timed replay
    K = args.steps
    wall, mean_ms, dist = timed_steps(step, stream, K, args.warmup, args.flush_iters, dev)
    wall /= calls
    mean_ms /= calls
    if dist is not None and calls > 1:
        dist = {k: (round(v / calls, 2) if k.startswith("p") else v) for k, v in dist.items()}

    e = 1 if fp8 else W.ELEM_BYTES[wl.dtype]
    kv = wl.kv_bytes() // W.ELEM_BYTES[wl.dtype] * e
    kv_unique = wl.kv_bytes_unique() // W.ELEM_BYTES[wl.dtype] * e
    shared = kv_unique < kv                            # blocks named by several sequences
    roof_bytes = kv_unique if shared else kv
    ms_per_step = wall * 1e3 / K
    value = kv / (wall / K) / 1e9
    achieved = roof_bytes / (mean_ms / 1e3) / 1e9
    # the launch the library picks: the vector-ALU core for fp32, and with one
    # query head per kv head (with partitions, or from 1024 (sequence, kv
    # head) pairs; over fp8 pools then cut into partitions by the library)
    mha = wl.num_heads == wl.num_kv_heads and (ps > 0 or wl.num_seqs * wl.num_kv_heads >= 1024)
    if wl.dtype == "f32":
        kernel = "pa_decode_valu_kernel" + ("+pa_reduce_kernel" if ps > 0 else "")
    elif mha and fp8:                                  # fed from the work queue, partitions merged
        kernel = "pa_decode_valu_kernel+pa_reduce_kernel+pa_queue_reset_kernel"
    elif mha:                                          # partitions merged, or longest sequence first
        kernel = "pa_decode_valu_kernel+" + ("pa_reduce_kernel" if ps > 0 else "pa_order_by_length_kernel")
    else:
        kernel = "pa_decode_mfma_kernel+pa_reduce_kernel" if ps > 0 else "pa_decode_sk_kernel+pa_sk_merge_kernel"
    if fp8:
        kernel += "|fp8"
    traffic = traffic_for(kernel, f"cfg{cfg}")            # measured HBM bytes per step, if taken on these sources
    out_host = out.cpu().double().numpy()
    err = None
    if refs:
        err = max(float(np.max(np.abs(out_host[s] - r))) for s, r in refs.items())
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype + ("/e4m3 KV" if fp8 else ""),
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[cfg] + (", over e4m3 (fp8) K/V pools" if fp8 else ""),
            "num_seqs": wl.num_seqs, "num_heads": wl.num_heads, "num_kv_heads": wl.num_kv_heads,
            "head_size": wl.head_size, "block_size": wl.block_size, "num_blocks": wl.num_blocks,
            "total_tokens": int(wl.seq_lens.sum()), "max_seq_len": wl.max_seq_len,
            "partition_size": ps, "flags": flags, "seed": args.seed, "parallelism": "none (1 GPU)",
            "launch": f"HIP graph replay, {args.graph_calls} calls per graph" if args.graph else "eager",
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_flushed": dist,
        "kv_bytes_per_step": kv,
        "kv_bytes_unique": kv_unique,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "launch_us": round(mean_ms * 1e3, 2),
        "scatter_us": scatter_us,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_flushed_p50": (round(roof_bytes / (dist["p50"] / 1e6) / 1e9 / HBM_PEAK_GBS, 4)
                                 if dist else None),
            "traffic": traffic,
            "frac_traffic": round(traffic / (mean_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4) if traffic else None,
            "kernel": kernel,
            "bytes_per_launch": roof_bytes,
            "bytes": "unique K/V rows (a shared block counts once)" if shared else "K/V rows of the valid tokens",
        },
        "cpu_baseline": cb,
        "max_abs_err_vs_oracle": err,
    }
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n
    return rec


if __name__ == "__main__":
    main()
