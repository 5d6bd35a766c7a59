#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = one ``paged_attention_decode`` call over the whole batch (for the
split path: the partition kernel plus the log-sum-exp reduce), with the
inputs already resident in HBM.  Prints ONE JSON line:

  value        KV GB/s = (bytes of K and V of the valid tokens) / (wall time per step)
  ms_per_step  wall time per step between two device synchronisations
  roofline     the decode launch: algorithmic KV bytes / its mean duration from
               HIP events on the launch stream, against 8000 GB/s HBM3E peak
  cpu_baseline the float64 oracle, single thread, on a bounded sample of the
               same workload (first sequences, ~10 s of CPU work)

Workload (default): 8B-shaped GQA decode batch, 256 sequences, 32 query / 8
kv heads, head_size 128, bf16, block_size 16, lognormal lengths (median 1024,
sigma 1, clipped to [16, 4096]), shuffled block pool.  Synthetic N(0, 1) data.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention: KV GB/s and % of HBM peak; us per decode step"
# partition size the timed launch uses per workload (0 = the library's balanced split)
DEFAULT_PARTITION = {1: 0, 2: 0, 3: 0, 4: 0, 5: 0}
# the shared-prefix workload names the same blocks from many sequences
DEFAULT_FLAGS = {5: 1}
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_291_amd", "csrc", "pagedattn.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--partition", type=int, default=-1, help="tokens per partition; -1 = workload default")
    ap.add_argument("--flags", type=int, default=-1, help="decode flags (1 = shared blocks); -1 = workload default")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def traffic_for(kernel_name: str, workload: str):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel_name}|{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, seconds: float, gpu_out):
    """Time the oracle (single thread) on the first sequences of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from paged_kv_cache_291_amd import workloads as W

    q, kc, vc = W.raw_numpy(wl.query), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache)
    done, tok, elapsed, err = 0, 0, 0.0, 0.0
    with threadpool_limits(1):
        while done < wl.num_seqs and elapsed < seconds:
            t0 = time.perf_counter()
            ref = oracle.paged_decode_ref(q, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, wl.dtype,
                                          seqs=[done])
            elapsed += time.perf_counter() - t0
            g = gpu_out[done].double().numpy()
            err = max(err, float(np.max(np.abs(g - ref[0]))))
            tok += int(wl.seq_lens[done])
            done += 1
    kv = tok * wl.num_kv_heads * wl.head_size * 2 * W.ELEM_BYTES[wl.dtype]
    return {
        "value": round(kv / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {done} of {wl.num_seqs} sequences ({tok} tokens, {kv} KV bytes) of the same "
                  f"workload, float64 NumPy, one thread, {elapsed:.2f} s",
    }, err


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the sharding design is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import paged_kv_cache_291_amd as P
    from paged_kv_cache_291_amd import workloads as W

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    P.load_library()
    cfg = args.config
    ps = DEFAULT_PARTITION[cfg] if args.partition < 0 else args.partition
    flags = DEFAULT_FLAGS.get(cfg, 0) if args.flags < 0 else args.flags

    t0 = time.time()
    wl = W.make_config(cfg, args.seed, poison=False)
    print(f"[bench] workload cfg{cfg} generated in {time.time() - t0:.1f}s: S={wl.num_seqs} "
          f"tokens={int(wl.seq_lens.sum())} kv_bytes={wl.kv_bytes()}", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    q = wl.query.to(dev)
    kc, vc = wl.k_cache.to(dev), wl.v_cache.to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    out = torch.empty_like(q)
    ws = None
    need = P.decode_workspace_bytes(q, bt, wl.block_size, ps, wl.max_seq_len)
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if wl.slot_mapping is not None:
        P.reshape_and_cache(wl.new_key.to(dev), wl.new_value.to(dev), kc, vc,
                            torch.from_numpy(wl.slot_mapping).to(dev))
    stream = torch.cuda.current_stream()

    def step():
        P.paged_attention_decode(out, q, kc, vc, bt, sl, wl.scale, partition_size=ps,
                                 max_seq_len=wl.max_seq_len, workspace=ws, flags=flags, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        evs[k][0].record(stream)
        step()
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    launch_ms = np.array([a.elapsed_time(b) for a, b in evs])

    kv = wl.kv_bytes()
    ms_per_step = wall * 1e3 / K
    value = kv / (wall / K) / 1e9
    mean_launch_s = float(launch_ms.mean()) / 1e3
    achieved = kv / mean_launch_s / 1e9
    workload = {1: "tiny MHA paged decode (4 seqs, 8/8 heads, D=64, fp32)",
                2: "13B-shaped MHA paged decode (64 seqs, 40/40 heads, D=128, fp16)",
                3: "8B-shaped GQA paged decode (256 seqs, 32/8 heads, D=128, bf16)",
                4: "long-context GQA paged decode (8 seqs x 32768, 64/8 heads, D=128, bf16)",
                5: "shared-prefix GQA paged decode (128 seqs, 1024-token shared prefix, 32/8 heads, bf16)"}[cfg]
    if wl.dtype == "f32":
        kernel = "pa_decode_valu_kernel" + ("+pa_reduce_kernel" if ps > 0 else "")
    else:
        kernel = "pa_decode_mfma_kernel+pa_reduce_kernel" if ps > 0 else "pa_decode_sk_kernel+pa_sk_merge_kernel"
    out_host = out.cpu()
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
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload,
            "num_seqs": wl.num_seqs, "num_heads": wl.num_heads, "num_kv_heads": wl.num_kv_heads,
            "head_size": wl.head_size, "block_size": wl.block_size, "num_blocks": wl.num_blocks,
            "total_tokens": int(wl.seq_lens.sum()), "max_seq_len": wl.max_seq_len,
            "partition_size": ps, "flags": flags, "seed": args.seed, "parallelism": "none (1 GPU)",
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "kv_bytes_per_step": kv,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "launch_us": {"mean": round(float(launch_ms.mean()) * 1e3, 2),
                      "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(launch_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(kernel, f"cfg{cfg}"),
            "kernel": kernel,
            "bytes_per_launch": kv,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cb, err = cpu_baseline(wl, args.cpu_seconds, out_host)
        rec["cpu_baseline"] = cb
        rec["max_abs_err_vs_oracle_on_cpu_sample"] = err
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
