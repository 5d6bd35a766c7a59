"""The online-softmax rescale with a live running state, on every
matrix-core path, against the float64 oracle element by element.

devpress.csdn.net vLLM architecture article, section 3, part 2 step 4: the
attention over the gathered blocks may be fused FlashAttention-style, i.e.
computed as an online softmax whose running maximum, sum and accumulator are
rescaled whenever a new maximum arrives.  The kernels rescale lazily (only
when a step's maximum beats the reference by more than 8 in base 2), which
N(0, 1) data never triggers after a segment's first block.  These batches
plant score spikes and climbs (``rescale_cases``), assert from the inputs
alone that the rescale of a state holding keys is reached (and on rows in
both halves of the 16-row tile, so the per-row factor transpose matters),
then compare every output element with the oracle at the plain max-abs
bound: 1e-2 for bf16 outputs, 2e-3 for fp16 (values are N(0, 1/16), so the
final rounding stays far inside it).

Paths: decode through the balanced split and a fixed 512-token split;
multi-token rows through the balanced split with one and two tiles per
kv-head wave, the many-tile LDS kernel, and, past the split's sequence limit, the
one-wave-per-tile kernel and the LDS kernel with two tiles; 16-bit and fp8
pools; a large positive and a large negative score scale.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_291_amd as P
from paged_kv_cache_291_amd import workloads as W

import rescale_cases as RC
from helpers import TOL

pytestmark = pytest.mark.gpu

DECODE_SHAPES = [(32, 8, 128), (16, 2, 128), (8, 8, 64), (16, 8, 64)]
KINDS = ["bf16", "f16", "e4m3"]


def _dtype_of(kv):
    return "bf16" if kv == "e4m3" else kv


def _decode_lens(seed, S=40):
    rng = np.random.default_rng(seed)
    return rng.integers(900, 2600, size=S)


def _run_decode(case, ps):
    wl, pools = case.wl, case.pools
    dev = "cuda"
    q = case.query.to(dev)
    out = torch.empty_like(q)
    args = (out, q, pools.k.to(dev), pools.v.to(dev), torch.from_numpy(wl.block_tables).to(dev),
            torch.from_numpy(wl.seq_lens).to(dev), wl.scale)
    if pools.kind == "e4m3":
        P.paged_attention_decode_fp8(*args, pools.k_scale, pools.v_scale, partition_size=ps,
                                     max_seq_len=wl.max_seq_len)
    else:
        P.paged_attention_decode(*args, partition_size=ps, max_seq_len=wl.max_seq_len)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def _oracle_decode(case):
    wl, pools = case.wl, case.pools
    kw = dict(kv_dtype="e4m3", k_scale=pools.k_scale, v_scale=pools.v_scale) if pools.kind == "e4m3" else {}
    return oracle.paged_decode_ref(W.raw_numpy(case.query), W.raw_numpy(pools.k), W.raw_numpy(pools.v),
                                   wl.block_tables, wl.seq_lens, wl.scale, wl.dtype, **kw)


def _check(g, ref, dtype, what):
    diff = np.abs(g - ref)
    worst = float(diff.max()) if diff.size else 0.0
    print(f"  {what}: max-abs {worst:.3e} (bound {TOL[dtype]})", flush=True)
    assert np.isfinite(g).all(), what
    assert worst <= TOL[dtype], what


@pytest.mark.parametrize("kv", KINDS)
@pytest.mark.parametrize("Hq,Hkv,D", DECODE_SHAPES)
def test_decode_rescale(Hq, Hkv, D, kv):
    seed = 1000 + Hq + 3 * Hkv + D + KINDS.index(kv)
    lens = _decode_lens(seed)
    case = RC.make_case(seed, lens, np.ones(len(lens)), Hq, Hkv, D, _dtype_of(kv), kv)
    nblk = RC.valid_blocks(case.wl.seq_lens, case.wl.max_blocks_per_seq)
    ref = _oracle_decode(case)
    G = Hq // Hkv
    for ps, segs in ((0, RC.balanced_segments(nblk, Hkv)), (512, RC.fixed_segments(nblk, 512))):
        ev, rows, amb = RC.events_over(case, segs)
        print(f"decode {kv} {Hq}/{Hkv} D={D} ps={ps}: {ev} rescales of live states on rows {sorted(rows)}, "
              f"{amb} ambiguous replays", flush=True)
        assert ev >= 100 and len(rows) == G and rows <= set(range(G))
        _check(_run_decode(case, ps), ref, case.wl.dtype, f"ps={ps}")


def test_decode_rescale_large_scale():
    """A score scale of 4 on N(0, 1/16) keys: scores spread over tens of
    base-2 units and block maxima overtake the reference often."""
    lens = _decode_lens(77)
    case = RC.make_case(77, lens, np.ones(len(lens)), 32, 8, 128, "bf16", "bf16", plant_seqs=[], scale=4.0)
    case.plans = {(s, kvh): None for s in range(len(lens)) for kvh in range(8)}
    nblk = RC.valid_blocks(case.wl.seq_lens, case.wl.max_blocks_per_seq)
    ev, rows, _ = RC.events_over(case, RC.balanced_segments(nblk, 8))
    print(f"decode scale 4: {ev} rescales of live states on rows {sorted(rows)}", flush=True)
    assert ev >= 100 and rows == {0, 1, 2, 3}
    _check(_run_decode(case, 0), _oracle_decode(case), "bf16", "scale 4, ps=0")


# ---- multi-token rows

def _run_prefill(case, max_q):
    wl, pools = case.wl, case.pools
    dev = "cuda"
    q = case.query.to(dev)
    out = torch.empty_like(q)
    kw = dict(k_scale=pools.k_scale, v_scale=pools.v_scale) if pools.kind == "e4m3" else {}
    P.paged_attention_prefill(out, q, pools.k.to(dev), pools.v.to(dev), torch.from_numpy(wl.block_tables).to(dev),
                              torch.from_numpy(wl.seq_lens).to(dev), torch.from_numpy(case.starts).to(dev),
                              wl.scale, max_query_len=max_q, **kw)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def _oracle_prefill(case):
    wl, pools = case.wl, case.pools
    kw = dict(kv_dtype="e4m3", k_scale=pools.k_scale, v_scale=pools.v_scale) if pools.kind == "e4m3" else {}
    return oracle.paged_prefill_ref(W.raw_numpy(case.query), W.raw_numpy(pools.k), W.raw_numpy(pools.v),
                                    wl.block_tables, wl.seq_lens, case.starts, wl.scale, wl.dtype, **kw)


# path: (Hq, Hkv, D, query rows per sequence (lo, hi), sequences, big batch)
MQ_PATHS = {
    "split-1tile": (32, 8, 128, (1, 4), 40, False),
    "split-1tile-G8": (16, 2, 128, (1, 2), 40, False),
    "split-2tiles": (32, 8, 128, (5, 8), 40, False),
    "lds": (32, 8, 128, (20, 64), 12, False),
    "lds-G8": (16, 2, 64, (10, 40), 12, False),
    "wave-per-tile": (8, 2, 64, (1, 4), 16, True),
    "lds-2tiles-big-batch": (8, 2, 64, (5, 8), 16, True),
}
BIG_SHORT = 16384                     # short sequences added past the split's limit


def _mq_case(path, kv, scale=None):
    Hq, Hkv, D, (lo, hi), S, big = MQ_PATHS[path]
    seed = 2000 + sorted(MQ_PATHS).index(path) * 7 + KINDS.index(kv)
    rng = np.random.default_rng(seed)
    lens = rng.integers(700, 2000, size=S)
    nq = rng.integers(lo, hi + 1, size=S)
    nq[0] = hi
    plant_seqs = list(range(S))
    if big:
        lens = np.concatenate([lens, 1 + np.arange(BIG_SHORT) % 3])
        nq = np.concatenate([nq, np.ones(BIG_SHORT, dtype=nq.dtype)])
    case = RC.make_case(seed, lens, nq, Hq, Hkv, D, _dtype_of(kv), kv, plant_seqs=plant_seqs, scale=scale)
    return case, int(nq.max())


def _mq_events(path, case, max_q):
    wl = case.wl
    Hq, Hkv = wl.num_heads, wl.num_kv_heads
    G = Hq // Hkv
    starts = case.starts
    nq_of = lambda s: int(starts[s + 1] - starts[s])          # noqa: E731
    tiles = -(-max_q * G // 16)
    if path.startswith("split"):
        nblk = RC.valid_blocks(wl.seq_lens, wl.max_blocks_per_seq)
        segs = RC.balanced_segments(nblk, Hkv, tiles, wl.head_size)
        return RC.events_over(case, segs, 1, lambda s: [16 * t // G for t in range(tiles)])
    tpt = 16 // G
    waves = lambda s: list(range(0, nq_of(s), tpt))            # noqa: E731
    unit = 1 if path == "wave-per-tile" else 2
    return RC.events_over(case, None, unit, waves)


@pytest.mark.parametrize("kv", KINDS)
@pytest.mark.parametrize("path", list(MQ_PATHS))
def test_multi_token_rescale(path, kv):
    case, max_q = _mq_case(path, kv)
    ev, rows, amb = _mq_events(path, case, max_q)
    print(f"{path} {kv}: {ev} rescales of live states on rows {sorted(rows)}, {amb} ambiguous replays", flush=True)
    assert ev >= 100
    assert any(r < 4 for r in rows) and any(r >= 4 for r in rows)
    g = _run_prefill(case, max_q)
    _check(g, _oracle_prefill(case), case.wl.dtype, path)


@pytest.mark.parametrize("scale", [4.0, -4.0])
@pytest.mark.parametrize("path", ["split-1tile", "lds"])
def test_multi_token_rescale_large_scale(path, scale):
    """Planted jumps plus a large score scale of either sign (the many-tile
    kernel moves a negative scale's sign into the query)."""
    case, max_q = _mq_case(path, "bf16", scale=scale)
    ev, rows, _ = _mq_events(path, case, max_q)
    print(f"{path} scale {scale}: {ev} rescales of live states on rows {sorted(rows)}", flush=True)
    assert ev >= 100
    _check(_run_prefill(case, max_q), _oracle_prefill(case), "bf16", f"{path} scale {scale}")
