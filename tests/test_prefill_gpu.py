"""Multi-token causal queries over the paged cache on the GPU against the
float64 oracle: edge lengths and query counts (n = 1 is decode, n = L is a
whole prompt), every head size, group size and type, fp8 pools, contract
violations, and the chunked-prefill and verification batches at full size
checked on every row."""

from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_291_amd as P
from paged_kv_cache_291_amd import workloads as W
from helpers import assert_parity

pytestmark = pytest.mark.gpu

LENS = [1, 2, 16, 17, 40, 64, 100, 300, 513, 33, 7, 600]
NQ = [1, 2, 16, 5, 40, 3, 1, 33, 17, 0, 7, 64]


def _case(seed, Hq, Hkv, D, dtype, lens=LENS, nq=NQ):
    wl = W.make_random(seed, len(lens), Hq, Hkv, D, dtype, lens, extra_table_cols=1)
    starts = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = W.random_rows(seed, 99, (int(starts[-1]), Hq, D), dtype)
    return wl, starts, q


def _gpu(wl, starts, q, kc=None, vc=None, fp8=None, max_q=0, bt=None, sl=None, scale=None):
    out = torch.empty_like(q, device="cuda")
    kw = {} if fp8 is None else dict(k_scale=fp8[0], v_scale=fp8[1])
    P.paged_attention_prefill(out, q.cuda(), (kc if kc is not None else wl.k_cache).cuda(),
                              (vc if vc is not None else wl.v_cache).cuda(),
                              torch.from_numpy(wl.block_tables if bt is None else bt).cuda(),
                              torch.from_numpy(wl.seq_lens if sl is None else sl).cuda(),
                              torch.from_numpy(starts).cuda(), wl.scale if scale is None else scale,
                              max_query_len=max_q, **kw)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


SWEEP = [(dt, D, Hq, Hkv) for dt in ("bf16", "f16") for D in (64, 128) for (Hq, Hkv) in ((4, 4), (4, 2), (8, 2), (16, 2))]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", SWEEP)
def test_prefill_sweep(dtype, D, Hq, Hkv):
    seed = zlib.crc32(f"prefill-{dtype}-{D}-{Hq}-{Hkv}".encode()) % 10000
    wl, starts, q = _case(seed, Hq, Hkv, D, dtype)
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, dtype)
    for max_q in (0, max(NQ)):
        g = _gpu(wl, starts, q, max_q=max_q)
        assert_parity(g, ref, dtype, f"prefill {dtype} D={D} {Hq}/{Hkv} max_q={max_q}")


# Query counts around the many-tile kernel's unit of work (2 tiles per wave,
# 16 per workgroup): with G = 8 a tile is 2 tokens, so n = 8 is the smallest
# batch it takes (4 tiles), 32 fills one workgroup and 33 starts a second
# whose first wave has one token; cached prefixes from 0 to 101 tokens put the
# causal diagonal at many offsets inside a block pair.
LDS_LENS = [8, 10, 46, 48, 65, 33, 64, 165, 40, 31, 129, 200]
LDS_NQ = [8, 9, 31, 32, 33, 33, 63, 64, 24, 16, 65, 100]


@pytest.mark.parametrize("dtype,D,Hq,Hkv,fp8", [("bf16", 128, 16, 2, False), ("f16", 64, 16, 2, False),
                                                ("bf16", 128, 32, 8, True), ("f16", 64, 8, 1, True)])
def test_many_tile_kernel_edges(dtype, D, Hq, Hkv, fp8):
    seed = zlib.crc32(f"lds-{dtype}-{D}-{Hq}-{Hkv}-{fp8}".encode()) % 10000
    wl, starts, q = _case(seed, Hq, Hkv, D, dtype, LDS_LENS, LDS_NQ)
    if fp8:
        kc8, vc8 = W.with_fp8_pools(wl, seed)
        ks, vs = 1.0 / 128, 1.0 / 96
        g = _gpu(wl, starts, q, kc8, vc8, fp8=(ks, vs))
        ref = oracle.paged_prefill_ref(W.raw_numpy(q), kc8.numpy(), vc8.numpy(), wl.block_tables, wl.seq_lens,
                                       starts, wl.scale, dtype, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    else:
        g = _gpu(wl, starts, q)
        ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                       wl.block_tables, wl.seq_lens, starts, wl.scale, dtype)
    assert_parity(g, ref, dtype, f"many-tile {dtype} D={D} {Hq}/{Hkv} fp8={fp8}")


# At most 8 query tiles per (sequence, kv head): the many-tile kernel runs
# workgroups of 8 tiles (4 waves).  G = 8: 16 tokens fill them, G = 4: 32.
SMALL_LENS = [8, 10, 46, 48, 65, 33, 64, 165, 40, 31, 129, 200]
SMALL_NQ = {8: [5, 6, 9, 16, 16, 12, 7, 16, 3, 16, 11, 14], 4: [9, 12, 17, 32, 31, 24, 13, 32, 20, 16, 30, 28]}


@pytest.mark.parametrize("dtype,D,Hq,Hkv,fp8", [("bf16", 128, 16, 2, False), ("f16", 64, 16, 2, False),
                                                ("bf16", 128, 32, 8, False), ("bf16", 128, 32, 8, True)])
def test_small_group_kernel_edges(dtype, D, Hq, Hkv, fp8):
    G = Hq // Hkv
    nq = np.minimum(SMALL_NQ[G], SMALL_LENS).tolist()
    assert 2 < max(nq) * G / 16 <= 8
    seed = zlib.crc32(f"small-{dtype}-{D}-{Hq}-{Hkv}-{fp8}".encode()) % 10000
    wl, starts, q = _case(seed, Hq, Hkv, D, dtype, SMALL_LENS, nq)
    if fp8:
        kc8, vc8 = W.with_fp8_pools(wl, seed)
        ks, vs = 1.0 / 128, 1.0 / 96
        g = _gpu(wl, starts, q, kc8, vc8, fp8=(ks, vs))
        ref = oracle.paged_prefill_ref(W.raw_numpy(q), kc8.numpy(), vc8.numpy(), wl.block_tables, wl.seq_lens,
                                       starts, wl.scale, dtype, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    else:
        g = _gpu(wl, starts, q)
        ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                       wl.block_tables, wl.seq_lens, starts, wl.scale, dtype)
    assert_parity(g, ref, dtype, f"8-tile groups {dtype} D={D} {Hq}/{Hkv} fp8={fp8}")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8)])
def test_prefill_fp8_pools(Hq, Hkv):
    wl, starts, q = _case(600 + Hq, Hq, Hkv, 128, "bf16")
    kc8, vc8 = W.with_fp8_pools(wl, 61)
    ks, vs = 1.0 / 128, 1.0 / 96
    g = _gpu(wl, starts, q, kc8, vc8, fp8=(ks, vs))
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), kc8.numpy(), vc8.numpy(), wl.block_tables, wl.seq_lens, starts,
                                   wl.scale, "bf16", kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    assert_parity(g, ref, "bf16", f"prefill fp8 {Hq}/{Hkv}")


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
@pytest.mark.parametrize("lens,nq", [([300, 40, 64, 17], [64, 40, 17, 3]),     # 64 tokens x 4 heads: 16 tiles
                                     ([300, 40, 64, 17], [4, 3, 1, 4])])      # <= 16 rows: balanced split
def test_prefill_non_positive_scale(scale, lens, nq):
    """The many-tile kernel scales scores after the row maximum, so a negative
    scale moves its sign into the query, and a zero one gives equal weights
    over the visible keys."""
    wl, starts, q = _case(91, 32, 8, 128, "bf16", lens, nq)
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, scale, "bf16")
    g = _gpu(wl, starts, q, scale=scale)
    assert_parity(g, ref, "bf16", f"prefill scale {scale} max_q={max(nq)}")


@pytest.mark.parametrize("D,nq", [(64, [3, 4, 2, 5]), (128, [3, 4, 2, 12])])
def test_prefill_contract_violations_give_nan_rows(D, nq):
    """Out-of-contract sequences give NaN rows; 12 query tokens of 4 heads per
    kv head take the many-tile kernel."""
    lens = [40, 20, 30, 50]
    wl, starts, q = _case(71, 8, 2, D, "bf16", lens, nq)
    bt, sl = wl.block_tables.copy(), wl.seq_lens.copy()
    sl[1] = 3                                             # fewer tokens than query rows
    sl[2] = bt.shape[1] * 16 + 1                          # past the table row
    bt[3, 1] = wl.num_blocks                              # id outside the pool
    g = _gpu(wl, starts, q, bt=bt, sl=sl)
    for s in (1, 2, 3):
        assert np.isnan(g[starts[s]:starts[s + 1]]).all(), s
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, "bf16", seqs=[0])
    assert_parity(g[:3], ref[:3], "bf16", "rows beside the out-of-contract ones")


def test_many_tile_longest_first_contract_violations():
    """40 sequences (the many-tile kernel orders them longest first): zero
    query rows, equal lengths, and out-of-contract sequences (more query rows
    than tokens, a length past the table row, an id outside the pool) give NaN
    rows; every other row against the oracle."""
    rng = np.random.default_rng(40)
    lens = rng.integers(12, 300, size=40).tolist()
    lens[5] = lens[6] = lens[7] = 77
    nq = [12] * 40
    nq[8], nq[9] = 0, 9
    wl, starts, q = _case(73, 16, 4, 128, "bf16", lens, nq)
    bt, sl = wl.block_tables.copy(), wl.seq_lens.copy()
    sl[1] = 3
    sl[2] = bt.shape[1] * 16 + 1
    bt[3, 1] = wl.num_blocks
    g = _gpu(wl, starts, q, bt=bt, sl=sl)
    bad = [1, 2, 3]
    for s in bad:
        assert np.isnan(g[starts[s]:starts[s + 1]]).all(), s
    good = [s for s in range(40) if s not in bad]
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, "bf16", seqs=good)
    rows = np.concatenate([np.arange(starts[s], starts[s + 1]) for s in good])
    assert_parity(g[rows], ref[rows], "bf16", "many-tile, 40 sequences longest first, beside out-of-contract ones")


def test_chunked_prefill_batch_full_size():
    """8 sequences of 4096 tokens whose last 512 are the query chunk (8B head
    shape): every row against the oracle."""
    S, L, n, Hq, Hkv, D = 8, 4096, 512, 32, 8, 128
    wl, starts, q = _case(72, Hq, Hkv, D, "bf16", [L] * S, [n] * S)
    g = _gpu(wl, starts, q)
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, "bf16")
    assert_parity(g, ref, "bf16", "chunked prefill 8 x (3584 + 512), every row")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("dtype,D,Hq,Hkv", [("bf16", 128, 32, 8), ("f16", 64, 8, 8), ("bf16", 64, 16, 2)])
def test_few_query_rows_per_sequence(dtype, D, Hq, Hkv, fp8):
    """Speculative verification: a few rows per sequence, one tile per (sequence, kv head)."""
    lens = [1, 3, 16, 17, 200, 513, 40, 2]
    nq = [1, 3, 2, 3, 3, 1, 0, 2]
    wl, starts, q = _case(80 + Hq + D, Hq, Hkv, D, dtype, lens, nq)
    if fp8:
        kc8, vc8 = W.with_fp8_pools(wl, 81)
        g = _gpu(wl, starts, q, kc8, vc8, fp8=(1 / 128, 1 / 96), max_q=3)
        ref = oracle.paged_prefill_ref(W.raw_numpy(q), kc8.numpy(), vc8.numpy(), wl.block_tables, wl.seq_lens,
                                       starts, wl.scale, dtype, kv_dtype="e4m3", k_scale=1 / 128, v_scale=1 / 96)
    else:
        g = _gpu(wl, starts, q, max_q=3)
        ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                       wl.block_tables, wl.seq_lens, starts, wl.scale, dtype)
    assert_parity(g, ref, dtype, f"verify-shaped {dtype} D={D} {Hq}/{Hkv} fp8={fp8}")


@pytest.mark.parametrize("dtype,Hq,Hkv,max_q", [("bf16", 32, 8, 4), ("f16", 64, 8, 2), ("bf16", 16, 16, 16),
                                               ("bf16", 32, 8, 8), ("f16", 64, 8, 4), ("bf16", 32, 8, 16),
                                               ("bf16", 16, 16, 48), ("f16", 8, 2, 12), ("bf16", 4, 1, 8),
                                               ("f16", 8, 1, 4)])
def test_few_rows_many_segments_per_range(dtype, Hq, Hkv, max_q):
    """Speculative verification over hundreds of short sequences, so that a
    workgroup's range holds several sequences: a first segment that began in
    an earlier range and ends inside this one (its record is held until the
    range's last segment), one that runs past the range's end as well, and
    sequences without query rows in between.  Up to 16 rows per kv head is
    one tile per wave; 17..32 rows are two tiles, held by one wave per kv
    head, where fewer than 1024 (sequence, kv head) pairs (one kv head here)
    keep the split; more pairs, or more rows, go to the LDS kernel, which runs
    the sequences longest first.  Every row against the oracle."""
    rng = np.random.default_rng(Hq * 10 + Hkv + max_q)
    S = 600
    lens = rng.integers(1, 200, size=S)
    lens[::29] = rng.integers(400, 900, size=len(lens[::29]))   # some sequences span several ranges
    nq = rng.integers(0, max_q + 1, size=S)
    nq[::11] = 0
    nq = np.minimum(nq, lens)
    wl, starts, q = _case(700 + Hq + Hkv, Hq, Hkv, 128, dtype, lens, nq)
    g = _gpu(wl, starts, q, max_q=max_q)
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, dtype)
    assert_parity(g, ref, dtype, f"{S} short sequences {dtype} {Hq}/{Hkv} up to {max_q} rows")


@pytest.mark.parametrize("dtype,Hq,Hkv,max_q", [("bf16", 32, 8, 8), ("f16", 64, 8, 4), ("bf16", 32, 8, 4), ("bf16", 4, 1, 8)])
def test_few_rows_many_segments_fp8_pools(dtype, Hq, Hkv, max_q):
    """Few query rows per sequence over fp8 (e4m3) pools and hundreds of short
    sequences: one tile per kv head on the split; two tiles on the split (one
    kv head: fewer than 1024 pairs) or on the LDS kernel, longest first (eight
    kv heads); every row against the oracle."""
    rng = np.random.default_rng(Hq * 20 + Hkv + max_q)
    S = 400
    lens = rng.integers(1, 200, size=S)
    lens[::23] = rng.integers(400, 900, size=len(lens[::23]))
    nq = np.minimum(rng.integers(0, max_q + 1, size=S), lens)
    wl, starts, q = _case(800 + Hq + max_q, Hq, Hkv, 128, dtype, lens, nq)
    kc8, vc8 = W.with_fp8_pools(wl, 83)
    ks, vs = 1.0 / 128, 1.0 / 96
    g = _gpu(wl, starts, q, kc8, vc8, fp8=(ks, vs), max_q=max_q)
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), kc8.numpy(), vc8.numpy(), wl.block_tables, wl.seq_lens, starts,
                                   wl.scale, dtype, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    assert_parity(g, ref, dtype, f"{S} short sequences over fp8 pools {dtype} {Hq}/{Hkv} up to {max_q} rows")


@pytest.mark.parametrize("nqv", [4, 5, 8, 16])
def test_verify_8b_batch_full_size(nqv):
    """Speculative verification on the 8B-shaped batch (4 query rows per
    sequence: one 16-row tile per kv head, the balanced split with causal
    rows; 5 and 8: two tiles, 16: four tiles, the many-tile kernel run
    longest sequence first), every row against the oracle."""
    wl = W.make_config(3, 0, poison=True)
    S = wl.num_seqs
    nq = np.full(S, nqv, np.int32)
    starts = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = W.random_rows(3, 900, (int(starts[-1]), wl.num_heads, wl.head_size), "bf16")
    g = _gpu(wl, starts, q, max_q=nqv)
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, "bf16")
    assert_parity(g, ref, "bf16", f"verify 8B batch, {nqv} rows per sequence, every row")


def test_split_path_contract_violations():
    lens, nq = [40, 20, 30, 50, 16], [3, 4, 2, 4, 1]
    wl, starts, q = _case(73, 8, 2, 64, "bf16", lens, nq)
    bt, sl = wl.block_tables.copy(), wl.seq_lens.copy()
    sl[1] = 3                                             # fewer tokens than query rows
    sl[2] = bt.shape[1] * 16 + 1                          # past the table row
    bt[3, 1] = wl.num_blocks                              # id outside the pool
    g = _gpu(wl, starts, q, bt=bt, sl=sl, max_q=4)        # 4 rows x 4 heads: the split path
    for s in (1, 2, 3):
        assert np.isnan(g[starts[s]:starts[s + 1]]).all(), s
    ref = oracle.paged_prefill_ref(W.raw_numpy(q), W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                   wl.block_tables, wl.seq_lens, starts, wl.scale, "bf16", seqs=[0, 4])
    for s in (0, 4):
        r = slice(starts[s], starts[s + 1])
        assert_parity(g[r], ref[r], "bf16", f"sequence {s} beside the out-of-contract ones")
