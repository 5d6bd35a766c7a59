"""FP8 (OCP e4m3) KV pools on the GPU: the quantising scatter bit-exact against
the oracle, decode over fp8 pools against the float64 oracle (edge-length sweep
in every split mode, and the 8B-shaped batch at full size on every
sequence), and block copies of fp8 pools."""

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

K_SCALE, V_SCALE = 1.0 / 128, 1.0 / 96
EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 33, 64, 511, 512, 513, 600, 1025]


def same_codes(a: np.ndarray, b: np.ndarray) -> bool:
    """Byte-equal, except that any NaN code (0x7F, 0xFF) matches any other."""
    na, nb = (a & 0x7F) == 0x7F, (b & 0x7F) == 0x7F
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb]))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fp8_scatter_bit_exact(dtype):
    T, Hkv, D, NB, BS = 40, 8, 128, 16, 16
    key = W.random_rows(700, 0, (T, Hkv, D), dtype) * 3
    value = W.random_rows(700, 1, (T, Hkv, D), dtype)
    special = torch.tensor([0.0, -0.0, 1e-30, -1e-30, 448.0 * K_SCALE, 449 * K_SCALE, 1e6, -1e6,
                            float("inf"), float("-inf"), float("nan"), 1.0625 * K_SCALE, 1.1875 * K_SCALE,
                            2.0 ** -10 * K_SCALE, 3 * 2.0 ** -11 * K_SCALE, 7.5 * 2.0 ** -9 * K_SCALE])
    key[0, 0, :len(special)] = special.to(key.dtype)
    kc = torch.full((NB, BS, Hkv, D), 0x7F, dtype=torch.uint8)
    vc = kc.clone()
    slots = np.random.default_rng(3).choice(NB * BS, size=T, replace=False).astype(np.int32)
    slots[5] = -1
    want_k, want_v = oracle.reshape_and_cache_fp8_ref(W.raw_numpy(key), W.raw_numpy(value), kc.numpy(), vc.numpy(),
                                                      slots, dtype, K_SCALE, V_SCALE)
    dk, dv = kc.cuda(), vc.cuda()
    print(f"fp8 scatter from {dtype}", flush=True)
    P.reshape_and_cache_fp8(key.cuda(), value.cuda(), dk, dv, torch.from_numpy(slots).cuda(), K_SCALE, V_SCALE)
    torch.cuda.synchronize()
    assert same_codes(dk.cpu().numpy(), want_k)
    assert same_codes(dv.cpu().numpy(), want_v)


def _fp8_case(wl, seed):
    kc8, vc8 = W.with_fp8_pools(wl, seed)
    return kc8, vc8


def _run_fp8(wl, kc8, vc8, ps, flags=0):
    q = wl.query.cuda()
    out = torch.empty_like(q)
    P.paged_attention_decode_fp8(out, q, kc8.cuda(), vc8.cuda(), torch.from_numpy(wl.block_tables).cuda(),
                                 torch.from_numpy(wl.seq_lens).cuda(), wl.scale, K_SCALE, V_SCALE,
                                 partition_size=ps, max_seq_len=wl.max_seq_len, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def _ref_fp8(wl, kc8, vc8, seqs=None):
    return oracle.paged_decode_ref(W.raw_numpy(wl.query), kc8.numpy(), vc8.numpy(), wl.block_tables, wl.seq_lens,
                                   wl.scale, wl.dtype, seqs=seqs, kv_dtype="e4m3", k_scale=K_SCALE,
                                   v_scale=V_SCALE)


SWEEP = [(dt, D, Hq, Hkv) for dt in ("bf16", "f16") for D in (64, 128) for (Hq, Hkv) in ((4, 4), (4, 2), (8, 2), (16, 2))]


@pytest.mark.parametrize("ps", [0, 16, 512])
@pytest.mark.parametrize("dtype,D,Hq,Hkv", SWEEP)
def test_fp8_decode_sweep(dtype, D, Hq, Hkv, ps):
    seed = zlib.crc32(f"fp8-{dtype}-{D}-{Hq}-{Hkv}-{ps}".encode()) % 10000
    wl = W.make_random(seed, len(EDGE_LENS), Hq, Hkv, D, dtype, EDGE_LENS, extra_table_cols=2)
    kc8, vc8 = _fp8_case(wl, seed)
    g = _run_fp8(wl, kc8, vc8, ps)
    ref = _ref_fp8(wl, kc8, vc8)
    assert_parity(g, ref, dtype, f"fp8 {dtype} D={D} {Hq}/{Hkv} ps={ps}")
    assert (g[0] == 0).all()


def test_fp8_decode_8b_batch_full_size():
    wl = W.make_config(3, 0, poison=True)
    kc8, vc8 = _fp8_case(wl, 33)
    ref = _ref_fp8(wl, kc8, vc8)
    for ps in (0, 512):
        g = _run_fp8(wl, kc8, vc8, ps)
        assert_parity(g, ref, "bf16", f"fp8 8B batch ps={ps}, every sequence")


def test_fp8_decode_13b_batch_full_size():
    """64 sequences x 40 heads without grouping: every row, with the partitions
    the library picks and with 512-token partitions (both on the vector-ALU
    core fed from the work queue, reading the fp8 codes)."""
    wl = W.make_config(2, 0, poison=True)
    kc8, vc8 = _fp8_case(wl, 34)
    ref = _ref_fp8(wl, kc8, vc8)
    for ps in (0, 512):
        g = _run_fp8(wl, kc8, vc8, ps)
        assert_parity(g, ref, wl.dtype, f"fp8 13B batch ps={ps}, every sequence")


@pytest.mark.parametrize("Hkv", [5, 6, 10])
def test_fp8_mha_queue_head_groups(Hkv):
    """Without grouping, fp8 pools take workgroups of up to 4 kv heads fed from
    the work queue; 5, 6 and 10 kv heads give 1, 3 and 2 heads per workgroup.
    16-token partitions make many items per sequence, empty ones included."""
    seed = 900 + Hkv
    wl = W.make_random(seed, len(EDGE_LENS), Hkv, Hkv, 128, "f16", EDGE_LENS, extra_table_cols=3)
    kc8, vc8 = _fp8_case(wl, seed)
    ref = _ref_fp8(wl, kc8, vc8)
    for ps in (16, 64):
        g = _run_fp8(wl, kc8, vc8, ps)
        assert_parity(g, ref, "f16", f"fp8 MHA {Hkv} heads ps={ps}")


def test_fp8_mha_queue_library_partitions():
    """1024 (sequence, kv head) pairs without a partition size: the library
    cuts partitions, doubling 256 tokens until the records fit the workspace
    sized for partition_size 0 (256 seqs up to 4096 tokens: 2048-token
    partitions; with max_seq_len 2048: 1024).  Sequences longer than the
    partitions cover (max_seq_len 2048 passed) break the contract and give NaN
    rows; the others are unaffected."""
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 300, size=256)
    lens[[3, 100, 255]] = [4096, 2049, 2048]
    lens[[7, 8]] = [0, 16]
    wl = W.make_random(78, 256, 4, 4, 64, "bf16", lens, extra_table_cols=1)
    kc8, vc8 = _fp8_case(wl, 78)
    need = P.pa_decode_workspace_size(256, 4, 64, 4096, 0)
    for msl, bad in ((4096, []), (2048, [3, 100])):
        ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")   # stale contents must not matter
        q = wl.query.cuda()
        out = torch.empty_like(q)
        P.paged_attention_decode_fp8(out, q, kc8.cuda(), vc8.cuda(), torch.from_numpy(wl.block_tables).cuda(),
                                     torch.from_numpy(wl.seq_lens).cuda(), wl.scale, K_SCALE, V_SCALE,
                                     partition_size=0, max_seq_len=msl, workspace=ws)
        torch.cuda.synchronize()
        g = out.cpu().double().numpy()
        good = [s for s in range(256) if s not in bad]
        assert_parity(g[good], _ref_fp8(wl, kc8, vc8)[good], "bf16", f"fp8 MHA library partitions msl={msl}")
        for s in bad:
            assert np.isnan(g[s]).all()


def test_fp8_mha_few_long_sequences():
    """Fewer than 1024 (sequence, kv head) pairs, long sequences: the queued
    launch with the library's partitions (not the matrix-core split)."""
    lens = [0, 1, 17, 255, 256, 257, 1999, 2000]
    wl = W.make_random(911, len(lens), 40, 40, 128, "f16", lens, extra_table_cols=1)
    kc8, vc8 = _fp8_case(wl, 911)
    g = _run_fp8(wl, kc8, vc8, 0)
    assert_parity(g, _ref_fp8(wl, kc8, vc8), "f16", "fp8 MHA few long sequences")
    assert (g[0] == 0).all()


def test_fp8_mha_queue_graph_replays():
    """The queued launch (counter reset, decode, reduce) captured in a HIP graph
    replays to the eager bytes, with eager work between replays."""
    wl = W.make_config(2, 1, poison=True)
    kc8, vc8 = _fp8_case(wl, 35)
    q = wl.query.cuda()
    dk, dv = kc8.cuda(), vc8.cuda()
    bt, sl = torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(wl.seq_lens).cuda()
    ws = torch.empty(P.pa_decode_workspace_size(wl.num_seqs, wl.num_heads, wl.head_size, wl.max_seq_len, 0),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step(o=out):
        P.paged_attention_decode_fp8(o, q, dk, dv, bt, sl, wl.scale, K_SCALE, V_SCALE, partition_size=0,
                                     max_seq_len=wl.max_seq_len, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    ref = _ref_fp8(wl, kc8, vc8)
    queries = [wl.query.cuda().clone()] + [W.random_rows(2, 60 + i, tuple(q.shape), wl.dtype).cuda()
                                          for i in range(2)]
    for i, qi in enumerate(queries + queries[:1]):
        print(f"fp8 13B graph replay {i}", flush=True)
        q.copy_(qi)
        eager = torch.empty_like(out)
        step(eager)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        if i == 0 or i == len(queries):
            assert_parity(out.cpu().double().numpy(), ref, wl.dtype, f"fp8 13B graph replay {i} vs oracle")


def test_fp8_copy_blocks_bit_exact():
    NB, BS, Hkv, D = 200, 16, 8, 128
    kc = W.random_fp8_codes(5, (NB, BS, Hkv, D))
    vc = W.random_fp8_codes(6, (NB, BS, Hkv, D))
    ids = np.random.default_rng(4).permutation(NB)
    src, dst = ids[:60].astype(np.int32), ids[60:120].astype(np.int32)
    want_k, want_v = oracle.copy_blocks_ref(kc.numpy(), vc.numpy(), src, dst)
    dk, dv = kc.cuda(), vc.cuda()
    P.copy_blocks(dk, dv, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), want_k) and np.array_equal(dv.cpu().numpy(), want_v)
