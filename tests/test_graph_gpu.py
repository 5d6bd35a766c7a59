"""A decode step (and a whole serving step: copies, scatter, decode) captured
in a HIP graph replays to the same bytes as eager calls, and reads its inputs
live: inputs changed in place between replays change the output exactly as
they would eagerly.  Eager work and synchronisations run between replays.
Every replay's output is also compared with the float64 oracle over the
inputs of that replay (devpress.csdn.net vLLM architecture article, section
1: the worker captures the step in a graph to cut launch overhead)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from dataclasses import replace

import oracle
import paged_kv_cache_291_amd as P
from paged_kv_cache_291_amd import workloads as W
from helpers import assert_parity, oracle_decode, to_device

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("cfg,ps", [(3, 0), (1, 0), (2, 512), (4, 0)])
def test_decode_graph_replays_match_eager(cfg, ps):
    wl = W.make_config(cfg, 0, poison=True)
    d = to_device(wl)
    ws_bytes = P.decode_workspace_bytes(d["q"], d["bt"], wl.block_size, ps, wl.max_seq_len)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    flags = P.PA_FLAG_SHARED_BLOCKS if cfg == 5 else 0

    def step(o=out):
        P.paged_attention_decode(o, d["q"], d["kc"], d["vc"], d["bt"], d["sl"], wl.scale, partition_size=ps,
                                 max_seq_len=wl.max_seq_len, workspace=ws if ws_bytes else None, flags=flags)

    g = _capture(step)
    queries = [d["q"].clone()] + [W.random_rows(cfg, 50 + i, tuple(d["q"].shape), wl.dtype).cuda() for i in range(3)]
    for i, qi in enumerate(queries + queries[:1]):
        print(f"cfg{cfg} ps={ps} replay {i}", flush=True)
        d["q"].copy_(qi)
        eager = torch.empty_like(out)
        step(eager)                                            # eager work between replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        ref = oracle_decode(replace(wl, query=qi.cpu()))
        assert_parity(out.cpu().double().numpy(), ref, wl.dtype, f"cfg{cfg} ps={ps} replay {i} vs oracle")


def test_serving_step_graph():
    """copy_blocks + reshape_and_cache + decode captured together; the slot
    mapping, copy pairs, new rows and lengths are updated in place per replay."""
    S, Hq, Hkv, D, BS = 32, 32, 8, 128, 16
    mgr = P.BlockManager(2000, BS, 64, 64)
    rng = np.random.default_rng(3)
    kc = torch.zeros((2000, BS, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for s in range(S):
        slots = mgr.allocate(s, int(rng.integers(20, 300)))
        k = W.random_rows(9, 2 * s, (len(slots), Hkv, D), "bf16").cuda()
        v = W.random_rows(9, 2 * s + 1, (len(slots), Hkv, D), "bf16").cuda()
        P.reshape_and_cache(k, v, kc, vc, torch.from_numpy(slots).cuda())
    for s in range(8):                                         # shared partly filled blocks
        mgr.fork(s, S + s)
    seqs = list(range(S + 8))
    n = len(seqs)
    # fixed-size device buffers the graph reads; per step only their contents change
    slot_d = torch.empty(n, dtype=torch.int32, device="cuda")
    src_d = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dst_d = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    newk = torch.empty((n, Hkv, D), dtype=torch.bfloat16, device="cuda")
    newv = torch.empty_like(newk)
    q = torch.empty((n, Hq, D), dtype=torch.bfloat16, device="cuda")
    bt_d = torch.empty((n, 64), dtype=torch.int32, device="cuda")
    sl_d = torch.empty(n, dtype=torch.int32, device="cuda")
    ws = torch.empty(P.pa_decode_workspace_size(n, Hq, D, 64 * BS, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step(o=out, kc_=kc, vc_=vc):
        P.copy_blocks(kc_, vc_, src_d, dst_d)
        P.reshape_and_cache(newk, newv, kc_, vc_, slot_d)
        P.paged_attention_decode(o, q, kc_, vc_, bt_d, sl_d, D ** -0.5, max_seq_len=64 * BS, workspace=ws)

    def prepare(i):
        slots = mgr.append_batch(seqs)
        src, dst = mgr.take_copies()
        src_d.fill_(-1)
        dst_d.fill_(-1)
        if len(src):
            src_d[:len(src)] = torch.from_numpy(src).cuda()
            dst_d[:len(dst)] = torch.from_numpy(dst).cuda()
        slot_d.copy_(torch.from_numpy(slots))
        newk.copy_(W.random_rows(10, 3 * i, (n, Hkv, D), "bf16"))
        newv.copy_(W.random_rows(10, 3 * i + 1, (n, Hkv, D), "bf16"))
        q.copy_(W.random_rows(10, 3 * i + 2, (n, Hq, D), "bf16"))
        bt, sl = mgr.block_tables(seqs)
        bt_d.copy_(torch.from_numpy(bt))
        sl_d.copy_(torch.from_numpy(sl))
        return len(src)

    g = None
    copies = 0
    for i in range(5):
        copies += prepare(i)
        kc_e, vc_e = kc.clone(), vc.clone()
        eager = torch.empty_like(out)
        step(eager, kc_e, vc_e)                                # eager on copies of the pools
        torch.cuda.synchronize()
        if g is None:
            g = _capture(lambda: step())                       # the capture's warm-up runs step i
            torch.cuda.synchronize()
            kc.copy_(kc_e)
            vc.copy_(vc_e)
        else:
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
        print(f"serving replay {i}: {copies} copies so far", flush=True)
        assert torch.equal(out, eager) or i == 0
        assert torch.equal(kc, kc_e) and torch.equal(vc, vc_e)
        if i > 0:                                              # a replay: the pools hold what it scattered
            ref = oracle.paged_decode_ref(W.raw_numpy(q.cpu()), W.raw_numpy(kc.cpu()), W.raw_numpy(vc.cpu()),
                                          bt_d.cpu().numpy(), sl_d.cpu().numpy(), D ** -0.5, "bf16")
            assert_parity(out.cpu().double().numpy(), ref, "bf16", f"serving replay {i} vs oracle")
    assert copies > 0
