"""GPU parity of reshape_and_cache: whole pools must be byte-identical to the
oracle's scatter (every byte, targeted or not)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_291_amd as P
from paged_kv_cache_291_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bytes(t: torch.Tensor) -> bytes:
    return W.raw_numpy(t.cpu()).tobytes()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Hkv,D", [(1, 64), (8, 128), (40, 128), (2, 64)])
def test_scatter_bit_exact(dtype, Hkv, D):
    rng = np.random.default_rng(Hkv * 1000 + D)
    NB, BS, T = 37, 16, 50
    tdt = W.TORCH_DTYPES[dtype]
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(tdt)
    kc, vc, key, value = mk(NB, BS, Hkv, D), mk(NB, BS, Hkv, D), mk(T, Hkv, D), mk(T, Hkv, D)
    slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int32)
    slots[[3, 17, 40]] = [-1, -5, -2147483648]
    slots[41] = NB * BS                                   # past the pool: skipped
    want_k, want_v = oracle.reshape_and_cache_ref(W.raw_numpy(key), W.raw_numpy(value),
                                                  W.raw_numpy(kc), W.raw_numpy(vc),
                                                  np.where(slots < NB * BS, slots, -1))
    dkc, dvc = kc.cuda(), vc.cuda()
    P.reshape_and_cache(key.cuda(), value.cuda(), dkc, dvc, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert _bytes(dkc) == want_k.tobytes()
    assert _bytes(dvc) == want_v.tobytes()


def test_scatter_nan_payload_preserved():
    key = torch.tensor([[[float("nan"), -0.0, float("inf"), 1.0] * 16]], dtype=torch.bfloat16)
    key.view(torch.int16)[0, 0, 0] = 0x7FA1                # a NaN with a payload
    value = -key
    kc = torch.zeros(2, 16, 1, 64, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    dkc, dvc = kc.cuda(), vc.cuda()
    P.reshape_and_cache(key.cuda(), value.cuda(), dkc, dvc, torch.tensor([21], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    want_k, want_v = oracle.reshape_and_cache_ref(W.raw_numpy(key), W.raw_numpy(value),
                                                  W.raw_numpy(kc), W.raw_numpy(vc), np.array([21]))
    assert _bytes(dkc) == want_k.tobytes() and _bytes(dvc) == want_v.tobytes()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config5_scatter_bit_exact(seed):
    wl = W.make_config(5, seed, poison=True)
    want_k, want_v = oracle.reshape_and_cache_ref(W.raw_numpy(wl.new_key), W.raw_numpy(wl.new_value),
                                                  W.raw_numpy(wl.k_cache), W.raw_numpy(wl.v_cache),
                                                  wl.slot_mapping)
    dkc, dvc = wl.k_cache.cuda(), wl.v_cache.cuda()
    P.reshape_and_cache(wl.new_key.cuda(), wl.new_value.cuda(), dkc, dvc,
                        torch.from_numpy(wl.slot_mapping).cuda())
    torch.cuda.synchronize()
    assert _bytes(dkc) == want_k.tobytes()
    assert _bytes(dvc) == want_v.tobytes()


def test_scatter_empty_is_noop():
    kc = torch.randn(4, 16, 2, 64).cuda()
    before = kc.clone()
    empty = torch.empty(0, 2, 64).cuda()
    P.reshape_and_cache(empty, empty, kc, kc, torch.empty(0, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert torch.equal(kc, before)
