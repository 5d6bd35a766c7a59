"""Seeded synthetic inputs for paged decode attention.

This module only draws and lays out inputs: sequence lengths, a shuffled
physical block pool, block tables, slot mappings and N(0, 1) query/key/value
values.  It holds none of the attention arithmetic, and both the HIP path and
the float64 oracle are fed from it.

Layouts (csdn vLLM architecture article, section 3, part 1):
  query         [num_seqs, num_heads, head_size]
  block_tables  [num_seqs, max_blocks_per_seq]   int32, unused entries = -1
  k/v cache     [num_blocks, block_size, num_kv_heads, head_size]
  seq_lens      [num_seqs]                        int32
Token t of sequence s is stored in physical block ``block_tables[s, t // BS]``
at offset ``t % BS`` (BS = 16 tokens per block, aiflowlearn vLLM course page,
section on cutting the KV cache into pages).

Pool blocks no table names, and the dead slots after the last token of a
sequence, hold NaN when ``poison=True`` (freed blocks are reused and hold
stale data, yangyitao vLLM preface, "from OS to GPU" figure) and zeros when
``poison=False`` (timing runs).  Values are drawn in float32 and rounded to
nearest-even into the workload's element type by torch on the CPU.

Random streams: ``numpy.random.default_rng(SeedSequence([291, cfg, seed]))``,
drawn in a fixed order: seq_lens, block permutation, slot targets, q, k, v.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
_CHUNK = 1 << 24  # values per draw chunk


@dataclass
class Workload:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    seq_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray      # int32 [S, max_blocks_per_seq]
    query: torch.Tensor           # CPU [S, Hq, D]
    k_cache: torch.Tensor         # CPU [NB, BS, Hkv, D]
    v_cache: torch.Tensor
    scale: float
    partition_size: int = 0
    new_key: Optional[torch.Tensor] = None     # CPU [T, Hkv, D]
    new_value: Optional[torch.Tensor] = None
    slot_mapping: Optional[np.ndarray] = None  # int32 [T]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    def kv_bytes(self) -> int:
        """Bytes of K and V that one decode step must read: valid tokens only."""
        e = ELEM_BYTES[self.dtype]
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_size * 2 * e

    def kv_bytes_unique(self) -> int:
        """Bytes of the distinct K/V rows the step reads: a slot named by
        several sequences (a shared prefix) counts once."""
        e = ELEM_BYTES[self.dtype]
        slots = [_slots_of(self.block_tables, s, np.arange(int(L)), self.block_size)
                 for s, L in enumerate(self.seq_lens.tolist()) if L > 0]
        n = len(np.unique(np.concatenate(slots))) if slots else 0
        return n * self.num_kv_heads * self.head_size * 2 * e


def raw_numpy(t: torch.Tensor) -> np.ndarray:
    """Stored elements of a CPU tensor as numpy: float32, float16, or the
    16-bit patterns (int16) of bfloat16."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy()


def _rng(cfg: int, seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([291, cfg, seed]))


def _workers() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0, 1) values, drawn in float32 chunks of 2^24 and rounded to ``dtype``.

    One 64-bit key is taken from ``rng``; chunk i is drawn from its own stream
    ``SeedSequence([key, i])``, so the values depend on the seed only, not on
    how many threads draw them.
    """
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=TORCH_DTYPES[dtype])
    key = int(rng.integers(0, 2 ** 63))

    def fill(i):
        a, b = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng(np.random.SeedSequence([key, i]))
        out[a:b] = torch.from_numpy(g.standard_normal(b - a, dtype=np.float32)).to(out.dtype)

    nchunks = -(-n // _CHUNK)
    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.view(*shape)


def _tables_from_ids(ids: np.ndarray, nblk: np.ndarray, max_blocks: int) -> np.ndarray:
    """Hand consecutive chunks of ``ids`` to the sequences, ``nblk[s]`` each."""
    tables = np.full((len(nblk), max_blocks), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(nblk.tolist()):
        tables[s, :n] = ids[pos:pos + n]
        pos += n
    return tables


def _slots_of(tables: np.ndarray, s: int, t: np.ndarray, bs: int) -> np.ndarray:
    return tables[s, t // bs].astype(np.int64) * bs + t % bs


def _fill_pool(rng, dtype, num_blocks, bs, hkv, d, slots: np.ndarray, poison: bool) -> torch.Tensor:
    """Pool with N(0, 1) rows at ``slots`` (in that order) and NaN/zero elsewhere."""
    tdt = TORCH_DTYPES[dtype]
    pool = (torch.full if poison else lambda shape, v, dtype: torch.zeros(shape, dtype=dtype))(
        (num_blocks * bs, hkv, d), float("nan"), dtype=tdt)
    if len(slots):
        pool.index_copy_(0, torch.from_numpy(slots), _normal(rng, (len(slots), hkv, d), dtype))
    return pool.view(num_blocks, bs, hkv, d)


def build(name: str, dtype: str, seq_lens: np.ndarray, tables: np.ndarray, num_blocks: int,
          num_heads: int, num_kv_heads: int, head_size: int, block_size: int,
          rng: np.random.Generator, poison: bool = True, partition_size: int = 0,
          shared_prefix_tokens: int = 0, new_token_slots: Optional[np.ndarray] = None,
          meta: Optional[dict] = None) -> Workload:
    """Draw q, then k, then v for a given table layout.

    Rows the tables share (the first ``shared_prefix_tokens`` tokens of every
    sequence after the first) are drawn once.  Positions listed in
    ``new_token_slots`` are left empty in the pool: their K/V is drawn as
    ``new_key``/``new_value`` for a later scatter.
    """
    S = len(seq_lens)
    bs = block_size
    slots = []
    for s in range(S):
        t0 = shared_prefix_tokens if s > 0 else 0
        slots.append(_slots_of(tables, s, np.arange(t0, int(seq_lens[s])), bs))
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    if new_token_slots is not None:
        slots = slots[~np.isin(slots, new_token_slots)]
    q = _normal(rng, (S, num_heads, head_size), dtype)
    kc = _fill_pool(rng, dtype, num_blocks, bs, num_kv_heads, head_size, slots, poison)
    nk = None if new_token_slots is None else _normal(rng, (len(new_token_slots), num_kv_heads, head_size), dtype)
    vc = _fill_pool(rng, dtype, num_blocks, bs, num_kv_heads, head_size, slots, poison)
    nv = None if new_token_slots is None else _normal(rng, (len(new_token_slots), num_kv_heads, head_size), dtype)
    return Workload(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_size=head_size, block_size=bs, seq_lens=np.asarray(seq_lens, np.int32),
                    block_tables=tables, query=q, k_cache=kc, v_cache=vc,
                    scale=1.0 / math.sqrt(head_size), partition_size=partition_size,
                    new_key=nk, new_value=nv,
                    slot_mapping=None if new_token_slots is None else new_token_slots.astype(np.int32),
                    meta=dict(meta or {}))


CONFIG_NAMES = {
    1: "tiny MHA paged decode: 4 seqs, 8/8 heads, D=64, fp32, L~U[1,64], 64-block pool",
    2: "13B-shaped MHA decode: 64 seqs, 40/40 heads, D=128, fp16, L~U[128,2048], 12000-block pool",
    3: "8B-shaped GQA decode: 256 seqs, 32/8 heads, D=128, bf16, L~lognormal(median 1024, sigma 1) clipped [16,4096]",
    4: "long-context GQA decode: 8 seqs x 32768, 64/8 heads, D=128, bf16, partition 512 + LSE reduce",
    5: "shared-prefix batch: 128 seqs, 1024-token shared prefix (64 blocks) + U[16,512] private tails, 32/8 heads, bf16",
}


def make_config(cfg: int, seed: int = 0, poison: bool = True) -> Workload:
    """The five synthetic workloads (stand-ins for the pages' model shapes)."""
    rng = _rng(cfg, seed)
    bs = 16
    if cfg == 1:
        lens = rng.integers(1, 65, size=4).astype(np.int32)
        nblk = -(-lens // bs)
        perm = rng.permutation(64)
        tables = _tables_from_ids(perm, nblk, 4)
        return build("cfg1", "f32", lens, tables, 64, 8, 8, 64, bs, rng, poison,
                     meta={"cfg": 1, "seed": seed})
    if cfg == 2:
        lens = rng.integers(128, 2049, size=64).astype(np.int32)
        nblk = -(-lens // bs)
        perm = rng.permutation(12000)
        tables = _tables_from_ids(perm, nblk, 2048 // bs)
        return build("cfg2", "f16", lens, tables, 12000, 40, 40, 128, bs, rng, poison,
                     meta={"cfg": 2, "seed": seed})
    if cfg == 3:
        z = rng.standard_normal(256)
        lens = np.clip(np.round(1024.0 * np.exp(z)), 16, 4096).astype(np.int32)
        nblk = -(-lens // bs)
        nb = int(math.ceil(1.1 * int(nblk.sum())))
        perm = rng.permutation(nb)
        tables = _tables_from_ids(perm, nblk, 4096 // bs)
        return build("cfg3", "bf16", lens, tables, nb, 32, 8, 128, bs, rng, poison,
                     meta={"cfg": 3, "seed": seed})
    if cfg == 4:
        lens = np.full(8, 32768, dtype=np.int32)
        nblk = -(-lens // bs)
        nb = int(math.ceil(1.1 * int(nblk.sum())))
        perm = rng.permutation(nb)
        tables = _tables_from_ids(perm, nblk, 32768 // bs)
        return build("cfg4", "bf16", lens, tables, nb, 64, 8, 128, bs, rng, poison,
                     partition_size=512, meta={"cfg": 4, "seed": seed})
    if cfg == 5:
        S, prefix_blocks = 128, 64
        tails = rng.integers(16, 513, size=S).astype(np.int32)
        lens = (prefix_blocks * bs + tails).astype(np.int32)
        tail_blk = -(-tails // bs)
        nb = int(math.ceil(1.1 * (prefix_blocks + int(tail_blk.sum()))))
        perm = rng.permutation(nb)
        tables = np.full((S, prefix_blocks + 512 // bs), -1, dtype=np.int32)
        tables[:, :prefix_blocks] = perm[:prefix_blocks]
        tables[:, prefix_blocks:] = _tables_from_ids(perm[prefix_blocks:], tail_blk, 512 // bs)
        # slot targets: the new token of each sequence sits at its last position
        new_slots = np.array([_slots_of(tables, s, np.array([lens[s] - 1]), bs)[0] for s in range(S)],
                             dtype=np.int64)
        return build("cfg5", "bf16", lens, tables, nb, 32, 8, 128, bs, rng, poison,
                     shared_prefix_tokens=prefix_blocks * bs, new_token_slots=new_slots,
                     meta={"cfg": 5, "seed": seed, "prefix_blocks": prefix_blocks})
    raise ValueError(f"unknown config {cfg}")


def make_random(seed: int, num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                dtype: str, seq_lens, block_size: int = 16, pool_factor: float = 1.5,
                poison: bool = True, partition_size: int = 0, extra_table_cols: int = 0) -> Workload:
    """Small workload with given lengths and a shuffled pool (for sweeps)."""
    rng = np.random.default_rng(np.random.SeedSequence([291, 100, seed]))
    lens = np.asarray(seq_lens, dtype=np.int32).reshape(num_seqs)
    nblk = -(-lens // block_size)
    need = int(nblk.sum())
    nb = max(1, int(math.ceil(pool_factor * need)))
    perm = rng.permutation(nb)
    max_blocks = max(1, int(nblk.max()) if num_seqs else 1) + extra_table_cols
    tables = _tables_from_ids(perm, nblk, max_blocks)
    return build(f"random{seed}", dtype, lens, tables, nb, num_heads, num_kv_heads, head_size,
                 block_size, rng, poison, partition_size=partition_size, meta={"seed": seed})


def permute_blocks(wl: Workload, seed: int) -> Workload:
    """Same logical content, physical block ids shuffled: block b moves to
    ``perm[b]`` and every table entry is rewritten to match."""
    rng = np.random.default_rng(np.random.SeedSequence([291, 200, seed]))
    nb = wl.num_blocks
    perm = rng.permutation(nb)
    idx = torch.from_numpy(perm.astype(np.int64))
    kc = torch.empty_like(wl.k_cache).index_copy_(0, idx, wl.k_cache)
    vc = torch.empty_like(wl.v_cache).index_copy_(0, idx, wl.v_cache)
    t = wl.block_tables
    tables = np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)
    slots = None
    if wl.slot_mapping is not None:
        sm = wl.slot_mapping.astype(np.int64)
        slots = np.where(sm >= 0, perm[np.maximum(sm, 0) // wl.block_size] * wl.block_size
                         + np.maximum(sm, 0) % wl.block_size, -1).astype(np.int32)
    return replace(wl, k_cache=kc, v_cache=vc, block_tables=tables, slot_mapping=slots,
                   name=wl.name + "_perm")


def unshare_prefix(wl: Workload, prefix_blocks: int) -> Workload:
    """Copy-on-write resolved: every sequence after the first gets private
    copies of the shared prefix blocks (appended to the pool)."""
    S, nb = wl.num_seqs, wl.num_blocks
    shared = wl.block_tables[0, :prefix_blocks].astype(np.int64)
    extra = (S - 1) * prefix_blocks
    kc = torch.cat([wl.k_cache, wl.k_cache[torch.from_numpy(np.tile(shared, S - 1))]])
    vc = torch.cat([wl.v_cache, wl.v_cache[torch.from_numpy(np.tile(shared, S - 1))]])
    tables = wl.block_tables.copy()
    for s in range(1, S):
        tables[s, :prefix_blocks] = nb + (s - 1) * prefix_blocks + np.arange(prefix_blocks)
    assert kc.shape[0] == nb + extra
    return replace(wl, k_cache=kc, v_cache=vc, block_tables=tables, name=wl.name + "_private")


def random_rows(seed: int, stream: int, shape, dtype: str) -> torch.Tensor:
    """N(0, 1) tensor of ``shape`` in ``dtype`` from its own seeded stream."""
    return _normal(np.random.default_rng(np.random.SeedSequence([291, 200, seed, stream])), shape, dtype)


def random_fp8_codes(seed: int, shape, poison_mask=None) -> torch.Tensor:
    """uint8 OCP e4m3 codes drawn uniformly from the finite ones (every code
    except 0x7F and 0xFF); where ``poison_mask`` is true, the NaN code 0x7F."""
    rng = np.random.default_rng(np.random.SeedSequence([291, 400, seed]))
    codes = rng.integers(0, 0x7F, size=shape, dtype=np.uint8) | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)
    if poison_mask is not None:
        codes[np.asarray(poison_mask)] = 0x7F
    return torch.from_numpy(codes)


def with_fp8_pools(wl: Workload, seed: int):
    """The workload's tables, lengths and query with fp8 code pools of the
    same shape: random finite codes where the 16-bit pools hold data, the NaN
    code where they hold the NaN poison.  Returns (k_codes, v_codes)."""
    km = torch.isnan(wl.k_cache.float()).numpy()
    vm = torch.isnan(wl.v_cache.float()).numpy()
    return random_fp8_codes(2 * seed, km.shape, km), random_fp8_codes(2 * seed + 1, vm.shape, vm)
