"""Inputs that force the online-softmax rescale with a live running state.

The matrix-core kernels keep a per-row reference maximum and only rescale the
running sum and accumulator when a block's (or, in the many-tile kernel, a
block pair's) maximum score exceeds that reference by more than 8 in base-2
units (devpress.csdn.net vLLM architecture article, section 3, part 2 step 4:
the attention step may be fused FlashAttention-style, i.e. an online softmax
whose running state is rescaled as the maximum grows).  N(0, 1) data never
climbs that far inside one segment, so these cases plant score jumps:

* spikes: one key of a row gets a score 9.5 (base 2) above every earlier key
  the row sees, once or twice per row, at seeded positions;
* climbs: a row's scores rise by a seeded slope per block (natural units),
  so the block maxima overtake the reference every few blocks;
* background keys are scaled by 1/4 and values by 1/4 (N(0, 1/16) data), so
  the mass already accumulated when a jump arrives stays a sizeable part of
  the result and a wrong rescale factor shows in the output.

Rows of one kv head share its keys, so the rows of a wave get different
plans and therefore different rescale factors in the same step.

The segment model mirrors the launches' work split (which blocks one wave
streams with one running state), and ``count_rescales`` replays the lazy
rule on float64 scores of the stored inputs, so a test can assert from the
inputs alone that the rescale with a live state is reached, and how often.
This module only builds inputs and counts; it holds no attention arithmetic
and imports nothing from the product.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

import oracle
from paged_kv_cache_291_amd import workloads as W

LOG2E = 1.0 / math.log(2.0)
THRESHOLD = 8.0                       # base-2 units: the kernels' rescale rule
SPIKE_JUMP = 9.5                      # base-2 units above every earlier visible key
BS = 16
# the work split of the launches: 256 workgroups over the head groups
SPLIT_WORKGROUPS = 256


@dataclass
class KvPools:
    """Pools as the kernels see them, plus how to read and write rows of them.

    ``kind``: "bf16" / "f16" (16-bit pools of the query type) or "e4m3"
    (fp8 code pools; the effective value is code value * scale)."""
    kind: str
    k: torch.Tensor
    v: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0

    def read_k(self, slots: np.ndarray, kvh: int) -> np.ndarray:
        rows = self.k.view(-1, *self.k.shape[2:])[torch.from_numpy(slots), kvh]
        if self.kind == "e4m3":
            return oracle.E4M3_VALUES[rows.numpy()] * self.k_scale
        return rows.double().numpy()

    def write_k(self, slots: np.ndarray, kvh: int, x: np.ndarray) -> None:
        flat = self.k.view(-1, *self.k.shape[2:])
        flat[torch.from_numpy(slots), kvh] = _store(x, self.kind, self.k_scale)


def _store(x: np.ndarray, kind: str, scale: float) -> torch.Tensor:
    """Round float64 values to the pool's element type (nearest-even); fp8
    values are saturated to the format's range first."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if kind == "e4m3":
        return (t / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return t.to(W.TORCH_DTYPES[kind])


def pools_for(wl: W.Workload, kv: str, k_scale: float = 1.0 / 64, v_scale: float = 1.0 / 256) -> KvPools:
    """Background pools: the workload's values scaled by 1/4 (K and V); for
    kv == "e4m3" those values stored as fp8 codes with the given scales
    (NaN poison stays NaN)."""
    k = wl.k_cache * 0.25
    v = wl.v_cache * 0.25
    if kv == "e4m3":
        return KvPools("e4m3", _store(k.double().numpy(), "e4m3", k_scale),
                       _store(v.double().numpy(), "e4m3", v_scale), k_scale, v_scale)
    return KvPools(wl.dtype, k, v)


def seq_slots(bt_row: np.ndarray, L: int) -> np.ndarray:
    t = np.arange(L)
    return bt_row[t // BS].astype(np.int64) * BS + t % BS


def plant(pools: KvPools, bt_row: np.ndarray, L: int, kvh: int, qrows: list, scale: float,
          visible: int, rng: np.random.Generator, plans=None):
    """Plant spikes and climbs for the query rows ``qrows`` (float64 vectors)
    of one (sequence, kv head) into the K pool, over keys ``[0, visible)``.

    Each row gets one plan: "climb", "one", "two" or "none" (seeded, at most
    one climb per kv head).  Spikes sit at keys >= 32 (never in the first
    block pair) and every key carries at most one spike.  Returns the plans.
    """
    slots = seq_slots(bt_row, L)
    K = pools.read_k(slots, kvh)
    R = len(qrows)
    if plans is None:
        kinds = ["climb", "one", "two", "none", "one", "two"]
        rng.shuffle(kinds)
        plans = [kinds[i % len(kinds)] for i in range(R)]
        if plans.count("climb") > 1:
            plans = [p if p != "climb" or i == plans.index("climb") else "one" for i, p in enumerate(plans)]
    nblk_vis = visible // BS
    for r, kind in enumerate(plans):
        if kind != "climb" or nblk_vis < 4:
            continue
        q = qrows[r]
        u = q / (float(q @ q) * scale)                 # adds 1 to row r's natural score
        b0 = int(rng.integers(1, max(2, nblk_vis // 3)))
        slope = float(rng.uniform(0.8, 1.4))
        top = 28.0 if pools.kind == "e4m3" else 60.0
        t = np.arange(visible)
        rise = np.clip((t // BS - b0 + 1) * slope, 0.0, top)
        K[:visible] += rise[:, None] * u[None, :]
    pools.write_k(slots, kvh, K)
    K = pools.read_k(slots, kvh)
    taken = set()
    spikes = []
    for r, kind in enumerate(plans):
        n = {"one": 1, "two": 2}.get(kind, 0)
        if n == 0 or visible <= 48:
            continue
        cand = [int(x) for x in rng.choice(np.arange(32, visible), size=min(8, visible - 32), replace=False)]
        picks = sorted(c for c in cand if c not in taken)[:n]
        for t in picks:
            taken.add(t)
            spikes.append((t, r))
    for t, r in sorted(spikes):
        q = qrows[r]
        z_prev = scale * (K[:t] @ q)
        target = float(z_prev.max()) + SPIKE_JUMP / LOG2E
        z_now = scale * float(K[t] @ q)
        K[t] = K[t] + (target - z_now) * q / (float(q @ q) * scale)
        pools.write_k(slots[t:t + 1], kvh, K[t:t + 1])
        K[t] = pools.read_k(slots[t:t + 1], kvh)[0]
    return plans


# ---- which blocks one wave streams with one running state

def valid_blocks(seq_lens: np.ndarray, max_blocks: int) -> np.ndarray:
    L = np.asarray(seq_lens, dtype=np.int64)
    ok = (L > 0) & (L <= max_blocks * BS)
    return np.where(ok, -(-L // BS), 0)


def heads_per_workgroup(num_kv_heads: int, waves: int = 8) -> int:
    for d in range(waves, 1, -1):
        if num_kv_heads % d == 0:
            return d
    return 1


def balanced_segments(nblk: np.ndarray, num_kv_heads: int, tiles: int = 1, head_size: int = 128):
    """Per sequence, the [b0, b1) block runs of the balanced split: the
    batch's blocks laid end to end and cut into 256 / head-groups equal
    ranges (a head group is up to 8 kv heads; up to 4 when a wave holds two
    tiles of 128-wide heads)."""
    hpw = heads_per_workgroup(num_kv_heads, 4 if tiles == 2 and head_size == 128 else 8)
    nwg = max(SPLIT_WORKGROUPS // (num_kv_heads // hpw), 1)
    cum = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)
    U = int(cum[-1])
    cuts = [(r * U) // nwg for r in range(nwg + 1)]
    segs = []
    for s in range(len(nblk)):
        c0, c1 = int(cum[s]), int(cum[s + 1])
        runs = []
        for r in range(nwg):
            a, b = max(c0, cuts[r]), min(c1, cuts[r + 1])
            if a < b:
                runs.append((a - c0, b - c0))
        segs.append(runs)
    return segs


def fixed_segments(nblk: np.ndarray, partition_size: int):
    per = partition_size // BS
    return [[(b, min(b + per, int(n))) for b in range(0, int(n), per)] for n in nblk]


# ---- the lazy rule replayed on float64 scores

def count_rescales(Z: np.ndarray, row_last: np.ndarray, b0: int, b1: int, unit: int = 1):
    """Replay one wave's running maxima over blocks [b0, b1) in steps of
    ``unit`` blocks.  ``Z``: base-2 scores ``[16, keys]`` of the wave's 16
    rows (zeros for padding rows); ``row_last``: each row's last visible key.
    A step rescales when any row's step maximum exceeds its reference by more
    than THRESHOLD; every row then takes the larger of the two.  Returns the
    rows whose reference rose by at least 1 with a finite old reference
    (a rescale by a factor <= 1/2 of a running state that holds keys), and
    whether a decision fell within 0.01 of the threshold (then the replay
    stops: float32 rounding could decide it either way)."""
    nkeys = Z.shape[1]
    m = np.full(16, -np.inf)
    events = []
    key_ids = np.arange(nkeys)
    for u in range(b0, b1, unit):
        k0, k1 = u * BS, min((u + unit) * BS, nkeys)
        if k0 >= nkeys:
            break
        vis = key_ids[None, k0:k1] <= row_last[:, None]
        zz = np.where(vis, Z[:, k0:k1], -np.inf)
        bm = zz.max(axis=1)
        with np.errstate(invalid="ignore"):              # -inf - -inf: a row with nothing visible yet
            d = bm - (m + THRESHOLD)
        fin = np.isfinite(d)
        if np.any(fin & (np.abs(d) < 0.01)):
            return events, True
        if np.any(d > 0):
            m_new = np.maximum(m, bm)
            for r in range(16):
                if np.isfinite(m[r]) and m_new[r] >= m[r] + 1.0 and m_new[r] - m[r] < 100.0:
                    events.append(r)
            m = m_new
    return events, False


@dataclass
class Case:
    """A planted batch and the query rows per (sequence, kv head)."""
    wl: W.Workload
    pools: KvPools
    query: torch.Tensor                  # [T, Hq, D] (decode: T = S)
    starts: np.ndarray                   # int32 [S + 1] (decode: 0..S)
    plans: dict


def _qrows(query_np: np.ndarray, dtype: str, a: int, n: int, kvh: int, G: int):
    rows = []
    for i in range(n):
        q = oracle.decode_values(query_np[a + i], dtype)
        for j in range(G):
            rows.append(q[kvh * G + j])
    return rows


def make_case(seed: int, lens, nq, Hq: int, Hkv: int, D: int, dtype: str, kv: str, plant_seqs=None,
              scale: float | None = None) -> Case:
    """A random batch (``make_random``), its pools scaled to the background
    level, and planted jumps for every (sequence, kv head) of
    ``plant_seqs`` (default: all), aimed at the sequence's query rows: ``nq``
    rows per sequence (its last tokens; 1 per sequence for decode)."""
    lens = np.asarray(lens, dtype=np.int32)
    nq = np.asarray(nq, dtype=np.int32)
    wl = W.make_random(seed, len(lens), Hq, Hkv, D, dtype, lens, extra_table_cols=1)
    if scale is not None:
        wl = replace(wl, scale=float(scale))
    pools = pools_for(wl, kv)
    starts = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    query = W.random_rows(seed, 77, (int(starts[-1]), Hq, D), dtype)
    qn = W.raw_numpy(query)
    rng = np.random.default_rng(np.random.SeedSequence([291, 300, seed]))
    G = Hq // Hkv
    plans = {}
    for s in (range(len(lens)) if plant_seqs is None else plant_seqs):
        L, n = int(lens[s]), int(nq[s])
        if n == 0 or L < 64:
            continue
        for kvh in range(Hkv):
            rows = _qrows(qn, dtype, int(starts[s]), n, kvh, G)
            plans[(s, kvh)] = plant(pools, wl.block_tables[s], L, kvh, rows, wl.scale, L - n + 1, rng)
    return Case(wl, pools, query, starts, plans)


def wave_scores(case: Case, s: int, kvh: int, tok0: int) -> tuple:
    """Base-2 scores and last visible keys of one wave's 16 rows: rows
    r = (token tok0 + r // G, head r % G) of (sequence s, kv head kvh);
    rows past the sequence's query rows are padding (zero query, they see
    every key)."""
    wl = case.wl
    G = wl.num_heads // wl.num_kv_heads
    L = int(wl.seq_lens[s])
    a, n = int(case.starts[s]), int(case.starts[s + 1] - case.starts[s])
    K = case.pools.read_k(seq_slots(wl.block_tables[s], L), kvh)
    qn = W.raw_numpy(case.query)
    Z = np.zeros((16, L))
    last = np.full(16, L - 1)
    for r in range(16):
        tok = tok0 + r // G
        if tok < n:
            q = oracle.decode_values(qn[a + tok], wl.dtype)[kvh * G + r % G]
            Z[r] = wl.scale * (K @ q) * LOG2E
            last[r] = L - n + tok
    return Z, last


def events_over(case: Case, segs, unit: int = 1, tiles_of=None):
    """Rescale events over the given segments for every planted (sequence,
    kv head) and its tile waves.  ``segs[s]``: [b0, b1) runs of sequence s
    (None: the whole visible range of each wave); ``tiles_of(s)``: first
    tokens of the sequence's waves (default one wave at token 0).  Returns
    (events, rows with events, ambiguous replays)."""
    wl = case.wl
    events, rows, ambiguous = 0, set(), 0
    for (s, kvh) in case.plans:
        for tok0 in (tiles_of(s) if tiles_of else [0]):
            Z, last = wave_scores(case, s, kvh, tok0)
            runs = segs[s] if segs is not None else [(0, int(last.max()) // BS + 1)]
            for (b0, b1) in runs:
                ev, amb = count_rescales(Z, last, b0, b1, unit)
                events += len(ev)
                rows.update(ev)
                ambiguous += amb
    return events, rows, ambiguous
