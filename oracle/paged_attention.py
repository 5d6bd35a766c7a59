"""Plain, slow, float64 reference for paged decode attention (CPU, NumPy).

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, the smoke check
and the CPU-baseline leg of the benchmark are its only callers.

Sources (pages on the subject, cited by title and section):

* devpress.csdn.net article on the vLLM architecture, section 3 ("PagedAttention
  kernel: from concept to CUDA"):
  - part 1 (inputs): ``query[num_seqs, num_heads, head_size]``,
    ``block_tables[num_seqs, max_blocks_per_seq]``,
    ``k_cache[num_physical_blocks, block_size, num_kv_heads, head_size]`` and a
    ``v_cache`` of the same form;
  - part 2 (kernel flow): for each sequence (1) take its block table,
    (2) take its actual length and the number of logical blocks it covers,
    (3) gather K/V from the physical blocks the table names into a logically
    contiguous K_seq / V_seq, (4) run standard attention of the sequence's
    query against them, (5) write the output back.
* aiflowlearn.net vLLM course page, section on how the KV cache is cut into
  pages: a block holds the K/V of 16 tokens.
* yangyitao.com vLLM book preface, section "from OS to GPU" (block-pool
  figure): blocks are handed out on demand from one pool and freed blocks are
  reused, so the pool holds arbitrary data outside the blocks a table names.

Readings where the pages are silent (each is listed in the design notes):

* scale is an argument (1/sqrt(head_size) in every workload);
* query head h reads kv head ``h // (num_heads // num_kv_heads)``;
* the one query attends to all ``seq_lens[s]`` cached tokens, no mask;
* token t of a sequence lives in logical block ``t // block_size`` at offset
  ``t % block_size`` of physical block ``block_tables[s, t // block_size]``;
* ``seq_lens[s] == 0`` gives an all-zero output row;
* q, caches and output share one element type; the oracle decodes those
  values exactly into float64 and keeps its output in float64.

This is the definition of the result written out: exact softmax attention over
the gathered rows.  A matmul and an exp are the only library steps; nothing is
blocked, fused or reordered beyond the formula.
"""

from __future__ import annotations

import math

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def decode_values(raw, dtype: str) -> np.ndarray:
    """Decode stored elements into float64, exactly.

    ``raw`` holds the elements as stored: float32 values for ``"f32"``,
    float16 values (or their uint16/int16 bit patterns) for ``"f16"``, and the
    uint16/int16 bit patterns for ``"bf16"``.  bfloat16 is, by its definition,
    the upper half of an IEEE-754 binary32 word, so its value is the binary32
    whose top 16 bits are the pattern and whose low 16 bits are zero.
    Every value of the three formats is exactly representable in float64.
    """
    a = np.asarray(raw)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError(f"f32 data must be float32, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "f16":
        if a.dtype in (np.uint16, np.int16):
            a = a.view(np.float16)
        if a.dtype != np.float16:
            raise TypeError(f"f16 data must be float16 or 16-bit patterns, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype not in (np.uint16, np.int16):
            raise TypeError(f"bf16 data must be 16-bit patterns, got {a.dtype}")
        word = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return word.view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        if a.dtype not in (np.uint8, np.int8):
            raise TypeError(f"e4m3 data must be 8-bit codes, got {a.dtype}")
        return E4M3_VALUES[a.view(np.uint8)]
    raise ValueError(f"unknown dtype {dtype!r}; expected one of {DTYPES}")


def e4m3_value(code: int) -> float:
    """Value of an OCP 8-bit float E4M3 code (the OCP 8-bit floating point
    specification's E4M3 encoding): sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6; there are no
    infinities, and S.1111.111 is NaN, so the largest finite value is
    1.75 * 2^8 = 448."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0


def quantize_e4m3_ref(x, scale: float) -> np.ndarray:
    """Codes of ``x / scale`` in E4M3, the way the fp8 pools store them.

    Reading (the pages name quantisation but no format, see the design
    notes): the product ``x * inv`` is taken in float32 with
    ``inv = float32(1 / scale)``; values beyond +-448 saturate to +-448; NaN
    gives the NaN code; everything else rounds to the nearest E4M3 value,
    ties to the even code (the one whose lowest bit is 0).  ``x`` holds
    values exactly representable in float32.
    """
    inv = np.float32(1.0 / np.float64(scale))
    y = (np.asarray(x, dtype=np.float64).astype(np.float32) * inv).astype(np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    codes = np.array([c for c in range(256) if not np.isnan(E4M3_VALUES[c])])
    values = E4M3_VALUES[codes]
    for i, v in enumerate(flat.tolist()):
        if v != v:
            out[i] = 0x7F
            continue
        v = min(max(v, -E4M3_MAX), E4M3_MAX)
        dist = np.abs(values - v)
        near = codes[dist == dist.min()].tolist()
        if len(near) > 1:                         # a tie, or +0 / -0
            signed = [c for c in near if (c & 0x80) == (0x80 if np.signbit(v) else 0)]
            near = signed or near
            even = [c for c in near if c % 2 == 0]
            near = even or near
        out[i] = near[0]
    return out.reshape(y.shape)


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head that query head ``h`` reads: contiguous groups of
    ``num_heads // num_kv_heads`` query heads share one KV head (grouped-query
    attention; the csdn inputs list lets num_heads and num_kv_heads differ)."""
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return h // (num_heads // num_kv_heads)


def gather_rows(cache, table_row, seq_len: int, kv_head: int) -> np.ndarray:
    """Gather one KV head's rows of one sequence in logical token order.

    csdn section 3, part 2 steps (2)-(3): token t sits in logical block
    ``t // block_size`` at offset ``t % block_size``; the table maps the
    logical block to a physical block of the pool.  Only the first
    ``ceil(seq_len / block_size)`` table entries are read.
    Returns the raw stored elements, shape ``[seq_len, head_size]``.
    """
    block_size = cache.shape[1]
    t = np.arange(int(seq_len))
    phys = np.asarray(table_row)[t // block_size].astype(np.int64)
    return np.asarray(cache)[phys, t % block_size, kv_head, :]


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Standard attention of one query vector over ``L`` key/value rows.

    csdn section 3, part 2 step (4).  ``z_t = scale * <q, K_t>``,
    ``p = softmax(z)`` (the max is subtracted before exp, which changes nothing
    mathematically), ``out = sum_t p_t V_t``.  Returns ``(out, p)``; with
    ``L == 0`` the output is zero and ``p`` is empty.
    """
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=np.float64), np.zeros(0, dtype=np.float64)
    z = scale * (K @ q)
    e = np.exp(z - z.max())
    p = e / e.sum()
    return p @ V, p


def _check_shapes(query, k_cache, v_cache, block_tables, seq_lens):
    S, Hq, D = query.shape
    NB, BS, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must both be [blocks, block_size, kv_heads, head_size]")
    if block_tables.shape[0] != S or len(seq_lens) != S:
        raise ValueError("block_tables and seq_lens need one row per sequence")
    if Hq % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return S, Hq, D, NB, BS, Hkv


def paged_decode_ref(query, k_cache, v_cache, block_tables, seq_lens, scale: float,
                     dtype: str, seqs=None, kv_dtype: str | None = None, k_scale: float = 1.0,
                     v_scale: float = 1.0) -> np.ndarray:
    """Paged decode attention, float64: csdn section 3, parts 1-2, steps (1)-(5).

    For every sequence s (or only those in ``seqs``) and query head h: gather
    the rows of KV head ``kv_head_of(h)`` through the block table, run
    ``softmax_attention`` with ``query[s, h]``, and store the result.
    Returns float64 ``[len(seqs), num_heads, head_size]`` (all sequences when
    ``seqs`` is None), in the order of ``seqs``.  With ``kv_dtype`` the pools
    hold that type (``"e4m3"`` codes) and their values are multiplied by
    ``k_scale`` / ``v_scale``.
    """
    S, Hq, D, NB, BS, Hkv = _check_shapes(query, k_cache, v_cache, block_tables, seq_lens)
    seqs = range(S) if seqs is None else list(seqs)
    kvt = kv_dtype or dtype
    out = np.zeros((len(seqs), Hq, D), dtype=np.float64)
    for row, s in enumerate(seqs):
        L = int(seq_lens[s])
        q = decode_values(query[s], dtype)                              # [Hq, D]
        for kvh in range(Hkv):
            K = decode_values(gather_rows(k_cache, block_tables[s], L, kvh), kvt) * k_scale
            V = decode_values(gather_rows(v_cache, block_tables[s], L, kvh), kvt) * v_scale
            for h in range(Hq):
                if kv_head_of(h, Hq, Hkv) == kvh:
                    out[row, h], _ = softmax_attention(q[h], K, V, scale)
    return out


def paged_decode_probs_ref(query, k_cache, v_cache, block_tables, seq_lens, scale: float,
                           dtype: str, s: int, h: int) -> np.ndarray:
    """Softmax row ``p`` (length ``seq_lens[s]``) of sequence s, head h."""
    S, Hq, D, NB, BS, Hkv = _check_shapes(query, k_cache, v_cache, block_tables, seq_lens)
    L = int(seq_lens[s])
    kvh = kv_head_of(h, Hq, Hkv)
    K = decode_values(gather_rows(k_cache, block_tables[s], L, kvh), dtype)
    V = decode_values(gather_rows(v_cache, block_tables[s], L, kvh), dtype)
    _, p = softmax_attention(decode_values(query[s, h], dtype), K, V, scale)
    return p


def paged_decode_partials_ref(query, k_cache, v_cache, block_tables, seq_lens, scale: float,
                              dtype: str, partition_size: int, seqs=None):
    """Split-context partials, float64.

    Partition p of sequence s covers tokens
    ``[p * partition_size, min((p + 1) * partition_size, L))``; only the
    ``ceil(L / partition_size)`` non-empty partitions exist.  For each one:
    ``m_p = max_t z_t``, ``l_p = sum_t exp(z_t - m_p)`` and
    ``o_p = sum_t exp(z_t - m_p) V_t / l_p`` with ``z_t = scale <q, K_t>``.
    Returns ``{(s, h): [(m_p, l_p, o_p), ...]}``.
    """
    S, Hq, D, NB, BS, Hkv = _check_shapes(query, k_cache, v_cache, block_tables, seq_lens)
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    seqs = range(S) if seqs is None else list(seqs)
    parts = {}
    for s in seqs:
        L = int(seq_lens[s])
        q = decode_values(query[s], dtype)
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            K = decode_values(gather_rows(k_cache, block_tables[s], L, kvh), dtype)
            V = decode_values(gather_rows(v_cache, block_tables[s], L, kvh), dtype)
            plist = []
            for p0 in range(0, L, partition_size):
                Kp, Vp = K[p0:p0 + partition_size], V[p0:p0 + partition_size]
                z = scale * (Kp @ q[h])
                m = z.max()
                e = np.exp(z - m)
                l = e.sum()
                plist.append((m, l, (e @ Vp) / l))
            parts[(s, h)] = plist
    return parts


def lse_combine_ref(plist, head_size: int) -> np.ndarray:
    """Merge partition partials by log-sum-exp weighting.

    ``M = max_p m_p``, ``w_p = l_p exp(m_p - M)``,
    ``out = sum_p w_p o_p / sum_p w_p``; no partitions gives zeros.
    """
    if not plist:
        return np.zeros(head_size, dtype=np.float64)
    M = max(m for m, _, _ in plist)
    w = np.array([l * math.exp(m - M) for m, l, _ in plist])
    o = np.stack([o for _, _, o in plist])
    return (w @ o) / w.sum()


def reshape_and_cache_ref(key, value, k_cache, v_cache, slot_mapping):
    """Scatter each new token's K/V row into its cache slot (returns copies).

    csdn section 4, point 3 (gather-scatter replaces contiguous access) and
    section 2, step 4 (a new token is appended to its sequence's blocks):
    token i goes to physical block ``slot // block_size`` at offset
    ``slot % block_size``; a negative slot means "no write".  Elements are
    copied as stored (no conversion), so the result is bit-exact by
    construction.  ``key``/``value``: ``[num_tokens, num_kv_heads, head_size]``.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    block_size = kc.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        kc[blk, off] = key[i]
        vc[blk, off] = value[i]
    return kc, vc


def copy_blocks_ref(k_cache, v_cache, src, dst):
    """Copy whole blocks in both pools: block ``dst[i]`` becomes a copy of
    block ``src[i]`` as it was before the call (returns copies).

    csdn section 1: reference counts give copy-on-write, so a shared block is
    copied before a sequence writes into it.  Pairs naming a block outside the
    pool are skipped.  Elements are copied as stored (bit-exact).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb = kc.shape[0]
    for s, d in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        if 0 <= s < nb and 0 <= d < nb:
            kc[d] = k_cache[s]
            vc[d] = v_cache[s]
    return kc, vc


def reshape_and_cache_fp8_ref(key, value, k_cache, v_cache, slot_mapping, dtype: str, k_scale: float,
                              v_scale: float):
    """Scatter with quantisation: as ``reshape_and_cache_ref``, but the rows
    of ``key`` / ``value`` (stored as ``dtype``) are written as E4M3 codes of
    ``x / k_scale`` / ``x / v_scale`` (``quantize_e4m3_ref``).  Returns copies
    of the code pools."""
    kq = quantize_e4m3_ref(decode_values(key, dtype), k_scale)
    vq = quantize_e4m3_ref(decode_values(value, dtype), v_scale)
    return reshape_and_cache_ref(kq, vq, k_cache, v_cache, slot_mapping)


def paged_prefill_ref(query, k_cache, v_cache, block_tables, seq_lens, query_start, scale: float, dtype: str,
                      seqs=None, kv_dtype: str | None = None, k_scale: float = 1.0,
                      v_scale: float = 1.0) -> np.ndarray:
    """Several new tokens per sequence attending over the paged cache, causally.

    yangyitao.com vLLM book preface (overview figure and its list): prefill,
    decode and speculative decoding are one operation, giving a request N new
    tokens; is96.com essay: chunked prefill cuts a long prompt into pieces
    processed step by step.  Reading: the ``n = query_start[s+1] -
    query_start[s]`` query rows of sequence s (packed in ``query[T, Hq, D]``)
    are its last n tokens, whose K/V are already in the cache, so row i sits at
    position ``p = seq_lens[s] - n + i`` and attends to tokens ``0 .. p``
    (causal; decode is ``n = 1``).  Returns float64 ``[T, Hq, D]`` (rows of
    sequences outside ``seqs`` stay zero).
    """
    T, Hq, D = query.shape
    NB, BS, Hkv, Dk = k_cache.shape
    S = len(seq_lens)
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or len(query_start) != S + 1:
        raise ValueError("shape mismatch")
    kvt = kv_dtype or dtype
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        a, b, L = int(query_start[s]), int(query_start[s + 1]), int(seq_lens[s])
        n = b - a
        if n > L:
            raise ValueError("a sequence has more query rows than tokens")
        for kvh in range(Hkv):
            K = decode_values(gather_rows(k_cache, block_tables[s], L, kvh), kvt) * k_scale
            V = decode_values(gather_rows(v_cache, block_tables[s], L, kvh), kvt) * v_scale
            for i in range(n):
                p = L - n + i
                q = decode_values(query[a + i], dtype)
                for h in range(Hq):
                    if kv_head_of(h, Hq, Hkv) == kvh:
                        out[a + i, h], _ = softmax_attention(q[h], K[:p + 1], V[:p + 1], scale)
    return out
