"""Seeded random operation traces for the block manager (test input generator).

Holds no block-manager logic: it only draws operations.  Whether an operation
is valid is decided by the manager under test, so invalid ones (unknown or
duplicate ids, oversize requests) are drawn on purpose now and then.
"""

from __future__ import annotations

import numpy as np


def random_trace(seed: int, n_ops: int, max_seqs: int, block_size: int, max_tokens: int):
    """A list of (op, args) with op in allocate / append / fork / free."""
    rng = np.random.default_rng(np.random.SeedSequence([291, 7, seed]))
    live: list[int] = []
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        free_ids = [i for i in range(max_seqs) if i not in live]
        if r < 0.03:                                       # deliberately odd requests
            kind = rng.integers(0, 4)
            if kind == 0:
                ops.append(("free", (int(rng.integers(0, max_seqs)),)))
            elif kind == 1:
                ops.append(("allocate", (int(rng.integers(0, max_seqs)), int(rng.integers(0, 40 * max_tokens)))))
            elif kind == 2:
                ops.append(("append", (int(rng.integers(0, max_seqs)), int(rng.integers(0, 40 * max_tokens)))))
            else:
                ops.append(("fork", (int(rng.integers(0, max_seqs)), int(rng.integers(0, max_seqs)))))
            continue
        if (r < 0.30 or not live) and free_ids:
            s = int(rng.choice(free_ids))
            n = int(rng.integers(0, max_tokens + 1))
            ops.append(("allocate", (s, n)))
            live.append(s)
        elif r < 0.70 and live:
            s = int(rng.choice(live))
            n = 1 if rng.random() < 0.6 else int(rng.integers(0, 2 * block_size + 3))
            ops.append(("append", (s, n)))
        elif r < 0.82 and live and free_ids:
            p = int(rng.choice(live))
            c = int(rng.choice(free_ids))
            ops.append(("fork", (p, c)))
            live.append(c)
        elif live:
            s = int(rng.choice(live))
            ops.append(("free", (s,)))
            live.remove(s)
    return ops
