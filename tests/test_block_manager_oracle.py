"""Pins of the block-manager oracle (CPU): the pages' block-pool figure,
brute-force contents through the tables, reference-count conservation,
all-or-nothing operations, and planted mistakes that each pin must catch."""

from __future__ import annotations

import copy
import json
import os

import pytest

from oracle.block_manager import BlockManagerRef, BlockManagerError, Capacity, InvalidArg, NoBlocks, blocks_for
from bm_traces import random_trace

HERE = os.path.dirname(os.path.abspath(__file__))


def run_op(m, op, args):
    if op == "allocate":
        return m.allocate(*args)
    if op == "append":
        return m.append_slots(*args)
    if op == "fork":
        return m.fork(*args)
    return m.free_seq(*args)


def test_block_pool_figure():
    """[preface] 'from OS to GPU' figure: A -> B1/B3/B7, B -> B2/B5, freed B4/B6 -> a new request."""
    g = json.load(open(os.path.join(HERE, "golden", "block_manager_figure.json")))
    m = BlockManagerRef(g["num_blocks"], g["block_size"], 8, 8)
    ids = {}
    for op, name, *rest in g["ops"]:
        seq = ids.setdefault(name, len(ids))
        run_op(m, op, (seq, *rest))
    for name, want in g["tables"].items():
        assert m.block_table(ids[name]) == want, name
        assert m.seq_len(ids[name]) == g["seq_lens"][name]
    assert m.num_free() == g["num_free"]
    assert set(g["tables"]["C"]) == {4, 6}


class ContentModel:
    """Brute-force device memory: every slot holds the id of the token written
    there; copies move whole blocks.  A sequence's tokens, read back through
    its table, must be exactly the tokens it was given (a fork inherits its
    parent's)."""

    def __init__(self, m):
        self.m = m
        self.mem = {}
        self.want = {}
        self.next = 1

    def apply(self, op, args):
        before = copy.deepcopy((self.m.tables, self.m.lens, self.m.free, self.m.ref, self.m.copies))
        try:
            res = run_op(self.m, op, args)
        except BlockManagerError:
            after = (self.m.tables, self.m.lens, self.m.free, self.m.ref, self.m.copies)
            assert after == before, f"failed {op}{args} changed the state"
            return False
        bs = self.m.block_size
        for src, dst in self.m.take_copies():           # copies land before the new tokens
            for o in range(bs):
                if src * bs + o in self.mem:
                    self.mem[dst * bs + o] = self.mem[src * bs + o]
                else:
                    self.mem.pop(dst * bs + o, None)
        if op in ("allocate", "append"):
            seq = args[0]
            toks = list(range(self.next, self.next + len(res)))
            self.next += len(res)
            for slot, v in zip(res, toks):
                self.mem[slot] = v
            self.want[seq] = (self.want.get(seq, []) if op == "append" else []) + toks
        elif op == "fork":
            self.want[args[1]] = list(self.want[args[0]])
        else:
            del self.want[args[0]]
        return True

    def check(self):
        m, bs = self.m, self.m.block_size
        for s, toks in self.want.items():
            t = m.block_table(s)
            assert len(t) == blocks_for(len(toks), bs) and m.seq_len(s) == len(toks)
            got = [self.mem.get(t[i // bs] * bs + i % bs) for i in range(len(toks))]
            assert got == toks, f"sequence {s} reads {got} instead of {toks}"
        # reference counts are the number of table entries naming a block; the
        # pool holds exactly the unreferenced blocks, once each
        cnt = [0] * m.num_blocks
        for t in m.tables.values():
            for b in t:
                cnt[b] += 1
        assert cnt == m.ref
        assert sorted(m.free) == [b for b in range(m.num_blocks) if cnt[b] == 0]
        assert len(set(m.free)) == len(m.free)


@pytest.mark.parametrize("seed", range(12))
def test_contents_through_tables(seed):
    bs = [1, 2, 4, 16][seed % 4]
    m = BlockManagerRef(num_blocks=40 + seed, block_size=bs, max_seqs=10, max_blocks_per_seq=12)
    cm = ContentModel(m)
    ok = 0
    for op, args in random_trace(seed, 600, 10, bs, 3 * bs):
        ok += cm.apply(op, args)
        cm.check()
    assert ok > 300


def test_closed_forms():
    m = BlockManagerRef(10, 4, 4, 10)
    assert m.allocate(0, 9) == list(range(9))          # a fresh pool hands out 0, 1, 2 in order
    assert m.block_table(0) == [0, 1, 2] and m.num_free() == 7
    assert m.append_slots(0, 3) == [9, 10, 11]         # fills block 2
    assert m.append_slots(0, 1) == [12]                # block 3
    m.fork(0, 1)
    assert [m.ref_count(b) for b in range(4)] == [2, 2, 2, 2]
    assert m.append_slots(1, 1) == [4 * 4 + 1]         # shared, partly filled: copied to block 4
    assert m.take_copies() == [(3, 4)]
    assert m.ref_count(3) == 1 and m.ref_count(4) == 1
    assert m.append_slots(0, 1) == [13]                # block 3 is now private: written in place
    assert m.take_copies() == []
    m.free_seq(0)                                      # 0, 1, 2 shared with seq 1; 3 freed
    assert m.free[-1] == 3 and m.ref_count(0) == 1
    m.free_seq(1)
    assert m.num_free() == 10
    assert m.free[-5:] == [3, 0, 1, 2, 4]              # table order: 0, 1, 2, 4 on top of 3


def test_full_shared_block_is_not_copied():
    m = BlockManagerRef(6, 4, 3, 6)
    m.allocate(0, 8)
    m.fork(0, 1)
    assert m.append_slots(1, 1) == [2 * 4]             # new block 2, nothing copied
    assert m.take_copies() == []


def test_errors_leave_state_unchanged():
    m = BlockManagerRef(4, 4, 3, 3)
    m.allocate(0, 5)
    snap = copy.deepcopy(m.__dict__)
    for op, args, exc in [("allocate", (0, 1), InvalidArg), ("allocate", (3, 1), InvalidArg),
                          ("allocate", (1, 13), Capacity), ("allocate", (1, -1), InvalidArg),
                          ("append", (2, 1), InvalidArg), ("append", (0, 8), Capacity),
                          ("fork", (1, 2), InvalidArg), ("fork", (0, 0), InvalidArg),
                          ("free", (2,), InvalidArg)]:
        with pytest.raises(exc):
            run_op(m, op, args)
        assert m.__dict__ == snap
    m.allocate(1, 8)                                   # pool now empty
    with pytest.raises(NoBlocks):
        m.append_slots(0, 4)
    m.fork(0, 2)
    with pytest.raises(NoBlocks):                      # the copy needs a block
        m.append_slots(2, 1)


def test_freed_copy_destination_is_dropped():
    m = BlockManagerRef(6, 4, 3, 6)
    m.allocate(0, 2)
    m.fork(0, 1)
    m.append_slots(1, 1)
    m.free_seq(1)
    assert m.take_copies() == []


# ---- planted mistakes: each must be caught by the pins above


class NoCopy(BlockManagerRef):
    def append_slots(self, seq, n):
        L = self.lens.get(seq, 0)
        if seq in self.tables and n > 0 and L % self.block_size and self.ref[self.tables[seq][-1]] > 1:
            self.ref[self.tables[seq][-1]] += 0            # forgets copy-on-write
            res = []
            for _ in range(n):
                t = self.tables[seq]
                if self.lens[seq] % self.block_size == 0:
                    t.append(self._take())
                res.append(self._slot(seq, self.lens[seq]))
                self.lens[seq] += 1
            return res
        return super().append_slots(seq, n)


class NoDecrement(BlockManagerRef):
    def free_seq(self, seq):
        t = self.tables.pop(seq)
        del self.lens[seq]
        for b in t:
            if self.ref[b] == 1:
                self.ref[b] = 0
                self.free.append(b)


class FifoPool(BlockManagerRef):
    def _take(self):
        b = self.free.pop(0)
        self.ref[b] = 1
        return b


@pytest.mark.parametrize("cls", [NoCopy, NoDecrement])
def test_planted_mistakes_fail_content_pins(cls):
    failed = False
    for seed in range(6):
        m = cls(num_blocks=40, block_size=4, max_seqs=10, max_blocks_per_seq=12)
        cm = ContentModel(m)
        try:
            for op, args in random_trace(seed, 400, 10, 4, 12):
                cm.apply(op, args)
                cm.check()
        except AssertionError:
            failed = True
            break
    assert failed


def test_planted_pool_order_fails_figure():
    g = json.load(open(os.path.join(HERE, "golden", "block_manager_figure.json")))
    m = FifoPool(g["num_blocks"], g["block_size"], 8, 8)
    m.free = list(range(g["num_blocks"]))              # FIFO from the front
    ids = {}
    for op, name, *rest in g["ops"]:
        seq = ids.setdefault(name, len(ids))
        run_op(m, op, (seq, *rest))
    assert m.block_table(ids["C"]) != g["tables"]["C"]


def test_append_batch_is_sequential_appends_or_nothing():
    import random
    for seed in range(20):
        r = random.Random(seed)
        m = BlockManagerRef(30, 4, 8, 8)
        for op, args in random_trace(seed, 60, 8, 4, 12):
            try:
                run_op(m, op, args)
            except BlockManagerError:
                pass
        live = sorted(m.tables)
        if not live:
            continue
        batch = r.sample(live, r.randint(1, len(live)))
        seq = copy.deepcopy(m)
        try:
            want = [seq.append_slots(s, 1)[0] for s in batch]
        except BlockManagerError:
            want = None
        snap = copy.deepcopy(m.__dict__)
        try:
            got = m.append_batch(batch)
        except BlockManagerError:
            got = None
            assert m.__dict__ == snap                      # nothing changed
        assert got == want
        if got is not None:
            assert m.__dict__ == seq.__dict__
