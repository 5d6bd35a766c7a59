"""Plain reference model of the paged KV block manager (pure Python).

TEST INFRASTRUCTURE ONLY (see the package docstring): tests are its only
callers; the native manager behind the C ABI shares no code with it.

Sources (pages on the subject, cited by title and section):

* devpress.csdn.net article on the vLLM architecture, section 1 (the engine
  process's KV-cache manager): GPU memory is cut into fixed-size blocks kept
  in one global pool of free blocks; the manager answers a sequence's request
  for blocks and keeps the mapping from its logical blocks to physical ones;
  reference counts give copy-on-write, so blocks can be shared (beam search).
* same article, section 2, part 2 (scheduling and memory): when a request is
  scheduled the manager takes physical blocks from the free pool and builds
  the sequence's block table; part 4 (sampling): a new token joins its
  sequence, and if that needs a new physical block the manager is asked again.
* yangyitao.com vLLM book preface, section "from OS to GPU" (block-pool
  figure): blocks are handed out on demand; blocks a finished request frees go
  straight to new requests.
* aiflowlearn.net vLLM course page: a block holds 16 tokens (any block size
  works here).

Readings where the pages are silent (each is listed in the design notes):

* the free pool is a stack: the block freed last is handed out first (in the
  figure, blocks a finished request frees are handed straight to the next
  one); a new pool hands out block 0 first, then 1, 2, ...;
* a sequence's blocks are released in table order (logical block 0 first), so
  its last block is on top of the pool afterwards;
* token t of a sequence goes to slot ``table[t // block_size] * block_size +
  t % block_size``;
* copy-on-write happens on the first write into a shared block: a sequence
  that appends while its last block is partly filled and shared (reference
  count > 1) gets a fresh block in its place and a (shared, fresh) copy is
  queued; a full shared last block is never written, so appending past it
  only takes a new block;
* ``fork`` makes a child that shares all of the parent's blocks (the
  beam-search case of section 1);
* every operation either succeeds or leaves the state unchanged: not enough
  free blocks raises ``NoBlocks``, a table longer than ``max_blocks_per_seq``
  raises ``Capacity``, an unknown / duplicate sequence or a bad size raises
  ``InvalidArg``;
* a queued copy whose destination block is freed before the copies are taken
  is dropped (its data would belong to nobody).
"""

from __future__ import annotations


class BlockManagerError(Exception):
    status = -1


class InvalidArg(BlockManagerError):
    status = -1


class NoBlocks(BlockManagerError):
    status = -5


class Capacity(BlockManagerError):
    status = -6


def blocks_for(num_tokens: int, block_size: int) -> int:
    return -(-num_tokens // block_size)


class BlockManagerRef:
    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int):
        if num_blocks < 0 or block_size <= 0 or max_seqs < 0 or max_blocks_per_seq < 0:
            raise InvalidArg("bad sizes")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks - 1, -1, -1))   # top of the stack is the end
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.copies: list[tuple[int, int]] = []

    # -- helpers
    def _check_new(self, seq: int):
        if not (0 <= seq < self.max_seqs) or seq in self.tables:
            raise InvalidArg(f"sequence {seq} is not a free id")

    def _check_live(self, seq: int):
        if seq not in self.tables:
            raise InvalidArg(f"sequence {seq} does not exist")

    def _take(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def _slot(self, seq: int, t: int) -> int:
        return self.tables[seq][t // self.block_size] * self.block_size + t % self.block_size

    # -- operations
    def allocate(self, seq: int, num_tokens: int) -> list[int]:
        """A new sequence holding num_tokens tokens (its prompt): fresh blocks."""
        self._check_new(seq)
        if num_tokens < 0:
            raise InvalidArg("negative length")
        nb = blocks_for(num_tokens, self.block_size)
        if nb > self.max_blocks_per_seq:
            raise Capacity("table full")
        if nb > len(self.free):
            raise NoBlocks("pool exhausted")
        self.tables[seq] = [self._take() for _ in range(nb)]
        self.lens[seq] = num_tokens
        return [self._slot(seq, t) for t in range(num_tokens)]

    def append_slots(self, seq: int, n: int) -> list[int]:
        """n new tokens at the end of seq; returns their slots."""
        self._check_live(seq)
        if n < 0:
            raise InvalidArg("negative count")
        L = self.lens[seq]
        table = self.tables[seq]
        grow = blocks_for(L + n, self.block_size) - len(table)
        cow = n > 0 and L % self.block_size != 0 and self.ref[table[-1]] > 1
        if blocks_for(L + n, self.block_size) > self.max_blocks_per_seq:
            raise Capacity("table full")
        if grow + (1 if cow else 0) > len(self.free):
            raise NoBlocks("pool exhausted")
        if cow:
            old = table[-1]
            new = self._take()
            self.ref[old] -= 1
            table[-1] = new
            self.copies.append((old, new))
        for _ in range(grow):
            table.append(self._take())
        self.lens[seq] = L + n
        return [self._slot(seq, t) for t in range(L, L + n)]

    def append_batch(self, seqs) -> list[int]:
        """One more token for each sequence of the batch, in order; all or
        nothing (the state is restored if any append fails)."""
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("duplicate sequence in the batch")
        for s in seqs:                                     # errors: ids, then capacity, then blocks
            self._check_live(s)
        for s in seqs:
            if blocks_for(self.lens[s] + 1, self.block_size) > self.max_blocks_per_seq:
                raise Capacity("table full")
        saved = ({k: list(v) for k, v in self.tables.items()}, dict(self.lens), list(self.free),
                 list(self.ref), list(self.copies))
        try:
            return [self.append_slots(s, 1)[0] for s in seqs]
        except BlockManagerError:
            self.tables, self.lens, self.free, self.ref, self.copies = saved
            raise

    def fork(self, parent: int, child: int):
        """child shares every block of parent."""
        self._check_live(parent)
        self._check_new(child)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int):
        """Release seq; blocks nobody else holds go back on top of the pool."""
        self._check_live(seq)
        released = []
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                released.append(b)
        del self.lens[seq]
        if released:
            gone = set(released)
            self.copies = [(s, d) for (s, d) in self.copies if d not in gone]

    def take_copies(self) -> list[tuple[int, int]]:
        out, self.copies = self.copies, []
        return out

    # -- queries
    def num_free(self) -> int:
        return len(self.free)

    def ref_count(self, block: int) -> int:
        return self.ref[block]

    def seq_len(self, seq: int) -> int:
        return self.lens.get(seq, -1)

    def block_table(self, seq: int) -> list[int]:
        self._check_live(seq)
        return list(self.tables[seq])

    def block_tables(self, seqs) -> tuple[list[list[int]], list[int]]:
        """Rows padded with -1 to max_blocks_per_seq, and the lengths."""
        rows, lens = [], []
        for s in seqs:
            t = self.block_table(s)
            rows.append(t + [-1] * (self.max_blocks_per_seq - len(t)))
            lens.append(self.lens[s])
        return rows, lens
