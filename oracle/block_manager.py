"""Plain reference of the host-side block bookkeeping. TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may use this module; the product's block manager is the C++
one behind include/pa.h (pa_bm_*), which shares no code with it.

What the pages fix:

* "How PagedAttention works", section "A strong answer": the pool is split
  into blocks of one size, every sequence has its own table of block ids, at
  most a sequence's final block has unused slots; the feature table: a shared
  prefix is a single set of blocks counted by reference, a fork shares its
  parent's blocks and copies a block only when a branch writes to it (copy on
  write), preemption moves whole blocks out to host memory;
* same page, section "What interviewers probe next": admitting a request needs
  ceil(prompt tokens / block size) free blocks plus at least one to grow into,
  and a small watermark reserve is kept so decode steps do not starve;
* lihaoran.work explainer, section "How many tail slots remain unused?": a
  sequence of T positions holds ceil(T / b) blocks, an empty one none.

Readings where the pages are silent (the C++ manager follows the same ones):

* allocation order: the lowest-numbered free block first (device and host
  pools alike), so placements are reproducible;
* the watermark applies to admission only; growth of running sequences may
  use the reserve;
* a batch of appends is all-or-nothing: if the pool cannot cover every fresh
  block the batch needs, nothing changes and NoSpace is raised;
* swap-out copies each of the sequence's blocks to its own host block (blocks
  shared with other sequences stay on the device for them); swap-in gives
  each host block a fresh device block.  A swapped-out sequence cannot grow,
  fork or be read until it is swapped back in.
"""

from __future__ import annotations

import heapq


class NoSpace(Exception):
    """The pool cannot cover the request; the scheduler must wait or preempt."""


def blocks_for(tokens: int, block_size: int) -> int:
    """ceil(tokens / block_size): the lihaoran.work explainer, section "How many
    tail slots remain unused?"."""
    if tokens < 0 or block_size <= 0:
        raise ValueError("bad sizes")
    return -(-tokens // block_size)


class _Pool:
    def __init__(self, n: int):
        self.free = list(range(n))       # a heap: lowest id out first
        heapq.heapify(self.free)
        self.ref = [0] * n

    def take(self) -> int:
        if not self.free:
            raise NoSpace("pool exhausted")
        blk = heapq.heappop(self.free)
        self.ref[blk] = 1
        return blk

    def drop(self, blk: int) -> None:
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            heapq.heappush(self.free, blk)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, watermark: int = 0,
                 num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or watermark < 0 or num_host_blocks < 0:
            raise ValueError("bad sizes")
        self.block_size = block_size
        self.watermark = watermark
        self.dev = _Pool(num_blocks)
        self.host = _Pool(num_host_blocks)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.swapped: set[int] = set()

    # -- admission ------------------------------------------------------------
    def can_admit(self, prompt_tokens: int) -> bool:
        """ceil(prompt / b) blocks plus one to grow into, above the watermark."""
        need = blocks_for(prompt_tokens, self.block_size) + 1
        return len(self.dev.free) - self.watermark >= need

    def admit(self, seq: int, prompt_tokens: int) -> None:
        if seq in self.tables:
            raise ValueError("sequence id in use")
        if not self.can_admit(prompt_tokens):
            raise NoSpace("admission")
        self.tables[seq] = [self.dev.take() for _ in range(blocks_for(prompt_tokens, self.block_size))]
        self.lens[seq] = prompt_tokens

    # -- sharing --------------------------------------------------------------
    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (reference counts + 1)."""
        if parent not in self.tables or child in self.tables or parent in self.swapped:
            raise ValueError("bad fork")
        self.tables[child] = list(self.tables[parent])
        for blk in self.tables[child]:
            self.dev.ref[blk] += 1
        self.lens[child] = self.lens[parent]

    # -- growth ---------------------------------------------------------------
    def append_slots(self, seqs):
        """Reserve the slot of each sequence's next token (position lens[seq]).

        A sequence whose blocks are all full takes a fresh block; one whose
        last block is shared gets a private copy first (copy on write: the
        pair (shared, copy) is reported and the shared block loses one
        reference).  Returns (slots, cow_pairs).  All or nothing."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.tables or s in self.swapped
                                              for s in seqs):
            raise ValueError("bad sequence list")
        fresh = sum(1 for s in seqs if self._needs_block(s))
        if fresh > len(self.dev.free):
            raise NoSpace("append")
        slots, cow = [], []
        b = self.block_size
        for s in seqs:
            pos = self.lens[s]
            table = self.tables[s]
            if pos % b == 0:
                table.append(self.dev.take())
            elif self.dev.ref[table[-1]] > 1:
                shared = table[-1]
                copy = self.dev.take()
                self.dev.drop(shared)
                table[-1] = copy
                cow.append((shared, copy))
            slots.append(table[pos // b] * b + pos % b)
            self.lens[s] = pos + 1
        return slots, cow

    def _needs_block(self, s: int) -> bool:
        pos = self.lens[s]
        return pos % self.block_size == 0 or self.dev.ref[self.tables[s][-1]] > 1

    # -- release and preemption -------------------------------------------------
    def release(self, seq: int) -> None:
        if seq not in self.tables:
            raise ValueError("unknown sequence")
        pool = self.host if seq in self.swapped else self.dev
        for blk in self.tables.pop(seq):
            pool.drop(blk)
        del self.lens[seq]
        self.swapped.discard(seq)

    def swap_out(self, seq: int):
        """Move the sequence to host blocks; returns (device, host) pairs."""
        if seq not in self.tables or seq in self.swapped:
            raise ValueError("bad swap-out")
        table = self.tables[seq]
        if len(table) > len(self.host.free):
            raise NoSpace("host pool")
        pairs = []
        for i, blk in enumerate(table):
            h = self.host.take()
            pairs.append((blk, h))
            self.dev.drop(blk)
            table[i] = h
        self.swapped.add(seq)
        return pairs

    def swap_in(self, seq: int):
        """Bring a swapped-out sequence back; returns (host, device) pairs."""
        if seq not in self.swapped:
            raise ValueError("bad swap-in")
        table = self.tables[seq]
        if len(table) > len(self.dev.free):
            raise NoSpace("swap-in")
        pairs = []
        for i, h in enumerate(table):
            d = self.dev.take()
            pairs.append((h, d))
            self.host.drop(h)
            table[i] = d
        self.swapped.discard(seq)
        return pairs

    # -- decode inputs ----------------------------------------------------------
    def decode_inputs(self, seqs, max_blocks: int, pad_block: int):
        """Block-table rows (padded with pad_block) and lengths for a batch."""
        tables, lens = [], []
        for s in seqs:
            if s not in self.tables or s in self.swapped or len(self.tables[s]) > max_blocks:
                raise ValueError("bad batch")
            row = self.tables[s] + [pad_block] * (max_blocks - len(self.tables[s]))
            tables.append(row)
            lens.append(self.lens[s])
        return tables, lens

    def free_blocks(self) -> int:
        return len(self.dev.free)

    def free_host_blocks(self) -> int:
        return len(self.host.free)
