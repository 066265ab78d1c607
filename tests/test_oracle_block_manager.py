"""Pins for the block-manager oracle: the pages' numbers, the copy-on-write
and sharing rules, and a ledger invariant under random operation streams.
The planted-mistake tests swap a wrong piece into the oracle (on the CPU) and
assert that a pin then fails."""

import numpy as np
import pytest

import oracle
from oracle import block_manager as obm
from oracle.block_manager import BlockManager, NoSpace


def pin_request_blocks():
    """A 600 + 250 token chat request holds 54 blocks of 16 ("How PagedAttention
    works", worked example: 850 tokens -> 54 blocks)."""
    bm = BlockManager(100, 16)
    bm.admit(1, 600)
    bm.append_slots([1])
    for _ in range(249):
        bm.append_slots([1])
    return len(bm.tables[1]) == 54 and bm.free_blocks() == 46


def pin_admission_rule():
    """Admission needs ceil(prompt / 16) + 1 free blocks above the watermark
    (same page, "What interviewers probe next")."""
    need = -(-600 // 16) + 1                       # 39
    ok = BlockManager(need, 16).can_admit(600)
    short = BlockManager(need - 1, 16).can_admit(600)
    wm_ok = BlockManager(need + 5, 16, watermark=5).can_admit(600)
    wm_short = BlockManager(need + 4, 16, watermark=5).can_admit(600)
    bm = BlockManager(need - 1, 16)
    try:
        bm.admit(7, 600)
        raised = False
    except NoSpace:
        raised = True
    return ok and not short and wm_ok and not wm_short and raised and bm.free_blocks() == need - 1


def pin_shared_prefix():
    """A 2,000-token prefix shared by 200 sequences is one set of 125 blocks with
    a reference count of 200 (same page, the 2,000-token, 200-conversation case)."""
    bm = BlockManager(400, 16)
    bm.admit(0, 2000)
    for s in range(1, 200):
        bm.fork(0, s)
    used = {b for t in bm.tables.values() for b in t}
    return (len(used) == 125 and all(bm.dev.ref[b] == 200 for b in used)
            and bm.free_blocks() == 400 - 125)


def pin_copy_on_write():
    """A fork copies only the block that diverges, once: the child's first
    append into a shared, partly filled block gets a private copy; the parent
    keeps its block; a fork whose last block is full copies nothing."""
    bm = BlockManager(20, 4)
    bm.admit(1, 10)                               # blocks 0,1,2; block 2 half full
    bm.fork(1, 2)
    slots, cow = bm.append_slots([2])
    if cow != [(2, 3)] or slots != [3 * 4 + 2] or bm.tables[1] != [0, 1, 2]:
        return False
    if bm.dev.ref[2] != 1 or bm.dev.ref[3] != 1 or bm.dev.ref[0] != 2:
        return False
    slots, cow = bm.append_slots([1, 2])          # parent writes its own block now
    if cow != [] or slots != [2 * 4 + 2, 3 * 4 + 3]:
        return False
    bm2 = BlockManager(20, 4)
    bm2.admit(1, 8)                               # two full blocks
    bm2.fork(1, 2)
    slots, cow = bm2.append_slots([2])
    return cow == [] and slots == [2 * 4] and bm2.tables[2] == [0, 1, 2]


def _ledger_ok(bm):
    """Reference counts equal the number of tables holding each block, the free
    list is exactly the unreferenced blocks, and every resident sequence of
    length T holds ceil(T / b) blocks."""
    for pool, swapped in ((bm.dev, False), (bm.host, True)):
        count = [0] * len(pool.ref)
        for s, t in bm.tables.items():
            if (s in bm.swapped) == swapped:
                for b in t:
                    count[b] += 1
        if count != pool.ref or sorted(pool.free) != [b for b, c in enumerate(count) if c == 0]:
            return False
    return all(len(t) == oracle.block_layout(bm.lens[s], bm.block_size)[0]
               for s, t in bm.tables.items())


def random_ops(bm, rng, steps, ids):
    """Admit / fork / append / release / swap at random; returns the log of
    every result (the parity test replays the same stream on the C++ side)."""
    log = []
    for _ in range(steps):
        live = sorted(s for s in bm.tables if s not in bm.swapped)
        op = rng.integers(0, 7)
        try:
            if op == 0 or not live:
                s = next(ids)
                n = int(rng.integers(0, 40))
                log.append(("admit", s, n, bm.can_admit(n)))
                bm.admit(s, n)
            elif op == 1:
                s = next(ids)
                p = int(rng.choice(live))
                log.append(("fork", p, s))
                bm.fork(p, s)
            elif op in (2, 3):
                batch = [int(x) for x in rng.choice(live, size=min(len(live), 3), replace=False)]
                log.append(("append", batch, bm.append_slots(batch)))
            elif op == 4:
                s = int(rng.choice(live))
                log.append(("release", s))
                bm.release(s)
            elif op == 5:
                s = int(rng.choice(live))
                log.append(("swap_out", s, bm.swap_out(s)))
            elif bm.swapped:
                s = sorted(bm.swapped)[0]
                log.append(("swap_in", s, bm.swap_in(s)))
        except NoSpace:
            log.append(("nospace",))
    return log


def pin_ledger_random_streams():
    rng = np.random.default_rng(41)
    for trial in range(4):
        bm = BlockManager(60, 4, watermark=trial, num_host_blocks=30)
        random_ops(bm, rng, 300, iter(range(10_000)))
        if not _ledger_ok(bm):
            return False
    return True


def _lookup(k_pool, v_pool, table, n, bs):
    """Position-by-position read of a sequence through its table (test side)."""
    return (np.stack([k_pool[table[t // bs], :, t % bs] for t in range(n)]),
            np.stack([v_pool[table[t // bs], :, t % bs] for t in range(n)]))


def pin_swap_round_trip_content():
    """Preemption moves a sequence's content, not just its ids ("How
    PagedAttention works", feature table: blocks swap to host memory and
    back).  Content is moved with the oracle's block swap along the pairs the
    manager reports; in between, another sequence reuses the freed device
    blocks and overwrites them.  The swapped sequence read through its new
    table afterwards is byte-identical to before, and so is the fork that
    still shares its first block on the device."""
    rng = np.random.default_rng(53)
    bs, hkv, d = 4, 2, 3
    bm = BlockManager(10, bs, num_host_blocks=6)
    dev_k = np.full((10, hkv, bs, d), np.nan)
    dev_v = np.full((10, hkv, bs, d), np.nan)
    host_k = np.full((6, hkv, bs, d), np.nan)
    host_v = np.full((6, hkv, bs, d), np.nan)

    def write(seq, start, n):
        for t in range(start, start + n):
            blk = bm.tables[seq][t // bs]
            dev_k[blk, :, t % bs] = rng.standard_normal((hkv, d))
            dev_v[blk, :, t % bs] = rng.standard_normal((hkv, d))

    bm.admit(1, 11)                        # 3 blocks, the last one 3/4 full
    write(1, 0, 11)
    bm.fork(1, 2)                          # shares all three blocks
    slots, cow = bm.append_slots([2])      # 2 copies the shared last block
    oracle.copy_blocks(dev_k, dev_v, cow)
    write(2, 11, 1)
    before1 = _lookup(dev_k, dev_v, list(bm.tables[1]), 11, bs)
    before2 = _lookup(dev_k, dev_v, list(bm.tables[2]), 12, bs)
    oracle.swap_blocks(host_k, host_v, dev_k, dev_v, bm.swap_out(1))
    bm.admit(3, 8)                         # takes the device block 1 gave up
    write(3, 0, 8)
    oracle.swap_blocks(dev_k, dev_v, host_k, host_v, bm.swap_in(1))
    after1 = _lookup(dev_k, dev_v, list(bm.tables[1]), 11, bs)
    after2 = _lookup(dev_k, dev_v, list(bm.tables[2]), 12, bs)
    same = all(np.array_equal(x, y) for x, y in zip(before1 + before2, after1 + after2))
    return same and bm.free_host_blocks() == 6


ALL_PINS = [pin_request_blocks, pin_admission_rule, pin_shared_prefix, pin_copy_on_write,
            pin_ledger_random_streams, pin_swap_round_trip_content]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin):
    assert pin()


def test_no_space_leaves_state_unchanged():
    bm = BlockManager(3, 4)
    bm.admit(1, 4)
    bm.admit(2, 4)                                 # one block left
    before = (bm.free_blocks(), {s: list(t) for s, t in bm.tables.items()}, dict(bm.lens))
    with pytest.raises(NoSpace):
        bm.append_slots([1, 2])                    # both need a fresh block
    assert (bm.free_blocks(), bm.tables, bm.lens) == before


# ---- planted mistakes ---------------------------------------------------------

def _can_admit_no_growth(self, prompt_tokens):
    return len(self.dev.free) - self.watermark >= obm.blocks_for(prompt_tokens, self.block_size)


def _fork_no_refcount(self, parent, child):
    self.tables[child] = list(self.tables[parent])
    self.lens[child] = self.lens[parent]


def _append_no_cow(self, seqs):
    slots = []
    for s in seqs:
        pos = self.lens[s]
        if pos % self.block_size == 0:
            self.tables[s].append(self.dev.take())
        slots.append(self.tables[s][pos // self.block_size] * self.block_size + pos % self.block_size)
        self.lens[s] = pos + 1
    return slots, []


def _release_leaks(self, seq):
    self.tables.pop(seq)
    del self.lens[seq]
    self.swapped.discard(seq)


def _swap_in_pairs_misordered(self, seq):
    """Reports the (host, device) pairs in reverse while the table keeps its order."""
    pairs = BlockManager.__dict__["_orig_swap_in"](self, seq)
    return [(h, d) for (h, _), (_, d) in zip(pairs, reversed(pairs))]


def _swap_out_keeps_device_ids(self, seq):
    """Moves the blocks to the host in the ledger but leaves the table naming
    the old device ids."""
    table = list(self.tables[seq])
    pairs = BlockManager.__dict__["_orig_swap_out"](self, seq)
    self.tables[seq] = table
    return pairs


PLANTED = [("can_admit", _can_admit_no_growth), ("fork", _fork_no_refcount),
           ("append_slots", _append_no_cow), ("release", _release_leaks),
           ("swap_in", _swap_in_pairs_misordered), ("swap_out", _swap_out_keeps_device_ids)]


@pytest.mark.parametrize("name,bad", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_mistake_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(BlockManager, "_orig_swap_in", BlockManager.swap_in, raising=False)
    monkeypatch.setattr(BlockManager, "_orig_swap_out", BlockManager.swap_out, raising=False)
    monkeypatch.setattr(BlockManager, name, bad)
    failed = False
    for pin in ALL_PINS:
        try:
            if not pin():
                failed = True
        except Exception:
            failed = True
    assert failed, f"no pin caught {bad.__name__}"
