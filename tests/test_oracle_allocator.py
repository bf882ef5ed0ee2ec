"""Pins of the oracle's block allocator (CPU only): a hand-traced example of the rules,
the invariants of refcounted sharing after every operation on seeded random traces, and
all-or-nothing exhaustion."""

import numpy as np
import pytest

from oracle import measures as M
from oracle.allocator import Allocator, InvalidOp, NoBlocks


def test_hand_traced_example():
    """4 blocks of 2 slots, free order [2, 0, 3, 1]; every value below worked out by hand
    from the rules (one block at a time, non-adjacent blocks, slot = block*bs + offset,
    copy-on-write of a shared partial tail, release in logical order)."""
    a = Allocator(4, 2, [2, 0, 3, 1])
    a.add(1)
    slots, cow = a.append(1, 3)          # block 2 (slots 4, 5), then block 0 (slot 0)
    assert slots == [4, 5, 0] and cow == []
    assert a.dump() == ([1, 0, 1, 0], [3, 1])
    a.fork(1, 2)                         # both blocks now held twice
    assert a.dump() == ([2, 0, 2, 0], [3, 1])
    slots, cow = a.append(2, 1)          # tail block 0 is shared and partial -> COW to 3
    assert slots == [7] and cow == [(0, 3)]
    assert a.dump() == ([1, 0, 2, 1], [1])
    slots, cow = a.append(1, 1)          # block 0 is private again: no copy
    assert slots == [1] and cow == []
    slots, cow = a.append(1, 1)          # block 0 full -> next free block 1
    assert slots == [2] and cow == []
    assert a.dump() == ([1, 1, 2, 1], [])
    with pytest.raises(NoBlocks):
        a.append(2, 2)                   # needs one more block, none free
    assert a.dump() == ([1, 1, 2, 1], []) and a.stats()["exhaustion_events"] == 1
    a.release(1)                         # blocks 2, 0, 1 lose a reference in logical order
    assert a.dump() == ([0, 0, 1, 1], [0, 1])
    t, L = a.block_table([2], 3)
    assert t == [[2, 3, -1]] and L == [4]
    a.release(2)
    assert a.dump() == ([0, 0, 0, 0], [0, 1, 2, 3])


def test_first_token_takes_one_block_next_block_when_full():
    """A request is given one block; when it fills it gets a second, which need not be
    adjacent to the first."""
    a = Allocator(8, 16, [5, 2, 7, 0, 1, 3, 4, 6])
    a.add(0)
    s, _ = a.append(0, 1)
    assert s == [5 * 16] and a.stats()["used"] == 1
    s, _ = a.append(0, 15)
    assert s == list(range(81, 96)) and a.stats()["used"] == 1
    s, _ = a.append(0, 1)
    assert s == [2 * 16] and a.stats()["used"] == 2


def test_waste_stat_is_sum_of_unused_slots():
    a = Allocator(100, 16)
    lens = [1, 16, 17, 200, 31]
    for i, L in enumerate(lens):
        a.add(i)
        a.append(i, L)
    assert a.stats()["waste_slots"] == sum(M.unused_slots(L, block_size=16) for L in lens)
    assert a.stats()["waste_slots"] == 15 + 0 + 15 + 8 + 1


def test_invalid_ops_leave_state_unchanged():
    a = Allocator(4, 4)
    a.add(0)
    a.append(0, 5)
    before = (a.dump(), {k: (list(v.blocks), v.n) for k, v in a.seqs.items()})
    for bad in (lambda: a.add(0), lambda: a.append(9, 1), lambda: a.fork(9, 1),
                lambda: a.fork(0, 0), lambda: a.release(9)):
        with pytest.raises(InvalidOp):
            bad()
    assert before == (a.dump(), {k: (list(v.blocks), v.n) for k, v in a.seqs.items()})


def check_invariants(a: Allocator):
    bs = a.block_size
    held = [b for s in a.seqs.values() for b in s.blocks]
    # every reference is a block-table entry of some sequence
    assert sum(a.refcount) == len(held)
    for b in range(a.num_blocks):
        assert a.refcount[b] == held.count(b)
    # free and used partition the pool
    free = list(a.free)
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(a.num_blocks) if a.refcount[b] == 0}
    # a sequence holds exactly ceil(n / bs) blocks
    for s in a.seqs.values():
        assert len(s.blocks) == -(-s.n // bs)
        assert len(set(s.blocks)) == len(s.blocks)


def random_trace(seed, n_ops=400, num_blocks=48, bs=4):
    """Seeded random operations; returns the list of (op, args, outcome)."""
    rng = np.random.default_rng(seed)
    a = Allocator(num_blocks, bs, rng.permutation(num_blocks))
    live, next_id, log = [], 0, []
    for _ in range(n_ops):
        r = rng.random()
        try:
            if r < 0.15 or not live:
                a.add(next_id); live.append(next_id); log.append(("add", next_id, None)); next_id += 1
            elif r < 0.65:
                s = int(rng.choice(live)); n = int(rng.integers(1, 3 * bs))
                slots, cow = a.append(s, n)
                log.append(("append", (s, n), (slots, cow)))
                # written slots are never in a block held by another sequence
                for sl in slots:
                    assert a.refcount[sl // bs] == 1
            elif r < 0.8:
                p = int(rng.choice(live)); a.fork(p, next_id); live.append(next_id)
                log.append(("fork", (p, next_id), None)); next_id += 1
            else:
                s = int(rng.choice(live)); a.release(s); live.remove(s); log.append(("free", s, None))
        except NoBlocks:
            log.append(("noblocks", None, a.dump()))
        check_invariants(a)
    return a, log


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_invariants(seed):
    a, log = random_trace(seed)
    assert any(op == "noblocks" for op, _, _ in log) or seed > 2  # small pools hit exhaustion
    assert any(op == "append" and out[1] for op, _, out in log)    # some copy-on-write happened


def test_slots_are_unique_among_live_tokens():
    """No two live (sequence, position) pairs that are not shared map to one slot: every
    sequence's slots for positions it wrote privately are distinct from all others'."""
    a = Allocator(64, 4, np.random.default_rng(0).permutation(64))
    owner = {}
    for s in range(6):
        a.add(s)
        slots, _ = a.append(s, 7 + s)
        for sl in slots:
            assert sl not in owner
            owner[sl] = s


# --------------------------------------------------------------------------- swapping

def test_hand_traced_swap():
    """Device pool of 4 blocks of 2 slots (free order [2, 0, 3, 1]), host pool of 3.  Every
    value worked out by hand from the swap rules: each distinct block met walking the listed
    sequences in order gets the next host block, references move with it, device references
    drop as in a release."""
    a = Allocator(4, 2, [2, 0, 3, 1])
    a.set_host_blocks(3)
    a.add(1)
    a.append(1, 3)                       # blocks [2, 0]
    a.fork(1, 2)                         # 2 shares [2, 0]
    a.add(3)
    a.append(3, 1)                       # block 3
    assert a.dump() == ([2, 0, 2, 1], [1])
    pairs = a.swap_out([2, 3])           # 2's blocks 2, 0, then 3's block 3
    assert pairs == [(2, 0), (0, 1), (3, 2)]
    assert a.dump() == ([1, 0, 1, 0], [1, 3])          # 2 and 0 still held by 1; 3 freed
    assert a.dump_host() == ([1, 1, 1], [])
    assert a.is_swapped(2) and a.is_swapped(3) and not a.is_swapped(1)
    assert a.stats()["swapped_seqs"] == 2 and a.stats()["waste_slots"] == 1
    with pytest.raises(NoBlocks):
        a.swap_out([1])                  # needs 2 host blocks, none free
    with pytest.raises(InvalidOp):
        a.append(2, 1)
    with pytest.raises(InvalidOp):
        a.block_table([3], 2)
    a.release(1)                         # device blocks 2, 0 -> free tail
    assert a.dump() == ([0, 0, 0, 0], [1, 3, 2, 0])
    pairs = a.swap_in([3, 2])            # 3's host block 2, then 2's host blocks 0, 1
    assert pairs == [(2, 1), (0, 3), (1, 2)]
    assert a.dump() == ([0, 1, 1, 1], [0])
    assert a.dump_host() == ([0, 0, 0], [2, 0, 1])
    t, L = a.block_table([2, 3], 2)
    assert t == [[3, 2], [1, -1]] and L == [3, 1]


def test_swap_exhaustion_and_invalid_leave_state_unchanged():
    a = Allocator(4, 2)
    a.set_host_blocks(2)
    for s in (0, 1):
        a.add(s)
        a.append(s, 4)                   # 0: [0, 1], 1: [2, 3]
    snap = lambda: (a.dump(), a.dump_host(), {k: (list(v.blocks), v.n, v.swapped) for k, v in a.seqs.items()})
    before = snap()
    with pytest.raises(NoBlocks):
        a.swap_out([0, 1])               # 4 host blocks needed, 2 free
    assert snap() == before and a.stats()["exhaustion_events"] == 0
    for bad in (lambda: a.swap_out([0, 0]), lambda: a.swap_out([7]), lambda: a.swap_in([0]),
                lambda: a.set_host_blocks(-1)):
        with pytest.raises(InvalidOp):
            bad()
        assert snap() == before
    a.swap_out([0])
    a.add(2)
    a.append(2, 4)                       # takes the two freed device blocks
    before = snap()
    with pytest.raises(NoBlocks):
        a.swap_in([0])                   # no device block free
    assert snap() == before and a.stats()["exhaustion_events"] == 1
    with pytest.raises(InvalidOp):
        a.set_host_blocks(4)             # refused while a sequence is swapped out
    a.release(0)                         # a swapped sequence can be released
    assert a.dump_host() == ([0, 0], [0, 1]) and a.stats()["swapped_seqs"] == 0


def check_pool_invariants(a: Allocator):
    """Both pools: refcount = number of table entries naming the block, free queue = the
    blocks with refcount 0, each listed once."""
    for swapped, ref, free in ((False, a.refcount, a.free), (True, a.host_refcount, a.host_free)):
        held = [b for s in a.seqs.values() if s.swapped == swapped for b in s.blocks]
        for b in range(len(ref)):
            assert ref[b] == held.count(b)
        assert sorted(free) == [b for b in range(len(ref)) if ref[b] == 0]
    for s in a.seqs.values():
        assert len(s.blocks) == -(-s.n // a.block_size) and len(set(s.blocks)) == len(s.blocks)


@pytest.mark.parametrize("seed", range(6))
def test_swap_preserves_every_sequence_contents(seed):
    """The page-table definition, with the cache simulated as token ids: tokens are written
    at the slots the allocator returns, copy-on-write and swap pairs copy whole blocks between
    the simulated pools, and after every operation each sequence read through its table (in
    whichever pool holds it) must give exactly the tokens appended to it (a fork inherits its
    parent's).  A block released while still held, a wrong pair or a lost reference would
    let a later write or copy overwrite some sequence's tokens."""
    rng = np.random.default_rng(500 + seed)
    N, NH, bs = 24, 20, int(rng.choice([1, 2, 4]))
    a = Allocator(N, bs, rng.permutation(N))
    a.set_host_blocks(NH)
    dev = np.full((N, bs), -1, np.int64)
    host = np.full((NH, bs), -1, np.int64)
    want = {}
    live, nid, tok = [], 0, 0
    swaps = 0
    for _ in range(600):
        r = rng.random()
        try:
            resident = [s for s in live if not a.seqs[s].swapped]
            swapped = [s for s in live if a.seqs[s].swapped]
            if r < 0.1 or not live:
                a.add(nid); want[nid] = []; live.append(nid); nid += 1
            elif r < 0.45 and resident:
                s = int(rng.choice(resident)); n = int(rng.integers(1, 2 * bs + 1))
                slots, cow = a.append(s, n)
                for src, dst in cow:
                    dev[dst] = dev[src]
                for sl in slots:
                    dev[sl // bs, sl % bs] = tok
                    want[s].append(tok)
                    tok += 1
            elif r < 0.55 and resident:
                p = int(rng.choice(resident)); a.fork(p, nid); want[nid] = list(want[p]); live.append(nid); nid += 1
            elif r < 0.7 and resident:
                k = int(rng.integers(1, min(4, len(resident)) + 1))
                ids = [int(x) for x in rng.choice(resident, size=k, replace=False)]
                for d, h in a.swap_out(ids):
                    host[h] = dev[d]
                swaps += 1
            elif r < 0.85 and swapped:
                k = int(rng.integers(1, min(4, len(swapped)) + 1))
                ids = [int(x) for x in rng.choice(swapped, size=k, replace=False)]
                for h, d in a.swap_in(ids):
                    dev[d] = host[h]
                swaps += 1
            elif live:
                s = int(rng.choice(live)); a.release(s); live.remove(s); del want[s]
        except NoBlocks:
            pass
        check_pool_invariants(a)
        for s in live:
            q = a.seqs[s]
            pool = host if q.swapped else dev
            got = [int(pool[q.blocks[j // bs], j % bs]) for j in range(q.n)]
            assert got == want[s], (s, q)
    assert swaps > 20


# --------------------------------------------------------------------------- prefix caching

def test_hand_traced_prefix_cache():
    """6 blocks of 2 slots, free order [4, 1, 5, 0, 2, 3].  Worked out by hand from the rules:
    a full block is registered under the whole token prefix up to its end; a prompt takes the
    registered blocks of its block-boundary prefixes from block 0 on, up to the first miss; a
    registered block at refcount 0 stays registered until the free queue hands it out."""
    a = Allocator(6, 2, [4, 1, 5, 0, 2, 3])
    n, slots = a.add_prompt(1, [7, 8, 9, 10, 11])      # nothing cached: blocks 4, 1, 5
    assert n == 0 and slots == [8, 9, 2, 3, 10]
    assert a.dump_cached() == [0, 1, 0, 0, 1, 0]       # (7,8) -> 4, (7,8,9,10) -> 1
    n, slots = a.add_prompt(2, [7, 8, 9, 10, 12, 13])  # two hits, then block 0 for (12, 13)
    assert n == 4 and slots == [0, 1]
    assert a.dump() == ([1, 2, 0, 0, 2, 1], [2, 3])
    assert a.dump_cached() == [1, 1, 0, 0, 1, 0]       # (7,8,9,10,12,13) -> 0
    n, slots = a.add_prompt(3, [8, 7, 9, 10])          # (8, 7) is not (7, 8): no hit at all
    assert n == 0 and slots == [4, 5, 6, 7]
    assert a.dump() == ([1, 2, 1, 1, 2, 1], [])
    a.release(2)                                       # 4, 1, 0 lose a reference; 0 is free
    a.release(1)                                       # then 4, 1, 5: 4 and 1 free
    assert a.dump() == ([0, 0, 1, 1, 0, 0], [0, 4, 1, 5])
    assert a.dump_cached() == [1, 1, 1, 1, 1, 0]       # free blocks keep their registration
    n, slots = a.add_prompt(4, [7, 8, 9, 10, 12])      # hits 4 and 1 out of the free queue
    assert n == 4 and slots == [0]                     # head 0 is handed out: (7,8,9,10,12,13) evicted
    assert a.dump() == ([1, 1, 1, 1, 1, 0], [5])
    assert a.dump_cached() == [0, 1, 1, 1, 1, 0]
    st = a.stats()
    assert (st["cached_blocks"], st["cache_hit_blocks"], st["cache_evictions"]) == (4, 4, 1)
    a.append(4, 1)                                     # ids unknown from now on
    a.append(4, 2, [1, 2])                             # block 0 fills: nothing registered
    assert a.dump_cached() == [0, 1, 1, 1, 1, 0]


def test_prompt_exhaustion_leaves_state_unchanged():
    a = Allocator(3, 2)
    a.add_prompt(0, [1, 2, 3, 4])                      # blocks 0, 1 registered
    a.release(0)                                       # both free but registered
    snap = (a.dump(), a.dump_cached(), a.stats())
    with pytest.raises(NoBlocks):
        a.add_prompt(1, [1, 2, 3, 4, 5, 6, 7, 8])      # 2 hits + 2 fresh > 1 other free block
    assert (a.dump(), a.dump_cached()) == snap[:2] and a.stats()["exhaustion_events"] == 1
    n, _ = a.add_prompt(1, [1, 2, 3, 4, 5, 6])         # 2 hits + 1 fresh fits
    assert n == 4


@pytest.mark.parametrize("seed", range(6))
def test_prefix_cache_serves_only_equal_prefixes(seed):
    """The definition of a cache hit, checked by simulation: every slot of the simulated cache
    holds the identity of the whole token prefix through that token (the K/V of a token
    depends on all tokens before it).  Tokens are written only at the slots the allocator
    returns (a prompt's cached tokens are not written); copy-on-write and swap pairs copy
    whole blocks.  After every operation each sequence read through its table must give the
    prefix identities of exactly its own tokens.  Keying blocks by their own tokens only, a
    hit past a miss or a registration that outlives a block being handed out fail it."""
    rng = np.random.default_rng(900 + seed)
    N, NH, bs = 40, 24, int(rng.choice([1, 2, 4]))
    a = Allocator(N, bs, rng.permutation(N))
    a.set_host_blocks(NH)
    ident = {}
    pid = lambda toks: ident.setdefault(tuple(toks), len(ident))
    dev = np.full((N, bs), -1, np.int64)
    host = np.full((NH, bs), -1, np.int64)
    want = {}                                          # sequence -> its token ids (None: unknown)
    vals = {}                                          # sequence -> expected slot values
    systems = [list(rng.integers(0, 3, size=int(rng.integers(1, 4 * bs + 1)))) for _ in range(3)]
    live, nid, hits = [], 0, 0
    for _ in range(700):
        r = rng.random()
        resident = [s for s in live if not a.seqs[s].swapped]
        swapped = [s for s in live if a.seqs[s].swapped]
        try:
            if r < 0.25 or not live:
                toks = list(systems[int(rng.integers(0, 3))]) + list(rng.integers(0, 3, size=int(rng.integers(0, 2 * bs))))
                n_cached, slots = a.add_prompt(nid, toks)
                hits += n_cached
                for j, sl in enumerate(slots):
                    dev[sl // bs, sl % bs] = pid(toks[: n_cached + j + 1])
                want[nid] = list(toks)
                vals[nid] = [pid(toks[: j + 1]) for j in range(len(toks))]
                live.append(nid); nid += 1
            elif r < 0.5 and resident:
                s = int(rng.choice(resident)); k = int(rng.integers(1, 2 * bs + 1))
                known = want[s] is not None and rng.random() < 0.9
                ids = [int(x) for x in rng.integers(0, 3, size=k)]
                slots, cow = a.append(s, k, ids if known else None)
                for src, dst in cow:
                    dev[dst] = dev[src]
                if known:
                    want[s] = want[s] + ids
                    new = [pid(want[s][: len(vals[s]) + j + 1]) for j in range(k)]
                else:
                    want[s] = None
                    new = [10_000_000 + len(ident) + j for j in range(k)]   # unknown content
                    ident[("unknown", len(ident))] = len(ident)
                for sl, v in zip(slots, new):
                    dev[sl // bs, sl % bs] = v
                vals[s] = vals[s] + new
            elif r < 0.6 and resident:
                p = int(rng.choice(resident)); a.fork(p, nid)
                want[nid] = None if want[p] is None else list(want[p]); vals[nid] = list(vals[p])
                live.append(nid); nid += 1
            elif r < 0.7 and resident:
                ids = [int(x) for x in rng.choice(resident, size=min(len(resident), 2), replace=False)]
                for d, h in a.swap_out(ids):
                    host[h] = dev[d]
            elif r < 0.8 and swapped:
                ids = [int(x) for x in rng.choice(swapped, size=min(len(swapped), 2), replace=False)]
                for h, d in a.swap_in(ids):
                    dev[d] = host[h]
            elif live:
                s = int(rng.choice(live)); a.release(s); live.remove(s)
        except NoBlocks:
            pass
        check_pool_invariants(a)
        for s in live:
            q = a.seqs[s]
            pool = host if q.swapped else dev
            assert [int(pool[q.blocks[j // bs], j % bs]) for j in range(q.n)] == vals[s], s
        for key, b in a.cache.items():                 # registered blocks hold their prefix
            assert [int(x) for x in dev[b]] == [pid(key[: len(key) - bs + i + 1]) for i in range(bs)]
    assert hits > 0
