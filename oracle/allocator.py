"""Block allocator model (oracle; test infrastructure only).

What the pages fix:

* The cache is split into fixed-size blocks of ``block_size`` token slots; a request's
  a request's tokens may sit in any free blocks, and a per-request block table maps logical
  block j to a physical block, as an operating system's page table maps pages ("KV Cache Optimization and
  PagedAttention", prose on paging; "PagedAttention: Optimizing KV Cache Utilization in
  Large Language Models", "The Mechanics of PagedAttention").
* Blocks are granted on demand: a request holds one block and gets the next when that one
  fills; the next need not be adjacent ("KV Cache Management", "The Solution:
  PagedAttention (vLLM)").
* Requests can point at the same physical blocks for a shared prefix, with
  copy-on-write ("KV Cache Optimization and PagedAttention", prose on sharing;
  "KV Cache Management", "The Bonus: Zero-Copy Sharing").
* A batch can run out of blocks mid-generation; the caller must handle it
  ("PagedAttention: ...", "Conclusion").

Readings where the pages are silent (the plainest ones the rest supports):

* Which free block is granted: a FIFO queue; grants pop the head, releases push to the
  tail.  The initial order is given by the caller.
* Slot of a token: ``physical_block * block_size + (position mod block_size)``.
* Copy-on-write: when a token is appended into a partially filled last block that other
  sequences also hold (refcount > 1), a fresh block is granted, the pair (old, new) is
  reported so the caller copies the whole block, the old block loses one reference and the
  new one replaces it in this sequence's table.  A shared block is never written.
* Fork shares the parent's whole current block list (every block gains one reference).
* Release walks the sequence's blocks in logical order; blocks whose refcount reaches 0
  join the free queue tail in that order.
* A multi-token append is all-or-nothing: if the free queue cannot cover it, nothing
  changes and the exhaustion counter is incremented.

Preemption by swapping ("PagedAttention: ...", "Conclusion": requests that run out of
blocks are preempted and their KV cache recomputed or swapped).  The pages name swapping
only; the reading taken here:

* Swapped-out blocks go to a second pool of host blocks, with its own FIFO free queue
  (identity order) and refcounts.
* Swapping out a set of sequences gives every distinct device block they hold one host
  block (the pair is reported so the caller copies the block), in the order the blocks are
  met walking the sequences in the given order, each in logical order.  Every reference of
  the set moves to the host block, and the device references are dropped exactly as a
  release drops them.  Swapping in is the same with the pools exchanged.
* A block that a sequence outside the set also holds is copied and stays with that holder,
  so the two stop sharing it.
* A swapped-out sequence cannot be appended to, forked or listed in a block table; it can
  be swapped in or released (releasing its host blocks).
* A swap is all-or-nothing; a swap-in refused for lack of device blocks counts as an
  exhaustion event, a swap-out refused for lack of host blocks does not.

Prefix caching ("KV Cache Management", "The Bonus: Zero-Copy Sharing": a system prompt
shared by many users is computed and stored once and their tables all point at it; "KV
Cache Optimization and PagedAttention", first paragraph: prefix caching).  Readings:

* A full block is registered under its content, the tuple of every token id from position
  0 to the block's end, when a sequence whose token ids are all known fills it, unless that
  content is already registered to another block.
* A sequence added with its prompt takes, from block 0 on, the registered block of each
  prefix that ends at a block boundary, and stops at the first one that is not registered;
  the tokens so covered are reported as cached.  The rest of the prompt is appended.
* A registered block whose refcount reaches 0 stays registered in the free queue; a hit
  takes it out of the queue; when the queue hands it out again its registration is dropped.
* Token ids are known for sequences created empty or by a prompt and grown only by appends
  that give ids; an append without ids (of at least one token) makes them unknown for good.
  A fork copies its parent's ids.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field


class NoBlocks(Exception):
    """Raised when the free queue cannot cover an append; the state is unchanged."""


class InvalidOp(Exception):
    """Raised for unknown/duplicate sequence ids; the state is unchanged."""


@dataclass
class _Seq:
    blocks: list = field(default_factory=list)   # device ids, or host ids while swapped
    n: int = 0
    swapped: bool = False
    tokens: list = field(default_factory=list)   # every token id held, or None if unknown


class Allocator:
    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidOp("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidOp("initial free order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.seqs: dict[int, _Seq] = {}
        self.exhaustion_events = 0
        self.host_free = deque()
        self.host_refcount = []
        self.cache = {}            # token-id prefix (tuple) ending at a block end -> block
        self.cached_key = {}       # block -> its prefix
        self.cache_hit_blocks = 0
        self.cache_evictions = 0

    def _grant(self) -> int:
        """The free queue's head; a registered block loses its registration."""
        b = self.free.popleft()
        if b in self.cached_key:
            del self.cache[self.cached_key.pop(b)]
            self.cache_evictions += 1
        return b

    def _resident(self, seq_id: int) -> _Seq:
        if seq_id not in self.seqs:
            raise InvalidOp(f"unknown sequence {seq_id}")
        if self.seqs[seq_id].swapped:
            raise InvalidOp(f"sequence {seq_id} is swapped out")
        return self.seqs[seq_id]

    # -- operations -------------------------------------------------------------------
    def add(self, seq_id: int) -> None:
        if seq_id in self.seqs:
            raise InvalidOp(f"sequence {seq_id} already exists")
        self.seqs[seq_id] = _Seq()

    def _blocks_needed(self, s: _Seq, n_tokens: int) -> int:
        bs = self.block_size
        need = 0
        if n_tokens > 0 and s.n % bs != 0 and self.refcount[s.blocks[-1]] > 1:
            need += 1                                   # copy-on-write of the shared tail
        for t in range(n_tokens):
            if (s.n + t) % bs == 0:
                need += 1                               # a fresh block for this token
        return need

    def append(self, seq_id: int, n_tokens: int, token_ids=None):
        """Append n_tokens to a sequence (their ids, if given, register the blocks they
        fill).  Returns (slots, cow_pairs)."""
        s = self._resident(seq_id)
        if n_tokens < 0:
            raise InvalidOp("negative token count")
        if token_ids is not None and len(token_ids) != n_tokens:
            raise InvalidOp("token ids do not match the count")
        if self._blocks_needed(s, n_tokens) > len(self.free):
            self.exhaustion_events += 1
            raise NoBlocks(f"sequence {seq_id}: not enough free blocks")
        bs = self.block_size
        if token_ids is None and n_tokens > 0:
            s.tokens = None
        slots, cow = [], []
        for t in range(n_tokens):
            if s.n % bs == 0:
                b = self._grant()
                self.refcount[b] = 1
                s.blocks.append(b)
            elif self.refcount[s.blocks[-1]] > 1:
                old = s.blocks[-1]
                new = self._grant()
                self.refcount[old] -= 1
                self.refcount[new] = 1
                s.blocks[-1] = new
                cow.append((old, new))
            slots.append(s.blocks[-1] * bs + s.n % bs)
            s.n += 1
            if s.tokens is not None:
                s.tokens.append(int(token_ids[t]))
                if s.n % bs == 0 and tuple(s.tokens) not in self.cache:
                    assert s.blocks[-1] not in self.cached_key
                    self.cache[tuple(s.tokens)] = s.blocks[-1]
                    self.cached_key[s.blocks[-1]] = tuple(s.tokens)
        return slots, cow

    def add_prompt(self, seq_id: int, token_ids):
        """Create a sequence holding the prompt: registered blocks whose prefix matches are
        taken from block 0 on (up to the first miss), the rest is appended.  Returns
        (cached tokens, slots of the rest)."""
        if seq_id in self.seqs:
            raise InvalidOp(f"sequence {seq_id} already exists")
        token_ids = [int(t) for t in token_ids]
        bs = self.block_size
        hits = []
        while (len(hits) + 1) * bs <= len(token_ids):
            key = tuple(token_ids[: (len(hits) + 1) * bs])
            if key not in self.cache:
                break
            hits.append(self.cache[key])
        n_cached = len(hits) * bs
        need = -(-(len(token_ids) - n_cached) // bs)
        if need > len(self.free) - sum(1 for b in hits if self.refcount[b] == 0):
            self.exhaustion_events += 1
            raise NoBlocks(f"sequence {seq_id}: not enough free blocks")
        for b in hits:
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
        self.cache_hit_blocks += len(hits)
        self.seqs[seq_id] = _Seq(blocks=list(hits), n=n_cached, tokens=token_ids[:n_cached])
        slots, _ = self.append(seq_id, len(token_ids) - n_cached, token_ids[n_cached:])
        return n_cached, slots

    def append_batch(self, seq_ids, n_tokens):
        """Appends to several distinct sequences in order, all or nothing: the appends are
        tried on a copy of the state, which replaces the state only if all succeed."""
        import copy
        if len(set(seq_ids)) != len(seq_ids):
            raise InvalidOp("a sequence is listed twice")
        for s, n in zip(seq_ids, n_tokens):             # bad arguments before exhaustion
            self._resident(s)
            if n < 0:
                raise InvalidOp("negative token count")
        trial = copy.deepcopy(self)
        slots, cow = [], []
        try:
            for s, n in zip(seq_ids, n_tokens):
                sl, cw = trial.append(s, n)
                slots += sl
                cow += cw
        except NoBlocks:
            self.exhaustion_events += 1
            raise
        self.__dict__.update(trial.__dict__)
        return slots, cow

    def fork(self, parent: int, child: int) -> None:
        p = self._resident(parent)
        if child in self.seqs:
            raise InvalidOp(f"sequence {child} already exists")
        for b in p.blocks:
            self.refcount[b] += 1
        self.seqs[child] = _Seq(blocks=list(p.blocks), n=p.n,
                                tokens=None if p.tokens is None else list(p.tokens))

    def release(self, seq_id: int) -> None:
        if seq_id not in self.seqs:
            raise InvalidOp(f"unknown sequence {seq_id}")
        s = self.seqs.pop(seq_id)
        refcount, free = (self.host_refcount, self.host_free) if s.swapped else (self.refcount, self.free)
        for b in s.blocks:
            refcount[b] -= 1
            if refcount[b] == 0:
                free.append(b)

    # -- preemption by swapping ---------------------------------------------------------
    def set_host_blocks(self, num_host_blocks: int) -> None:
        if num_host_blocks < 0:
            raise InvalidOp("negative host pool size")
        if any(s.swapped for s in self.seqs.values()):
            raise InvalidOp("sequences are swapped out")
        self.host_free = deque(range(num_host_blocks))
        self.host_refcount = [0] * num_host_blocks

    def _swap(self, seq_ids, to_host: bool):
        if len(set(seq_ids)) != len(seq_ids):
            raise InvalidOp("a sequence is listed twice")
        for sid in seq_ids:
            if sid not in self.seqs:
                raise InvalidOp(f"unknown sequence {sid}")
            if self.seqs[sid].swapped == to_host:
                raise InvalidOp(f"sequence {sid} is in the wrong state for this swap")
        if to_host:
            src_ref, src_free, dst_ref, dst_free = self.refcount, self.free, self.host_refcount, self.host_free
        else:
            src_ref, src_free, dst_ref, dst_free = self.host_refcount, self.host_free, self.refcount, self.free
        distinct = {b for sid in seq_ids for b in self.seqs[sid].blocks}
        if len(distinct) > len(dst_free):
            if not to_host:
                self.exhaustion_events += 1
            raise NoBlocks("not enough free blocks in the destination pool")
        moved = {}
        pairs = []
        grant = self.host_free.popleft if to_host else self._grant
        for sid in seq_ids:
            s = self.seqs[sid]
            new_blocks = []
            for b in s.blocks:
                if b not in moved:
                    moved[b] = grant()
                    pairs.append((b, moved[b]))
                dst_ref[moved[b]] += 1
                src_ref[b] -= 1
                if src_ref[b] == 0:
                    src_free.append(b)
                new_blocks.append(moved[b])
            s.blocks = new_blocks
            s.swapped = to_host
        return pairs

    def swap_out(self, seq_ids):
        """Moves the sequences to the host pool.  Returns the (device, host) block pairs."""
        return self._swap(list(seq_ids), True)

    def swap_in(self, seq_ids):
        """Moves the sequences back to the device pool.  Returns the (host, device) pairs."""
        return self._swap(list(seq_ids), False)

    def is_swapped(self, seq_id: int) -> bool:
        if seq_id not in self.seqs:
            raise InvalidOp(f"unknown sequence {seq_id}")
        return self.seqs[seq_id].swapped

    def dump_host(self):
        """(host refcounts, host free queue in order)."""
        return list(self.host_refcount), list(self.host_free)

    # -- views ------------------------------------------------------------------------
    def block_table(self, seq_ids, max_blocks: int):
        """Rows of physical block ids padded with -1, and the token counts."""
        tables, lens = [], []
        for sid in seq_ids:
            s = self._resident(sid)
            if len(s.blocks) > max_blocks:
                raise InvalidOp(f"sequence {sid} holds {len(s.blocks)} blocks > {max_blocks}")
            tables.append(list(s.blocks) + [-1] * (max_blocks - len(s.blocks)))
            lens.append(s.n)
        return tables, lens

    def stats(self) -> dict:
        bs = self.block_size
        used = sum(1 for r in self.refcount if r > 0)
        waste = 0
        for s in self.seqs.values():
            if not s.swapped:
                waste += -(-s.n // bs) * bs - s.n        # final-block waste per resident holder
        return {
            "free": len(self.free),
            "used": used,
            "refs": sum(self.refcount),
            "exhaustion_events": self.exhaustion_events,
            "waste_slots": waste,
            "host_free": len(self.host_free),
            "host_used": sum(1 for r in self.host_refcount if r > 0),
            "swapped_seqs": sum(1 for s in self.seqs.values() if s.swapped),
            "cached_blocks": len(self.cache),
            "cache_hit_blocks": self.cache_hit_blocks,
            "cache_evictions": self.cache_evictions,
        }

    def dump_cached(self):
        """1 for each block registered in the prefix cache, else 0."""
        return [1 if b in self.cached_key else 0 for b in range(self.num_blocks)]

    def dump(self):
        """(refcounts, free queue in order) for bit-exact comparison."""
        return list(self.refcount), list(self.free)
