"""Block allocator model (oracle; test infrastructure only).

What the pages fix:

* The cache is split into fixed-size blocks of ``block_size`` token slots; a request's
  tokens go into whatever blocks are free, and a per-request block table maps logical
  block j to a physical block, like an OS page table ("KV Cache Optimization and
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

    def append(self, seq_id: int, n_tokens: int):
        """Append n_tokens to a sequence.  Returns (slots, cow_pairs)."""
        s = self._resident(seq_id)
        if n_tokens < 0:
            raise InvalidOp("negative token count")
        if self._blocks_needed(s, n_tokens) > len(self.free):
            self.exhaustion_events += 1
            raise NoBlocks(f"sequence {seq_id}: not enough free blocks")
        bs = self.block_size
        slots, cow = [], []
        for _ in range(n_tokens):
            if s.n % bs == 0:
                b = self.free.popleft()
                self.refcount[b] = 1
                s.blocks.append(b)
            elif self.refcount[s.blocks[-1]] > 1:
                old = s.blocks[-1]
                new = self.free.popleft()
                self.refcount[old] -= 1
                self.refcount[new] = 1
                s.blocks[-1] = new
                cow.append((old, new))
            slots.append(s.blocks[-1] * bs + s.n % bs)
            s.n += 1
        return slots, cow

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
        self.seqs[child] = _Seq(blocks=list(p.blocks), n=p.n)

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
        for sid in seq_ids:
            s = self.seqs[sid]
            new_blocks = []
            for b in s.blocks:
                if b not in moved:
                    moved[b] = dst_free.popleft()
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
        }

    def dump(self):
        """(refcounts, free queue in order) for bit-exact comparison."""
        return list(self.refcount), list(self.free)
