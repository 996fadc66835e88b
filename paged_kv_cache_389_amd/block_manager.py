"""Host-side block manager: physical block pool, block tables, reference counts,
fork and copy-on-write.

This is the host logic that produces the integer inputs of the three device
calls (block tables, context lengths, slot mappings, copy pairs).  It does no
device work.

Behaviour, from the pages:

* The KV memory is a pool of equal-sized physical blocks; a sequence is a run
  of logical blocks that map to arbitrary physical blocks through a per-
  sequence block table ("Memory Optimization in LLM Serving with
  PagedAttention", section "How PagedAttention Works", items 1-3).
* A block is taken from the pool only when the sequence needs it; nothing is
  reserved up front, so only the last block of a sequence is partly filled
  (same section, the two bullets after the list; "vLLM and PagedAttention:
  How Ideas from Operating Systems Accelerated LLM Inference", paragraph on the
  solution).
* Sequences may share physical blocks (parallel sampling, beam search,
  common prefixes).  Each block carries a reference count.  Before appending
  into a shared block (count above one) the sequence gets a fresh block, the
  content is copied into it, the table entry is redirected to the copy, and
  only then is the token written ("Memory Optimization ...", section
  "Advanced Capabilities: Memory Sharing with Copy-on-Write"; "vLLM and
  PagedAttention ...", paragraph on sharing).
* When device memory runs short, whole sequences are evicted by swapping
  their blocks to a pool in CPU memory and brought back later ("vLLM and
  PagedAttention ...", paragraph on the engine).

Readings where the pages are silent:

* The count of the old block drops by one when a holder moves to its copy.
* A holder that finds the count at one writes in place (no copy).
* Slot numbering: slot ``b * block_size + o`` is offset ``o`` of block ``b``.
* Free blocks are handed out from the end of a free list; its initial order
  may be given (a seeded permutation gives random placement).
* Copy-on-write pairs wait until the caller takes them (one batch for one
  copy_blocks call, which copies them in parallel).  Until then a block they
  name does not return to the free list even when its count drops to zero,
  and a pending destination cannot be the source of another copy, so the
  batch never reads a block it writes.
* A swap moves a group of sequences that holds every reference to its
  blocks (a prompt and its forks): each distinct block moves once, keeps its
  count, and every table of the group is rewritten.
"""

from __future__ import annotations

import numpy as np


class OutOfBlocks(RuntimeError):
    """The pool has no free block; the manager's state is left unchanged."""


class Sequence:
    """One sequence's logical view: its block table and its token count."""

    __slots__ = ("seq_id", "table", "length", "on_host")

    def __init__(self, seq_id: int):
        self.seq_id = seq_id
        self.table: list[int] = []
        self.length = 0
        self.on_host = False   # the table indexes the host pool (swapped out)

    def __repr__(self):
        where = "host" if self.on_host else "device"
        return f"Sequence(id={self.seq_id}, len={self.length}, {where} table={self.table})"


class BlockManager:
    """A pool of ``num_blocks`` physical blocks of ``block_size`` token slots."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None,
                 num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            # pop() takes from the end, so block 0 is handed out first
            self._free = list(range(self.num_blocks - 1, -1, -1))
        else:
            order = [int(b) for b in free_order]
            if sorted(order) != list(range(self.num_blocks)):
                raise ValueError("free_order must be a permutation of the pool")
            self._free = order
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)
        self._next_id = 0
        # copy-on-write pairs (src, dst) emitted since the last take_copy_pairs()
        self._pending_copies: list[tuple[int, int]] = []
        # blocks named by a pending pair, and those among them whose count
        # fell to zero: they stay off the free list until the pairs are taken,
        # so no block is both a source and a destination of one batch of copies
        self._pending_blocks: set[int] = set()
        self._held_for_copy: list[int] = []
        # the host pool that swapped-out blocks live in
        self.num_host_blocks = int(num_host_blocks)
        self._host_free = list(range(self.num_host_blocks - 1, -1, -1))
        self.host_refcount = np.zeros(self.num_host_blocks, dtype=np.int64)

    # ------------------------------------------------------------------ pool
    @property
    def num_free(self) -> int:
        return len(self._free)

    def free_blocks(self) -> list[int]:
        return list(self._free)

    def _take(self) -> int:
        if not self._free:
            raise OutOfBlocks(f"pool of {self.num_blocks} blocks is exhausted")
        b = self._free.pop()
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] < 0:
            raise AssertionError(f"block {b} released more often than held")
        if self.refcount[b] == 0:
            if b in self._pending_blocks:
                self._held_for_copy.append(b)
            else:
                self._free.append(b)

    # ------------------------------------------------------------- sequences
    def new_sequence(self) -> Sequence:
        seq = Sequence(self._next_id)
        self._next_id += 1
        return seq

    def append_slot(self, seq: Sequence) -> int:
        """Reserve the slot of the sequence's next token and return it.

        Takes a new block when the last one is full (or there is none);
        performs copy-on-write when the last block is partly filled and shared.
        Raises :class:`OutOfBlocks` without changing any state if the pool
        cannot supply the block.
        """
        if seq.on_host:
            raise ValueError("the sequence is swapped out; swap it in first")
        bs = self.block_size
        offset = seq.length % bs
        if offset == 0:
            seq.table.append(self._take())
        else:
            last = seq.table[-1]
            if self.refcount[last] > 1:
                if any(last == d for _, d in self._pending_copies):
                    # its content is still being copied in: one batch of copies
                    # runs in parallel, so it cannot also be a source
                    raise ValueError(
                        f"block {last} is the destination of a pending copy; take the "
                        "pending pairs (and apply them and the step's writes) first")
                fresh = self._take()
                self.refcount[last] -= 1
                seq.table[-1] = fresh
                self._pending_copies.append((last, fresh))
                self._pending_blocks.update((last, fresh))
        slot = seq.table[seq.length // bs] * bs + offset
        seq.length += 1
        return slot

    def extend(self, seq: Sequence, num_tokens: int) -> np.ndarray:
        """Append ``num_tokens`` tokens; returns their slots (int64)."""
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        bs = self.block_size
        need = -(-(seq.length + num_tokens) // bs) - len(seq.table)
        shared_tail = (seq.length % bs != 0 and num_tokens > 0
                       and self.refcount[seq.table[-1]] > 1)
        if need + int(shared_tail) > self.num_free:
            raise OutOfBlocks(
                f"need {need + int(shared_tail)} blocks, {self.num_free} free")
        return np.array([self.append_slot(seq) for _ in range(num_tokens)],
                        dtype=np.int64)

    def fork(self, parent: Sequence) -> Sequence:
        """A child that shares every block of ``parent`` (counts go up by one)."""
        child = self.new_sequence()
        child.table = list(parent.table)
        child.length = parent.length
        for b in child.table:
            self.refcount[b] += 1
        return child

    def free(self, seq: Sequence) -> None:
        """Drop the sequence's hold on its blocks; unreferenced blocks return."""
        for b in reversed(seq.table):
            if seq.on_host:
                self.host_refcount[b] -= 1
                if self.host_refcount[b] == 0:
                    self._host_free.append(b)
            else:
                self._release(b)
        seq.table = []
        seq.length = 0
        seq.on_host = False

    # ------------------------------------------------------------------ swap
    def _group_blocks(self, seqs, on_host: bool):
        """Distinct blocks of the group in first-use order, checked to be
        held by the group alone."""
        order, count = [], {}
        for s in seqs:
            if s.on_host != on_host:
                raise ValueError(f"sequence {s.seq_id} is not on the "
                                 f"{'host' if on_host else 'device'}")
            for b in s.table:
                if b not in count:
                    order.append(b)
                    count[b] = 0
                count[b] += 1
        refs = self.host_refcount if on_host else self.refcount
        for b in order:
            if count[b] != refs[b]:
                raise ValueError(f"block {b} is also held outside the group")
        if not on_host and any(b in self._pending_blocks for b in order):
            raise ValueError("the group's blocks are named by pending copy-on-write pairs; "
                             "take the pairs (and apply them) before swapping")
        return order

    def _move(self, seqs, order, to_host: bool) -> np.ndarray:
        src_refs, dst_refs = ((self.refcount, self.host_refcount) if to_host
                              else (self.host_refcount, self.refcount))
        src_free, dst_free = ((self._free, self._host_free) if to_host
                              else (self._host_free, self._free))
        mapping = {}
        for b in order:
            d = dst_free.pop()
            dst_refs[d] = src_refs[b]
            src_refs[b] = 0
            src_free.append(b)
            mapping[b] = d
        for s in seqs:
            s.table = [mapping[b] for b in s.table]
            s.on_host = to_host
        return np.array([(b, mapping[b]) for b in order], dtype=np.int64).reshape(-1, 2)

    def swap_out(self, seqs) -> np.ndarray:
        """Move the group's blocks to the host pool.  Returns int64 [n, 2]
        (device block, host block) pairs, one per distinct block, for
        swap_blocks; raises :class:`OutOfBlocks` (state unchanged) when the
        host pool is short."""
        seqs = list(seqs)
        order = self._group_blocks(seqs, on_host=False)
        if len(order) > len(self._host_free):
            raise OutOfBlocks(f"need {len(order)} host blocks, {len(self._host_free)} free")
        return self._move(seqs, order, to_host=True)

    def swap_in(self, seqs) -> np.ndarray:
        """Move the group's blocks back to the device pool.  Returns int64
        [n, 2] (host block, device block) pairs; raises :class:`OutOfBlocks`
        (state unchanged) when the device pool is short."""
        seqs = list(seqs)
        order = self._group_blocks(seqs, on_host=True)
        if len(order) > len(self._free):
            raise OutOfBlocks(f"need {len(order)} device blocks, {len(self._free)} free")
        return self._move(seqs, order, to_host=False)

    def take_copy_pairs(self) -> np.ndarray:
        """Copy-on-write pairs emitted since the last call, as int64 [n, 2].
        Their destinations are distinct and none is a source, as
        copy_blocks requires; blocks of these pairs that were freed
        meanwhile return to the free list now."""
        pairs = np.array(self._pending_copies, dtype=np.int64).reshape(-1, 2)
        self._pending_copies = []
        self._pending_blocks = set()
        self._free.extend(self._held_for_copy)
        self._held_for_copy = []
        return pairs

    def held_for_copy(self) -> list[int]:
        """Unreferenced blocks kept off the free list until the pending
        copy-on-write pairs that name them are taken."""
        return list(self._held_for_copy)

    def pending_copy_pairs(self) -> list[tuple[int, int]]:
        """The pairs take_copy_pairs() would return, without taking them."""
        return list(self._pending_copies)

    # ------------------------------------------------------------ exports
    def block_table_array(self, seqs, width: int | None = None, pad: int = 0):
        """int32 ``[len(seqs), width]`` block tables, padded with ``pad``."""
        need = max((len(s.table) for s in seqs), default=0)
        width = need if width is None else int(width)
        if width < need:
            raise ValueError("width is smaller than the longest block table")
        arr = np.full((len(seqs), max(width, 1)), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            arr[i, :len(s.table)] = s.table
        return arr

    def context_lens(self, seqs) -> np.ndarray:
        return np.array([s.length for s in seqs], dtype=np.int32)

    def utilisation(self, seqs) -> float:
        """Filled token slots over allocated slots, each shared block counted
        once (the page-level memory figure the pages quote)."""
        allocated = int(np.count_nonzero(self.refcount)) * self.block_size
        if allocated == 0:
            return 1.0
        filled = {}
        for s in seqs:
            for j, b in enumerate(s.table):
                used = min(self.block_size, s.length - j * self.block_size)
                filled[b] = max(filled.get(b, 0), used)
        return sum(filled.values()) / allocated


# ------------------------------------------------------- grouped decode lists
TILE_TOKENS = 16   # tokens per tile of the grouped decode kernel


def share_groups(block_tables, context_lens, max_members: int) -> list[list[int]]:
    """Sequences grouped by the physical block holding their first tokens
    (forks of one prompt share it), in batch order, at most ``max_members``
    per group; a sequence of length zero, or one that shares nothing, forms
    a group of its own."""
    by_first: dict[int, list[int]] = {}
    singles = []
    for s in range(len(context_lens)):
        if int(context_lens[s]) <= 0:
            singles.append([s])
            continue
        by_first.setdefault(int(block_tables[s][0]), []).append(s)
    groups = []
    for seqs in by_first.values():
        groups.extend(seqs[i:i + max_members] for i in range(0, len(seqs), max_members))
    return groups + singles


def group_tiles(block_tables, context_lens, groups, block_size: int, max_members: int):
    """Inputs of the grouped decode call for ``groups`` (lists of sequence
    indices, each at most ``max_members`` long and no sequence twice).

    Returns ``(members, tiles, tile_start)``: int32 ``[G, max_members]``
    (-1 pads), int32 ``[T, 4]`` rows ``(block, tile, mask, 0)`` and int32
    ``[G + 1]``.  Group j's rows ``tile_start[j] .. tile_start[j+1]`` name
    every distinct (physical block, 16-token tile index) its members reach,
    with bit m of the mask set for each member m whose table maps that tile
    to that block; a tile shared by several members appears once."""
    if block_size % TILE_TOKENS:
        raise ValueError("block_size must be a multiple of 16")
    tpb = block_size // TILE_TOKENS
    num_groups = len(groups)
    members = np.full((num_groups, max_members), -1, dtype=np.int32)
    seqs, grp_of, mem_of = [], [], []
    for j, grp in enumerate(groups):
        if len(grp) > max_members:
            raise ValueError(f"group {j} has {len(grp)} members, more than {max_members}")
        members[j, :len(grp)] = grp
        seqs.extend(int(x) for x in grp)
        grp_of.extend([j] * len(grp))
        mem_of.extend(range(len(grp)))
    seqs = np.asarray(seqs, dtype=np.int64)
    if len(np.unique(seqs)) != len(seqs):
        raise ValueError("a sequence is in two groups")
    lens = np.asarray(context_lens, dtype=np.int64)[seqs] if len(seqs) else np.zeros(0, np.int64)
    ntile = -(-np.maximum(lens, 0) // TILE_TOKENS)
    # one row per (member, tile index), then one per distinct (group, tile, block)
    total = int(ntile.sum())
    first = np.repeat(np.cumsum(ntile) - ntile, ntile)
    t = np.arange(total, dtype=np.int64) - first
    seq_rep = np.repeat(seqs, ntile)
    blk = np.asarray(block_tables)[seq_rep, t // tpb].astype(np.int64)
    grp = np.repeat(np.asarray(grp_of, dtype=np.int64), ntile)
    bit = np.left_shift(1, np.repeat(np.asarray(mem_of, dtype=np.int64), ntile))
    order = np.lexsort((blk, t, grp))
    blk, t, grp, bit = blk[order], t[order], grp[order], bit[order]
    new = np.ones(total, dtype=bool)
    if total:
        new[1:] = (grp[1:] != grp[:-1]) | (t[1:] != t[:-1]) | (blk[1:] != blk[:-1])
    heads = np.nonzero(new)[0]
    tiles = np.zeros((len(heads), 4), dtype=np.int32)
    if len(heads):
        tiles[:, 0] = blk[heads]
        tiles[:, 1] = t[heads]
        tiles[:, 2] = np.bitwise_or.reduceat(bit, heads)
    start = np.searchsorted(grp[heads], np.arange(num_groups + 1)).astype(np.int32)
    return members, tiles, start
