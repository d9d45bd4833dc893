"""Dict model of the block allocator (test infrastructure).

Semantics, from the pages (cited by title and section):

* "What is PagedAttention?" (qubittool glossary), "How It Works: Map Logical to
  Physical Blocks": each sequence's logical blocks map through a block table to
  physical blocks that need not be adjacent; a prefill takes enough blocks for its
  tokens; a decode step appends into the partly filled last block and takes a new
  block only when that one is full; an allocation that cannot be met must fail
  explicitly instead of disturbing another sequence (here: the call fails and the
  state is left exactly as it was).
* Same page, "Share Without Mutating State", and "PagedAttention: Optimizing KV Cache
  in vLLM" (grasp.study), §4 "Advanced Benefit: Zero-Cost Sharing with Copy-on-Write":
  sequences may point at the same immutable blocks; a reference count per block
  counts its users and a block returns to the free pool when it reaches zero; before
  a sequence writes into a block whose count exceeds one, it gets a fresh block with a
  copy of the shared one, only its own table entry changes, and the old block's count
  drops by one.
* §2 "The Solution" of the same lesson: only a sequence's last block can be partly
  empty, so the waste per sequence stays under one block.

The model hands out free blocks last-in-first-out, starting from ``free_order[0]``.
No test relies on which IDs it picks: tests compare the sharing structure, lengths,
copy-on-write counts and free counts, all of which the semantics fix.
"""
from __future__ import annotations

import copy

OK, INVALID_ARG, UNSUPPORTED, OUT_OF_BLOCKS, UNKNOWN_SEQ = 0, 1, 2, 3, 4


class AllocError(Exception):
    def __init__(self, status, msg=""):
        super().__init__(msg or str(status))
        self.status = status


def _ceil_div(a, b):
    return -(-a // b)


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(INVALID_ARG)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks))
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = list(reversed(order))       # pop() hands out order[0] first
        self.ref = [0] * num_blocks
        self.seqs: dict[int, list] = {}         # id -> [blocks, length]

    # ---- helpers -------------------------------------------------------------------
    def _pop(self):
        b = self.free.pop()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _snapshot(self):
        return copy.deepcopy((self.free, self.ref, self.seqs))

    def _restore(self, snap):
        self.free, self.ref, self.seqs = snap

    def _slot(self, blocks, pos):
        return blocks[pos // self.bs] * self.bs + pos % self.bs

    def _append_one(self, sid, cows):
        blocks, n = self.seqs[sid]
        if n % self.bs == 0:
            if not self.free:
                raise AllocError(OUT_OF_BLOCKS)
            blocks.append(self._pop())
        else:
            tail = blocks[-1]
            if self.ref[tail] > 1:
                if not self.free:
                    raise AllocError(OUT_OF_BLOCKS)
                nb = self._pop()
                self.ref[tail] -= 1
                blocks[-1] = nb
                cows.append((tail, nb))
        slot = self._slot(blocks, n)
        self.seqs[sid][1] = n + 1
        return slot

    # ---- API -----------------------------------------------------------------------
    def seq_create(self, sid: int, length: int):
        if sid in self.seqs or length < 0:
            raise AllocError(INVALID_ARG)
        need = _ceil_div(length, self.bs)
        if need > len(self.free):
            raise AllocError(OUT_OF_BLOCKS)
        blocks = [self._pop() for _ in range(need)]
        self.seqs[sid] = [blocks, length]
        return [self._slot(blocks, p) for p in range(length)]

    def fork(self, parent: int, child: int, prefix_len: int):
        if parent not in self.seqs:
            raise AllocError(UNKNOWN_SEQ)
        pblocks, plen = self.seqs[parent]
        if child in self.seqs or not (0 <= prefix_len <= plen):
            raise AllocError(INVALID_ARG)
        shared = pblocks[:_ceil_div(prefix_len, self.bs)]
        for b in shared:
            self.ref[b] += 1
        self.seqs[child] = [list(shared), prefix_len]

    def extend(self, sid: int, n: int):
        if sid not in self.seqs:
            raise AllocError(UNKNOWN_SEQ)
        if n < 0:
            raise AllocError(INVALID_ARG)
        snap = self._snapshot()
        cows, slots = [], []
        try:
            for _ in range(n):
                slots.append(self._append_one(sid, cows))
        except AllocError:
            self._restore(snap)
            raise
        return slots, cows

    def append(self, sids):
        if len(set(sids)) != len(sids):
            raise AllocError(INVALID_ARG)
        for s in sids:
            if s not in self.seqs:
                raise AllocError(UNKNOWN_SEQ)
        snap = self._snapshot()
        cows, slots = [], []
        try:
            for s in sids:
                slots.append(self._append_one(s, cows))
        except AllocError:
            self._restore(snap)
            raise
        return slots, cows

    def swap_to(self, other: "AllocatorModel", sid: int):
        """Moves sequence `sid` into `other` ("What is PagedAttention?", "How It Works: Map
        Logical to Physical Blocks": swap is one of the explicit responses to an allocation
        that cannot be met).  Reading taken (the pages do not detail it): `other` gives
        every logical block a fresh block of its own, so sharing does not survive the
        move; the sequence then leaves this allocator as by free_seq.  All-or-nothing.
        Returns the (block here, block in other) pair of each logical block, in order."""
        if other is self or other.bs != self.bs:
            raise AllocError(INVALID_ARG)
        if sid not in self.seqs:
            raise AllocError(UNKNOWN_SEQ)
        if sid in other.seqs:
            raise AllocError(INVALID_ARG)
        blocks, length = self.seqs[sid]
        if len(blocks) > len(other.free):
            raise AllocError(OUT_OF_BLOCKS)
        fresh = [other._pop() for _ in blocks]
        other.seqs[sid] = [fresh, length]
        self.free_seq(sid)
        return list(zip(blocks, fresh))

    def free_seq(self, sid: int):
        if sid not in self.seqs:
            raise AllocError(UNKNOWN_SEQ)
        blocks, _ = self.seqs.pop(sid)
        for b in blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def tables(self, sids, max_blocks: int):
        rows, lens = [], []
        for s in sids:
            if s not in self.seqs:
                raise AllocError(UNKNOWN_SEQ)
            blocks, n = self.seqs[s]
            if len(blocks) > max_blocks:
                raise AllocError(INVALID_ARG)
            rows.append(list(blocks) + [-1] * (max_blocks - len(blocks)))
            lens.append(n)
        return rows, lens

    @property
    def num_free(self) -> int:
        return len(self.free)

    def stats(self) -> dict:
        """Pool occupancy: blocks in use and shared, and how many of their slots hold a token
        ("PagedAttention: Optimizing KV Cache in vLLM", §2: only a sequence's last block can be
        partly empty; §4: a shared block is stored once however many tables point at it)."""
        holders = {}
        for blocks, n in self.seqs.values():
            for j, b in enumerate(blocks):
                holders.setdefault(b, []).append(min(self.bs, n - j * self.bs))
        return {"num_blocks": self.num_blocks, "free_blocks": len(self.free),
                "used_blocks": len(holders), "shared_blocks": sum(1 for h in holders.values() if len(h) > 1),
                "logical_blocks": sum(len(b) for b, _ in self.seqs.values()),
                "tokens": sum(n for _, n in self.seqs.values()),
                "stored_tokens": sum(max(h) for h in holders.values()), "num_seqs": len(self.seqs)}

    def prefix_groups(self, sids, max_chunk: int):
        """Column chunks for reading shared leading blocks once per group: a group is a run of
        listed sequences whose first block is the same block with a count above one (any other
        sequence is a group of its own), cut into chunks of at most ``max_chunk`` sequences.
        Per listed sequence: the index of its chunk's first sequence, the chunk's source (the
        member with the most leading blocks held by several sequences, the first such on a
        tie), and how many leading table entries it has equal to the source's -- at the
        source, the most of any other member (0 alone).  Sharing blocks is the pages' own
        structure ("PagedAttention: Optimizing KV Cache in vLLM", §4: sharers' tables point at
        the same physical blocks); the chunking is this library's."""
        if max_chunk < 1:
            raise AllocError(INVALID_ARG)
        rows = []
        for sid in sids:
            if sid not in self.seqs:
                raise AllocError(UNKNOWN_SEQ)
            rows.append(self.seqs[sid][0])
        n = len(rows)

        def head(i):
            b = rows[i]
            return b[0] if b and self.ref[b[0]] > 1 else None

        def lead(i):
            c = 0
            while c < len(rows[i]) and self.ref[rows[i][c]] > 1:
                c += 1
            return c

        first, src, blocks = [0] * n, [0] * n, [0] * n
        i = 0
        while i < n:
            end = i + 1
            if head(i) is not None:
                while end < n and head(end) == head(i):
                    end += 1
            for c0 in range(i, end, max_chunk):
                members = list(range(c0, min(end, c0 + max_chunk)))
                best = max(lead(k) for k in members)
                source = next(k for k in members if lead(k) == best)
                for k in members:
                    first[k], src[k] = c0, source
                    same = 0
                    while (same < len(rows[k]) and same < len(rows[source])
                           and rows[k][same] == rows[source][same]):
                        same += 1
                    blocks[k] = same
                blocks[source] = max([blocks[k] for k in members if k != source], default=0)
            i = end
        return first, src, blocks

    # ---- invariants ----------------------------------------------------------------
    def check_invariants(self):
        check_allocator_state(self.num_blocks, self.bs, set(self.free), self.ref,
                              {s: (b, n) for s, (b, n) in self.seqs.items()})


def check_allocator_state(num_blocks, bs, free_set, ref, seqs):
    """Invariants any correct allocator state satisfies (used on the model and the C++ one).

    seqs: id -> (blocks, length); ref: per-block reference counts; free_set: free IDs.
    """
    counts = [0] * num_blocks
    for blocks, n in seqs.values():
        assert len(blocks) == _ceil_div(n, bs), "blocks must cover exactly the tokens"
        # Waste bound: only the last block may be partly empty, by less than one block.
        assert 0 <= len(blocks) * bs - n < bs or (n == 0 and not blocks)
        for b in blocks:
            assert 0 <= b < num_blocks
            counts[b] += 1
        assert len(set(blocks)) == len(blocks), "a sequence never holds a block twice"
    for b in range(num_blocks):
        assert ref[b] == counts[b], f"refcount of block {b}: {ref[b]} != {counts[b]} users"
        assert (ref[b] == 0) == (b in free_set), f"block {b} free/used mismatch"
    assert len(free_set) + sum(1 for c in counts if c > 0) == num_blocks
