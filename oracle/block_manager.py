"""Oracle: a plain Python model of the paged KV block manager.

Test infrastructure only (see the package docstring).

What the pages fix, and where:

* Blocks are handed out on demand from a shared pool, any free block will do,
  and no contiguity is needed ("KV Cache与长上下文管理", the section on
  fragmentation: two freed 2048-token regions still serve a 4096-token request
  once allocation is by page; "One Deep Concept #01", §3 Problem and §4 Core
  Innovation).
* Each block carries a reference count; a sequence that appends to a block
  whose count is above one first copies that block, drops the shared count by
  one and writes into the copy, whose count is one ("PagedAttention — 把 KV
  cache 当虚拟内存页来管理", 核心要点 and 实践案例 / 案例 3, with a count of 4 for
  four samples sharing a prompt block).
* A sliding window is a ring of pages: the oldest page is marked invalid, the
  new token is written into it and only the page-table order changes; no KV
  data moves, whatever the context length ("KV Cache与长上下文管理", the section
  on the second problem paging solves; "PagedAttention的终极用途", part 三).

Readings of what the pages leave open (this project's choices):

* Free-list order: a FIFO queue, initially in the order the caller passes (the
  tests pass a seeded permutation); allocation pops the head; a block whose
  count drops to zero is pushed to the tail, in logical order within a sequence.
* Copy-on-write happens only for the last, partly filled block, when the new
  token's offset is above zero and the block's count is above one. A token at
  offset zero opens a fresh block and copies nothing.
* Ring: when a sequence already holds ``window_blocks`` live blocks and needs a
  new one, its oldest live block is evicted. If no other sequence holds it
  (count one) its physical id is reused as the new last block; otherwise its
  count drops by one and a fresh block comes from the free list. The table row
  stays in logical order (front dropped, id pushed to the back). The live
  context is ``tokens appended - block_size * blocks evicted``.
* Swapping ("KV Cache与长上下文管理", the fourth point: only a paged cache can
  swap page by page, cold pages to host memory and back on demand, instead of
  moving a whole contiguous cache). The unit here is one sequence's live
  blocks: ``swap_out`` gives each of them a block of a host pool (a FIFO free
  list of its own, ascending ids unless an order is given), in logical order,
  and returns the ``(device, host)`` copy pairs; a device block that no one
  else holds returns to the device free list (tail, logical order), a shared
  one only loses a count, so the sequences still holding it are untouched.
  ``swap_in`` takes one device block per host block from the device free list
  and returns the ``(host, device)`` pairs; the host blocks return to the tail
  of the host free list. Blocks shared before a swap-out come back as private
  copies. A swapped-out sequence cannot append, fork or be exported for decode;
  freeing it returns its host blocks.
* Prefix caching ("KV Cache与长上下文管理", section 二, item 2: a system prompt
  or a common history prefix is stored once and reused by many users).
  ``add_seq_prefix`` registers a sequence from its token ids. Every full block
  is looked up under the key (physical block before it, or -1 for the first;
  the block's token ids): a live block registered under that key is shared
  (its count rises by one) and its tokens get slot -1 (nothing to write);
  otherwise a fresh block is taken and registered. Keying on the previous
  physical block makes a match imply that the whole prefix matches. The
  partly filled last block is never shared. A block leaves the index when its
  count drops to zero. Only managers without a ring use it (an evicted or
  reused block would leave stale keys behind).
* Every call is atomic: on error nothing changes.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np


class BMError(Exception):
    code = -5     # state error


class InvalidArg(BMError):
    code = -1


class OutOfBlocks(BMError):
    code = -3


class OutOfRange(BMError):
    code = -4


class StateError(BMError):
    code = -5


class Unsupported(BMError):
    code = -2


@dataclass
class _Seq:
    table: list = field(default_factory=list)   # live physical blocks, logical order
    tokens: int = 0                              # tokens appended in total
    evicted: int = 0                             # blocks dropped by the ring
    swapped: bool = False                        # table holds host-pool block ids


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None,
                 window_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or window_blocks < 0:
            raise InvalidArg("bad geometry")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.window = window_blocks
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.seqs: dict[int, _Seq] = {}
        self.num_host_blocks = 0
        self.host_free: deque = deque()
        self.prefix: dict = {}          # (previous block or -1, token ids) -> block
        self.prefix_key: dict = {}      # block -> its key in self.prefix

    # -- queries -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def ref_count(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise OutOfRange("block id")
        return self.ref[block]

    def context_len(self, seq: int) -> int:
        st = self._get(seq)
        return st.tokens - self.block_size * st.evicted

    def table(self, seq: int):
        st = self._get(seq)
        return list(st.table), self.context_len(seq)

    def export(self, seqs, cap: int):
        """Tables ``[n][cap]`` (unused entries -1) and live context lengths ``[n]``."""
        rows = np.full((len(seqs), cap), -1, dtype=np.int32)
        ctx = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            st = self._resident(s)
            if len(st.table) > cap:
                raise OutOfRange("table row longer than cap")
        for i, s in enumerate(seqs):
            st = self.seqs[s]
            rows[i, :len(st.table)] = st.table
            ctx[i] = self.context_len(s)
        return rows, ctx

    # -- mutations -----------------------------------------------------------
    def add_seq(self, seq: int, prefill_tokens: int) -> np.ndarray:
        """Register ``seq`` with ``prefill_tokens`` tokens; returns their slots."""
        if seq in self.seqs:
            raise StateError("sequence exists")
        if prefill_tokens < 0:
            raise InvalidArg("negative prefill")
        nb = -(-prefill_tokens // self.block_size)
        if self.window and nb > self.window:
            raise InvalidArg("prefill longer than the window")
        if nb > len(self.free):
            raise OutOfBlocks("pool exhausted")
        st = _Seq()
        for _ in range(nb):
            b = self.free.popleft()
            self.ref[b] = 1
            st.table.append(b)
        st.tokens = prefill_tokens
        self.seqs[seq] = st
        bs = self.block_size
        return np.array([st.table[t // bs] * bs + t % bs for t in range(prefill_tokens)],
                        dtype=np.int64)

    def add_seq_prefix(self, seq: int, tokens):
        """Register ``seq`` from its token ids, sharing cached full blocks.

        Returns ``(slots, shared_blocks)``: the slots of the tokens to write
        (-1 for tokens of shared blocks) and how many leading blocks were shared.
        """
        if self.window:
            raise Unsupported("prefix caching with a ring")
        if seq in self.seqs:
            raise StateError("sequence exists")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        n = len(tokens)
        nb = -(-n // bs)
        plan, prev = [], -1
        for i in range(nb):
            chunk = tuple(tokens[i * bs:(i + 1) * bs])
            hit = self.prefix.get((prev, chunk)) if len(chunk) == bs else None
            if hit is None:
                break
            plan.append(hit)
            prev = hit
        shared = len(plan)
        if nb - shared > len(self.free):
            raise OutOfBlocks("pool exhausted")
        st = _Seq()
        prev = -1
        for i in range(nb):
            chunk = tuple(tokens[i * bs:(i + 1) * bs])
            if i < shared:
                b = plan[i]
                self.ref[b] += 1
            else:
                b = self.free.popleft()
                self.ref[b] = 1
                if len(chunk) == bs:
                    self.prefix[(prev, chunk)] = b
                    self.prefix_key[b] = (prev, chunk)
            st.table.append(b)
            prev = b
        st.tokens = n
        self.seqs[seq] = st
        slots = np.array([-1 if t // bs < shared else st.table[t // bs] * bs + t % bs for t in range(n)],
                         dtype=np.int64)
        return slots, shared

    def _release(self, b: int) -> None:
        """Drop one count of device block ``b``; at zero it is free and unindexed."""
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)
            key = self.prefix_key.pop(b, None)
            if key is not None:
                del self.prefix[key]

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (each count rises by one)."""
        p = self._resident(parent)
        if child in self.seqs:
            raise StateError("child exists")
        for b in p.table:
            self.ref[b] += 1
        self.seqs[child] = _Seq(list(p.table), p.tokens, p.evicted)

    def append(self, seq: int):
        """Make room for one new token; returns ``(slot, copy_src, copy_dst)``.

        ``copy_src``/``copy_dst`` are -1 when no block has to be copied first.
        """
        st = self._resident(seq)
        bs = self.block_size
        offset = st.tokens % bs
        src = dst = -1
        if offset == 0:
            if self.window and len(st.table) == self.window:
                oldest = st.table[0]
                if self.ref[oldest] == 1:
                    st.table.pop(0)
                    st.table.append(oldest)          # reuse in place: no data moves
                else:
                    if not self.free:
                        raise OutOfBlocks("pool exhausted")
                    st.table.pop(0)
                    self.ref[oldest] -= 1
                    b = self.free.popleft()
                    self.ref[b] = 1
                    st.table.append(b)
                st.evicted += 1
            else:
                if not self.free:
                    raise OutOfBlocks("pool exhausted")
                b = self.free.popleft()
                self.ref[b] = 1
                st.table.append(b)
        else:
            last = st.table[-1]
            if self.ref[last] > 1:
                if not self.free:
                    raise OutOfBlocks("pool exhausted")
                b = self.free.popleft()
                self.ref[last] -= 1
                self.ref[b] = 1
                st.table[-1] = b
                src, dst = last, b
        st.tokens += 1
        return st.table[-1] * bs + offset, src, dst

    def free_seq(self, seq: int) -> None:
        st = self._get(seq)
        if st.swapped:
            self.host_free.extend(st.table)
        else:
            for b in st.table:
                self._release(b)
        del self.seqs[seq]

    # -- swapping ------------------------------------------------------------
    def set_host_blocks(self, num_host_blocks: int, free_order=None) -> None:
        """Give the manager a host pool of ``num_host_blocks`` blocks (once)."""
        if self.num_host_blocks:
            raise StateError("host pool already set")
        if num_host_blocks <= 0:
            raise InvalidArg("host pool size")
        order = list(range(num_host_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_host_blocks)):
            raise InvalidArg("host free order must be a permutation of the host pool")
        self.num_host_blocks = num_host_blocks
        self.host_free = deque(order)

    def num_host_free(self) -> int:
        return len(self.host_free)

    def is_swapped(self, seq: int) -> bool:
        return self._get(seq).swapped

    def swap_out(self, seq: int):
        """Move ``seq``'s live blocks to the host pool; returns ``[(device, host)]``."""
        st = self._resident(seq)
        if not self.num_host_blocks:
            raise StateError("no host pool")
        if len(st.table) > len(self.host_free):
            raise OutOfBlocks("host pool exhausted")
        pairs = []
        for b in st.table:
            hb = self.host_free.popleft()
            pairs.append((b, hb))
            self._release(b)
        st.table = [hb for _, hb in pairs]
        st.swapped = True
        return pairs

    def swap_in(self, seq: int):
        """Bring ``seq``'s blocks back into the device pool; returns ``[(host, device)]``."""
        st = self._get(seq)
        if not st.swapped:
            raise StateError("sequence is resident")
        if len(st.table) > len(self.free):
            raise OutOfBlocks("pool exhausted")
        pairs = []
        for hb in st.table:
            b = self.free.popleft()
            self.ref[b] = 1
            pairs.append((hb, b))
            self.host_free.append(hb)
        st.table = [b for _, b in pairs]
        st.swapped = False
        return pairs

    # -- helpers -------------------------------------------------------------
    def _get(self, seq: int) -> _Seq:
        if seq not in self.seqs:
            raise StateError("unknown sequence")
        return self.seqs[seq]

    def _resident(self, seq: int) -> _Seq:
        st = self._get(seq)
        if st.swapped:
            raise StateError("sequence is swapped out")
        return st
