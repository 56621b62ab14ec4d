"""Oracle: mixed-precision pages — an fp16 hot tail block, int8 cold blocks.

Test infrastructure only (see the package docstring).

What the pages say: pages used often stay in FP16, pages used rarely are
stored quantised to INT8, and cold pages are backed up in host memory
("PagedAttention 的技术溯源与演进脉络", §4.1 on page thrashing, item 2: mixed-
precision page management); FP16 -> INT8 KV compression halves the memory
("KV Cache与长上下文管理", section 二.3).

Reading taken (this project's): the hot page of a sequence is its newest
block — the one every decode step writes — kept in an fp16 pool, one block
per sequence for the sequence's whole life; every older block is cold, in an
int8 pool with one fp16 scale per (block, head) for K and V. When the hot
block is full and the next token arrives, the block is *demoted*: its 16
rows are quantised in one group per (block, head) into a fresh cold block
(the int8 rule of :mod:`oracle.cache_ops` with the whole block written at
once, so ``s = fp16(max|x| / 127)`` and no earlier scale is involved), and the
hot block is reused from offset 0 for the new token. Cold blocks are written
once and never change, so they can be shared by reference count (a fork
shares them; the child gets its own hot block, a copy of the parent's).
Prefill writes full blocks straight into the cold pool (same rule) and the
remainder into the hot block. Block size 16.

The cold pool may also hold int4 codes (the same page lists INT4 after INT8
as the next compression step): the same demotion with codes in [-7, 7] and
``s = fp16(max|x| / 7)`` (:func:`oracle.cache_ops.write_kv_int4`'s rule).

Layout: a sequence of ``ctx`` tokens has ``max(0, ceil(ctx / 16) - 1)`` cold
blocks holding tokens ``[0, 16 * n_cold)`` and its hot block holding tokens
``[16 * n_cold, ctx)`` (1 to 16 of them when ``ctx > 0``).
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

from . import attention, cache_ops
from .block_manager import InvalidArg, OutOfBlocks, OutOfRange, StateError

BS = 16


@dataclass
class _MSeq:
    cold: list = field(default_factory=list)    # cold blocks, logical order
    hot: int = -1                                # the hot block
    tokens: int = 0


class MixedBlockManager:
    """Free lists and reference counts of the two pools (FIFO, as in R5)."""

    def __init__(self, num_cold: int, num_hot: int, cold_order=None, hot_order=None):
        if num_cold <= 0 or num_hot <= 0:
            raise InvalidArg("pool sizes")
        co = list(range(num_cold)) if cold_order is None else [int(b) for b in cold_order]
        ho = list(range(num_hot)) if hot_order is None else [int(b) for b in hot_order]
        if sorted(co) != list(range(num_cold)) or sorted(ho) != list(range(num_hot)):
            raise InvalidArg("free orders must be permutations")
        self.num_cold, self.num_hot = num_cold, num_hot
        self.cold_free = deque(co)
        self.hot_free = deque(ho)
        self.ref = [0] * num_cold
        self.seqs: dict[int, _MSeq] = {}

    def _get(self, seq):
        if seq not in self.seqs:
            raise StateError("unknown sequence")
        return self.seqs[seq]

    def add_seq(self, seq: int, prefill_tokens: int):
        """Returns ``(cold_slots, hot_slots)``, each ``[prefill_tokens]`` with -1
        for the tokens that go to the other pool."""
        if seq in self.seqs:
            raise StateError("sequence exists")
        if prefill_tokens < 0:
            raise InvalidArg("negative prefill")
        n = prefill_tokens
        n_cold = max(0, -(-n // BS) - 1)
        if not self.hot_free or n_cold > len(self.cold_free):
            raise OutOfBlocks("pool exhausted")
        st = _MSeq()
        for _ in range(n_cold):
            b = self.cold_free.popleft()
            self.ref[b] = 1
            st.cold.append(b)
        st.hot = self.hot_free.popleft()
        st.tokens = n
        self.seqs[seq] = st
        cold = np.full(n, -1, dtype=np.int64)
        hot = np.full(n, -1, dtype=np.int64)
        for t in range(n):
            if t < BS * n_cold:
                cold[t] = st.cold[t // BS] * BS + t % BS
            else:
                hot[t] = st.hot * BS + (t - BS * n_cold)
        return cold, hot

    def append(self, seq: int):
        """Room for one token: ``(hot_slot, demote_src_hot, demote_dst_cold)``
        (the last two -1 when no block is demoted)."""
        st = self._get(seq)
        src = dst = -1
        if st.tokens > 0 and st.tokens % BS == 0:
            if not self.cold_free:
                raise OutOfBlocks("cold pool exhausted")
            dst = self.cold_free.popleft()
            self.ref[dst] = 1
            st.cold.append(dst)
            src = st.hot
        off = st.tokens - BS * len(st.cold)
        st.tokens += 1
        return st.hot * BS + off, src, dst

    def fork(self, parent: int, child: int):
        """``child`` shares the parent's cold blocks and gets a copy of its hot
        block; returns the (parent hot, child hot) pair to copy."""
        p = self._get(parent)
        if child in self.seqs:
            raise StateError("child exists")
        if not self.hot_free:
            raise OutOfBlocks("hot pool exhausted")
        for b in p.cold:
            self.ref[b] += 1
        h = self.hot_free.popleft()
        self.seqs[child] = _MSeq(list(p.cold), h, p.tokens)
        return p.hot, h

    def free_seq(self, seq: int) -> None:
        st = self._get(seq)
        for b in st.cold:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.cold_free.append(b)
        self.hot_free.append(st.hot)
        del self.seqs[seq]

    def context_len(self, seq: int) -> int:
        return self._get(seq).tokens

    def export(self, seqs, cap: int):
        """Cold tables ``[n][cap]`` (-1 padded), hot blocks ``[n]``, contexts ``[n]``."""
        for s in seqs:
            if len(self._get(s).cold) > cap:
                raise OutOfRange("table row longer than cap")
        rows = np.full((len(seqs), cap), -1, dtype=np.int32)
        hot = np.zeros(len(seqs), dtype=np.int32)
        ctx = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            st = self.seqs[s]
            rows[i, :len(st.cold)] = st.cold
            hot[i] = st.hot
            ctx[i] = st.tokens
        return rows, hot, ctx


def demote(hot_k, hot_v, cold_k, cold_ks, cold_v, cold_vs, pairs, qmax: int = 127) -> None:
    """Quantise whole hot blocks into cold blocks: for every ``(hot, cold)``
    pair and head, the block's 16 rows form one group written at once (codes
    in [-qmax, qmax]: 127 for int8 cold blocks, 7 for int4)."""
    H = hot_k.shape[1]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        for h in range(H):
            cache_ops._quantise_group(cold_k, cold_ks, int(dst), h, list(range(BS)),
                                      list(hot_k[src, h].astype(np.float32)), BS, qmax)
            cache_ops._quantise_group(cold_v, cold_vs, int(dst), h, list(range(BS)),
                                      list(hot_v[src, h].astype(np.float32)), BS, qmax)


def gather(cold, cold_scale, hot, cold_row, hot_block: int, ctx: int) -> np.ndarray:
    """Rows ``[ctx][H][D]`` (float64) of one sequence: dequantised cold rows,
    then the hot block's fp16 rows."""
    n_cold = max(0, -(-ctx // BS) - 1)
    t = np.arange(BS * n_cold)
    phys = np.asarray(cold_row, dtype=np.int64)[t // BS]
    c = cold[phys, :, t % BS, :].astype(np.float64) * cold_scale[phys, :].astype(np.float64)[:, :, None]
    hrows = hot[hot_block, :, :ctx - BS * n_cold, :].astype(np.float64).transpose(1, 0, 2)
    return np.concatenate([c, hrows], axis=0)


def decode(q, cold_k, cold_ks, cold_v, cold_vs, hot_k, hot_v, cold_tables, hot_blocks, context_lens,
           scale: float | None = None) -> np.ndarray:
    """Attention of every sequence over its mixed-precision rows, float64."""
    S, H, D = q.shape
    scale = attention.default_scale(D) if scale is None else scale
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        K = gather(cold_k, cold_ks, hot_k, cold_tables[s], int(hot_blocks[s]), ctx)
        V = gather(cold_v, cold_vs, hot_v, cold_tables[s], int(hot_blocks[s]), ctx)
        out[s] = attention.attend(q[s], K, V, scale)
    return out
