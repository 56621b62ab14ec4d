"""One decode step of the paged KV cache, end to end.

A step appends one token to each sequence of a batch and attends with it:

1. host block manager (native): one slot per sequence, copy-on-write pairs,
   ring evictions, then the batch's table rows and live context lengths —
   all written into pinned staging buffers by two library calls;
2. asynchronous uploads of those buffers on the step's stream;
3. ``pa_copy_blocks`` for the copy-on-write pairs (only when there are any);
4. ``pa_write_kv`` of the new K/V rows into their slots;
5. ``pa_decode`` (single pass, or split-K partitions plus the reduce kernel).

The host never waits for the device inside a step: staging buffers rotate
through a small ring guarded by events, so the host prepares step k+1 while
the device still runs step k.
"""

from __future__ import annotations

import numpy as np
import torch

from . import native as N


class PagedDecodeEngine:
    def __init__(self, num_blocks: int, num_heads: int, head_dim: int, kv_dtype: int,
                 max_seqs: int, max_blocks_per_seq: int, *, window_blocks: int = 0,
                 free_order=None, device="cuda", partition_tokens: int = 0,
                 pool_fill=None, staging_depth: int = 3, longest_first: bool = True):
        self.device = torch.device(device)
        self.num_heads, self.head_dim = num_heads, head_dim
        self.pool = N.new_pool(num_blocks, num_heads, head_dim, kv_dtype, device=self.device, fill=pool_fill)
        self.bm = N.BlockManager(num_blocks, N.BLOCK_SIZE, free_order=free_order, window_blocks=window_blocks)
        self.max_seqs = max_seqs
        self.cap = max_blocks_per_seq
        self.partition_tokens = partition_tokens
        # Dispatch sequences longest first (pa_decode_ordered): the host knows
        # every context length, so the schedule costs one argsort per step.
        self.longest_first = longest_first
        dev = self.device
        # Everything a step uploads lives in one packed buffer so that a step
        # makes a single host-to-device copy:
        #   slots int64 [max_seqs] | ctx int32 [max_seqs] | order int32 [max_seqs]
        #   | pairs int32 [max_seqs][2] | tables int32 [max_seqs][cap]
        self._off_ctx = 8 * max_seqs
        self._off_order = self._off_ctx + 4 * max_seqs
        self._off_pairs = self._off_order + 4 * max_seqs
        self._off_tables = self._off_pairs + 8 * max_seqs
        self._stage_bytes = self._off_tables + 4 * max_seqs * self.cap
        self._dev_stage = torch.zeros(self._stage_bytes, dtype=torch.uint8, device=dev)
        self.slots, self.ctx, self.order, self.pairs, self.tables = self._views(self._dev_stage)
        self.tables.fill_(-1)
        self.workspace = None
        self._ws_bytes = 0
        self._staging = []
        for _ in range(staging_depth):
            buf = torch.empty(self._stage_bytes, dtype=torch.uint8, pin_memory=True)
            slots, ctx, order, pairs, tables = self._views(buf)
            self._staging.append({"buf": buf, "slots": slots.numpy(), "ctx": ctx.numpy(),
                                  "order": order.numpy(), "pairs": pairs.numpy(),
                                  "tables": tables.numpy(), "event": None})
        self._next = 0
        self.last_ctx = np.zeros(0, dtype=np.int32)
        self.last_pairs = 0

    def _views(self, buf):
        """(slots, ctx, order, pairs, tables) views of a packed staging buffer."""
        m = self.max_seqs
        slots = buf[:self._off_ctx].view(torch.int64)
        ctx = buf[self._off_ctx:self._off_order].view(torch.int32)
        order = buf[self._off_order:self._off_pairs].view(torch.int32)
        pairs = buf[self._off_pairs:self._off_tables].view(torch.int32).view(m, 2)
        tables = buf[self._off_tables:self._stage_bytes].view(torch.int32).view(m, self.cap)
        return slots, ctx, order, pairs, tables

    # -- setup -----------------------------------------------------------------
    def add_sequence(self, seq: int, k_rows=None, v_rows=None, prefill_tokens: int | None = None):
        """Register ``seq`` and write its prefill rows ``[n][heads][head_dim]``."""
        n = int(k_rows.shape[0]) if k_rows is not None else int(prefill_tokens or 0)
        slots = self.bm.add_seq(seq, n)
        if n and k_rows is not None:
            N.pa_write_kv(self.pool, k_rows, v_rows, torch.from_numpy(slots).to(self.device))
        return slots

    def fork(self, parent: int, child: int) -> None:
        self.bm.fork(parent, child)

    def free_sequence(self, seq: int) -> None:
        self.bm.free_seq(seq)

    def _workspace_for(self, n: int, max_ctx: int):
        need = N.pa_decode_workspace_bytes(self.pool, n, max_ctx, self.partition_tokens)
        if need > self._ws_bytes:
            # Grow geometrically so that a growing context does not reallocate every step.
            self._ws_bytes = max(need, int(self._ws_bytes * 1.5))
            self.workspace = torch.empty(self._ws_bytes // 4 + 1, dtype=torch.float32, device=self.device)
        return self.workspace

    # -- the step ---------------------------------------------------------------
    def step(self, seqs, k_new, v_new, q, out, *, decode: bool = True, stream=None,
             decode_events=None) -> None:
        """Append one token per sequence of ``seqs`` (order = rows of k_new/q) and decode.

        ``decode_events``: optional (start, end) torch events recorded on the
        step's stream right before and after the decode launch(es).
        """
        seqs = np.asarray(seqs, dtype=np.int64)
        n = seqs.size
        if n > self.max_seqs:
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, f"batch of {n} > max_seqs {self.max_seqs}")
        st = self._staging[self._next]
        self._next = (self._next + 1) % len(self._staging)
        if st["event"] is not None:
            st["event"].synchronize()         # the uploads that last read this buffer are done
        _, pairs = self.bm.append_batch(seqs, slots_out=st["slots"], pairs_out=st["pairs"])
        npairs = int(pairs.shape[0])
        tables_np = st["tables"][:n]
        ctx_np = st["ctx"][:n]
        self.bm.export(seqs, self.cap, tables_out=tables_np, ctx_out=ctx_np)
        max_ctx = int(ctx_np.max()) if n else 0
        if decode and self.longest_first:
            st["order"][:n] = np.argsort(-ctx_np, kind="stable")
        self.last_ctx = ctx_np.copy()
        self.last_pairs = npairs
        self.last_pair_list = pairs.copy()
        self.last_slots = st["slots"][:n].copy()

        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        with torch.cuda.stream(cur):
            # One copy: everything up to the end of this batch's table rows.
            upto = self._off_tables + 4 * n * self.cap if decode else self._off_tables
            self._dev_stage[:upto].copy_(st["buf"][:upto], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(cur)
            st["event"] = ev
            if npairs:
                N.pa_copy_blocks(self.pool, self.pairs[:npairs], stream=cur)
            N.pa_write_kv(self.pool, k_new, v_new, self.slots[:n], stream=cur)
            if decode:
                ws = self._workspace_for(n, max_ctx) if self.partition_tokens else None
                if decode_events is not None:
                    decode_events[0].record(cur)
                N.pa_decode(self.pool, q, out, self.tables[:n], self.ctx[:n], max_ctx,
                            partition_tokens=self.partition_tokens, workspace=ws, stream=cur,
                            seq_order=self.order[:n] if self.longest_first else None)
                if decode_events is not None:
                    decode_events[1].record(cur)

    def decode(self, seqs, q, out, *, partition_tokens=None, stream=None, longest_first=None) -> None:
        """Decode the batch as it stands (no append): tables and contexts uploaded first."""
        seqs = np.asarray(seqs, dtype=np.int64)
        n = seqs.size
        tables, ctx = self.bm.export(seqs, self.cap)
        max_ctx = int(ctx.max()) if n else 0
        ptok = self.partition_tokens if partition_tokens is None else partition_tokens
        lf = self.longest_first if longest_first is None else longest_first
        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        with torch.cuda.stream(cur):
            self.tables[:n].copy_(torch.from_numpy(tables))
            self.ctx[:n].copy_(torch.from_numpy(ctx))
            if lf:
                self.order[:n].copy_(torch.from_numpy(np.argsort(-ctx, kind="stable").astype(np.int32)))
            ws = None
            if ptok:
                need = N.pa_decode_workspace_bytes(self.pool, n, max_ctx, ptok)
                ws = torch.empty(need // 4 + 1, dtype=torch.float32, device=self.device)
            N.pa_decode(self.pool, q, out, self.tables[:n], self.ctx[:n], max_ctx,
                        partition_tokens=ptok, workspace=ws, stream=cur,
                        seq_order=self.order[:n] if lf else None)
        self.last_ctx = ctx
