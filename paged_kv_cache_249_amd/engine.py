"""One decode step of the paged KV cache, end to end.

A step appends one token to each sequence of a batch and attends with it:

1. host block manager (native): one slot per sequence, copy-on-write pairs,
   ring evictions, then the batch's table rows and live context lengths —
   all written into a pinned staging buffer by two library calls, plus the
   longest-first dispatch order;
2. ``pa_stage_copy`` uploads that buffer with one small kernel on the step's
   stream (``overlap_uploads=True`` moves it to an auxiliary stream that the
   step's kernels wait on with an event; measured, the cross-stream wait costs
   about what the overlap saves, so it is off by default);
3. ``pa_copy_blocks`` for the copy-on-write pairs (only when there are any);
4. ``pa_write_kv`` of the new K/V rows into their slots and
5. ``pa_decode_ordered`` (single pass, or split-K partitions plus the reduce
   kernel) — for float pools both in one launch, ``pa_write_decode``.

The host never waits for the device inside a step: pinned staging buffers
rotate through a small ring guarded by events, and two device staging buffers
alternate so an upload never overwrites the tables a running decode reads.
"""

from __future__ import annotations

import numpy as np
import torch

from . import native as N


class PagedDecodeEngine:
    def __init__(self, num_blocks: int, num_heads: int, head_dim: int, kv_dtype: int,
                 max_seqs: int, max_blocks_per_seq: int, *, window_blocks: int = 0,
                 free_order=None, device="cuda", partition_tokens: int = 0,
                 pool_fill=None, staging_depth: int = 3, longest_first: bool = True,
                 overlap_uploads: bool = False, fuse_write: bool = True, block_size: int = N.BLOCK_SIZE):
        self.device = torch.device(device)
        self.num_heads, self.head_dim = num_heads, head_dim
        self.kv_dtype = kv_dtype
        self.block_size = block_size
        self.pool = N.new_pool(num_blocks, num_heads, head_dim, kv_dtype, device=self.device, fill=pool_fill,
                               block_size=block_size)
        self.bm = N.BlockManager(num_blocks, block_size, free_order=free_order, window_blocks=window_blocks)
        self.max_seqs = max_seqs
        self.cap = max_blocks_per_seq
        self.partition_tokens = partition_tokens
        # Dispatch sequences longest first (pa_decode_ordered): the host knows
        # every context length, so the schedule costs one argsort per step.
        self.longest_first = longest_first
        # Float pools write the new token inside the decode launch (pa_write_decode).
        self.fuse_write = fuse_write and kv_dtype != N.PA_I8
        dev = self.device
        # Everything a step uploads lives in one packed buffer:
        #   slots int64 [max_seqs] | ctx int32 [max_seqs] | order int32 [max_seqs]
        #   | pairs int32 [max_seqs][2] | tables int32 [max_seqs][cap]
        self._off_ctx = 8 * max_seqs
        self._off_order = self._off_ctx + 4 * max_seqs
        self._off_pairs = self._off_order + 4 * max_seqs
        self._off_tables = self._off_pairs + 8 * max_seqs
        self._stage_bytes = -(-(self._off_tables + 4 * max_seqs * self.cap) // 16) * 16
        self._dev = []
        for _ in range(2):
            v = self._views(torch.zeros(self._stage_bytes, dtype=torch.uint8, device=dev))
            v["tables"].fill_(-1)
            v["released"] = None          # event: the last kernel reading this buffer is done
            self._dev.append(v)
        self._cur = 0
        self.workspace = None
        self._ws_bytes = 0
        self._staging = []
        for _ in range(staging_depth):
            v = self._views(torch.empty(self._stage_bytes, dtype=torch.uint8, pin_memory=True))
            v = {k: (t if k == "buf" else t.numpy()) for k, t in v.items()}
            v["event"] = None             # event: the upload that last read this buffer is done
            self._staging.append(v)
        self._next = 0
        self._aux = torch.cuda.Stream(device=dev) if overlap_uploads else None
        self.last_ctx = np.zeros(0, dtype=np.int32)
        self.last_pairs = 0

    def _views(self, buf):
        m = self.max_seqs
        return {
            "buf": buf,
            "slots": buf[:self._off_ctx].view(torch.int64),
            "ctx": buf[self._off_ctx:self._off_order].view(torch.int32),
            "order": buf[self._off_order:self._off_pairs].view(torch.int32),
            "pairs": buf[self._off_pairs:self._off_tables].view(torch.int32).view(m, 2),
            "tables": buf[self._off_tables:self._off_tables + 4 * m * self.cap].view(torch.int32).view(m, self.cap),
        }

    # Device views of the staging buffer the latest step used.
    @property
    def slots(self):
        return self._dev[self._cur]["slots"]

    @property
    def tables(self):
        return self._dev[self._cur]["tables"]

    @property
    def ctx(self):
        return self._dev[self._cur]["ctx"]

    @property
    def order(self):
        return self._dev[self._cur]["order"]

    # -- setup -----------------------------------------------------------------
    def add_sequence(self, seq: int, k_rows=None, v_rows=None, prefill_tokens: int | None = None):
        """Register ``seq`` and write its prefill rows ``[n][heads][head_dim]``."""
        n = int(k_rows.shape[0]) if k_rows is not None else int(prefill_tokens or 0)
        slots = self.bm.add_seq(seq, n)
        if n and k_rows is not None:
            N.pa_write_kv(self.pool, k_rows, v_rows, torch.from_numpy(slots).to(self.device))
        return slots

    def add_sequence_prefix(self, seq: int, tokens, k_rows, v_rows):
        """Register ``seq`` from its token ids, sharing cached full blocks
        (prefix caching), and write the rows of the tokens not shared.
        Returns the number of shared blocks."""
        slots, shared = self.bm.add_seq_prefix(seq, tokens)
        if slots.size and shared * self.block_size < slots.size:
            N.pa_write_kv(self.pool, k_rows, v_rows, torch.from_numpy(slots).to(self.device))
        return shared

    def fork(self, parent: int, child: int) -> None:
        self.bm.fork(parent, child)

    def free_sequence(self, seq: int) -> None:
        self.bm.free_seq(seq)

    # -- swapping --------------------------------------------------------------
    def enable_swap(self, host_blocks: int, host_free_order=None) -> None:
        """Give the engine a host pool of ``host_blocks`` blocks in pinned memory."""
        self.host = N.HostPool(self.pool, host_blocks)
        self.bm.set_host_pool(host_blocks, host_free_order)

    def swap_out(self, seqs, stream=None) -> np.ndarray:
        """Move the blocks of ``seqs`` to the host pool; returns the (device, host) pairs."""
        return self._swap(seqs, True, stream)

    def swap_in(self, seqs, stream=None) -> np.ndarray:
        """Bring ``seqs`` back into the device pool; returns the (host, device) pairs."""
        return self._swap(seqs, False, stream)

    def _swap(self, seqs, out: bool, stream) -> np.ndarray:
        # The manager moves one sequence at a time; if one fails, the copies of
        # those already moved are still issued before the error propagates.
        done, err = [], None
        for s in np.asarray(seqs, dtype=np.int64).reshape(-1):
            try:
                done.append(self.bm.swap_out(int(s)) if out else self.bm.swap_in(int(s)))
            except N.PagedKVError as e:
                err = e
                break
        pairs = np.concatenate(done) if done else np.zeros((0, 2), np.int32)
        if pairs.shape[0]:
            cur = torch.cuda.current_stream(self.device) if stream is None else stream
            host = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).pin_memory()
            with torch.cuda.stream(cur):
                dev = host.to(self.device, non_blocking=True)
                for i in range(0, pairs.shape[0], 65535):
                    N.pa_swap_blocks(self.pool, self.host, dev[i:i + 65535],
                                     N.PA_SWAP_OUT if out else N.PA_SWAP_IN, stream=cur)
        if err is not None:
            raise err
        return pairs

    def _workspace_for(self, n: int, max_ctx: int, ptok: int):
        need = N.pa_decode_workspace_bytes(self.pool, n, max_ctx, ptok)
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
            st["event"].synchronize()         # the upload that last read this buffer is done
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
        self._cur ^= 1
        dv = self._dev[self._cur]
        # Everything up to the end of this batch's table rows, in one upload.
        upto = self._off_tables + 4 * n * self.cap if decode else self._off_tables
        upto = -(-upto // 16) * 16
        up = self._aux if self._aux is not None else cur
        if dv["released"] is not None and up is not cur:
            up.wait_event(dv["released"])     # no kernel still reads this device buffer
        N.pa_stage_copy(dv["buf"], st["buf"], upto, stream=up)
        uploaded = torch.cuda.Event()
        uploaded.record(up)
        st["event"] = uploaded
        if up is not cur:
            cur.wait_event(uploaded)
        with torch.cuda.stream(cur):
            if npairs:
                N.pa_copy_blocks(self.pool, dv["pairs"][:npairs], stream=cur)
            fused = decode and self.fuse_write
            if not fused:
                N.pa_write_kv(self.pool, k_new, v_new, dv["slots"][:n], stream=cur)
            if decode:
                ptok = self.partition_tokens
                ws = self._workspace_for(n, max_ctx, ptok) if ptok else None
                order = dv["order"][:n] if self.longest_first else None
                if decode_events is not None:
                    decode_events[0].record(cur)
                if fused:
                    N.pa_write_decode(self.pool, k_new, v_new, dv["slots"][:n], q, out, dv["tables"][:n],
                                      dv["ctx"][:n], max_ctx, partition_tokens=ptok, workspace=ws,
                                      stream=cur, seq_order=order)
                else:
                    N.pa_decode(self.pool, q, out, dv["tables"][:n], dv["ctx"][:n], max_ctx,
                                partition_tokens=ptok, workspace=ws, stream=cur, seq_order=order)
                if decode_events is not None:
                    decode_events[1].record(cur)
            done = torch.cuda.Event()
            done.record(cur)
            dv["released"] = done

    def decode(self, seqs, q, out, *, partition_tokens=None, stream=None, longest_first=None) -> None:
        """Decode the batch as it stands (no append): tables and contexts uploaded first."""
        seqs = np.asarray(seqs, dtype=np.int64)
        n = seqs.size
        tables, ctx = self.bm.export(seqs, self.cap)
        max_ctx = int(ctx.max()) if n else 0
        ptok = self.partition_tokens if partition_tokens is None else partition_tokens
        lf = self.longest_first if longest_first is None else longest_first
        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        dv = self._dev[self._cur]
        with torch.cuda.stream(cur):
            dv["tables"][:n].copy_(torch.from_numpy(tables))
            dv["ctx"][:n].copy_(torch.from_numpy(ctx))
            if lf:
                dv["order"][:n].copy_(torch.from_numpy(np.argsort(-ctx, kind="stable").astype(np.int32)))
            ws = None
            if ptok:
                need = N.pa_decode_workspace_bytes(self.pool, n, max_ctx, ptok)
                ws = torch.empty(need // 4 + 1, dtype=torch.float32, device=self.device)
            N.pa_decode(self.pool, q, out, dv["tables"][:n], dv["ctx"][:n], max_ctx,
                        partition_tokens=ptok, workspace=ws, stream=cur,
                        seq_order=dv["order"][:n] if lf else None)
            done = torch.cuda.Event()
            done.record(cur)
            dv["released"] = done
        self.last_ctx = ctx
