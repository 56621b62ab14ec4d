"""One decode step of the paged KV cache, end to end.

A step appends one token to each sequence of a batch and attends with it:

1. host block manager (native): one slot per sequence, copy-on-write pairs,
   ring evictions, then the batch's table rows and live context lengths —
   all written into a pinned staging buffer by two library calls, plus the
   longest-first dispatch order;
2. the step's kernels read that buffer in place over the host link (the
   default where pinned memory has the same address on the device: no upload
   and one kernel boundary less per step), or ``pa_stage_copy`` uploads it
   with one small kernel first (``host_tables=False``; ``overlap_uploads=True``
   then moves the upload to an auxiliary stream that the step's kernels wait
   on with an event; measured, that wait costs about what the overlap saves);
3. ``pa_copy_blocks`` for the copy-on-write pairs (only when there are any);
4. ``pa_write_kv`` of the new K/V rows into their slots and
5. ``pa_decode_ordered`` (single pass, or split-K partitions plus the reduce
   kernel) — for float pools both in one launch, ``pa_write_decode``.

The host never waits for the device inside a step: pinned staging buffers
rotate through a small ring guarded by events (a buffer is rewritten only
after the last kernel that reads it is done), and with uploads two device
staging buffers alternate so an upload never overwrites the tables a
running decode reads.
"""

from __future__ import annotations

import numpy as np
import torch

from . import native as N


class _Staging:
    """Upload of a step's small arrays in one packed buffer.

    ``fields`` is an ordered list of ``(name, torch dtype, per-sequence
    shape)``; the last field is the only one whose upload is cut to the batch
    (the table rows). Pinned host copies rotate through a ring guarded by
    events, and two device copies alternate, each released by an event after
    the last kernel that reads it.
    """

    def __init__(self, fields, max_seqs: int, device, depth: int, aux_stream: bool):
        self.fields, self.max_seqs, self.device = fields, max_seqs, device
        self.off, o = {}, 0
        for name, dt, shape in fields:
            self.off[name] = o
            o += max_seqs * int(np.prod(shape, dtype=np.int64)) * torch.empty(0, dtype=dt).element_size()
            o = -(-o // 8) * 8
        self.bytes = -(-o // 16) * 16
        self.dev = []
        for _ in range(2):
            v = self._views(torch.zeros(self.bytes, dtype=torch.uint8, device=device))
            v["released"] = None          # event: the last kernel reading this buffer is done
            self.dev.append(v)
        self.cur = 0
        self.ring = []
        for _ in range(depth):
            tv = self._views(torch.empty(self.bytes, dtype=torch.uint8, pin_memory=True))
            v = {k: (t if k == "buf" else t.numpy()) for k, t in tv.items()}
            v["t"] = tv                   # the same pinned memory as tensors
            v["event"] = None             # event: the last kernel that reads this buffer is done
            self.ring.append(v)
        self.next = 0
        self.aux = torch.cuda.Stream(device=device) if aux_stream else None

    def _views(self, buf):
        m, out = self.max_seqs, {"buf": buf}
        for name, dt, shape in self.fields:
            size = torch.empty(0, dtype=dt).element_size() * m * int(np.prod(shape, dtype=np.int64))
            o = self.off[name]
            out[name] = buf[o:o + size].view(dt).view(m, *shape) if shape else buf[o:o + size].view(dt)
        return out

    def host(self):
        """The next pinned buffer, once the upload that last read it is done."""
        st = self.ring[self.next]
        self.next = (self.next + 1) % len(self.ring)
        if st["event"] is not None:
            st["event"].synchronize()
        return st

    def upload(self, st, n: int, stream):
        """Copy ``st`` (the last field up to row ``n``) into the next device
        buffer; kernels on ``stream`` issued afterwards see it."""
        name, dt, shape = self.fields[-1]
        row = torch.empty(0, dtype=dt).element_size() * int(np.prod(shape, dtype=np.int64))
        upto = -(-(self.off[name] + row * n) // 16) * 16
        self.cur ^= 1
        dv = self.dev[self.cur]
        up = self.aux if self.aux is not None else stream
        if dv["released"] is not None and up is not stream:
            up.wait_event(dv["released"])     # no kernel still reads this device buffer
        N.pa_stage_copy(dv["buf"], st["buf"], upto, stream=up)
        uploaded = torch.cuda.Event()
        uploaded.record(up)
        st["event"] = uploaded
        if up is not stream:
            stream.wait_event(uploaded)
        return dv

    def release(self, dv, stream) -> None:
        done = torch.cuda.Event()
        done.record(stream)
        dv["released"] = done

    def in_place_ok(self) -> bool:
        """Whether kernels can read the pinned buffers at their host
        addresses (the tensors handed to them carry those addresses)."""
        return all(N.pa_host_view(st["buf"]) == st["buf"].data_ptr() for st in self.ring)

    def release_host(self, st, stream) -> None:
        """The kernels read ``st`` in place: it may be rewritten once they are done."""
        done = torch.cuda.Event()
        done.record(stream)
        st["event"] = done


def prefill_appends(bm, seqs, counts, cap: int):
    """The block-manager side of a chunked-prefill step, all or nothing.

    ``counts[i]`` tokens are appended to sequence ``seqs[i]`` (distinct ids,
    sequence order), registering unknown sequences. Returns the chunk's slots
    (int64, in row order) and copy-on-write pairs (int32 [k][2]). Before any
    state changes, every sequence's new context must fit ``cap`` table
    entries (else ``PA_ERR_OUT_OF_RANGE``) and none may be swapped out (else
    ``PA_ERR_STATE``). New sequences are registered empty and then appended
    token by token in the same undo-logged batch as the others, which places
    their blocks as registering them with their tokens would; if the batch
    fails (``PA_ERR_OUT_OF_BLOCKS``) it is undone, the new sequences are
    removed again, and the manager is exactly as before the call.
    """
    seqs = np.asarray(seqs, dtype=np.int64).reshape(-1)
    counts = np.asarray(counts, dtype=np.int64).reshape(-1)
    bs = bm.block_size
    new = []
    for s, c in zip(seqs.tolist(), counts.tolist()):
        if bm.has_seq(s):
            if bm.is_swapped(s):
                raise N.PagedKVError(N.PA_ERR_STATE, f"sequence {s} is swapped out")
            ctx = bm.table(s)[1] + c
        else:
            new.append(s)
            ctx = c
        if -(-ctx // bs) > cap:
            raise N.PagedKVError(N.PA_ERR_OUT_OF_RANGE,
                                 f"sequence {s}: {ctx} tokens need more than {cap} table entries")
    for s in new:
        bm.add_seq(s, 0)
    try:
        slots, pairs = bm.append_batch(np.repeat(seqs, counts))
    except N.PagedKVError:
        for s in new:
            bm.free_seq(s)
        raise
    return slots.copy(), pairs.copy()


class _Workspace:
    """Split-K workspace on the device, grown geometrically."""

    def __init__(self, device):
        self.device, self.buf, self.bytes = device, None, 0

    def get(self, need: int, stream):
        if need > self.bytes:
            self.bytes = max(need, int(self.bytes * 1.5))
            self.buf = torch.empty(self.bytes // 4 + 1, dtype=torch.float32, device=self.device)
        # Steps may run on different streams: the caching allocator must not
        # hand this memory out again (once it is replaced) before the last
        # kernel that uses it, on whichever stream, is done.
        self.buf.record_stream(stream)
        return self.buf


class PagedDecodeEngine:
    def __init__(self, num_blocks: int, num_heads: int, head_dim: int, kv_dtype: int,
                 max_seqs: int, max_blocks_per_seq: int, *, window_blocks: int = 0,
                 free_order=None, device="cuda", partition_tokens: int = 0,
                 pool_fill=None, staging_depth: int = 3, longest_first: bool = True,
                 overlap_uploads: bool = False, fuse_write: bool = True, block_size: int = N.BLOCK_SIZE,
                 host_tables=None):
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
        self.fuse_write = fuse_write and not N.is_quantised(kv_dtype)
        # Everything a step uploads lives in one packed buffer.
        self._stage = _Staging([("slots", torch.int64, ()), ("ctx", torch.int32, ()), ("order", torch.int32, ()),
                                ("pairs", torch.int32, (2,)), ("tables", torch.int32, (self.cap,))],
                               max_seqs, self.device, staging_depth, overlap_uploads)
        for v in self._stage.dev:
            v["tables"].fill_(-1)
        self.host_tables = self._stage.in_place_ok() if host_tables is None else host_tables
        if self.host_tables and not self._stage.in_place_ok():
            raise N.PagedKVError(N.PA_ERR_UNSUPPORTED, "pinned memory has a different device address")
        self._ws = _Workspace(self.device)
        self.last_ctx = np.zeros(0, dtype=np.int32)
        self.last_pairs = 0

    @property
    def workspace(self):
        return self._ws.buf

    # Device views of the device staging buffer last written (by decode(), or
    # by a step that uploads instead of reading the pinned buffer in place).
    @property
    def slots(self):
        return self._stage.dev[self._stage.cur]["slots"]

    @property
    def tables(self):
        return self._stage.dev[self._stage.cur]["tables"]

    @property
    def ctx(self):
        return self._stage.dev[self._stage.cur]["ctx"]

    @property
    def order(self):
        return self._stage.dev[self._stage.cur]["order"]

    # -- setup -----------------------------------------------------------------
    def add_sequence(self, seq: int, k_rows=None, v_rows=None, prefill_tokens: int | None = None):
        """Register ``seq`` and write its prefill rows ``[n][heads][head_dim]``."""
        n = int(k_rows.shape[0]) if k_rows is not None else int(prefill_tokens or 0)
        slots = self.bm.add_seq(seq, n)
        if n and k_rows is not None:
            N.pa_write_kv(self.pool, k_rows, v_rows, torch.from_numpy(slots).to(self.device))
        return slots

    def prefill(self, seqs, counts, k_rows, v_rows, q_rows, out, *, stream=None) -> None:
        """A chunked-prefill step: the next ``counts[i]`` tokens of each of
        ``seqs`` arrive together (rows of ``k_rows``/``v_rows``/``q_rows``
        ``[sum(counts)][heads][head_dim]`` in sequence order). Unknown
        sequences are registered; each token goes through the block manager
        (copy-on-write pairs included), the chunk's K/V is written into its
        slots, and the chunk's rows attend causally over their sequences'
        tables at once (``pa_prefill``), results in ``out``. fp16, int8 or
        int4 pools (a quantised pool codes each chunk's rows per (block, head)
        as it writes them), fp16 queries.

        The chunk is all or nothing: arguments and every sequence's table
        capacity are checked before any state changes, and the tokens go
        through one undo-logged batch append (new sequences are registered
        empty first and appended like the others, which places their blocks
        exactly as registering them with their tokens would). If the pool runs
        out of blocks, the appends are undone, the sequences registered by
        this call are removed, and the block manager is left exactly as it
        was (tables, contexts, reference counts and free list); nothing is
        launched."""
        seqs = np.asarray(seqs, dtype=np.int64).reshape(-1)
        counts = np.asarray(counts, dtype=np.int64).reshape(-1)
        if seqs.size != counts.size or (counts < 0).any():
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, "seqs and counts must pair up, counts >= 0")
        if np.unique(seqs).size != seqs.size:
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, "a sequence appears twice in one chunk")
        if self.kv_dtype not in (N.PA_F16, N.PA_I8, N.PA_I4):
            raise N.PagedKVError(N.PA_ERR_UNSUPPORTED, "chunked prefill attends over fp16, int8 or int4 pools")
        if self.bm.window_blocks:
            raise N.PagedKVError(N.PA_ERR_UNSUPPORTED, "chunked prefill over a sliding-window ring")
        R = int(counts.sum())
        if tuple(k_rows.shape[:1]) != (R,) or q_rows.shape != k_rows.shape or v_rows.shape != k_rows.shape:
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, "row counts do not match the chunk sizes")
        slots, pairs = prefill_appends(self.bm, seqs, counts, self.cap)
        tables, ctx = self.bm.export(seqs, self.cap)
        qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        with torch.cuda.stream(cur):
            if pairs.shape[0]:
                N.pa_copy_blocks(self.pool, torch.from_numpy(pairs).to(self.device), stream=cur)
            if R:
                sl = torch.from_numpy(slots.copy()).to(self.device, non_blocking=False)
                N.pa_write_kv(self.pool, k_rows, v_rows, sl, stream=cur)
                # Heaviest sequences first (pairs attended: n (2 ctx - n + 1) / 2),
                # so a long one does not stretch the launch's tail.
                work = counts * (2 * ctx.astype(np.int64) - counts + 1)
                order = torch.from_numpy(np.argsort(-work, kind="stable").astype(np.int32)).to(self.device)
                N.pa_prefill(self.pool, q_rows, out, torch.from_numpy(qs).to(self.device),
                             torch.from_numpy(tables).to(self.device), torch.from_numpy(ctx).to(self.device),
                             int(counts.max()), int(ctx.max()), stream=cur, seq_order=order)
        self.last_ctx = ctx.copy()
        self.last_pairs = int(pairs.shape[0])

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

    def _workspace_for(self, n: int, max_ctx: int, ptok: int, stream):
        return self._ws.get(N.pa_decode_workspace_bytes(self.pool, n, max_ctx, ptok), stream)

    # -- the step ---------------------------------------------------------------
    def step(self, seqs, k_new, v_new, q, out, *, decode: bool = True, stream=None,
             decode_events=None, copy_events=None) -> None:
        """Append one token per sequence of ``seqs`` (order = rows of k_new/q) and decode.

        ``decode_events`` / ``copy_events``: optional (start, end) torch events
        recorded on the step's stream right before and after the decode
        launch(es) / the copy-on-write launch (both recorded, with nothing
        between them, in a step without copies).
        """
        seqs = np.asarray(seqs, dtype=np.int64)
        n = seqs.size
        if n > self.max_seqs:
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, f"batch of {n} > max_seqs {self.max_seqs}")
        st = self._stage.host()
        _, pairs = self.bm.append_batch(seqs, slots_out=st["slots"], pairs_out=st["pairs"])
        npairs = int(pairs.shape[0])
        tables_np = st["tables"][:n]
        ctx_np = st["ctx"][:n]
        self.bm.export(seqs, self.cap, tables_out=tables_np, ctx_out=ctx_np)
        max_ctx = int(ctx_np.max()) if n else 0
        # Samples that share blocks go through one L2 together (PA_SCHED_SHARED).
        sched = N.PA_SCHED_SHARED if decode and self.bm.batch_shares(seqs) else N.PA_SCHED_HEADS
        if decode and self.longest_first:
            st["order"][:n] = np.argsort(-ctx_np, kind="stable")
        self.last_ctx = ctx_np.copy()
        self.last_pairs = npairs
        self.last_pair_list = pairs.copy()
        self.last_slots = st["slots"][:n].copy()

        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        # Everything up to the end of this batch's table rows, in one upload
        # (or none: the kernels read the pinned buffer in place).
        dv = st["t"] if self.host_tables else self._stage.upload(st, n if decode else 0, cur)
        with torch.cuda.stream(cur):
            if copy_events is not None:
                copy_events[0].record(cur)
            if npairs:
                N.pa_copy_blocks(self.pool, dv["pairs"][:npairs], stream=cur)
            if copy_events is not None:
                copy_events[1].record(cur)
            fused = decode and self.fuse_write
            if not fused:
                N.pa_write_kv(self.pool, k_new, v_new, dv["slots"][:n], stream=cur)
            if decode:
                ptok = self.partition_tokens
                ws = self._workspace_for(n, max_ctx, ptok, cur) if ptok else None
                order = dv["order"][:n] if self.longest_first else None
                if decode_events is not None:
                    decode_events[0].record(cur)
                if fused:
                    N.pa_write_decode(self.pool, k_new, v_new, dv["slots"][:n], q, out, dv["tables"][:n],
                                      dv["ctx"][:n], max_ctx, partition_tokens=ptok, workspace=ws,
                                      stream=cur, seq_order=order, schedule=sched)
                else:
                    N.pa_decode(self.pool, q, out, dv["tables"][:n], dv["ctx"][:n], max_ctx,
                                partition_tokens=ptok, workspace=ws, stream=cur, seq_order=order,
                                schedule=sched)
                if decode_events is not None:
                    decode_events[1].record(cur)
            if self.host_tables:
                self._stage.release_host(st, cur)
            else:
                self._stage.release(dv, cur)

    def decode(self, seqs, q, out, *, partition_tokens=None, stream=None, longest_first=None) -> None:
        """Decode the batch as it stands (no append): tables and contexts uploaded first."""
        seqs = np.asarray(seqs, dtype=np.int64)
        n = seqs.size
        tables, ctx = self.bm.export(seqs, self.cap)
        max_ctx = int(ctx.max()) if n else 0
        ptok = self.partition_tokens if partition_tokens is None else partition_tokens
        lf = self.longest_first if longest_first is None else longest_first
        sched = N.PA_SCHED_SHARED if self.bm.batch_shares(seqs) else N.PA_SCHED_HEADS
        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        dv = self._stage.dev[self._stage.cur]
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
                        seq_order=dv["order"][:n] if lf else None, schedule=sched)
            self._stage.release(dv, cur)
        self.last_ctx = ctx


class MixedDecodeEngine:
    """Decode steps over mixed-precision pages: an fp16 hot block per
    sequence (its newest tokens), int8 (or int4) cold blocks for everything older.

    A step: the manager appends one token per sequence (demoting full hot
    blocks into fresh cold blocks) and exports cold tables, hot blocks and
    contexts into the pinned staging buffer; one upload; ``pa_demote_blocks``
    for the demoted blocks; ``pa_write_kv`` of the new rows into the hot pool;
    ``pa_decode_mixed``.
    """

    def __init__(self, num_cold: int, num_hot: int, num_heads: int, head_dim: int, max_seqs: int,
                 max_cold_per_seq: int, *, cold_order=None, hot_order=None, device="cuda",
                 partition_tokens: int = 0, staging_depth: int = 3, longest_first: bool = True, host_tables=None,
                 cold_dtype: int = N.PA_I8):
        self.device = torch.device(device)
        self.num_heads, self.head_dim = num_heads, head_dim
        if not N.is_quantised(cold_dtype):
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, "cold blocks are int8 or int4")
        self.cold = N.new_pool(num_cold, num_heads, head_dim, cold_dtype, device=self.device, fill=0)
        self.hot = N.new_pool(num_hot, num_heads, head_dim, N.PA_F16, device=self.device, fill=0.0)
        self.mbm = N.MixedBlockManager(num_cold, num_hot, cold_order, hot_order)
        self.max_seqs = max_seqs
        self.cap = max_cold_per_seq
        self.partition_tokens = partition_tokens
        self.longest_first = longest_first
        self._stage = _Staging([("slots", torch.int64, ()), ("ctx", torch.int32, ()), ("order", torch.int32, ()),
                                ("hot", torch.int32, ()), ("pairs", torch.int32, (2,)),
                                ("tables", torch.int32, (self.cap,))],
                               max_seqs, self.device, staging_depth, False)
        for v in self._stage.dev:
            v["tables"].fill_(-1)
        self.host_tables = self._stage.in_place_ok() if host_tables is None else host_tables
        self._ws = _Workspace(self.device)
        self.last_ctx = np.zeros(0, dtype=np.int32)
        self.last_pairs = 0

    def add_sequence(self, seq: int, k_rows, v_rows) -> None:
        """Register ``seq`` with prefill rows ``[n][heads][head_dim]``: full
        blocks but the last are quantised into the cold pool, the rest goes to
        the sequence's hot block."""
        n = int(k_rows.shape[0])
        cold, hot = self.mbm.add_seq(seq, n)
        if n:
            if (cold >= 0).any():
                N.pa_write_kv(self.cold, k_rows, v_rows, torch.from_numpy(cold).to(self.device))
            N.pa_write_kv(self.hot, k_rows, v_rows, torch.from_numpy(hot).to(self.device))

    def fork(self, parent: int, child: int) -> None:
        src, dst = self.mbm.fork(parent, child)
        N.pa_copy_blocks(self.hot, torch.tensor([[src, dst]], dtype=torch.int32, device=self.device))

    def free_sequence(self, seq: int) -> None:
        self.mbm.free_seq(seq)

    def step(self, seqs, k_new, v_new, q, out, *, decode: bool = True, stream=None, decode_events=None) -> None:
        seqs = np.asarray(seqs, dtype=np.int64)
        n = seqs.size
        if n > self.max_seqs:
            raise N.PagedKVError(N.PA_ERR_INVALID_ARG, f"batch of {n} > max_seqs {self.max_seqs}")
        st = self._stage.host()
        _, pairs = self.mbm.append_batch(seqs, slots_out=st["slots"], pairs_out=st["pairs"])
        npairs = int(pairs.shape[0])
        ctx_np = st["ctx"][:n]
        self.mbm.export(seqs, self.cap, tables_out=st["tables"][:n], hot_out=st["hot"][:n], ctx_out=ctx_np)
        max_ctx = int(ctx_np.max()) if n else 0
        if decode and self.longest_first:
            st["order"][:n] = np.argsort(-ctx_np, kind="stable")
        sched = N.PA_SCHED_SHARED if decode and self.mbm.batch_shares(seqs) else N.PA_SCHED_HEADS
        self.last_ctx = ctx_np.copy()
        self.last_pairs = npairs
        cur = torch.cuda.current_stream(self.device) if stream is None else stream
        dv = st["t"] if self.host_tables else self._stage.upload(st, n if decode else 0, cur)
        with torch.cuda.stream(cur):
            if npairs:
                N.pa_demote_blocks(self.hot, self.cold, dv["pairs"][:npairs], stream=cur)
            N.pa_write_kv(self.hot, k_new, v_new, dv["slots"][:n], stream=cur)
            if decode:
                ptok = self.partition_tokens
                ws = self._ws.get(N.pa_decode_workspace_bytes(self.cold, n, max_ctx, ptok), cur) if ptok else None
                if decode_events is not None:
                    decode_events[0].record(cur)
                N.pa_decode_mixed(self.cold, self.hot, q, out, dv["tables"][:n], dv["hot"][:n], dv["ctx"][:n],
                                  max_ctx, partition_tokens=ptok, workspace=ws, stream=cur,
                                  seq_order=dv["order"][:n] if self.longest_first else None, schedule=sched)
                if decode_events is not None:
                    decode_events[1].record(cur)
            if self.host_tables:
                self._stage.release_host(st, cur)
            else:
                self._stage.release(dv, cur)
