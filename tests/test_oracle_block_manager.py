"""Pins for the oracle's block-manager model (CPU only)."""

import copy

import numpy as np
import pytest

import workloads as W
from oracle.block_manager import BlockManager, InvalidArg, OutOfBlocks, OutOfRange, StateError, Unsupported


def test_cow_worked_example(load_golden):
    g = load_golden("cow_ref4.json")
    bm = BlockManager(16, 16, free_order=range(16))
    bm.add_seq(0, 20)                          # block 0 full, block 1 holds 4 tokens
    for child in (1, 2, 3):
        bm.fork(0, child)
    shared = bm.table(0)[0][-1]
    assert bm.ref_count(shared) == g["initial_ref_count"]
    slot, src, dst = bm.append(1)
    assert g["after_first_append"]["copied"] and (src, dst) == (shared, bm.table(1)[0][-1])
    assert bm.ref_count(shared) == g["after_first_append"]["shared_ref_count"]
    assert bm.ref_count(dst) == g["after_first_append"]["copy_ref_count"]
    assert slot == dst * 16 + 4
    # Extension: the next two sharers copy too, the last one writes in place.
    assert bm.append(2)[1] == shared and bm.ref_count(shared) == 2
    assert bm.append(3)[1] == shared and bm.ref_count(shared) == 1
    s0, src0, _ = bm.append(0)
    assert src0 == -1 and s0 == shared * 16 + 4
    # The full first block stays shared by all four: full blocks are never copied.
    assert bm.ref_count(bm.table(0)[0][0]) == 4


def test_slot_follows_the_locate_rule(load_golden):
    g = load_golden("locate_worked_example.json")
    # Free list arranged so the sequence receives exactly the example's table.
    order = g["block_table"] + [b for b in range(8) if b not in g["block_table"]]
    bm = BlockManager(8, g["block_size"], free_order=order)
    slots = bm.add_seq(0, 35)
    assert bm.table(0)[0] == g["block_table"]
    assert slots[g["token_index"]] == g["physical"] * 16 + g["offset"]


def test_blocks_are_allocated_on_demand():
    bm = BlockManager(64, 16, free_order=W.free_order(3, 64))
    bm.add_seq(7, 0)
    for n in range(1, 200):
        bm.append(7)
        row, ctx = bm.table(7)
        assert ctx == n and len(row) == -(-n // 16)
    assert bm.num_free() == 64 - 13


def test_fragmentation_case(load_golden):
    g = load_golden("fragmentation_2048x2.json")
    blocks = lambda t: t // 16
    total = blocks(g["user_a_tokens"]) + 8 + blocks(g["user_b_tokens"]) + 8
    # Contiguous first-fit model: A | X | B | Y laid out back to back.
    layout = [("A", blocks(g["user_a_tokens"])), ("X", 8), ("B", blocks(g["user_b_tokens"])), ("Y", 8)]
    free_runs = [n for name, n in layout if name in ("A", "B")]
    assert (max(free_runs) >= blocks(g["new_user_tokens"])) == g["contiguous_allocation_succeeds"]
    # Paged: the same occupancy, then A and B leave; the new user still fits.
    bm = BlockManager(total, 16, free_order=range(total))
    bm.add_seq(0, g["user_a_tokens"])
    bm.add_seq(1, 128)
    bm.add_seq(2, g["user_b_tokens"])
    bm.add_seq(3, 128)
    assert bm.num_free() == 0
    bm.free_seq(0)
    bm.free_seq(2)
    ok = True
    try:
        bm.add_seq(4, g["new_user_tokens"])
    except OutOfBlocks:
        ok = False
    assert ok == g["paged_allocation_succeeds"]
    row, _ = bm.table(4)
    assert sorted(row) == list(range(128)) + list(range(136, 264))


def test_ring_moves_no_data_and_keeps_logical_order(load_golden):
    g = load_golden("ring_window.json")
    Wb = 4
    bm = BlockManager(32, 16, free_order=W.free_order(5, 32), window_blocks=Wb)
    bm.add_seq(0, 0)
    for _ in range(Wb * 16):
        bm.append(0)
    before, ctx = bm.table(0)
    free_before = bm.num_free()
    slot, src, dst = bm.append(0)               # token 64: the window is full
    after, ctx2 = bm.table(0)
    assert (src, dst) == (-1, -1)               # nothing copied
    assert after == before[1:] + [before[0]]    # oldest page reused as the newest
    assert slot == before[0] * 16               # the new token goes into it
    assert bm.num_free() == free_before         # no allocation at all
    assert ctx == 64 and ctx2 == 49
    assert g["kv_bytes_moved_per_slide"] == 0
    # Many more slides: the row stays W blocks, the live context stays in range.
    for _ in range(1000):
        bm.append(0)
        row, c = bm.table(0)
        assert len(row) == Wb and (Wb - 1) * 16 < c <= Wb * 16
        assert sorted(row) == sorted(before)


def test_ring_with_a_shared_oldest_block_takes_a_fresh_one():
    bm = BlockManager(16, 16, free_order=range(16), window_blocks=2)
    bm.add_seq(0, 32)
    bm.fork(0, 1)
    slot, src, dst = bm.append(1)
    row1, _ = bm.table(1)
    assert row1 == [1, 2] and bm.ref_count(0) == 1 and bm.ref_count(2) == 1
    assert (src, dst) == (-1, -1) and slot == 2 * 16


def _invariants(bm: BlockManager):
    refs = [0] * bm.num_blocks
    host_held = []
    for st in bm.seqs.values():
        if st.swapped:
            host_held += st.table
            continue
        for b in st.table:
            refs[b] += 1
    assert refs == bm.ref
    free = set(bm.free)
    used = {b for b in range(bm.num_blocks) if bm.ref[b] > 0}
    assert len(free) == len(bm.free)
    assert free.isdisjoint(used) and free | used == set(range(bm.num_blocks))
    # Host blocks: each held by exactly one swapped sequence, or free.
    assert len(set(host_held)) == len(host_held)
    assert len(set(bm.host_free)) == len(bm.host_free)
    assert set(host_held).isdisjoint(bm.host_free)
    assert set(host_held) | set(bm.host_free) == set(range(bm.num_host_blocks))
    # The prefix index only names live blocks, each under the key it was built with.
    for key, b in bm.prefix.items():
        assert bm.ref[b] > 0 and bm.prefix_key[b] == key
        assert key[0] == -1 or bm.ref[key[0]] > 0


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("seed", range(6))
def test_random_operation_sequences_keep_the_invariants(seed, bs):
    rng = W.rng(seed, 77)
    window = int(rng.integers(0, 2)) * int(rng.integers(2, 6))
    bm = BlockManager(48, bs, free_order=W.free_order(seed, 48), window_blocks=window)
    bm.set_host_blocks(40, W.free_order(seed + 100, 40))
    content = {}          # slot -> token id written there (models the pool)
    host = {}             # host slot -> token id (models the host pool)
    owner_tokens = {}     # seq -> list of token ids in logical order
    next_id = 0
    serial = 0            # unique id of every appended token
    live = []             # resident sequences
    swapped = []
    for _ in range(600):
        op = rng.integers(0, 12)
        try:
            if op == 0 or not live:
                s = next_id
                n = int(rng.integers(0, 40))
                if window:
                    n = min(n, window * bs)
                slots = bm.add_seq(s, n)
                ids = list(range(next_id * 1000, next_id * 1000 + n))
                for sl, tid in zip(slots, ids):
                    content[int(sl)] = tid
                owner_tokens[s] = ids
                live.append(s)
                next_id += 1
            elif op == 1:
                p = live[int(rng.integers(len(live)))]
                c = next_id
                bm.fork(p, c)
                owner_tokens[c] = list(owner_tokens[p])
                live.append(c)
                next_id += 1
            elif op == 2:
                s = live.pop(int(rng.integers(len(live))))
                bm.free_seq(s)
                del owner_tokens[s]
            elif op == 10:
                s = live[int(rng.integers(len(live)))]
                pairs = bm.swap_out(s)
                for d, h in pairs:                      # the copy the pairs ask for
                    for o in range(bs):
                        host.pop(h * bs + o, None)
                        if d * bs + o in content:
                            host[h * bs + o] = content[d * bs + o]
                live.remove(s)
                swapped.append(s)
                with pytest.raises(StateError):
                    bm.append(s)
                with pytest.raises(StateError):
                    bm.export([s], 64)
            elif op == 11 and swapped:
                s = swapped[int(rng.integers(len(swapped)))]
                pairs = bm.swap_in(s)
                for h, d in pairs:
                    # A device block taken for a swap-in was free: no live sequence reads it.
                    assert bm.ref[d] == 1
                    for o in range(bs):
                        content.pop(d * bs + o, None)
                        if h * bs + o in host:
                            content[d * bs + o] = host[h * bs + o]
                swapped.remove(s)
                live.append(s)
            elif op == 8 and not window:
                # A prompt built from a few shared templates, so full blocks repeat.
                s = next_id
                t = int(rng.integers(0, 3))
                n = int(rng.integers(0, 70))
                toks = [5000 + 100 * t + (i % 37) * 1000 * (1 + (i // 37) % 2) + i for i in range(n)]
                slots, shared = bm.add_seq_prefix(s, toks)
                assert (slots[:shared * bs] == -1).all() and (slots[shared * bs:] >= 0).all()
                for sl, tid in zip(slots, toks):
                    if sl >= 0:
                        content[int(sl)] = tid
                owner_tokens[s] = list(toks)
                live.append(s)
                next_id += 1
            elif op == 9 and swapped:
                s = swapped.pop(int(rng.integers(len(swapped))))
                bm.free_seq(s)
                del owner_tokens[s]
            else:
                s = live[int(rng.integers(len(live)))]
                shared_before = {b: bm.ref[b] for b in range(bm.num_blocks)}
                slot, src, dst = bm.append(s)
                if src >= 0:
                    # Copy-on-write only when the block was shared.
                    assert shared_before[src] > 1
                    for o in range(bs):
                        if src * bs + o in content:
                            content[dst * bs + o] = content[src * bs + o]
                # The block written into is never shared at write time.
                assert bm.ref[slot // bs] == 1
                tid = 10 ** 9 + serial
                serial += 1
                content[slot] = tid
                owner_tokens[s].append(tid)
        except OutOfBlocks:
            pass
        _invariants(bm)
        # Every live sequence reads back exactly its own tokens through its table.
        for s in live:
            row, ctx = bm.table(s)
            toks = owner_tokens[s][len(owner_tokens[s]) - ctx:]
            got = [content.get(row[t // bs] * bs + t % bs) for t in range(ctx)]
            assert got == toks
        for s in swapped:
            row, ctx = bm.table(s)
            toks = owner_tokens[s][len(owner_tokens[s]) - ctx:]
            assert [host.get(row[t // bs] * bs + t % bs) for t in range(ctx)] == toks


def test_calls_are_atomic_on_error():
    bm = BlockManager(4, 16, free_order=range(4))
    bm.add_seq(0, 48)
    bm.fork(0, 1)
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.add_seq(2, 33)
    assert bm.__dict__ == snap
    bm.add_seq(2, 16)                 # takes the last block
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.append(0)                  # offset 0: needs a fresh block
    assert bm.__dict__ == snap
    with pytest.raises(StateError):
        bm.fork(0, 1)
    with pytest.raises(StateError):
        bm.free_seq(9)
    with pytest.raises(StateError):
        bm.append(9)
    with pytest.raises(OutOfRange):
        bm.export([0], 2)
    with pytest.raises(InvalidArg):
        BlockManager(4, 16, free_order=[0, 0, 1, 2])
    assert bm.__dict__ == snap
    # Freeing the sharers releases the blocks back to the tail of the free list.
    bm.free_seq(0)
    assert bm.num_free() == 0
    bm.free_seq(1)
    assert list(bm.free) == [0, 1, 2]


def test_swap_round_trip_and_shared_blocks():
    bm = BlockManager(8, 16, free_order=range(8))
    bm.add_seq(0, 40)                        # blocks 0, 1, 2
    bm.fork(0, 1)                            # all three shared
    with pytest.raises(StateError):
        bm.swap_out(0)                       # no host pool yet
    bm.set_host_blocks(4)
    with pytest.raises(StateError):
        bm.set_host_blocks(4)
    pairs = bm.swap_out(1)
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    # The resident sharer is untouched; the blocks only lost one count.
    assert bm.table(0) == ([0, 1, 2], 40) and [bm.ref_count(b) for b in (0, 1, 2)] == [1, 1, 1]
    assert bm.table(1) == ([0, 1, 2], 40) and bm.is_swapped(1)
    assert bm.num_host_free() == 1 and bm.num_free() == 5
    with pytest.raises(StateError):
        bm.fork(1, 2)
    with pytest.raises(StateError):
        bm.swap_in(0)
    bm.add_seq(2, 20)                        # device blocks 3, 4
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.swap_out(2)                       # 2 host blocks needed, 1 free
    assert bm.__dict__ == snap and not bm.is_swapped(2)
    bm.free_seq(2)                           # device free list: 5 6 7 3 4
    snap = copy.deepcopy(bm.__dict__)
    back = bm.swap_in(1)                     # private copies, from the device free list head
    assert back == [(0, 5), (1, 6), (2, 7)]
    assert bm.table(1) == ([5, 6, 7], 40) and list(bm.host_free) == [3, 0, 1, 2]
    assert [bm.ref_count(b) for b in (0, 1, 2, 5, 6, 7)] == [1] * 6
    bm.__dict__.update(copy.deepcopy(snap))
    # Freeing a swapped-out sequence returns its host blocks to the tail.
    bm.free_seq(1)
    assert list(bm.host_free) == [3, 0, 1, 2]
    # Swap-out of a sole owner releases its device blocks in logical order.
    bm.swap_out(0)
    assert list(bm.free)[-3:] == [0, 1, 2]
    _invariants(bm)


def test_prefix_caching_shares_whole_matching_prefixes():
    bs = 16
    bm = BlockManager(32, bs, free_order=range(32))
    A = list(range(100, 150))                    # 3 full blocks + 2 tokens
    slots, shared = bm.add_seq_prefix(0, A)
    assert shared == 0 and (slots >= 0).all() and bm.table(0) == ([0, 1, 2, 3], 50)
    slots, shared = bm.add_seq_prefix(1, A)
    assert shared == 3 and (slots[:48] == -1).all()
    assert bm.table(1) == ([0, 1, 2, 4], 50) and slots[48] == 4 * bs
    assert [bm.ref_count(b) for b in range(5)] == [2, 2, 2, 1, 1]
    # Same first block, different second: only the first is shared.
    B = A[:16] + [7] * 16 + A[32:48]
    _, shared = bm.add_seq_prefix(2, B)
    assert shared == 1 and bm.table(2)[0] == [0, 5, 6]
    # A different first block breaks the chain even if later blocks match.
    C = [9] * 16 + A[16:48]
    _, shared = bm.add_seq_prefix(3, C)
    assert shared == 0 and bm.table(3)[0] == [7, 8, 9]
    # A full shared last block: the next append opens a fresh block, no copy.
    _, shared = bm.add_seq_prefix(4, A[:32])
    assert shared == 2
    slot, src, dst = bm.append(4)
    assert (src, dst) == (-1, -1) and slot == 10 * bs and bm.ref_count(1) == 3
    # Freed blocks leave the index: after every holder of A's blocks is gone,
    # A is built from scratch again.
    for s in (0, 1, 2, 4):
        bm.free_seq(s)
    assert all(bm.ref_count(b) == 0 for b in (0, 1, 2))
    _, shared = bm.add_seq_prefix(5, A)
    assert shared == 0
    _invariants(bm)
    # Atomic on error, and not offered with a ring.
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.add_seq_prefix(6, list(range(10**6, 10**6 + 40 * bs)))
    assert bm.__dict__ == snap
    with pytest.raises(StateError):
        bm.add_seq_prefix(5, A)
    with pytest.raises(Unsupported):
        BlockManager(8, 16, window_blocks=2).add_seq_prefix(0, A)


def test_prefix_caching_saves_the_shared_prompt_blocks():
    # Eight prompts of 1024 tokens, four samples each ("KV Cache与长上下文管理",
    # section 二 item 2: a common prefix is stored once): 8 x 64 prompt blocks
    # instead of 32 x 64.
    bm = BlockManager(4096, 16, free_order=W.free_order(3, 4096))
    for p in range(8):
        prompt = [p * 10**6 + i for i in range(1024)]
        for j in range(4):
            _, shared = bm.add_seq_prefix(p * 4 + j, prompt)
            assert shared == (0 if j == 0 else 64)
    assert 4096 - bm.num_free() == 8 * 64
