"""Pins for the oracle's mixed-precision pages (CPU only)."""

import copy
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import cache_ops as C
from oracle import mixed as M
from oracle.block_manager import OutOfBlocks, StateError

BS = 16


def _pools(NC, NH, H, D):
    return (np.zeros((NC, H, BS, D), np.int8), np.zeros((NC, H), np.float16),
            np.zeros((NC, H, BS, D), np.int8), np.zeros((NC, H), np.float16),
            np.zeros((NH, H, BS, D), np.float16), np.zeros((NH, H, BS, D), np.float16))


def _build(bm, pools, seq, K, V):
    """Prefill ``seq`` with rows K, V [n][H][D] through the manager's slots."""
    ck, cks, cv, cvs, hk, hv = pools
    cold, hot = bm.add_seq(seq, K.shape[0])
    C.write_kv_int8(ck, cks, cv, cvs, K.astype(np.float32), V.astype(np.float32), cold)
    C.write_kv(hk, hv, K, V, hot)


def _step(bm, pools, seq, k, v):
    ck, cks, cv, cvs, hk, hv = pools
    slot, src, dst = bm.append(seq)
    if src >= 0:
        M.demote(hk, hv, ck, cks, cv, cvs, [(src, dst)])
    C.write_kv(hk, hv, k[None], v[None], [slot])
    return src, dst


def test_exactly_representable_rows_decode_exactly():
    # Rows k/128 with integer k in [-127, 127] and one +-127/128 per (block,
    # head): the scale is exactly 1/128 and every code exact, so the mixed
    # decode must equal fp16 attention over the same rows exactly. A wrong
    # cold/hot split, offset or scale index fails this.
    rng = W.rng(60, 0)
    H, D, n = 3, 8, 75
    K = (rng.integers(-127, 128, size=(n, H, D)) / 128.0).astype(np.float16)
    V = (rng.integers(-127, 128, size=(n, H, D)) / 128.0).astype(np.float16)
    K[::BS, :, 0] = 127 / 128
    V[::BS, :, 1] = -127 / 128
    bm = M.MixedBlockManager(10, 4, cold_order=W.free_order(60, 10))
    pools = _pools(10, 4, H, D)
    _build(bm, pools, 0, K[:40], V[:40])
    for t in range(40, n):
        _step(bm, pools, 0, K[t], V[t])
    rows, hot, ctx = bm.export([0], 8)
    assert ctx[0] == n and (rows[0] >= 0).sum() == 4
    q = rng.standard_normal((1, H, D))
    got = M.decode(q, *pools, rows, hot, ctx)
    np.testing.assert_array_equal(got[0], A.attend(q[0], K, V, A.default_scale(D)))
    ck, cks = pools[0], pools[1]
    assert np.all(cks[rows[0][:4]] == np.float16(1 / 128))


def test_short_contexts_live_in_the_hot_block_only():
    rng = W.rng(61, 0)
    H, D = 2, 8
    bm = M.MixedBlockManager(4, 3)
    pools = _pools(4, 3, H, D)
    for seq, n in enumerate((1, 15, 16)):
        K = rng.standard_normal((n, H, D)).astype(np.float16)
        V = rng.standard_normal((n, H, D)).astype(np.float16)
        _build(bm, pools, seq, K, V)
        rows, hot, ctx = bm.export([seq], 4)
        assert (rows[0] < 0).all()
        q = rng.standard_normal((1, H, D))
        np.testing.assert_array_equal(M.decode(q, *pools, rows, hot, ctx)[0],
                                      A.attend(q[0], K, V, A.default_scale(D)))
    assert bm.cold_free == M.MixedBlockManager(4, 3).cold_free   # nothing cold yet


def test_demotion_happens_exactly_when_a_block_is_full():
    rng = W.rng(62, 0)
    H, D = 2, 16
    bm = M.MixedBlockManager(8, 2, cold_order=range(8))
    pools = _pools(8, 2, H, D)
    bm.add_seq(0, 0)
    events = []
    K = rng.standard_normal((50, H, D)).astype(np.float16)
    V = rng.standard_normal((50, H, D)).astype(np.float16)
    for t in range(50):
        src, dst = _step(bm, pools, 0, K[t], V[t])
        events.append((t, src, dst))
    assert [(t, d) for t, s, d in events if s >= 0] == [(16, 0), (32, 1), (48, 2)]
    # Demoted codes are within half a scale step of the fp16 rows.
    ck, cks = pools[0], pools[1]
    for blk, first in ((0, 0), (1, 16), (2, 32)):
        deq = ck[blk].astype(np.float64) * cks[blk].astype(np.float64)[:, None, None]
        src = K[first:first + 16].transpose(1, 0, 2).astype(np.float64)
        assert np.all(np.abs(deq - src) <= cks[blk].astype(np.float64)[:, None, None] / 2 + 1e-12)
    # Demotion is the int8 write rule with the whole block written at once.
    ck2, cks2 = np.zeros_like(ck), np.zeros_like(cks)
    C.write_kv_int8(ck2, cks2, ck2.copy(), cks2.copy(), K[:16].astype(np.float32), V[:16].astype(np.float32),
                    np.arange(16) + 5 * 16)
    assert np.array_equal(ck2[5], ck[0]) and np.array_equal(cks2[5], cks[0])


def test_fork_shares_cold_blocks_and_copies_the_hot_one():
    bm = M.MixedBlockManager(8, 4, cold_order=range(8), hot_order=range(4))
    bm.add_seq(0, 40)                      # cold 0, 1; hot 0 with 8 tokens
    src, dst = bm.fork(0, 1)
    assert (src, dst) == (0, 1)
    assert bm.ref == [2, 2, 0, 0, 0, 0, 0, 0]
    rows, hot, ctx = bm.export([0, 1], 4)
    assert rows[0].tolist() == rows[1].tolist() == [0, 1, -1, -1] and hot.tolist() == [0, 1]
    # Appends never write a cold block; each writes its own hot block.
    assert bm.append(1)[0] == 1 * 16 + 8 and bm.append(0)[0] == 0 * 16 + 8
    bm.free_seq(0)
    assert bm.ref[:2] == [1, 1] and list(bm.hot_free) == [2, 3, 0]
    bm.free_seq(1)
    assert list(bm.cold_free)[-2:] == [0, 1]
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.add_seq(5, 16 * 9 + 1)          # 9 cold blocks needed, 8 free
    assert bm.__dict__ == snap
    with pytest.raises(StateError):
        bm.append(0)


def test_gaussian_rows_meet_the_int8_bar():
    # N(0,1) rows, OPT-13B head size: mixed decode vs fp64 attention over the
    # unquantised rows within the int8 bar (2e-2 abs).
    rng = W.rng(63, 0)
    H, D, n = 4, 128, 700
    K = rng.standard_normal((n, H, D)).astype(np.float16)
    V = rng.standard_normal((n, H, D)).astype(np.float16)
    bm = M.MixedBlockManager(64, 2, cold_order=W.free_order(63, 64))
    pools = _pools(64, 2, H, D)
    _build(bm, pools, 0, K[:300], V[:300])
    for t in range(300, n):
        _step(bm, pools, 0, K[t], V[t])
    rows, hot, ctx = bm.export([0], 64)
    q = rng.standard_normal((1, H, D)).astype(np.float16)
    got = M.decode(q, *pools, rows, hot, ctx)[0]
    ref = A.attend(q[0], K, V, 1 / math.sqrt(D))
    assert np.abs(got - ref).max() <= 2e-2


@pytest.mark.parametrize("seed", range(4))
def test_random_operations_read_back_their_tokens(seed):
    rng = W.rng(seed, 64)
    H, D = 1, 4
    bm = M.MixedBlockManager(40, 12, cold_order=W.free_order(seed, 40), hot_order=W.free_order(seed + 1, 12))
    pools = _pools(40, 12, H, D)
    # Token t carries an integer in [1, 127] in every element, 127 at every
    # block start: each cold block's scale is exactly 1 and its codes exact,
    # so only an indexing error can change what reads back.
    val = lambda t: 127.0 if t % BS == 0 else float((t * 7) % 127 + 1)
    vals, live, nid = {}, [], 0
    for _ in range(300):
        op = int(rng.integers(0, 8))
        try:
            if op == 0 or not live:
                n = int(rng.integers(0, 60))
                x = np.array([[[val(i)] * D] for i in range(n)], np.float16).reshape(n, H, D)
                _build(bm, pools, nid, x, -x)
                vals[nid] = list(x[:, 0, 0])
                live.append(nid)
                nid += 1
            elif op == 1:
                p = live[int(rng.integers(len(live)))]
                src, dst = bm.fork(p, nid)
                C.copy_blocks([pools[4], pools[5]], [(src, dst)])
                vals[nid] = list(vals[p])
                live.append(nid)
                nid += 1
            elif op == 2:
                s = live.pop(int(rng.integers(len(live))))
                bm.free_seq(s)
            else:
                s = live[int(rng.integers(len(live)))]
                v = val(len(vals[s]))
                _step(bm, pools, s, np.full((H, D), v, np.float16), np.full((H, D), -v, np.float16))
                vals[s].append(v)
        except OutOfBlocks:
            pass
        for s in live:
            rows, hot, ctx = bm.export([s], 8)
            got = M.gather(pools[0], pools[1], pools[4], rows[0], hot[0], ctx[0])[:, 0, 0]
            assert np.array_equal(got, np.array(vals[s], np.float64))
        refs = [0] * 40
        for st in bm.seqs.values():
            for b in st.cold:
                refs[b] += 1
        assert refs == bm.ref
        assert sorted(list(bm.hot_free) + [st.hot for st in bm.seqs.values()]) == list(range(12))


def test_int4_cold_blocks_decode_exactly_when_representable():
    # Rows k/8 with integer k in [-7, 7] and one +-7/8 per (block, head): the
    # int4 scale is exactly 1/8 and every code exact, so mixed decode over
    # int4 cold blocks equals fp16 attention over the same rows exactly.
    rng = W.rng(65, 0)
    H, D, n = 2, 8, 75
    K = (rng.integers(-7, 8, size=(n, H, D)) / 8.0).astype(np.float16)
    V = (rng.integers(-7, 8, size=(n, H, D)) / 8.0).astype(np.float16)
    K[::BS, :, 0] = 7 / 8
    V[::BS, :, 1] = -7 / 8
    bm = M.MixedBlockManager(10, 4, cold_order=W.free_order(65, 10))
    ck, cks, cv, cvs, hk, hv = _pools(10, 4, H, D)
    cold, hot = bm.add_seq(0, 40)
    C.write_kv_int4(ck, cks, cv, cvs, K[:40].astype(np.float32), V[:40].astype(np.float32), cold)
    C.write_kv(hk, hv, K[:40], V[:40], hot)
    for t in range(40, n):
        slot, src, dst = bm.append(0)
        if src >= 0:
            M.demote(hk, hv, ck, cks, cv, cvs, [(src, dst)], qmax=7)
        C.write_kv(hk, hv, K[t][None], V[t][None], [slot])
    rows, hot, ctx = bm.export([0], 8)
    assert (rows[0] >= 0).sum() == 4 and np.abs(ck[rows[0][:4]]).max() <= 7
    assert np.all(cks[rows[0][:4]] == np.float16(1 / 8))
    q = rng.standard_normal((1, H, D))
    got = M.decode(q, ck, cks, cv, cvs, hk, hv, rows, hot, ctx)
    np.testing.assert_array_equal(got[0], A.attend(q[0], K, V, A.default_scale(D)))


def test_int4_demotion_is_the_whole_block_int4_write():
    rng = W.rng(66, 0)
    H, D = 2, 16
    hk = rng.standard_normal((3, H, BS, D)).astype(np.float16)
    hv = rng.standard_normal((3, H, BS, D)).astype(np.float16)
    ck, cks = np.zeros((4, H, BS, D), np.int8), np.zeros((4, H), np.float16)
    cv, cvs = np.zeros_like(ck), np.zeros_like(cks)
    M.demote(hk, hv, ck, cks, cv, cvs, [(2, 1)], qmax=7)
    wk, wks = np.zeros_like(ck), np.zeros_like(cks)
    C.write_kv_int4(wk, wks, wk.copy(), wks.copy(), hk[2].transpose(1, 0, 2).astype(np.float32),
                    hv[2].transpose(1, 0, 2).astype(np.float32), np.arange(BS) + 3 * BS)
    assert np.array_equal(wk[3], ck[1]) and np.array_equal(wks[3], cks[1])
    assert np.all(cks[1] == np.float16(np.abs(hk[2].astype(np.float32)).max(axis=(1, 2)) / np.float32(7)))
