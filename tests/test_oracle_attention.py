"""Pins for the attention and paging parts of the oracle (CPU only).

Each test ties the oracle to something other than its own formula: the pages'
worked example, a library routine the formula reduces to, closed forms worked
by hand, invariants, or brute force on tiny inputs.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import cache_ops as C
from oracle import paging as P


def test_locate_worked_example(load_golden):
    g = load_golden("locate_worked_example.json")
    phys, off = P.locate(g["token_index"], g["block_table"], g["block_size"])
    assert (phys, off) == (g["physical"], g["offset"])
    assert P.slot(g["token_index"], g["block_table"], g["block_size"]) == 3 * 16 + 2


def test_locate_every_token_of_the_example_table():
    # Brute force over the 48 tokens the example table covers: logical block
    # order must follow the table, offsets must run 0..15 inside each block.
    table = [7, 1, 3]
    seen = [P.locate(t, table, 16) for t in range(48)]
    assert [p for p, _ in seen] == [7] * 16 + [1] * 16 + [3] * 16
    assert [o for _, o in seen] == list(range(16)) * 3
    with pytest.raises(IndexError):
        P.locate(48, table, 16)


def _scatter_contiguous(K, table, num_blocks, bs=16):
    """Lay a contiguous [T][H][D] sequence out in a pool, block by block."""
    T, H, D = K.shape
    pool = np.full((num_blocks, H, bs, D), np.nan, dtype=K.dtype)
    for t in range(T):
        pool[table[t // bs], :, t % bs, :] = K[t]
    return pool


def test_gather_returns_the_contiguous_rows():
    rng = W.rng(11, 0)
    T, H, D, NB = 50, 3, 8, 9
    K = rng.standard_normal((T, H, D)).astype(np.float32)
    table = rng.permutation(NB)[:4]
    pool = _scatter_contiguous(K, table, NB)
    got = P.gather(pool, table, T)
    assert got.dtype == np.float64
    np.testing.assert_array_equal(got, K.astype(np.float64))


def test_attention_reduces_to_library_sdpa():
    # Special case that a library routine computes: torch's scaled dot-product
    # attention (float64, CPU) with one query row per head.
    rng = W.rng(12, 0)
    T, H, D = 37, 4, 16
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((T, H, D))
    V = rng.standard_normal((T, H, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None],
        torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None],
    )[0, :, 0, :].numpy()
    got = A.attend(q, K, V, A.default_scale(D))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_two_token_closed_form():
    # q = (2,0,0,0), k0 = 0, k1 = (ln 3, 0, 0, 0), d = 4: logits 0 and
    # 2 ln3 / sqrt(4) = ln 3, so the weights are exactly 1/4 and 3/4.
    # A missing 1/sqrt(d) would give 1/10, 9/10; a 1/d scale sqrt(3)-based weights.
    q = np.array([[2.0, 0, 0, 0]])
    K = np.array([[[0.0, 0, 0, 0]], [[math.log(3.0), 0, 0, 0]]])
    V = np.array([[[4.0, 0, -8, 1]], [[0.0, 4, 8, 1]]])
    got = A.attend(q, K, V, A.default_scale(4))
    np.testing.assert_allclose(got[0], [1.0, 3.0, 4.0, 1.0], rtol=0, atol=1e-14)


def test_attention_closed_forms():
    rng = W.rng(13, 0)
    H, D = 5, 32
    q = rng.standard_normal((H, D))
    # One token: the output is that token's value row.
    K1 = rng.standard_normal((1, H, D))
    V1 = rng.standard_normal((1, H, D))
    np.testing.assert_array_equal(A.attend(q, K1, V1, 0.3), V1[0])
    # q = 0 (or all keys equal): uniform weights, output is the mean of V.
    T = 29
    K = rng.standard_normal((T, H, D))
    V = rng.standard_normal((T, H, D))
    np.testing.assert_allclose(A.attend(np.zeros((H, D)), K, V, 0.2), V.mean(axis=0),
                               rtol=0, atol=1e-13)
    Keq = np.broadcast_to(K[:1], K.shape)
    np.testing.assert_allclose(A.attend(q, Keq, V, 0.2), V.mean(axis=0), rtol=0, atol=1e-13)
    # Constant value rows: the output is that constant.
    c = rng.standard_normal((H, D))
    np.testing.assert_allclose(A.attend(q, K, np.broadcast_to(c, V.shape), 0.2), c,
                               rtol=0, atol=1e-13)
    # No tokens: zeros.
    assert not A.attend(q, K[:0], V[:0], 0.2).any()


def test_softmax_weights_sum_to_one_and_follow_logits():
    rng = W.rng(14, 0)
    T, H, D = 40, 3, 8
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((T, H, D))
    w = A.softmax_weights(q, K, 0.5)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    z = np.einsum("thd,hd->ht", K, q)
    for h in range(H):
        order = np.argsort(z[h])
        assert np.all(np.diff(w[h][order]) >= 0)
    # The output is the weighted mean of V under these weights.
    V = rng.standard_normal((T, H, D))
    np.testing.assert_allclose(A.attend(q, K, V, 0.5), np.einsum("ht,thd->hd", w, V),
                               rtol=1e-12, atol=1e-13)


def _tiny_batch(seed=1):
    wl = W.tiny(seed)
    H, D, NB = wl.num_heads, wl.head_dim, wl.num_blocks
    order = W.free_order(seed, NB)
    tables, k_pool, v_pool = [], np.zeros((NB, H, 16, D), np.float32), np.zeros((NB, H, 16, D), np.float32)
    contig_k, contig_v = [], []
    used = 0
    for s, ctx in enumerate(wl.context_lens):
        nb = -(-ctx // 16)
        table = order[used:used + nb]
        used += nb
        K = W.normal_np((ctx, H, D), seed, W.STREAM_K, s)
        V = W.normal_np((ctx, H, D), seed, W.STREAM_V, s)
        C.write_kv(k_pool, v_pool, K, V, P.slots(ctx, table))
        tables.append(table)
        contig_k.append(K)
        contig_v.append(V)
    q = W.normal_np((wl.num_seqs, H, D), seed, W.STREAM_Q)
    return wl, q, k_pool, v_pool, tables, contig_k, contig_v


def test_paged_decode_equals_contiguous_brute_force():
    wl, q, k_pool, v_pool, tables, ck, cv = _tiny_batch()
    out = A.paged_decode(q, k_pool, v_pool, tables, wl.context_lens)
    scale = 1.0 / math.sqrt(wl.head_dim)
    for s in range(wl.num_seqs):
        # Brute force: a double loop over heads and tokens in plain Python.
        for h in range(wl.num_heads):
            z = [float(np.dot(q[s, h].astype(np.float64), ck[s][t, h].astype(np.float64))) * scale
                 for t in range(wl.context_lens[s])]
            mz = max(z)
            e = [math.exp(x - mz) for x in z]
            tot = sum(e)
            ref = sum((e[t] / tot) * cv[s][t, h].astype(np.float64) for t in range(len(z)))
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-12)


def test_physical_permutation_is_bit_exact():
    wl, q, k_pool, v_pool, tables, _, _ = _tiny_batch()
    out = A.paged_decode(q, k_pool, v_pool, tables, wl.context_lens)
    perm = W.relabel(1, wl.num_blocks)        # new physical id of every block
    k2 = np.empty_like(k_pool)
    v2 = np.empty_like(v_pool)
    k2[perm] = k_pool
    v2[perm] = v_pool
    tables2 = [perm[np.asarray(t)] for t in tables]
    out2 = A.paged_decode(q, k2, v2, tables2, wl.context_lens)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("ptok", [16, 48, 512, 10 ** 9])
def test_split_merge_equals_single_pass(ptok):
    rng = W.rng(15, ptok % 1000)
    T, H, D = 700, 3, 16
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((T, H, D)) * 3.0
    V = rng.standard_normal((T, H, D))
    full = A.attend(q, K, V, 0.25)
    np.testing.assert_allclose(A.split_decode(q, K, V, 0.25, ptok), full, rtol=1e-13, atol=1e-14)


def test_partition_partials_brute_force():
    rng = W.rng(16, 0)
    T, H, D = 40, 2, 4
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((T, H, D))
    V = rng.standard_normal((T, H, D))
    m, l, o = A.partition_partials(q, K, V, 0.5, 16, 32)
    for h in range(H):
        z = [0.5 * sum(q[h, d] * K[t, h, d] for d in range(D)) for t in range(16, 32)]
        assert m[h] == pytest.approx(max(z), abs=1e-14)
        assert l[h] == pytest.approx(sum(math.exp(x - max(z)) for x in z), rel=1e-14)
        # o is the attention over the partition alone.
        np.testing.assert_allclose(o[h], A.attend(q[h:h + 1], K[16:32, h:h + 1], V[16:32, h:h + 1], 0.5)[0],
                                   rtol=1e-13, atol=1e-14)
    # l >= 1 always (the max logit contributes exp(0)).
    assert np.all(l >= 1.0)


def test_kv_bytes_per_token_matches_the_note(load_golden):
    g = load_golden("kv_bytes_opt13b.json")
    per_token = C.kv_bytes_per_token(g["layers"], g["hidden"], g["bytes_fp16"])
    assert per_token == 819_200
    assert per_token / 1024 == g["printed_kb_per_token_approx"]
    per_request = per_token * g["tokens"] / 1024 ** 3
    assert per_request == 1.5625
    assert abs(per_request - g["printed_gb_per_2048_tokens_approx"]) < 0.05
    # One layer of the OPT-13B shape (40 heads x 128 = 5120) keeps 20,480 B per token.
    assert C.kv_bytes_per_token(1, 40 * 128, 2) == 20_480


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_paged_decode_at_any_block_size_equals_contiguous_attention(bs):
    # Pages of 16, 32 or 64 tokens only change where rows live: scattered
    # through random tables into a pool whose other slots hold NaN, every
    # sequence must give exactly the attention over its contiguous rows.
    rng = W.rng(13, bs)
    H, D, NB = 2, 8, 12
    ctxs = [1, bs - 1, bs, bs + 1, 3 * bs - 5]
    perm = rng.permutation(NB)
    kp = np.full((NB, H, bs, D), np.nan)
    vp = np.full((NB, H, bs, D), np.nan)
    tables, ks, vs, used = [], [], [], 0
    for ctx in ctxs:
        nb = -(-ctx // bs)
        table = perm[used:used + nb]
        used += nb
        K = rng.standard_normal((ctx, H, D))
        V = rng.standard_normal((ctx, H, D))
        C.write_kv(kp, vp, K, V, P.slots(ctx, table, bs), block_size=bs)
        tables.append(table)
        ks.append(K)
        vs.append(V)
    q = rng.standard_normal((len(ctxs), H, D))
    out = A.paged_decode(q, kp, vp, tables, ctxs, block_size=bs)
    for s in range(len(ctxs)):
        np.testing.assert_array_equal(out[s], A.attend(q[s], ks[s], vs[s], A.default_scale(D)))
    # The written slots are exactly the table's blocks at offsets t % bs.
    t = ctxs[-1] - 1
    assert P.slot(t, tables[-1], bs) == tables[-1][t // bs] * bs + t % bs
