"""Pins for the oracle's multi-token (prefill) attention over paged KV (CPU only).

Each test ties ``oracle.attention.paged_prefill`` to something other than its
own formula: torch's causal scaled dot-product attention (a library routine
the whole-prompt case reduces to), the separately pinned decode oracle run
once per token, a plain-Python brute force, closed forms worked by hand, and
invariants (causality, placement independence).
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import cache_ops as C
from oracle import paging as P


def _batch(ctxs, nqs, H=3, D=16, bs=16, seed=7, dtype=np.float32):
    """Pools holding each sequence's whole context, tables, and the queries
    of its last ``nq`` tokens, packed by sequence."""
    nbs = [-(-c // bs) for c in ctxs]
    NB = sum(nbs) + 3
    order = W.free_order(seed, NB)
    k_pool = np.zeros((NB, H, bs, D), dtype)
    v_pool = np.zeros((NB, H, bs, D), dtype)
    tables, ck, cv, used = [], [], [], 0
    for s, (ctx, nb) in enumerate(zip(ctxs, nbs)):
        table = order[used:used + nb]
        used += nb
        K = W.normal_np((ctx, H, D), seed, W.STREAM_K, s).astype(dtype)
        V = W.normal_np((ctx, H, D), seed, W.STREAM_V, s).astype(dtype)
        C.write_kv(k_pool, v_pool, K, V, P.slots(ctx, table, bs), bs)
        tables.append(table)
        ck.append(K)
        cv.append(V)
    qs = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int64)
    q = W.normal_np((int(qs[-1]), H, D), seed, W.STREAM_Q).astype(dtype)
    return q, k_pool, v_pool, tables, qs, ck, cv


def test_whole_prompt_reduces_to_library_causal_sdpa():
    # n == ctx: the mask aligned to the end of the context is the ordinary
    # causal mask, which torch computes (float64, CPU).
    ctxs = [1, 17, 40]
    q, kp, vp, tables, qs, ck, cv = _batch(ctxs, ctxs)
    out = A.paged_prefill(q, kp, vp, tables, ctxs, qs)
    for s, ctx in enumerate(ctxs):
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)
        K = torch.from_numpy(ck[s].astype(np.float64)).permute(1, 0, 2)
        V = torch.from_numpy(cv[s].astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
        np.testing.assert_allclose(out[qs[s]:qs[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("bs", [16, 32])
def test_each_token_equals_its_own_decode(bs):
    # The chunk's token at position p gets what the (separately pinned)
    # decode oracle gives for a context of p + 1 tokens.
    ctxs, nqs = [5, 33, 70, 16], [5, 3, 21, 1]
    q, kp, vp, tables, qs, _, _ = _batch(ctxs, nqs, bs=bs)
    out = A.paged_prefill(q, kp, vp, tables, ctxs, qs, block_size=bs)
    for s, (ctx, n) in enumerate(zip(ctxs, nqs)):
        for i in range(n):
            r = int(qs[s]) + i
            one = A.paged_decode(q[r:r + 1], kp, vp, [tables[s]], [ctx - n + i + 1], block_size=bs)
            np.testing.assert_allclose(out[r], one[0], rtol=1e-12, atol=1e-13)


def test_brute_force_double_loop():
    ctxs, nqs = [23, 9], [6, 9]
    q, kp, vp, tables, qs, ck, cv = _batch(ctxs, nqs, H=2, D=4)
    out = A.paged_prefill(q, kp, vp, tables, ctxs, qs, scale=0.3)
    for s, (ctx, n) in enumerate(zip(ctxs, nqs)):
        for i in range(n):
            r, p = int(qs[s]) + i, ctx - n + i
            for h in range(2):
                z = [0.3 * sum(float(q[r, h, d]) * float(ck[s][t, h, d]) for d in range(4))
                     for t in range(p + 1)]
                e = [math.exp(x - max(z)) for x in z]
                for d in range(4):
                    ref = sum(e[t] * float(cv[s][t, h, d]) for t in range(p + 1)) / sum(e)
                    assert abs(out[r, h, d] - ref) < 1e-12


def test_two_token_closed_forms():
    # One head, D = 2. The first token sees only itself: its output is v0
    # exactly. The second token with equal logits averages v0 and v1; with
    # logit gap log(3) it weighs them 1:3.
    k = np.array([[1.0, 0.0], [0.0, 1.0]])
    v = np.array([[2.0, -4.0], [6.0, 8.0]])
    kp = np.zeros((1, 1, 16, 2))
    vp = np.zeros((1, 1, 16, 2))
    kp[0, 0, :2], vp[0, 0, :2] = k, v
    q = np.array([[[5.0, -1.0]], [[0.7, 0.7]]])
    out = A.paged_prefill(q, kp, vp, [[0]], [2], [0, 2], scale=1.0)
    np.testing.assert_array_equal(out[0, 0], v[0])
    np.testing.assert_allclose(out[1, 0], (v[0] + v[1]) / 2, rtol=0, atol=1e-15)
    q2 = np.array([[[0.0, 0.0]], [[0.0, math.log(3.0)]]])
    out2 = A.paged_prefill(q2, kp, vp, [[0]], [2], [0, 2], scale=1.0)
    np.testing.assert_allclose(out2[1, 0], 0.25 * v[0] + 0.75 * v[1], rtol=0, atol=1e-14)


def test_later_tokens_do_not_reach_earlier_queries():
    # Changing K and V of the chunk's last token changes only the last query.
    ctxs, nqs = [40], [8]
    q, kp, vp, tables, qs, _, _ = _batch(ctxs, nqs)
    base = A.paged_prefill(q, kp, vp, tables, ctxs, qs)
    blk, off = P.locate(39, tables[0])
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[blk, :, off] += 3.0
    vp2[blk, :, off] -= 5.0
    moved = A.paged_prefill(q, kp2, vp2, tables, ctxs, qs)
    np.testing.assert_array_equal(moved[:7], base[:7])
    assert np.abs(moved[7] - base[7]).min() > 0


def test_placement_does_not_change_the_result():
    ctxs, nqs = [50, 20], [11, 4]
    q, kp, vp, tables, qs, ck, cv = _batch(ctxs, nqs, seed=3)
    out = A.paged_prefill(q, kp, vp, tables, ctxs, qs)
    # The same sequences laid out in identity order.
    H, D = q.shape[1:]
    ident, kp2, vp2, used = [], np.zeros_like(kp), np.zeros_like(vp), 0
    for s, ctx in enumerate(ctxs):
        nb = -(-ctx // 16)
        t = list(range(used, used + nb))
        used += nb
        C.write_kv(kp2, vp2, ck[s], cv[s], P.slots(ctx, t))
        ident.append(t)
    np.testing.assert_array_equal(A.paged_prefill(q, kp2, vp2, ident, ctxs, qs), out)


def test_empty_chunks_and_bad_lengths():
    ctxs, nqs = [10, 12], [0, 3]
    q, kp, vp, tables, qs, _, _ = _batch(ctxs, nqs)
    out = A.paged_prefill(q, kp, vp, tables, ctxs, qs)
    assert out.shape == (3,) + q.shape[1:]
    with pytest.raises(ValueError):
        A.paged_prefill(q, kp, vp, tables, [10, 2], qs)


@pytest.mark.parametrize("qmax", [127, 7])
def test_quantised_pools_reduce_to_library_causal_sdpa(qmax):
    # Rows k * 2^-e with integer |k| <= qmax, e depending on the logical block
    # (5, 6, 7, ...), and one entry of +-qmax in every (block, head): the
    # int8 (int4) write gives the scale 2^-e and the codes k exactly, so
    # prefill over the codes and scales must equal torch's causal attention
    # over the rows themselves. Blocks of one sequence carry different scales
    # and sit at scattered physical blocks, so a scale taken from the wrong
    # block, or by logical instead of physical index, fails.
    H, D, bs = 2, 8, 16
    ctxs = [40, 21]
    nbs = [-(-c // bs) for c in ctxs]
    NB = sum(nbs) + 5
    order = W.free_order(11, NB)
    kc = np.zeros((NB, H, bs, D), np.int8)
    vc = np.zeros((NB, H, bs, D), np.int8)
    ks = np.zeros((NB, H), np.float16)
    vs = np.zeros((NB, H), np.float16)
    rng = np.random.default_rng(11)
    tables, rows, used = [], [], 0
    for s, ctx in enumerate(ctxs):
        table = order[used:used + nbs[s]]
        used += nbs[s]
        e = np.array([5 + (t // bs + s) % 3 for t in range(ctx)], np.float64)
        K = rng.integers(-qmax, qmax + 1, size=(ctx, H, D)).astype(np.float64)
        V = rng.integers(-qmax, qmax + 1, size=(ctx, H, D)).astype(np.float64)
        for b in range(nbs[s]):
            K[b * bs, :, 0] = qmax
            V[b * bs, :, 1] = -qmax
        K *= 2.0 ** -e[:, None, None]
        V *= 2.0 ** -e[:, None, None]
        C.write_kv_int8(kc, ks, vc, vs, K.astype(np.float32), V.astype(np.float32),
                        P.slots(ctx, table, bs), bs, qmax=qmax)
        tables.append(table)
        rows.append((K, V))
    nqs = [ctxs[0], 9]
    qs = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int64)
    q = W.normal_np((int(qs[-1]), H, D), 11, W.STREAM_Q)
    out = A.paged_prefill(q, kc, vc, tables, ctxs, qs, block_size=bs, k_scale=ks, v_scale=vs)
    for s, ctx in enumerate(ctxs):
        n = nqs[s]
        K, V = rows[s]
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)
        Kt = torch.from_numpy(K).permute(1, 0, 2)
        Vt = torch.from_numpy(V).permute(1, 0, 2)
        # The chunk's rows are the context's last n: their causal mask is
        # aligned to the end of the context.
        mask = torch.ones(n, ctx, dtype=torch.bool).tril(diagonal=ctx - n)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=mask)
        np.testing.assert_allclose(out[qs[s]:qs[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
    # Without the scales the codes alone give a different answer.
    raw = A.paged_prefill(q, kc, vc, tables, ctxs, qs, block_size=bs)
    assert np.abs(raw - out).max() > 1e-3
