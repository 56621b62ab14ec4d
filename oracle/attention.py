"""Oracle: decode attention in float64.

Test infrastructure only (see the package docstring).

Definition: "One Deep Concept #01", §2 Background, gives attention as
softmax(Q K^T / sqrt(d)) V, with past keys and values kept in the KV cache so
that a new token computes only its own query ("KV Cache与长上下文管理", section
一: the new token's query meets every cached key and value). In decode there is
one query row per sequence and head, so for head h

    z_t = (q_h . k_{t,h}) * scale        scale = 1 / sqrt(head_dim)
    w_t = exp(z_t - max_u z_u) / sum_u exp(z_u - max_u z_u)
    out_h = sum_t w_t v_{t,h}

Paging changes where K and V live, not the result ("PagedAttention — 把 KV
cache 当虚拟内存页来管理", 踩过的坑: paging does not change the model's outputs,
only how the KV cache is stored and read), so the paged decode is this formula
over the rows gathered through the block table in logical order.

Partitions (split-K). For tokens in a range P the partial results are
``m_P = max z``, ``l_P = sum exp(z - m_P)`` and ``o_P = sum exp(z - m_P) v / l_P``.
Because softmax is unchanged by a common shift of its logits,
``out = sum_P exp(m_P - M) l_P o_P / sum_P exp(m_P - M) l_P`` with
``M = max_P m_P`` equals the unsplit result. The pages do not spell this merge
out; the long-context page only says to split a long sequence into several
attention units. It is derived here from the definition above.
"""

from __future__ import annotations

import math

import numpy as np

from . import paging


def default_scale(head_dim: int) -> float:
    """1 / sqrt(d), the logit scale of the attention formula."""
    return 1.0 / math.sqrt(head_dim)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Single-query attention per head.

    ``q``: [H][D]; ``K``, ``V``: [T][H][D] (contiguous, logical order).
    Returns [H][D] float64. ``T == 0`` gives zeros (nothing to attend to).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    H, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((H, D), dtype=np.float64)
    out = np.empty((H, D), dtype=np.float64)
    for h in range(H):
        z = (K[:, h, :] @ q[h]) * scale          # [T]
        e = np.exp(z - z.max())
        w = e / e.sum()
        out[h] = w @ V[:, h, :]
    return out


def softmax_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """The softmax weights ``w`` [H][T] of :func:`attend` (for invariant checks)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    z = np.einsum("thd,hd->ht", K, q) * scale
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def paged_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables,
                 context_lens, scale: float | None = None, block_size: int = 16,
                 k_scale: np.ndarray | None = None, v_scale: np.ndarray | None = None
                 ) -> np.ndarray:
    """Decode for a batch: ``q`` [S][H][D] -> out [S][H][D] (float64).

    Sequence ``s`` attends over its first ``context_lens[s]`` logical tokens,
    gathered through ``block_tables[s]``. For int8 pools pass the per-(block,
    head) scales; codes are dequantised exactly in float64.
    """
    q = np.asarray(q)
    S, H, D = q.shape
    if scale is None:
        scale = default_scale(D)
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        K = paging.gather(k_pool, block_tables[s], ctx, block_size, k_scale)
        V = paging.gather(v_pool, block_tables[s], ctx, block_size, v_scale)
        out[s] = attend(q[s], K, V, scale)
    return out


def partition_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       start: int, end: int):
    """(m, l, o) of tokens ``[start, end)`` for every head.

    ``m`` [H] is the largest logit, ``l`` [H] the sum of ``exp(z - m)`` and
    ``o`` [H][D] the attention output over the range alone.
    """
    q = np.asarray(q, dtype=np.float64)
    Kp = np.asarray(K[start:end], dtype=np.float64)
    Vp = np.asarray(V[start:end], dtype=np.float64)
    H, D = q.shape
    m = np.empty(H)
    l = np.empty(H)
    o = np.empty((H, D))
    for h in range(H):
        z = (Kp[:, h, :] @ q[h]) * scale
        m[h] = z.max()
        e = np.exp(z - m[h])
        l[h] = e.sum()
        o[h] = (e @ Vp[:, h, :]) / l[h]
    return m, l, o


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Merge partition results: ``m``, ``l`` [P][H], ``o`` [P][H][D] -> [H][D]."""
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    M = m.max(axis=0)                              # [H]
    w = np.exp(m - M[None, :]) * l                 # [P][H]
    return np.einsum("ph,phd->hd", w, o) / w.sum(axis=0)[:, None]


def split_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                 partition_tokens: int) -> np.ndarray:
    """One sequence decoded by partitions of ``partition_tokens`` and merged."""
    T = K.shape[0]
    parts = [partition_partials(q, K, V, scale, a, min(a + partition_tokens, T))
             for a in range(0, T, partition_tokens)]
    m = np.stack([p[0] for p in parts])
    l = np.stack([p[1] for p in parts])
    o = np.stack([p[2] for p in parts])
    return merge_partials(m, l, o)


def paged_prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables,
                  context_lens, query_start, scale: float | None = None,
                  block_size: int = 16, k_scale: np.ndarray | None = None,
                  v_scale: np.ndarray | None = None) -> np.ndarray:
    """Several new tokens of each sequence attend at once (float64).

    The attention formula of "One Deep Concept #01", §2 Background, takes a
    matrix of queries; during generation each token attends to the tokens
    before it and to itself ("PagedAttention的终极用途", part 一). So when the
    last ``n_s`` tokens of sequence ``s`` are processed together, the one at
    position ``p = ctx_s - n_s + i`` gets exactly what decoding it alone over
    the first ``p + 1`` tokens gives: logits of tokens after ``p`` are
    excluded (a causal mask aligned to the end of the context).

    ``q``: [N][H][D], rows ``query_start[s] .. query_start[s+1]`` belonging to
    sequence ``s`` in position order; their K and V are already in the pools.
    For int8 or int4 pools pass the codes (int4 unpacked) and the per-(block,
    head) scales, as for :func:`paged_decode`; codes are dequantised exactly in
    float64. Returns [N][H][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    N, H, D = q.shape
    if scale is None:
        scale = default_scale(D)
    out = np.zeros((N, H, D), dtype=np.float64)
    for s in range(len(context_lens)):
        a, b = int(query_start[s]), int(query_start[s + 1])
        n, ctx = b - a, int(context_lens[s])
        if n == 0:
            continue
        if n > ctx:
            raise ValueError("more new tokens than the context holds")
        K = paging.gather(k_pool, block_tables[s], ctx, block_size, k_scale)
        V = paging.gather(v_pool, block_tables[s], ctx, block_size, v_scale)
        pos = ctx - n + np.arange(n)                               # [n]
        allowed = np.arange(ctx)[None, :] <= pos[:, None]          # [n][ctx]
        for h in range(H):
            z = (q[a:b, h, :] @ K[:, h, :].T) * scale              # [n][ctx]
            z = np.where(allowed, z, -np.inf)
            e = np.exp(z - z.max(axis=1, keepdims=True))
            w = e / e.sum(axis=1, keepdims=True)
            out[a:b, h, :] = w @ V[:, h, :]
    return out
