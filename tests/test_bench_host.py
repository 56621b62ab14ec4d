"""Host-side arithmetic of the benchmark's figures (no GPU): the flop count
the prefill line is rated by, against a brute-force count of the (query,
attended token) pairs the causal definition gives."""

import numpy as np
import pytest

import bench


def brute_flops(ctx, nq, H, D):
    pairs = 0
    for c, n in zip(ctx, nq):
        for i in range(n):
            pos = c - n + i                  # position of chunk row i
            pairs += sum(1 for t in range(c) if t <= pos)
    return 4 * D * H * pairs                 # q.k and the weighted v sum, 2·D flops each


@pytest.mark.parametrize("ctx,nq", [([1], [1]), ([17, 100], [17, 3]), ([64, 50, 9], [0, 50, 1]),
                                    ([300], [129])])
def test_causal_prefill_flops_counts_attended_pairs(ctx, nq):
    assert bench.causal_prefill_flops(ctx, nq, 3, 64) == brute_flops(ctx, nq, 3, 64)


def test_prefill_workload_flops():
    # 16 whole prompts of 2048 tokens at 40 x 128: 4·128·40·16·(2048·2049/2).
    S, n = bench.PREFILL_SHAPE["S"], bench.PREFILL_SHAPE["n"]
    assert bench.causal_prefill_flops([n] * S, [n] * S, 40, 128) == 4 * 128 * 40 * S * n * (n + 1) // 2
    assert bench.causal_prefill_flops([n] * S, [n] * S, 40, 128) == 687_530_311_680
    # A decode is a one-row chunk: 4·D·ctx per head.
    rng = np.random.default_rng(0)
    ctx = [int(c) for c in rng.integers(1, 500, 7)]
    assert bench.causal_prefill_flops(ctx, [1] * 7, 2, 128) == 4 * 128 * 2 * sum(ctx)
