"""Pins for the oracle's write, copy and int8 / int4 quantise-on-write (CPU only)."""

import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import cache_ops as C
from oracle import paging as P


def test_write_then_gather_round_trip_f32_and_f16():
    rng = W.rng(21, 0)
    NB, H, D, n = 12, 3, 8, 40
    table = rng.permutation(NB)[:3]
    slots = P.slots(n, table)
    for dt in (np.float32, np.float16):
        kp = np.zeros((NB, H, 16, D), dt)
        vp = np.zeros((NB, H, 16, D), dt)
        k = rng.standard_normal((n, H, D)).astype(np.float32)
        v = rng.standard_normal((n, H, D)).astype(np.float32)
        C.write_kv(kp, vp, k, v, slots)
        np.testing.assert_array_equal(P.gather(kp, table, n), k.astype(dt).astype(np.float64))
        np.testing.assert_array_equal(P.gather(vp, table, n), v.astype(dt).astype(np.float64))


def test_write_rounds_to_nearest_even_into_f16():
    # Hand-worked fp16 ties: spacing of fp16 just above 1 is 2^-10.
    x = np.array([1 + 2 ** -11,            # tie between 1 and 1+2^-10 -> 1 (even)
                  1 + 3 * 2 ** -11,        # tie between 1+2^-10 and 1+2^-9 -> 1+2^-9 (even)
                  -(1 + 2 ** -11),
                  65520.0,                 # tie at the top -> overflows to +inf
                  2 ** -25,                # half the smallest subnormal -> 0 (even)
                  3 * 2 ** -25],           # 1.5 x smallest subnormal -> 2 x smallest subnormal
                 dtype=np.float32)
    expect = [1.0, 1 + 2 ** -9, -1.0, math.inf, 0.0, 2 ** -23]
    kp = np.zeros((1, 1, 16, x.size), np.float16)
    vp = np.zeros_like(kp)
    with np.errstate(over="ignore"):
        C.write_kv(kp, vp, x[None, None, :], x[None, None, :], [5])
    assert kp[0, 0, 5].astype(np.float64).tolist() == expect


def test_negative_slots_are_skipped():
    kp = np.full((2, 1, 16, 4), 7, np.float32)
    vp = kp.copy()
    C.write_kv(kp, vp, np.ones((2, 1, 4), np.float32), np.ones((2, 1, 4), np.float32), [-1, 17])
    assert (kp[1, 0, 1] == 1).all() and (kp == 7).sum() == kp.size - 4


def test_copy_blocks_copies_whole_blocks_only():
    rng = W.rng(22, 0)
    k = rng.standard_normal((6, 2, 16, 4)).astype(np.float16)
    ks = rng.standard_normal((6, 2)).astype(np.float16)
    before = k.copy()
    C.copy_blocks([k, ks], [(1, 4), (2, 5)])
    assert np.array_equal(k[4], before[1]) and np.array_equal(k[5], before[2])
    assert np.array_equal(k[:4], before[:4])
    assert np.array_equal(ks[4], ks[1])


def _int8_pools(NB=4, H=1, D=8):
    return (np.zeros((NB, H, 16, D), np.int8), np.zeros((NB, H), np.float16),
            np.zeros((NB, H, 16, D), np.int8), np.zeros((NB, H), np.float16))


def test_int8_hand_worked_codes():
    # max |x| = 127 -> scale = 127/127 = 1 exactly; codes are x rounded to
    # nearest even and clamped. A divisor of 128, or rounding half away from
    # zero, would change these codes.
    x = np.array([127.0, -63.5, 0.5, 1.5, 2.5, -2.5, 126.4, -127.0], np.float32)
    kc, ks, vc, vs = _int8_pools(D=8)
    C.write_kv_int8(kc, ks, vc, vs, x[None, None], x[None, None], [16])
    assert float(ks[1, 0]) == 1.0
    assert kc[1, 0, 0].tolist() == [127, -64, 0, 2, 2, -2, 126, -127]


def test_int8_requantise_when_the_scale_grows():
    # Row 0 opens the block with max 12.7 -> s_old = fp16(0.1) = 0.0999755859375.
    # Row 1 brings max 25.4 -> s_new = fp16(0.2) = 2 * s_old exactly, so old
    # codes are re-coded as rne(q / 2): 127 -> 64, 1 -> 0, 3 -> 2, -5 -> -2.
    kc, ks, vc, vs = _int8_pools(D=4)
    row0 = np.array([12.7, 0.1, 0.3, -0.5], np.float32)
    C.write_kv_int8(kc, ks, vc, vs, row0[None, None], row0[None, None], [0])
    assert float(ks[0, 0]) == 0.0999755859375
    assert kc[0, 0, 0].tolist() == [127, 1, 3, -5]
    row1 = np.array([25.4, 0.0, 0.0, 0.0], np.float32)
    C.write_kv_int8(kc, ks, vc, vs, row1[None, None], row1[None, None], [1])
    assert float(ks[0, 0]) == 0.199951171875
    assert kc[0, 0, 0].tolist() == [64, 0, 2, -2]
    assert kc[0, 0, 1].tolist() == [127, 0, 0, 0]
    # A smaller row later keeps the scale and leaves old rows alone.
    row2 = np.array([1.0, -1.0, 0.0, 0.0], np.float32)
    C.write_kv_int8(kc, ks, vc, vs, row2[None, None], row2[None, None], [2])
    assert float(ks[0, 0]) == 0.199951171875
    assert kc[0, 0, 0].tolist() == [64, 0, 2, -2]
    assert kc[0, 0, 2].tolist() == [5, -5, 0, 0]


def test_int8_zero_group_and_reopen():
    kc, ks, vc, vs = _int8_pools(D=4)
    kc[:] = 99
    z = np.zeros((1, 1, 4), np.float32)
    C.write_kv_int8(kc, ks, vc, vs, z, z, [3 * 16])
    assert float(ks[3, 0]) == 0.0 and kc[3, 0, 0].tolist() == [0, 0, 0, 0]
    # Offset 0 re-opens a block: its old scale is ignored even if larger.
    ks[2, 0] = 100.0
    x = np.array([[[1.27, 0, 0, 0]]], np.float32)
    C.write_kv_int8(kc, ks, vc, vs, x, x, [2 * 16])
    assert float(ks[2, 0]) == float(np.float16(np.float32(1.27) / np.float32(127)))
    assert kc[2, 0, 1].tolist() == [99, 99, 99, 99]     # other rows untouched


def test_int8_round_trip_bound_and_whole_block_group():
    rng = W.rng(23, 0)
    D = 128
    x = rng.standard_normal((16, 1, D)).astype(np.float32)
    kc, ks, vc, vs = _int8_pools(NB=2, D=D)
    C.write_kv_int8(kc, ks, vc, vs, x, x, np.arange(16) + 16)
    s = float(ks[1, 0])
    a = float(np.abs(x).max())
    assert s == float(np.float16(np.float32(a) / np.float32(127)))
    deq = kc[1, 0].astype(np.float64) * s
    err = np.abs(deq - x[:, 0].astype(np.float64))
    # |x - q s| <= s/2, except values clipped because fp16 rounded s below a/127.
    bound = s / 2 + np.maximum(0.0, np.abs(x[:, 0]) - 127 * s) + 1e-12
    assert np.all(err <= bound)


def test_int8_attention_error_within_two_hundredths():
    # The int8 bar: attention over dequantised codes vs the unquantised source.
    rng = W.rng(24, 0)
    T, H, D = 300, 4, 128
    NB = -(-T // 16)
    q = rng.standard_normal((H, D)).astype(np.float16)
    K = rng.standard_normal((T, H, D)).astype(np.float32)
    V = rng.standard_normal((T, H, D)).astype(np.float32)
    kc = np.zeros((NB, H, 16, D), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((NB, H), np.float16)
    vs = np.zeros_like(ks)
    table = np.arange(NB)
    for t in range(T):                      # one token per call, as in decode
        C.write_kv_int8(kc, ks, vc, vs, K[t:t + 1], V[t:t + 1], [P.slot(t, table)])
    out_q = A.paged_decode(q[None], kc, vc, [table], [T], k_scale=ks, v_scale=vs)[0]
    out_f = A.attend(q, K, V, A.default_scale(D))
    assert np.abs(out_q - out_f).max() < 2e-2


def test_swap_round_trip_is_a_relabelling():
    # Out to host blocks and back into other device blocks: every moved block
    # arrives bit for bit, blocks not named stay as they were, and decode
    # through the updated tables gives exactly the same result.
    from oracle import attention as A
    from oracle import paging as P
    rng = W.rng(21, 0)
    NB, NH, H, D, bs = 12, 6, 2, 8, 16
    kp = rng.standard_normal((NB, H, bs, D)).astype(np.float16)
    vp = rng.standard_normal((NB, H, bs, D)).astype(np.float16)
    ks = rng.standard_normal((NB, H)).astype(np.float16)
    hk = np.zeros((NH, H, bs, D), np.float16)
    hv = np.zeros_like(hk)
    hs = np.zeros((NH, H), np.float16)
    table, ctx = [7, 2, 9], 40
    q = rng.standard_normal((1, H, D))
    before = A.paged_decode(q, kp, vp, [table], [ctx])
    C.swap_blocks([kp, vp, ks], [hk, hv, hs], [(7, 4), (2, 0), (9, 5)], "out")
    assert np.array_equal(hk[[4, 0, 5]], kp[[7, 2, 9]]) and np.array_equal(hs[[4, 0, 5]], ks[[7, 2, 9]])
    untouched = kp[[0, 1, 3]].copy()
    kp[[7, 2, 9]] = np.nan                    # the device blocks are reused meanwhile
    C.swap_blocks([kp, vp, ks], [hk, hv, hs], [(4, 3), (0, 11), (5, 1)], "in")
    assert np.array_equal(kp[[3, 11, 1]], hk[[4, 0, 5]])
    assert np.array_equal(kp[0], untouched[0])
    after = A.paged_decode(q, kp, vp, [[3, 11, 1]], [ctx])
    assert np.array_equal(before, after)
    with pytest.raises(ValueError):
        C.swap_blocks([kp], [hk], [(0, 0)], "sideways")


# ---------------------------------------------------------------------------
# int4: the int8 group rule with codes in [-7, 7], and the nibble layout.

def test_int4_hand_worked_codes():
    # max |x| = 7 -> scale = 7/7 = 1 exactly; codes are x rounded to nearest
    # even and clamped to [-7, 7]. A divisor of 8 (or of 127) would change them.
    x = np.array([7.0, -3.5, 0.5, 1.5, 2.5, -2.5, 6.4, -7.0], np.float32)
    kc, ks, vc, vs = _int8_pools(D=8)
    C.write_kv_int4(kc, ks, vc, vs, x[None, None], x[None, None], [16])
    assert float(ks[1, 0]) == 1.0
    assert kc[1, 0, 0].tolist() == [7, -4, 0, 2, 2, -2, 6, -7]


def test_int4_requantise_when_the_scale_grows():
    # Row 0 opens the block with max 0.7 -> s_old = fp16(0.1) = 0.0999755859375.
    # Row 1 brings max 1.4 -> s_new = fp16(0.2) = 2 * s_old exactly, so old
    # codes are re-coded as rne(q / 2): 7 -> 4, 1 -> 0, 3 -> 2, -5 -> -2.
    kc, ks, vc, vs = _int8_pools(D=4)
    row0 = np.array([0.7, 0.1, 0.3, -0.5], np.float32)
    C.write_kv_int4(kc, ks, vc, vs, row0[None, None], row0[None, None], [0])
    assert float(ks[0, 0]) == 0.0999755859375
    assert kc[0, 0, 0].tolist() == [7, 1, 3, -5]
    row1 = np.array([1.4, 0.0, 0.0, -0.3], np.float32)
    C.write_kv_int4(kc, ks, vc, vs, row1[None, None], row1[None, None], [1])
    assert float(ks[0, 0]) == 0.199951171875
    assert kc[0, 0, 0].tolist() == [4, 0, 2, -2]
    assert kc[0, 0, 1].tolist() == [7, 0, 0, -2]


def test_int4_round_trip_bound():
    rng = W.rng(25, 0)
    D = 128
    x = rng.standard_normal((16, 1, D)).astype(np.float32)
    kc, ks, vc, vs = _int8_pools(NB=2, D=D)
    C.write_kv_int4(kc, ks, vc, vs, x, x, np.arange(16) + 16)
    s = float(ks[1, 0])
    assert s == float(np.float16(np.float32(np.abs(x).max()) / np.float32(7)))
    assert np.abs(kc[1, 0]).max() <= 7
    err = np.abs(kc[1, 0].astype(np.float64) * s - x[:, 0].astype(np.float64))
    bound = s / 2 + np.maximum(0.0, np.abs(x[:, 0]) - 7 * s) + 1e-12
    assert np.all(err <= bound)


def test_int4_nibble_layout():
    # Byte j of a row: code[2j] + 8 in the low nibble, code[2j+1] + 8 in the
    # high one.
    codes = np.array([[-7, 7, 0, 1, -1, 3, 5, -6]], np.int8)
    packed = C.pack_int4(codes)
    assert packed.dtype == np.uint8 and packed.tolist() == [[0xF1, 0x98, 0xB7, 0x2D]]
    assert np.array_equal(C.unpack_int4(packed), codes)
    allc = np.arange(-7, 8, dtype=np.int8)
    grid = np.stack(np.meshgrid(allc, allc, indexing="ij"), -1).reshape(-1, 2)
    assert np.array_equal(C.unpack_int4(C.pack_int4(grid)), grid)
    assert C.unpack_int4(np.zeros((1, 2), np.uint8)).tolist() == [[-8, -8, -8, -8]]
    with pytest.raises(ValueError):
        C.pack_int4(np.array([[8, 0]], np.int8))


def test_int4_exactly_representable_rows_decode_exactly():
    # Rows k/7 * 2^-3 with integer k in [-7, 7] and one +-7 per (block, head)
    # in every written group: the scale is exactly 2^-3 and every code exact,
    # so attention over the int4 codes equals fp64 attention over the rows.
    rng = W.rng(26, 0)
    T, H, D = 70, 2, 8
    NB = -(-T // 16)
    K = (rng.integers(-7, 8, size=(T, H, D)) / 8.0).astype(np.float32)
    V = (rng.integers(-7, 8, size=(T, H, D)) / 8.0).astype(np.float32)
    K[:, :, 0] = 7 / 8
    V[:, :, 1] = -7 / 8
    kc = np.zeros((NB, H, 16, D), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((NB, H), np.float16)
    vs = np.zeros_like(ks)
    table = W.free_order(26, NB)
    for t in range(T):
        C.write_kv_int4(kc, ks, vc, vs, K[t:t + 1], V[t:t + 1], [P.slot(t, table)])
    assert np.all(ks[table] == np.float16(1 / 8)) and np.all(vs[table] == np.float16(1 / 8))
    q = rng.standard_normal((1, H, D))
    got = A.paged_decode(q, kc, vc, [table], [T], k_scale=ks, v_scale=vs)[0]
    np.testing.assert_array_equal(got, A.attend(q[0], K, V, A.default_scale(D)))
