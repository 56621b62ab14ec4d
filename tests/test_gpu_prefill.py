"""GPU parity of pa_prefill (several new tokens per sequence attending at once
over paged fp16 KV) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import cache_ops as OC
from oracle import paging as OP

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# fp16 outputs: |gpu - ref| <= 5e-3 + 1e-2 |ref| elementwise (the stated bar).
ATOL, RTOL = 5e-3, 1e-2


def _pk():
    import paged_kv_cache_249_amd as pk
    return pk


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} out of tolerance; max abs {err.max():.3e} at "
                           f"{np.unravel_index(np.argmax(err - RTOL * np.abs(ref)), err.shape)}")


class Chunks:
    """Sequences whose whole contexts sit in a NaN-poisoned fp16 pool (seeded
    placement), with queries for the last ``nq[s]`` tokens of each."""

    def __init__(self, ctx, nq, H, D, bs=16, seed=0, write_chunk_on_gpu=False, key_gain=None):
        pk = _pk()
        self.ctx, self.nq, self.H, self.D, self.bs = list(ctx), list(nq), H, D, bs
        nbs = [-(-c // bs) for c in ctx]
        self.NB = sum(nbs) + 5
        order = W.free_order(seed, self.NB)
        self.tables, used = [], 0
        for nb in nbs:
            self.tables.append(order[used:used + nb])
            used += nb
        self.max_blocks = max(1, max(nbs))
        tab = np.full((len(ctx), self.max_blocks), -1, np.int32)
        for i, t in enumerate(self.tables):
            tab[i, :len(t)] = t
        self.k_pool = np.full((self.NB, H, bs, D), np.nan, np.float16)
        self.v_pool = np.full((self.NB, H, bs, D), np.nan, np.float16)
        self.qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
        R = int(self.qs[-1])
        kd_host, vd_host = self.k_pool.copy(), self.v_pool.copy()
        new_k, new_v, new_slots = [], [], []
        for s, c in enumerate(ctx):
            K = W.normal_np((c, H, D), seed, W.STREAM_K, s, dtype=np.float16)
            V = W.normal_np((c, H, D), seed, W.STREAM_V, s, dtype=np.float16)
            if key_gain is not None:
                # Keys scaled by a gain per position (then rounded to fp16 like the pool).
                K = (K.astype(np.float32) * key_gain(np.arange(c))[:, None, None].astype(np.float32)
                     ).astype(np.float16)
            slots = OP.slots(c, self.tables[s], bs)
            OC.write_kv(self.k_pool, self.v_pool, K, V, slots, block_size=bs)
            old = c - nq[s] if write_chunk_on_gpu else c
            OC.write_kv(kd_host, vd_host, K[:old], V[:old], slots[:old], block_size=bs)
            new_k.append(K[old:])
            new_v.append(V[old:])
            new_slots.append(slots[old:])
        self.q = W.normal_np((R, H, D), seed, W.STREAM_Q, dtype=np.float16)
        self.kd = torch.from_numpy(kd_host).to(DEV)
        self.vd = torch.from_numpy(vd_host).to(DEV)
        self.pool = pk.pa_alloc_pool(self.NB, bs, H, D, pk.PA_F16, self.kd, self.vd)
        if write_chunk_on_gpu:
            kn = torch.from_numpy(np.concatenate(new_k)).to(DEV)
            vn = torch.from_numpy(np.concatenate(new_v)).to(DEV)
            sl = torch.from_numpy(np.concatenate(new_slots).astype(np.int64)).to(DEV)
            pk.pa_write_kv(self.pool, kn, vn, sl)
        self.qd = torch.from_numpy(self.q).to(DEV)
        self.qsd = torch.from_numpy(self.qs).to(DEV)
        self.tabd = torch.from_numpy(tab).to(DEV)
        self.ctxd = torch.tensor(ctx, dtype=torch.int32, device=DEV)

    def gpu(self, max_query_len=None, max_ctx=None, sm_scale=0.0, seq_order=None):
        pk = _pk()
        out = torch.full_like(self.qd, float("nan"))
        order = None if seq_order is None else torch.tensor(seq_order, dtype=torch.int32, device=DEV)
        pk.pa_prefill(self.pool, self.qd, out, self.qsd, self.tabd, self.ctxd,
                      max(self.nq) if max_query_len is None else max_query_len,
                      max(self.ctx) if max_ctx is None else max_ctx, sm_scale, seq_order=order)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self, scale=None):
        return OA.paged_prefill(self.q, self.k_pool, self.v_pool, self.tables, self.ctx, self.qs,
                                scale=scale, block_size=self.bs)


# Whole prompts, partial chunks, an empty chunk, single rows, and chunks whose
# rows span several 64-row workgroups with ragged tails.
CTX = [1, 17, 100, 300, 64, 33, 250, 129]
NQ = [1, 17, 37, 130, 64, 0, 1, 129]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64])
def test_prefill_matches_the_oracle(D, bs):
    pk = _pk()
    b = Chunks(CTX, NQ, H=3, D=D, bs=bs, seed=bs + D)
    print(f"prefill D={D} bs={bs}", flush=True)
    got = b.gpu()
    assert pk.pa_check_errors(b.pool) == 0
    assert_close(got, b.oracle(), f"D={D} bs={bs}")


def test_dispatch_windows_cover_every_tile():
    # 6 sequences x 8 heads = 48 (sequence, head) groups: 6 per XCD, dealt
    # as a window of 4 groups and a partial one of 2, each with up to 4 row
    # tiles of 128 rows (whole prompts of 129..500 tokens, one chunk of 7).
    pk = _pk()
    ctx = [500, 129, 260, 384, 77, 450]
    nq = [500, 129, 260, 7, 77, 450]
    b = Chunks(ctx, nq, H=8, D=64, seed=83)
    print("prefill windows 6x8", flush=True)
    got = b.gpu()
    assert pk.pa_check_errors(b.pool) == 0
    assert_close(got, b.oracle(), "6 x 8 groups")


def test_prefill_after_gpu_write_of_the_chunk():
    # The chunk's own K and V go through pa_write_kv first, as a prefill step does.
    b = Chunks([200, 77, 16], [120, 77, 5], H=4, D=128, seed=5, write_chunk_on_gpu=True)
    assert_close(b.gpu(), b.oracle(), "write then prefill")


def test_prefill_explicit_scale_and_larger_bounds():
    b = Chunks([90, 40], [33, 40], H=2, D=64, seed=9)
    # Bounds larger than the batch needs change nothing.
    assert_close(b.gpu(max_query_len=200, max_ctx=16 * b.max_blocks, sm_scale=0.05), b.oracle(scale=0.05),
                 "scale 0.05")


def test_single_rows_equal_decode():
    # One new token per sequence: prefill is decode.
    b = Chunks([5, 300, 48, 1000], [1, 1, 1, 1], H=4, D=128, seed=11)
    got = b.gpu()
    ref = OA.paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.ctx)
    assert_close(got, ref, "single rows")


@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_logits_whose_max_moves_many_times(direction):
    # Keys whose scale grows (or shrinks) with position: each row's running
    # max of q.k climbs by far more than 2^8 in log2 units over its context,
    # so the kernel's reference max moves and the tiles are rescaled many
    # times (rising), or the first step already holds the max (falling).
    c = 700
    gain = (lambda t: 1.0 + t / 16.0) if direction == "rising" else (lambda t: 1.0 + (c - t) / 16.0)
    b = Chunks([c, 333, 96], [c, 200, 96], H=3, D=128, seed=17, key_gain=gain)
    got = b.gpu()
    ref = b.oracle()
    # Logits reach far beyond 8 (log2 units beyond 11): confirm the inputs do
    # what the test needs (block 10 holds tokens 160..175, gain 11 or 34).
    z = b.q[:c, 0].astype(np.float64) @ b.k_pool[b.tables[0][10], 0].astype(np.float64).T / np.sqrt(128)
    assert np.abs(z).max() > 8
    assert_close(got, ref, direction)


def test_table_rows_longer_than_the_kernel_keeps_in_lds():
    # A context of 33000 tokens needs 2063 table entries of 16-token blocks:
    # more than a workgroup keeps in LDS (2048), so the kernel reads the
    # table from memory as it walks; 64-token blocks (516 entries) keep it in
    # LDS. Both against the oracle, with a ragged chunk and a short sequence.
    # 66000 tokens in 32-token blocks (2063 entries) at head_dim 128: the
    # table read from memory with two 16-row slices per block.
    for ctx0, bs, D in ((33000, 16, 64), (33000, 64, 64), (66000, 32, 128)):
        b = Chunks([ctx0, 100], [70, 100], H=2, D=D, bs=bs, seed=23)
        print(f"prefill long table ctx={ctx0} bs={bs} D={D}", flush=True)
        got = b.gpu()
        assert _pk().pa_check_errors(b.pool) == 0
        assert_close(got, b.oracle(), f"ctx={ctx0} bs={bs} D={D}")


@pytest.mark.parametrize("ctx", [300, 33000])
def test_bad_table_entry_is_flagged(ctx):
    # An entry past the pool in sequence 0's row (table kept in LDS at 300
    # tokens, read from memory at 33000): the kernel flags it and reads an
    # in-bounds row instead; the other sequence is unaffected.
    pk = _pk()
    assert pk.pa_check_errors(None) == 0
    b = Chunks([ctx, 90], [40, 90], H=2, D=64, seed=29)
    tab = b.tabd.clone()
    tab[0, 3] = b.NB + 7
    b.tabd = tab
    got = b.gpu()
    assert pk.pa_check_errors(b.pool) & pk.PA_DEV_BAD_TABLE_ENTRY
    assert_close(got[40:], b.oracle()[40:], "good sequence beside a bad table row")


def test_dispatch_order_changes_nothing():
    # pa_prefill_ordered: any permutation of the batch gives the same bits.
    pk = _pk()
    b = Chunks(CTX, NQ, H=3, D=128, seed=61)
    ref = b.gpu()
    S = len(CTX)
    work = [n * (2 * c - n + 1) // 2 for c, n in zip(CTX, NQ)]
    rng = np.random.default_rng(61)
    for order in (sorted(range(S), key=lambda s: -work[s]), list(rng.permutation(S)), list(range(S))[::-1]):
        got = b.gpu(seq_order=order)
        assert pk.pa_check_errors(b.pool) == 0
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), order
    # An entry outside the batch is flagged and its work skipped; the rest is computed.
    bad = list(range(S))
    bad[2] = S + 3
    got = b.gpu(seq_order=bad)
    assert pk.pa_check_errors(b.pool) & pk.PA_DEV_BAD_CONTEXT
    r2 = slice(int(b.qs[2]), int(b.qs[3]))
    assert np.isnan(got[r2]).all()
    keep = np.ones(got.shape[0], bool)
    keep[r2] = False
    assert np.array_equal(got[keep].view(np.uint16), ref[keep].view(np.uint16))


def test_bad_lengths_flag_and_leave_rows_unwritten():
    pk = _pk()
    assert pk.pa_check_errors(None) == 0
    b = Chunks([40, 30], [10, 5], H=2, D=64, seed=13)
    # Sequence 1 claims a context shorter than its chunk.
    b.ctxd = torch.tensor([40, 3], dtype=torch.int32, device=DEV)
    got = b.gpu(max_ctx=40)
    assert pk.pa_check_errors(b.pool) & pk.PA_DEV_BAD_CONTEXT
    assert np.isnan(got[10:]).all()
    assert_close(got[:10], b.oracle()[:10], "good sequence beside a bad one")


def test_host_validation():
    pk = _pk()
    b = Chunks([20], [4], H=2, D=64, seed=1)
    # fp32 pools are not attended by pa_prefill.
    f32 = pk.new_pool(4, 2, 64, pk.PA_F32, device=DEV)
    with pytest.raises(pk.PagedKVError) as e:
        pk.pa_prefill(f32, b.qd, torch.empty_like(b.qd), b.qsd, b.tabd, b.ctxd, 4, 20)
    assert e.value.status == pk.PA_ERR_UNSUPPORTED
    out = torch.empty_like(b.qd)
    with pytest.raises(pk.PagedKVError) as e:
        pk.pa_prefill(b.pool, b.qd.float(), out.float(), b.qsd, b.tabd, b.ctxd, 4, 20)
    assert e.value.status == pk.PA_ERR_UNSUPPORTED
    with pytest.raises(pk.PagedKVError) as e:
        pk.pa_prefill(b.pool, b.qd, out, b.qsd, b.tabd, b.ctxd, 4, 20 + 16 * b.max_blocks)
    assert e.value.status == pk.PA_ERR_INVALID_ARG
    # Nothing to do: no launch, no error.
    pk.pa_prefill(b.pool, b.qd, out, b.qsd, b.tabd, b.ctxd, 0, 20)


def test_chunked_prefill_at_full_size_sampled_rows():
    # 16 sequences of 2048 tokens whose last 512 arrive as one chunk, 40
    # heads x 128 (the OPT-13B head shape), scattered 16-token blocks; the
    # oracle checks sampled rows one by one as decodes of their own prefix.
    S, ctx, n, H, D = 16, 2048, 512, 40, 128
    b = Chunks([ctx] * S, [n] * S, H=H, D=D, seed=21)
    got = b.gpu()
    rng = np.random.default_rng(0)
    for s in range(S):
        for i in sorted(set(rng.integers(0, n, 3).tolist()) | {0, n - 1}):
            r = int(b.qs[s]) + i
            ref = OA.paged_decode(b.q[r:r + 1], b.k_pool, b.v_pool, [b.tables[s]], [ctx - n + i + 1])
            assert_close(got[r:r + 1], ref, f"seq {s} row {i}")


class QuantChunks:
    """Sequences quantised into an int8 or int4 pool (one fp16 scale per
    (block, head), the oracle's quantiser; int4 packed two codes per byte)
    whose other bytes are random and whose unused blocks have NaN scales;
    queries for the last ``nq[s]`` tokens."""

    def __init__(self, ctx, nq, H, D, bs=16, seed=0, kv="i8"):
        pk = _pk()
        self.ctx, self.nq, self.bs = list(ctx), list(nq), bs
        nbs = [-(-c // bs) for c in ctx]
        NB = sum(nbs) + 5
        order = W.free_order(seed, NB)
        self.tables, used = [], 0
        for nb in nbs:
            self.tables.append(order[used:used + nb])
            used += nb
        self.max_blocks = max(nbs)
        tab = np.full((len(ctx), self.max_blocks), -1, np.int32)
        for i, t in enumerate(self.tables):
            tab[i, :len(t)] = t
        rng = np.random.default_rng(seed)
        if kv == "i8":
            kc = rng.integers(-128, 128, size=(NB, H, bs, D), dtype=np.int8)
            vc = rng.integers(-128, 128, size=(NB, H, bs, D), dtype=np.int8)
        else:   # random codes in [-7, 7] (every nibble 1..15), kept unpacked until the writes are done
            kc = rng.integers(-7, 8, size=(NB, H, bs, D), dtype=np.int8)
            vc = rng.integers(-7, 8, size=(NB, H, bs, D), dtype=np.int8)
        ks = np.full((NB, H), np.nan, np.float16)
        vs = np.full((NB, H), np.nan, np.float16)
        write = OC.write_kv_int8 if kv == "i8" else OC.write_kv_int4
        self.K, self.V = [], []
        for s, c in enumerate(ctx):
            K = W.normal_np((c, H, D), seed, W.STREAM_K, s, dtype=np.float32)
            V = W.normal_np((c, H, D), seed, W.STREAM_V, s, dtype=np.float32)
            write(kc, ks, vc, vs, K, V, OP.slots(c, self.tables[s], bs), block_size=bs)
            self.K.append(K)
            self.V.append(V)
        # The codes and scales the kernel reads (int4 codes unpacked here;
        # blocks nobody uses keep NaN scales).
        self.kc, self.vc, self.ks, self.vs = kc.copy(), vc.copy(), ks.copy(), vs.copy()
        if kv == "i4":
            kc, vc = OC.pack_int4(kc), OC.pack_int4(vc)
        self.qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
        self.q = W.normal_np((int(self.qs[-1]), H, D), seed, W.STREAM_Q, dtype=np.float16)
        t = {n: torch.from_numpy(a).to(DEV) for n, a in (("kc", kc), ("vc", vc), ("ks", ks), ("vs", vs))}
        self.t = t
        self.pool = pk.pa_alloc_pool(NB, bs, H, D, pk.PA_I8 if kv == "i8" else pk.PA_I4, t["kc"], t["vc"],
                                     t["ks"], t["vs"])
        self.qd = torch.from_numpy(self.q).to(DEV)
        self.qsd = torch.from_numpy(self.qs).to(DEV)
        self.tabd = torch.from_numpy(tab).to(DEV)
        self.ctxd = torch.tensor(ctx, dtype=torch.int32, device=DEV)

    def gpu(self):
        pk = _pk()
        out = torch.full_like(self.qd, float("nan"))
        pk.pa_prefill(self.pool, self.qd, out, self.qsd, self.tabd, self.ctxd, max(self.nq), max(self.ctx))
        torch.cuda.synchronize()
        assert pk.pa_check_errors(self.pool) == 0
        return out.cpu().numpy()

    def oracle(self):
        return OA.paged_prefill(self.q, self.kc, self.vc, self.tables, self.ctx, self.qs,
                                block_size=self.bs, k_scale=self.ks, v_scale=self.vs)


def Int8Chunks(*args, **kw):
    return QuantChunks(*args, kv="i8", **kw)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64])
def test_int8_prefill_matches_the_oracle(D, bs):
    # Against fp64 prefill over the same dequantised codes: the fp16 bar.
    b = Int8Chunks(CTX, NQ, H=3, D=D, bs=bs, seed=3 * bs + D)
    assert_close(b.gpu(), b.oracle(), f"int8 D={D} bs={bs}")


def test_int8_prefill_against_unquantised_rows():
    # Against fp64 attention over the unquantised source rows. The int8 bar
    # (2e-2 absolute) is the one stated for decode over thousands of tokens;
    # a prompt's first rows attend to a handful of tokens, so one block's
    # quantisation error shows through almost undiluted. Every row: the
    # kernel adds at most the fp16 bar to the error the quantisation itself
    # makes (the oracle over the dequantised codes); rows attending at least
    # 256 tokens: within 2e-2.
    b = Int8Chunks([300, 129], [130, 129], H=4, D=128, seed=41)
    got = b.gpu().astype(np.float64)
    deq = b.oracle()
    rows, attended = [], []
    for s, (c, n) in enumerate(zip(b.ctx, b.nq)):
        for i in range(n):
            p = c - n + i
            rows.append(OA.attend(b.q[int(b.qs[s]) + i], b.K[s][:p + 1], b.V[s][:p + 1], 1.0 / np.sqrt(128)))
            attended.append(p + 1)
    exact = np.stack(rows)
    attended = np.asarray(attended)
    quant_err = np.abs(deq - exact)
    assert (np.abs(got - exact) <= quant_err + 5e-3 + 1e-2 * np.abs(exact)).all()
    long_rows = attended >= 256
    assert long_rows.sum() >= 40
    assert np.abs(got - exact)[long_rows].max() <= 2e-2


def test_int8_prefill_table_read_from_memory():
    # 33000 tokens in 16-token blocks: the table row is walked from memory.
    b = Int8Chunks([33000, 50], [40, 50], H=2, D=64, seed=43)
    assert_close(b.gpu(), b.oracle(), "int8 long table")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64])
def test_int4_prefill_matches_the_oracle(D, bs):
    # Packed int4 codes against fp64 prefill over the same dequantised codes: the fp16 bar.
    b = QuantChunks(CTX, NQ, H=3, D=D, bs=bs, seed=5 * bs + D, kv="i4")
    assert_close(b.gpu(), b.oracle(), f"int4 D={D} bs={bs}")


def test_int4_prefill_table_read_from_memory():
    b = QuantChunks([33000, 50], [40, 50], H=2, D=128, seed=47, kv="i4")
    assert_close(b.gpu(), b.oracle(), "int4 long table")


@pytest.mark.parametrize("D", [64, 128])
def test_whole_prompt_of_4096_tokens(D):
    # One 4096-token prompt attending causally at once (32 row tiles per
    # (sequence, head), the longest walks) beside a short one.
    b = Chunks([4096, 70], [4096, 70], H=2, D=D, seed=53)
    got = b.gpu()
    assert _pk().pa_check_errors(b.pool) == 0
    assert_close(got, b.oracle(), f"4096-token prompt D={D}")


@pytest.mark.parametrize("kv", ["f16", "i8", "i4"])
@pytest.mark.parametrize("seed", [71, 72, 73])
def test_random_batches_against_the_oracle(kv, seed):
    # Seeded random batches: 12 sequences with contexts of 1..1500 tokens,
    # chunks of 0..ctx rows (whole prompts, single rows and empty chunks
    # included), a random head_dim and block size, dispatched in a random
    # order; every row against the oracle.
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64]))
    ctx = [int(c) for c in rng.integers(1, 1500, 12)]
    ctx[0] = 1
    nq = [int(rng.integers(0, c + 1)) for c in ctx]
    nq[1] = ctx[1]
    nq[2] = 0
    if kv == "f16":
        b = Chunks(ctx, nq, H=2, D=D, bs=bs, seed=seed)
        got = b.gpu(seq_order=list(rng.permutation(len(ctx))))
    else:
        b = QuantChunks(ctx, nq, H=2, D=D, bs=bs, seed=seed, kv=kv)
        got = b.gpu()
    assert _pk().pa_check_errors(b.pool) == 0
    assert_close(got, b.oracle(), f"{kv} seed={seed} D={D} bs={bs}")
