"""pa_decode_noalloc, the decode entry point that allocates nothing (its
split-K partials live in the library's static device scratch), against
pa_decode with a caller workspace, through the C ABI: two calls in a row,
the second smaller, each bit-identical to pa_decode and within the fp16 bar
of the oracle."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import cache_ops as OC
from oracle import paging as OP

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _batch(pk, ctx, H, D, seed):
    bs = 16
    nbs = [-(-c // bs) for c in ctx]
    NB = sum(nbs) + 3
    order = W.free_order(seed, NB)
    kp = np.full((NB, H, bs, D), np.nan, np.float16)
    vp = np.full((NB, H, bs, D), np.nan, np.float16)
    tables, used = [], 0
    for s, c in enumerate(ctx):
        t = order[used:used + nbs[s]]
        used += nbs[s]
        K = W.normal_np((c, H, D), seed, W.STREAM_K, s, dtype=np.float16)
        V = W.normal_np((c, H, D), seed, W.STREAM_V, s, dtype=np.float16)
        OC.write_kv(kp, vp, K, V, OP.slots(c, t, bs))
        tables.append(t)
    tab = np.full((len(ctx), max(nbs)), -1, np.int32)
    for s, t in enumerate(tables):
        tab[s, :len(t)] = t
    q = W.normal_np((len(ctx), H, D), seed, W.STREAM_Q, dtype=np.float16)
    kd, vd = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
    pool = pk.pa_alloc_pool(NB, bs, H, D, pk.PA_F16, kd, vd)
    ref = OA.paged_decode(q, kp, vp, tables, ctx)
    return dict(pool=pool, kd=kd, vd=vd, q=torch.from_numpy(q).to(DEV), tab=torch.from_numpy(tab).to(DEV),
                ctx=torch.tensor(ctx, dtype=torch.int32, device=DEV), maxc=max(ctx), ref=ref)


def _both(pk, b, ptok):
    S = b["q"].shape[0]
    ws = None
    if ptok:
        nb = pk.pa_decode_workspace_bytes(b["pool"], S, b["maxc"], ptok)
        ws = torch.full((nb // 4 + 1,), float("nan"), dtype=torch.float32, device=DEV)
    want = torch.empty_like(b["q"])
    pk.pa_decode(b["pool"], b["q"], want, b["tab"], b["ctx"], b["maxc"], partition_tokens=ptok, workspace=ws)
    got = torch.full_like(b["q"], float("nan"))
    pk.pa_decode_noalloc(b["pool"], b["q"], got, b["tab"], b["ctx"], b["maxc"], partition_tokens=ptok)
    torch.cuda.synchronize()
    assert pk.pa_check_errors(b["pool"]) == 0
    return want.cpu().numpy(), got.cpu().numpy()


def _close(got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    assert not (err > 5e-3 + 1e-2 * np.abs(ref)).any(), f"max abs {err.max():.3e}"


def test_noalloc_decode_matches_pa_decode_twice():
    import paged_kv_cache_249_amd as pk
    # First call: 24 sequences up to 3000 tokens, 8 heads x 128, partitions of
    # 64 tokens (many partitions per workgroup) -> about 3 MB of partials.
    rng = np.random.default_rng(91)
    ctx1 = [int(c) for c in rng.integers(1, 3000, 24)]
    ctx1[0] = 1
    b1 = _batch(pk, ctx1, 8, 128, 91)
    print(f"noalloc call 1: S={len(ctx1)} max ctx={max(ctx1)}", flush=True)
    for ptok in (64, 512, 0):
        want, got = _both(pk, b1, ptok)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"call 1 ptok={ptok}"
        _close(got, b1["ref"])
    # Second call, smaller: 5 sequences, 4 heads x 64, partitions of 32; the
    # scratch still holds call 1's partials.
    ctx2 = [700, 33, 1, 129, 64]
    b2 = _batch(pk, ctx2, 4, 64, 92)
    print(f"noalloc call 2: S={len(ctx2)} max ctx={max(ctx2)}", flush=True)
    for ptok in (32, 0):
        want, got = _both(pk, b2, ptok)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"call 2 ptok={ptok}"
        _close(got, b2["ref"])


def test_noalloc_decode_rejects_partials_beyond_the_scratch():
    import paged_kv_cache_249_amd as pk
    b = _batch(pk, [40, 20], 2, 64, 93)
    # 4096 sequences x 2 heads x 2048 partitions of 16 tokens: far past 32 MiB.
    ctx = torch.full((4096,), 16 * 2048, dtype=torch.int32, device=DEV)
    q = torch.zeros((4096, 2, 64), dtype=torch.float16, device=DEV)
    tab = torch.zeros((4096, 2048), dtype=torch.int32, device=DEV)
    need = pk.pa_decode_workspace_bytes(b["pool"], 4096, 16 * 2048, 16)
    assert need > pk.SCRATCH_BYTES
    with pytest.raises(pk.PagedKVError) as e:
        pk.pa_decode_noalloc(b["pool"], q, torch.empty_like(q), tab, ctx, 16 * 2048, partition_tokens=16)
    assert e.value.status == pk.PA_ERR_OUT_OF_RANGE
    # Nothing was launched: the pool's error word is clean and a valid call works.
    assert pk.pa_check_errors(b["pool"]) == 0
    want, got = _both(pk, b, 16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
