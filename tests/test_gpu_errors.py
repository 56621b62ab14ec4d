"""The device error model on the GPU: one error word per pool, read and
cleared atomically, and quantised writes that flag a block hit by two runs
of rows that are not adjacent.

Every bad input here is forced from the host and turned into a flag by the
kernels' own range checks; every kernel exits normally.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pk():
    import paged_kv_cache_249_amd as pk
    return pk


def _rows(n, H=2, D=64):
    return torch.ones((n, H, D), dtype=torch.float16, device=DEV)


def test_pools_keep_their_own_error_words():
    pk = _pk()
    a = pk.new_pool(8, 2, 64, pk.PA_F16, device=DEV, fill=0.0)
    b = pk.new_pool(8, 2, 64, pk.PA_F16, device=DEV, fill=0.0)
    print("error words: two pools", flush=True)
    assert pk.pa_check_errors(a) == 0 and pk.pa_check_errors(b) == 0
    r = _rows(1)
    pk.pa_write_kv(a, r, r, torch.tensor([8 * 16 + 1], dtype=torch.int64, device=DEV))   # a: slot past the pool
    pk.pa_copy_blocks(b, torch.tensor([[0, 9]], dtype=torch.int32, device=DEV))          # b: pair past the pool
    torch.cuda.synchronize()
    # Each word holds only its own pool's flag, and reading one leaves the other.
    assert pk.pa_check_errors(a) == pk.PA_DEV_BAD_SLOT
    assert pk.pa_check_errors(a) == 0
    assert pk.pa_check_errors(b) == pk.PA_DEV_BAD_PAIR
    assert pk.pa_check_errors(b) == 0
    # Flags raised on another stream are read after that stream's work.
    side = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(side):
        pk.pa_copy_blocks(a, torch.tensor([[12, 0]], dtype=torch.int32, device=DEV), stream=side)
        pk.pa_write_kv(b, r, r, torch.tensor([9 * 16], dtype=torch.int64, device=DEV), stream=side)
    assert pk.pa_check_errors(a, stream=side) == pk.PA_DEV_BAD_PAIR
    assert pk.pa_check_errors(b, stream=side) == pk.PA_DEV_BAD_SLOT
    # Calls tied to no pool flag the word read with pool = None, and no pool's.
    S, H, T, D = 1, 2, 16, 64
    k = torch.zeros((S, H, T, D), dtype=torch.float16, device=DEV)
    q = torch.zeros((S, H, D), dtype=torch.float16, device=DEV)
    out = torch.empty_like(q)
    pk.pa_decode_contiguous(k, k, q, out, torch.tensor([T + 5], dtype=torch.int32, device=DEV))
    assert pk.pa_check_errors(None) & pk.PA_DEV_BAD_CONTEXT
    assert pk.pa_check_errors(a) == 0 and pk.pa_check_errors(b) == 0
    # A freed pool's word is cleared before another pool takes it.
    pk.pa_write_kv(a, r, r, torch.tensor([8 * 16], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    pk.pa_free_pool(a)
    pools = [pk.new_pool(4, 2, 64, pk.PA_F16, device=DEV) for _ in range(8)]
    assert all(pk.pa_check_errors(p) == 0 for p in pools)


@pytest.mark.parametrize("kv", ["i8", "i4"])
def test_quantised_write_flags_runs_that_are_not_adjacent(kv):
    pk = _pk()
    code = pk.PA_I8 if kv == "i8" else pk.PA_I4
    NB = 700
    pool = pk.new_pool(NB, 2, 64, code, device=DEV, fill=0)
    print(f"quantised runs {kv}", flush=True)

    def write(slots):
        s = torch.tensor(slots, dtype=torch.int64, device=DEV)
        r = torch.randn((len(slots), 2, 64), dtype=torch.float32, device=DEV)
        pk.pa_write_kv(pool, r, r, s)
        return pk.pa_check_errors(pool)

    # Adjacent runs, one per block (a skipped row between two runs of one
    # block is a different matter: rows 0 and 2 below are not adjacent).
    assert write([5 * 16, 5 * 16 + 1, 7 * 16, -1, 9 * 16 + 3]) == 0
    assert write([5 * 16 + 2, 7 * 16 + 1, 5 * 16 + 3]) == pk.PA_DEV_BAD_RUN
    assert write([5 * 16 + 4, -1, 5 * 16 + 5]) == pk.PA_DEV_BAD_RUN
    # Duplicate slots inside one run.
    assert write([11 * 16, 11 * 16]) == pk.PA_DEV_BAD_RUN
    # Many runs: the scan over the rows before a run leader in its unrolled
    # steps. 600 rows into 600 distinct blocks are clean; a 601st row back in
    # block 3 is flagged.
    rows = [b * 16 for b in range(600)]
    assert write(rows) == 0
    assert write(rows + [3 * 16 + 5]) == pk.PA_DEV_BAD_RUN
    assert write([3 * 16 + 6] + rows[4:]) == 0
