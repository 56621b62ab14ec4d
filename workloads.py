"""Seeded synthetic inputs for paged decode attention.

This module is shared by the oracle side and the HIP side of every test and of
the benchmark. It holds only shapes, seeds and random draws: no attention,
paging, quantisation or block-management arithmetic lives here.

Every random value is drawn from a named substream so that each side can ask
for exactly the same tensor again:

* ``numpy.random.default_rng([seed, *stream])`` on the host (small cases, and
  anything the oracle must see in full);
* ``torch.Generator`` seeded with a 63-bit key derived from ``(seed, *stream)``
  on a device (large cases: the draws happen where the data will live, and the
  oracle receives a host copy of the rows it checks).

Value distribution: i.i.d. N(0, 1) drawn in float32 and rounded to nearest
even into the storage dtype, as the workloads on the pages state for K, V and
q ("K/V ~N(0,1)").

Workload shapes follow the five paged-decode cases: a tiny fp32 case, an
OPT-13B-shaped single layer (40 heads x 128 = hidden 5120, the model whose
per-token KV size the study note "PagedAttention — 把 KV cache 当虚拟内存页来管理"
works out in 实践案例 / 案例 1), a shared-prefix parallel-sampling batch, a
long-context split-K case and an int8 sliding-window ring.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BLOCK_SIZE = 16

# Named substreams (second element of the numpy seed sequence).
STREAM_CTX = 1
STREAM_POOL = 2       # initial free-list order of the block pool
STREAM_Q = 3
STREAM_K = 4
STREAM_V = 5
STREAM_KNEW = 6
STREAM_VNEW = 7
STREAM_POISON = 8
STREAM_PERM = 9       # extra physical relabelling used by invariance tests


def rng(seed: int, *stream: int) -> np.random.Generator:
    """A numpy generator for substream ``(seed, *stream)``."""
    return np.random.default_rng([int(seed)] + [int(x) for x in stream])


def torch_key(seed: int, *stream: int) -> int:
    """A 63-bit torch seed derived from ``(seed, *stream)`` (SHA-256 of the ids)."""
    h = hashlib.sha256(repr((int(seed),) + tuple(int(x) for x in stream)).encode())
    return int.from_bytes(h.digest()[:8], "little") & ((1 << 63) - 1)


def normal_np(shape, seed: int, *stream: int, dtype=np.float32) -> np.ndarray:
    """N(0,1) drawn in float32 on the host, rounded to ``dtype``."""
    x = rng(seed, *stream).standard_normal(size=shape, dtype=np.float32)
    return x.astype(dtype, copy=False)


def normal_torch(shape, seed: int, *stream: int, dtype=None, device="cpu"):
    """N(0,1) drawn in float32 by torch on ``device``, rounded to ``dtype``.

    On the CPU this delegates to :func:`normal_np` so host-only callers get the
    numpy stream; on a GPU the draw happens in device memory.
    """
    import torch

    dtype = dtype or torch.float32
    dev = torch.device(device)
    if dev.type == "cpu":
        np_dtype = {torch.float32: np.float32, torch.float16: np.float16}[dtype]
        return torch.from_numpy(normal_np(shape, seed, *stream, dtype=np_dtype))
    g = torch.Generator(device=dev)
    g.manual_seed(torch_key(seed, *stream))
    x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
    return x.to(dtype)


def free_order(seed: int, num_blocks: int) -> np.ndarray:
    """Initial order of the free list: a seeded permutation of the pool."""
    return rng(seed, STREAM_POOL).permutation(num_blocks).astype(np.int32)


def relabel(seed: int, num_blocks: int) -> np.ndarray:
    """A second, independent permutation of physical block ids."""
    return rng(seed, STREAM_PERM).permutation(num_blocks).astype(np.int32)


@dataclass
class Workload:
    """Shapes of one paged-decode workload (everything but the values)."""

    name: str
    seed: int
    num_heads: int
    head_dim: int
    kv_dtype: str            # "f32" | "f16" | "i8"
    q_dtype: str             # "f32" | "f16"
    context_lens: list       # tokens attended per sequence in the timed step
    num_blocks: int          # size of the physical pool
    block_size: int = BLOCK_SIZE
    partition_tokens: int = 0          # 0 = single pass
    prompts: int = 0                   # shared-prefix: number of prompts
    samples: int = 0                   # shared-prefix: samples per prompt
    prompt_tokens: int = 0
    private_tokens: int = 0
    window_blocks: int = 0             # ring size (0 = unbounded)
    generated_tokens: int = 0          # ring: tokens appended before the step
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "f16": 2, "i8": 1}[self.kv_dtype]


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tiny(seed: int = 1) -> Workload:
    """4 sequences, contexts {17, 33, 50, 100}, 8 heads x 64, fp32, pool of 64 blocks."""
    return Workload("tiny", seed, 8, 64, "f32", "f32", [17, 33, 50, 100], 64,
                    notes="fp32 q/K/V; one query per sequence")


def opt13b(seed: int = 2, num_seqs: int = 64, lo: int = 128, hi: int = 2048) -> Workload:
    """OPT-13B-shaped layer: contexts ~ U{lo..hi}, 40 heads x 128, fp16, pool 1.25x need."""
    ctx = rng(seed, STREAM_CTX).integers(lo, hi + 1, size=num_seqs).tolist()
    need = sum(_ceil_div(c, BLOCK_SIZE) for c in ctx)
    return Workload("opt13b", seed, 40, 128, "f16", "f16", ctx, _ceil_div(5 * need, 4),
                    notes="prefill ctx-1 tokens, then write the new token and decode")


def shared_prefix(seed: int = 3, prompts: int = 8, samples: int = 4,
                  prompt_tokens: int = 1024, private_tokens: int = 256,
                  heads: int = 40, head_dim: int = 128) -> Workload:
    """Parallel sampling: each prompt's blocks are shared by its samples (ref count = samples)."""
    ctx = [prompt_tokens + private_tokens] * (prompts * samples)
    need = prompts * _ceil_div(prompt_tokens, BLOCK_SIZE) \
        + prompts * samples * (_ceil_div(prompt_tokens + private_tokens, BLOCK_SIZE)
                               - prompt_tokens // BLOCK_SIZE)
    pool = _ceil_div(5 * need, 4)
    return Workload("shared_prefix", seed, heads, head_dim, "f16", "f16", ctx, pool,
                    prompts=prompts, samples=samples, prompt_tokens=prompt_tokens,
                    private_tokens=private_tokens)


def long_context(seed: int = 4, num_seqs: int = 4, ctx: int = 131072, heads: int = 32,
                 head_dim: int = 128, partition_tokens: int = 512) -> Workload:
    """Long contexts decoded by split-K partitions plus a reduce kernel."""
    need = num_seqs * _ceil_div(ctx, BLOCK_SIZE)
    return Workload("long_context", seed, heads, head_dim, "f16", "f16", [ctx] * num_seqs,
                    _ceil_div(5 * need, 4), partition_tokens=partition_tokens)


def int8_ring(seed: int = 5, num_seqs: int = 128, window_blocks: int = 256,
              generated_tokens: int = 8192, heads: int = 32, head_dim: int = 128) -> Workload:
    """Sliding-window ring of int8 KV with one fp16 scale per (block, head).

    ``generated_tokens`` counts every token appended, the timed one included.
    ``context_lens`` holds the nominal window (``window_blocks`` full blocks);
    how many tokens are live at the timed step is the block manager's answer.
    """
    need = num_seqs * window_blocks
    return Workload("int8_ring", seed, heads, head_dim, "i8", "f16",
                    [window_blocks * BLOCK_SIZE] * num_seqs,
                    _ceil_div(5 * need, 4), window_blocks=window_blocks,
                    generated_tokens=generated_tokens)


FULL = {
    "tiny": tiny,
    "opt13b": opt13b,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
    "int8_ring": int8_ring,
}
