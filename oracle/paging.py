"""Oracle: logical token -> (physical block, offset) through a block table.

Test infrastructure only (see the package docstring).

The study note "PagedAttention — 把 KV cache 当虚拟内存页来管理", 实践案例 /
案例 2, defines the lookup: the logical block of token ``t`` is ``t // block_size``,
its offset inside the block is ``t % block_size``, and the physical block is the
table entry at the logical block. Its worked example uses block size 16 and the
table ``[7, 1, 3]``; token 34 lands in physical block 3 at offset 2.

"One Deep Concept #01", §4 Core Innovation, states the same mapping as logical
KV blocks -> block table -> physical GPU blocks, with the model seeing a
continuous sequence.
"""

from __future__ import annotations

import numpy as np


def locate(token_index: int, block_table, block_size: int = 16):
    """(physical block, offset) of one logical token."""
    if token_index < 0:
        raise IndexError("token index must be non-negative")
    logical = token_index // block_size
    offset = token_index % block_size
    physical = int(block_table[logical])
    return physical, int(offset)


def slot(token_index: int, block_table, block_size: int = 16) -> int:
    """Flat slot number ``physical * block_size + offset`` of one token."""
    physical, offset = locate(token_index, block_table, block_size)
    return physical * block_size + offset


def slots(num_tokens: int, block_table, block_size: int = 16, first: int = 0) -> np.ndarray:
    """Slots of logical tokens ``first .. first+num_tokens-1`` (int64)."""
    return np.array([slot(t, block_table, block_size) for t in range(first, first + num_tokens)],
                    dtype=np.int64)


def gather(pool: np.ndarray, block_table, context_len: int, block_size: int = 16,
           scale: np.ndarray | None = None) -> np.ndarray:
    """Rows of one sequence in logical order, as float64.

    ``pool`` is ``[num_blocks][heads][block_size][head_dim]``; the result is
    ``[context_len][heads][head_dim]``. With ``scale`` (``[num_blocks][heads]``)
    the stored codes are dequantised as ``code * scale`` in float64.
    """
    t = np.arange(context_len, dtype=np.int64)
    logical = t // block_size
    offset = t % block_size
    physical = np.asarray(block_table, dtype=np.int64)[logical]
    rows = pool[physical, :, offset, :].astype(np.float64)          # [T][H][D]
    if scale is not None:
        rows = rows * scale[physical, :].astype(np.float64)[:, :, None]
    return rows
