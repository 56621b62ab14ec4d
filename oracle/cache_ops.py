"""Oracle: writing new K/V rows into slots, copying blocks, int8 and int4 quantise-on-write.

Test infrastructure only (see the package docstring).

Pool layout used throughout: ``pool[block][head][offset][dim]``; a slot is
``block * block_size + offset`` (the lookup of "PagedAttention — 把 KV cache
当虚拟内存页来管理", 实践案例 / 案例 2). New rows are ``new[i][head][dim]``.

* :func:`write_kv` — every row ``i`` with ``slot[i] >= 0`` goes to its slot,
  rounded to nearest even into the pool dtype. Negative slots are skipped.
* :func:`copy_blocks` — copy-on-write copies whole blocks: on the same page,
  实践案例 / 案例 3 makes the copy unit one block, not the whole prompt.
* :func:`swap_blocks` — swapping moves whole blocks between the device pool
  and a host pool of the same per-block layout ("KV Cache与长上下文管理", the
  fourth point on what paging makes possible: page-by-page swap in and out).
* :func:`write_kv_int8` — FP16 -> INT8 cache compression is listed by "KV
  Cache与长上下文管理" (section 二.3 and its summary list) without a scheme. The
  scheme here is this project's reading: symmetric int8 codes in [-127, 127]
  with one fp16 scale per (block, head), separately for K and V.

  Within one call the rows that land in one (block, head) form a group:
    a     = max |x| over the group (fp32)
    s_new = fp16(a / 127)                (IEEE fp32 divide, then RNE to fp16)
    s_old = 0 if the group writes offset 0 (a block being opened), else the
            stored scale
    s     = max(s_old, s_new)
  If ``s > s_old > 0`` every row of the block that the call does not write is
  re-coded: ``q' = clamp(rne(fp32(q) * s_old / s), -127, 127)`` (fp32 product,
  IEEE fp32 divide). New rows: ``q = clamp(rne(x / s), -127, 127)`` in fp32, or
  0 when ``s == 0``. The stored scale becomes ``s``.
  Parity unpinned beyond this definition: the pages fix no int8 scheme.
* :func:`write_kv_int4` — the same page's quantisation list goes on from INT8
  to INT4 (section 二.3 names both; the summary list runs FP16 -> INT8 ->
  INT4). Same group rule with codes in [-7, 7] and ``s_new = fp16(a / 7)``.
  The codes are kept here as plain integers ``[block][head][offset][dim]``;
  :func:`pack_int4` gives the stored bytes: two codes per byte, dim 2j in the
  low nibble and dim 2j+1 in the high one, each nibble holding ``code + 8``
  (1..15; a nibble never written is 0). This layout is this project's.
  Parity unpinned beyond this definition: the pages fix no int4 scheme.
"""

from __future__ import annotations

from collections import OrderedDict

import numpy as np

F32 = np.float32


def write_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             slot_mapping, block_size: int = 16) -> None:
    """Scatter rows into float pools in place (f32 or f16 pools)."""
    for i, sl in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if sl < 0:
            continue
        b, o = int(sl) // block_size, int(sl) % block_size
        k_pool[b, :, o, :] = np.asarray(k_new[i]).astype(k_pool.dtype)
        v_pool[b, :, o, :] = np.asarray(v_new[i]).astype(v_pool.dtype)


def copy_blocks(pools, pairs) -> None:
    """``pool[dst] = pool[src]`` for every (src, dst) pair, in pair order.

    ``pools`` is a list of arrays whose first axis is the block id (K, V and,
    for int8, the two scale arrays).
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        for p in pools:
            p[dst] = p[src].copy()


def swap_blocks(device_pools, host_pools, pairs, direction: str) -> None:
    """Copy whole blocks between two pools of the same per-block layout.

    ``direction == "out"``: ``host[h] = device[d]`` for every ``(d, h)``;
    ``direction == "in"``: ``device[d] = host[h]`` for every ``(h, d)``.
    ``device_pools`` / ``host_pools`` are matching lists (K, V and, for int8,
    the two scale arrays) whose first axis is the block id.
    """
    if direction not in ("out", "in"):
        raise ValueError(direction)
    for a, b in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        for dp, hp in zip(device_pools, host_pools):
            if direction == "out":
                hp[b] = dp[a].copy()
            else:
                dp[b] = hp[a].copy()


def _quantise_group(codes: np.ndarray, scales: np.ndarray, b: int, h: int,
                    offsets: list, rows: list, block_size: int, qmax: int = 127) -> None:
    """Apply the group rule to one (block, head) of one tensor; codes lie in
    [-qmax, qmax] (127: int8, 7: int4)."""
    x = np.stack([np.asarray(r, dtype=F32) for r in rows])          # [G][D] fp32
    a = np.max(np.abs(x)) if x.size else F32(0)
    s_new = np.float16(F32(a) / F32(qmax))
    opened = 0 in offsets
    s_old = F32(0.0) if opened else F32(scales[b, h])
    s = max(F32(s_old), F32(s_new))
    if s_old > 0 and s > s_old:
        for r in range(block_size):
            if r in offsets:
                continue
            old = codes[b, h, r, :].astype(F32)
            codes[b, h, r, :] = np.clip(np.rint((old * s_old) / F32(s)), -qmax, qmax).astype(np.int8)
    for o, row in zip(offsets, x):
        if s == 0:
            codes[b, h, o, :] = 0
        else:
            codes[b, h, o, :] = np.clip(np.rint(row / F32(s)), -qmax, qmax).astype(np.int8)
    scales[b, h] = np.float16(s)


def write_kv_int8(k_codes: np.ndarray, k_scale: np.ndarray, v_codes: np.ndarray,
                  v_scale: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                  slot_mapping, block_size: int = 16, qmax: int = 127) -> None:
    """Quantise-on-write into int8 pools with per-(block, head) fp16 scales."""
    groups: "OrderedDict[int, list]" = OrderedDict()
    for i, sl in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if sl < 0:
            continue
        groups.setdefault(int(sl) // block_size, []).append((int(sl) % block_size, i))
    H = k_codes.shape[1]
    for b, members in groups.items():
        offsets = [o for o, _ in members]
        for h in range(H):
            _quantise_group(k_codes, k_scale, b, h, offsets,
                            [k_new[i][h] for _, i in members], block_size, qmax)
            _quantise_group(v_codes, v_scale, b, h, offsets,
                            [v_new[i][h] for _, i in members], block_size, qmax)


def write_kv_int4(k_codes: np.ndarray, k_scale: np.ndarray, v_codes: np.ndarray,
                  v_scale: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                  slot_mapping, block_size: int = 16) -> None:
    """Quantise-on-write into int4 pools (codes in [-7, 7], kept unpacked as
    int8 ``[block][head][offset][dim]``) with per-(block, head) fp16 scales."""
    write_kv_int8(k_codes, k_scale, v_codes, v_scale, k_new, v_new, slot_mapping, block_size, qmax=7)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Stored bytes of int4 codes ``[..., D]`` (D even): byte j of a row holds
    ``code[2j] + 8`` in its low nibble and ``code[2j+1] + 8`` in its high one."""
    c = np.asarray(codes, dtype=np.int16)
    if np.any(np.abs(c) > 7):
        raise ValueError("int4 codes lie in [-7, 7]")
    n = (c + 8).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4` for bytes it produced: ``[..., D/2]`` ->
    int8 codes ``[..., 2 * (D/2)]``. A nibble of 0 (never written) reads -8."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = (b & 0x0F).astype(np.int8) - 8
    out[..., 1::2] = (b >> 4).astype(np.int8) - 8
    return out


def kv_bytes_per_token(layers: int, hidden: int, bytes_per_value: int) -> int:
    """KV cache bytes one token keeps: 2 (K and V) x layers x hidden x bytes.

    The note's 实践案例 / 案例 1 uses this to show why the cache is large.
    """
    return 2 * layers * hidden * bytes_per_value
