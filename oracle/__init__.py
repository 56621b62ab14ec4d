"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The product path (the HIP
library and its Python binding) never calls it, and this package never imports
the product path: the two share no code. The only module both sides use is
``workloads`` (seeded random inputs, no method arithmetic).

Everything here is plain, slow and meant to be checked by eye against the pages
it cites. Floating-point results are computed in float64 (numpy); integer and
byte results (slots, tables, block copies, int8 and int4 codes) are exact.

Sources, cited by page title and section:

* "PagedAttention — 把 KV cache 当虚拟内存页来管理" (estelledc.github.io study
  note on the 2023 paper): 实践案例 / 案例 1 (KV bytes per token), 案例 2 (block
  table lookup ``locate``), 案例 3 (reference counts and copy-on-write),
  踩过的坑 (block size 16; outputs are unchanged by paging).
* "One Deep Concept #01 — PagedAttention: From Operating System Virtual Memory
  to Large Language Model Memory Systems": §2 Background (the attention
  formula), §4 Core Innovation (logical blocks -> block table -> physical
  blocks).
* "KV Cache与长上下文管理" (staroceans.org): the section on the second problem
  paging solves (round-robin sliding window in O(1): invalidate the oldest
  page, write the new token into it, update the page-table order), the third
  (fragmentation), and the quantisation list (FP16 -> INT8 -> INT4).
* "PagedAttention的终极用途" (staroceans.org video script), part 三: the same
  sliding-window-by-table-edit statement.
* "PagedAttention 的技术溯源与演进脉络" (mjmagnets.cn), §4.1 item 2: mixed-
  precision page management (FP16 hot pages, INT8 rarely used pages, host
  backup for cold pages).

Modules:

* :mod:`oracle.paging` — ``locate``, slot numbers, gather through a table.
* :mod:`oracle.attention` — softmax(q K^T / sqrt(d)) V in fp64, partition
  partials (m, l, o) and their log-sum-exp merge, and several new tokens of a
  sequence attending at once (each over the context up to itself).
* :mod:`oracle.cache_ops` — scatter of new K/V rows into slots, block copy, and
  the int8 and int4 quantise-on-write rule (int4 codes and their nibble
  layout).
* :mod:`oracle.block_manager` — free list, reference counts, copy-on-write on
  append, the sliding-window ring, swapping to a host pool and prefix caching,
  as a plain Python model.
* :mod:`oracle.mixed` — mixed-precision pages: an fp16 hot tail block per
  sequence, int8 cold blocks demoted from it, and decode over both.

Parity unpinned (checked only against this oracle's own definition, because
the pages fix no value for it): the merge rule used when int8 rows are written
into a block that already holds rows (requantisation on a grown scale), and the
choice of which free block is handed out (a FIFO over a seeded permutation),
the swap and prefix-caching policies, and the hot/cold split of mixed pages.
"""

from . import attention, block_manager, cache_ops, mixed, paging  # noqa: F401
