"""Host-side block bookkeeping for copy-on-write.

Rows may reference the same physical block (a shared prompt prefix). Before a
decode step appends, a row whose new token falls in a block that other rows
still reference must get a private copy of that block: a fresh block is taken
from the free list, the shared block is cloned into it on the device
(``kv_copy_blocks``), and only the writer's table entry is repointed, so the
readers keep seeing the old block [SLM paged attention, "The architecture:
every piece explained" and "End-to-end flow"; PagedAttention, "Sharing is the
part that pays twice"]. Reference counts follow the table entries.

This module only decides which blocks to copy; it moves no data.
"""

from __future__ import annotations

import numpy as np


class OutOfBlocks(RuntimeError):
    """The free list ran out while planning copies (the caller must free or
    preempt rows first)."""


def refcounts(block_tables, seq_lens, block_size, num_blocks):
    """Reference count of every physical block: the number of (row, logical
    block) table entries within the rows' lengths that point at it."""
    tables = np.asarray(block_tables)
    counts = np.zeros(num_blocks, np.int32)
    for b, L in enumerate(np.asarray(seq_lens)):
        n = -(-int(L) // block_size) if L > 0 else 0
        for j in range(min(n, tables.shape[1])):
            blk = int(tables[b, j])
            if 0 <= blk < num_blocks:
                counts[blk] += 1
    return counts


def plan_copy_on_write(block_tables, seq_lens, block_size, refcount, free_blocks):
    """Plan the block copies that make every row's append target private.

    For each row b in order with L = seq_lens[b] >= 1, the new token goes to
    logical block (L-1) // block_size. If that block's reference count is
    above one, a block is popped from ``free_blocks`` (used as a stack), the
    pair (shared, fresh) is recorded, the row's table entry is repointed to
    the fresh block and one reference moves from the shared block to it. The
    last row still pointing at a block keeps it (its count is then one).

    block_tables [B][W] int32 and refcount [N] int32 are updated in place;
    free_blocks is a list of free block ids (popped from its end).
    Returns (src, dst) int32 arrays for kv_copy_blocks, to be run before the
    append of this step.
    """
    tables = block_tables
    src, dst = [], []
    W = tables.shape[1]
    N = refcount.shape[0]
    for b, L in enumerate(np.asarray(seq_lens)):
        L = int(L)
        if L < 1:
            continue
        j = (L - 1) // block_size
        if j >= W:
            continue
        blk = int(tables[b, j])
        if not (0 <= blk < N) or refcount[blk] <= 1:
            continue
        if not free_blocks:
            raise OutOfBlocks(f"no free block to copy block {blk} for row {b}")
        fresh = int(free_blocks.pop())
        src.append(blk)
        dst.append(fresh)
        tables[b, j] = fresh
        refcount[blk] -= 1
        refcount[fresh] = 1
    return np.asarray(src, np.int32), np.asarray(dst, np.int32)
