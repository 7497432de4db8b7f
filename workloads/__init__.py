"""Seeded synthetic inputs for paged decode attention.

This module is the only code that both the CPU oracle's tests and the HIP
path's tests/bench share. It builds inputs and nothing else: the host block
pool that hands out physical block ids (free list, reference counts), the
per-row block tables, and fp16 values drawn from a seeded normal
distribution. It holds none of the attention arithmetic.

Sources (page title, section):
  [Paged attention]     danielfleming.xyz/writing/inference/paged
  [PagedAttention]      deepconcepts.dev/c/llm-paged-attention
  [SLM paged attention] aicassindra.com/blogs/slm/slm_paged_attention.html

Pool layout (shared with every reader of the pool):
  K: [N][Hkv][D/8][bs][8]   -- 16-byte groups of 8 channels, token-minor
  V: [N][Hkv][D][bs]        -- channel-major, tokens contiguous
FP8 pools hold one byte per element (E4M3 codes):
  K: [N][Hkv][D/16][bs][16] -- 16-byte groups of 16 channels
  V: [N][Hkv][D][bs]
"""

from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional

import numpy as np


# ----------------------------------------------------------------------------
# Host block pool: the control plane the kernel's inputs come from.
# ----------------------------------------------------------------------------


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    """LIFO free list of physical block ids with per-block reference counts.

    Allocation pops from the top of the free list and freeing pushes back,
    both O(1) with no compaction [SLM paged attention, "The architecture:
    every piece explained"]; eviction only edits the free list [Paged
    attention, "What changed"]. A block shared by several tables carries a
    reference count and returns to the list only when the last holder frees
    it [SLM paged attention, "End-to-end flow"].
    """

    def __init__(self, num_blocks: int, initial_order: Optional[np.ndarray] = None):
        self.num_blocks = int(num_blocks)
        order = np.arange(num_blocks) if initial_order is None else np.asarray(initial_order)
        if sorted(order.tolist()) != list(range(num_blocks)):
            raise ValueError("initial free-list order must be a permutation of [0, N)")
        # the last element is the top of the stack
        self.free: List[int] = [int(x) for x in order[::-1]]
        self.refcount = np.zeros(num_blocks, np.int64)

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self, k: int) -> List[int]:
        if k > len(self.free):
            raise PoolExhausted(f"need {k} blocks, {len(self.free)} free")
        out = [self.free.pop() for _ in range(k)]
        for b in out:
            assert self.refcount[b] == 0, "allocated a block that is still referenced"
            self.refcount[b] = 1
        return out

    def share(self, blocks: List[int], extra_refs: int = 1) -> None:
        for b in blocks:
            if self.refcount[b] <= 0:
                raise ValueError(f"cannot share free block {b}")
            self.refcount[b] += extra_refs

    def release(self, blocks: List[int]) -> None:
        """Drop one reference from each block, in table order; a block whose
        count reaches zero is pushed back on the free list."""
        for b in blocks:
            if self.refcount[b] <= 0:
                raise ValueError(f"double free of block {b}")
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(int(b))


def churn(pool: BlockPool, events: int, rng: np.random.Generator, max_alloc: int = 16) -> None:
    """Run `events` seeded alloc/free events against the pool, then free every
    survivor oldest-first, so the free list ends up shuffled the way a
    serving history leaves it. Each event allocates k ~ U{1..max_alloc} blocks
    to a new owner with probability 1/2 (always, if no owner is live and k
    fits), otherwise frees a uniformly chosen live owner."""
    owners: List[List[int]] = []
    for _ in range(events):
        k = int(rng.integers(1, max_alloc + 1))
        do_alloc = (not owners) or (rng.random() < 0.5)
        if do_alloc and k <= pool.num_free():
            owners.append(pool.alloc(k))
        elif owners:
            i = int(rng.integers(0, len(owners)))
            pool.release(owners.pop(i))
    for blocks in owners:
        pool.release(blocks)


def blocks_for(length: int, block_size: int) -> int:
    """Blocks a sequence of `length` tokens occupies: whole blocks only."""
    return -(-int(length) // int(block_size))


def build_tables(
    pool: BlockPool,
    seq_lens: np.ndarray,
    block_size: int,
    width: int,
    shared_prefix_blocks: Optional[List[int]] = None,
    sharers: Optional[np.ndarray] = None,
) -> np.ndarray:
    """Block tables for rows whose lengths count the token being appended.

    Phase 1: each row, in row order, pops the blocks holding positions
    0 .. L-2 (sharers start from the shared prefix blocks). Phase 2: a row
    whose new position L-1 starts a block pops one fresh block and appends
    it [SLM paged attention, "End-to-end flow"]. Entries past a row's last
    block are -1.
    """
    B = len(seq_lens)
    tables = np.full((B, width), -1, np.int32)
    held: List[List[int]] = []
    for b in range(B):
        L = int(seq_lens[b])
        before = blocks_for(max(L - 1, 0), block_size)
        row: List[int] = []
        if sharers is not None and sharers[b]:
            row = list(shared_prefix_blocks)
        need = before - len(row)
        if need < 0:
            raise ValueError("a sharer must extend past the shared prefix")
        row += pool.alloc(need)
        held.append(row)
    for b in range(B):
        L = int(seq_lens[b])
        if L >= 1 and (L - 1) % block_size == 0:
            held[b] += pool.alloc(1)
    for b in range(B):
        row = held[b]
        if len(row) > width:
            raise ValueError("row needs more blocks than the table width")
        tables[b, : len(row)] = row
    return tables


# ----------------------------------------------------------------------------
# Values
# ----------------------------------------------------------------------------


def k_pool_shape(N, Hkv, D, bs):
    return (N, Hkv, D // 8, bs, 8)


def v_pool_shape(N, Hkv, D, bs):
    return (N, Hkv, D, bs)


def k_pool_shape_fp8(N, Hkv, D, bs):
    return (N, Hkv, D // 16, bs, 16)


def fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Random E4M3 bit patterns (uint8): a random sign bit, an exponent field
    drawn from a rounded normal around 6.5 (magnitudes mostly 2^-3 .. 2^2)
    and clipped to 0..14, and a uniform 3-bit mantissa. The NaN pattern
    (exponent 15, mantissa 7) never occurs. Bits only: no conversion."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    e = np.clip(np.rint(rng.normal(6.5, 1.5, size=shape)), 0, 14).astype(np.uint8)
    m = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign | (e << 3) | m).astype(np.uint8)


def normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws in float32 rounded to fp16 (round to nearest even)."""
    return rng.standard_normal(size=shape, dtype=np.float32).astype(np.float16)


def live_slot_mask(tables, seq_lens, bs, N) -> np.ndarray:
    """[N][bs] bool: True where a slot holds a token some row reads."""
    live = np.zeros((N, bs), bool)
    for b in range(tables.shape[0]):
        L = int(seq_lens[b])
        for j in range(blocks_for(L, bs)):
            n = min(bs, L - j * bs)
            live[tables[b, j], :n] = True
    return live


def poison_stale(k_pool, v_pool, tables, seq_lens, bs, value=np.nan) -> None:
    """Overwrite every pool slot no row reads (tails of last blocks, blocks no
    table lists) with `value`; the result must not depend on them."""
    N = k_pool.shape[0]
    dead = ~live_slot_mask(tables, seq_lens, bs, N)
    kd = np.broadcast_to(dead[:, None, None, :, None], k_pool.shape)
    vd = np.broadcast_to(dead[:, None, None, :], v_pool.shape)
    k_pool[kd] = value
    v_pool[vd] = value


def write_row(k_pool, v_pool, table_row, k_log, v_log, bs) -> None:
    """Store a row's logical K/V ([L][Hkv][D]) into the physical blocks its
    table lists (position t -> block table_row[t // bs], slot t % bs)."""
    L, Hkv, D = k_log.shape
    grp = k_pool.shape[-1]  # channels per 16-byte group: 8 (fp16) or 16 (fp8)
    for j in range(blocks_for(L, bs)):
        blk = int(table_row[j])
        lo, hi = j * bs, min(L, (j + 1) * bs)
        n = hi - lo
        kk = k_log[lo:hi].reshape(n, Hkv, D // grp, grp).transpose(1, 2, 0, 3)
        vv = v_log[lo:hi].transpose(1, 2, 0)
        k_pool[blk, :, :, :n, :] = kk
        v_pool[blk, :, :, :n] = vv


def read_row(k_pool, v_pool, table_row, L, bs):
    """Inverse of write_row: the row's logical [L][Hkv][D] K and V."""
    N, Hkv, ngrp, _, grp = k_pool.shape
    D = ngrp * grp
    k = np.empty((L, Hkv, D), k_pool.dtype)
    v = np.empty((L, Hkv, D), v_pool.dtype)
    for j in range(blocks_for(L, bs)):
        blk = int(table_row[j])
        lo, hi = j * bs, min(L, (j + 1) * bs)
        n = hi - lo
        k[lo:hi] = k_pool[blk, :, :, :n, :].transpose(2, 0, 1, 3).reshape(n, Hkv, D)
        v[lo:hi] = v_pool[blk, :, :, :n].transpose(2, 0, 1)
    return k, v


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class LayerData:
    q: np.ndarray        # [B][Hq][D] fp16
    k_new: np.ndarray    # [B][Hkv][D] fp16
    v_new: np.ndarray    # [B][Hkv][D] fp16
    k_pool: np.ndarray   # [N][Hkv][D/8][bs][8] fp16
    v_pool: np.ndarray   # [N][Hkv][D][bs] fp16


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    W: int
    N: int
    layers: int
    seq_lens: np.ndarray     # [B] int32, lengths after this step's append
    tables: np.ndarray       # [B][W] int32, -1 past each row's last block
    append: bool             # whether the step runs kv_append before attention
    seed: int
    scale: float
    shared_blocks: List[int] = dataclasses.field(default_factory=list)
    sharers: Optional[np.ndarray] = None
    _layer_fn: Optional[Callable[[int], LayerData]] = None

    def layer(self, i: int = 0) -> LayerData:
        return self._layer_fn(i)

    def kv_bytes_per_layer(self) -> int:
        """K+V bytes of every row at its own length (fp16)."""
        return int(np.sum(self.seq_lens.astype(np.int64))) * self.Hkv * self.D * 2 * 2

    def unique_kv_bytes_per_layer(self) -> int:
        """As kv_bytes_per_layer, but slots read by several rows count once."""
        live = live_slot_mask(self.tables, self.seq_lens, self.bs, self.N)
        return int(live.sum()) * self.Hkv * self.D * 2 * 2


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def _values(seed, B, Hq, Hkv, D, bs, N):
    def fn(layer: int) -> LayerData:
        rng = np.random.default_rng(seed + 1000 * layer)
        q = normal_f16(rng, (B, Hq, D))
        k_new = normal_f16(rng, (B, Hkv, D))
        v_new = normal_f16(rng, (B, Hkv, D))
        k_pool = normal_f16(rng, k_pool_shape(N, Hkv, D, bs))
        v_pool = normal_f16(rng, v_pool_shape(N, Hkv, D, bs))
        return LayerData(q, k_new, v_new, k_pool, v_pool)

    return fn


def make_workload(
    name, B, Hq, Hkv, D, bs, N, seq_lens, seed, *, layers=1, events=0, append=True, W=None,
    shared_prefix_tokens=0, sharers=None, max_alloc=16,
) -> Workload:
    seq_lens = np.asarray(seq_lens, np.int32)
    rng = np.random.default_rng(seed)
    pool = BlockPool(N, rng.permutation(N))
    churn(pool, events, rng, max_alloc=max_alloc)
    shared = []
    if shared_prefix_tokens:
        nshared = shared_prefix_tokens // bs
        shared = pool.alloc(nshared)
        pool.share(shared, int(np.sum(sharers)) - 1)
    if W is None:
        W = max(1, max(blocks_for(L, bs) for L in seq_lens))
    tables = build_tables(pool, seq_lens, bs, W, shared, sharers)
    return Workload(
        name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, W=W, N=N, layers=layers, seq_lens=seq_lens,
        tables=tables, append=append, seed=seed, scale=_scale(D), shared_blocks=shared,
        sharers=None if sharers is None else np.asarray(sharers, bool),
        _layer_fn=_values(seed, B, Hq, Hkv, D, bs, N),
    )


def tiny() -> Workload:
    """Batch 4, one layer, 2 query heads / 1 KV head, head_dim 64, block 16,
    lengths {5, 16, 33, 70}, a 32-block pool in seeded random order, one
    kv_append per row."""
    return make_workload("tiny", 4, 2, 1, 64, 16, 32, [5, 16, 33, 70], seed=1, W=5)


def uniform(L=1024, B=32, N=None, seed=2) -> Workload:
    """Qwen2.5-1.5B attention shape (12 query heads, 2 KV heads, head_dim 128),
    block 64, every row at length L, blocks from a shuffled pool."""
    N = N or max(1024, B * blocks_for(L, 64))
    return make_workload(f"uniform{L}", B, 12, 2, 128, 64, N, [L] * B, seed=seed, append=False)


def uniform4096() -> Workload:
    return uniform(L=4096, N=4096, seed=6)


def mixed() -> Workload:
    """The ragged batch: 31 rows at U{16..512} and one 4352-token row (4096
    prompt + 256 budget) at a seeded index; free list shuffled by 200
    alloc/free events."""
    rng = np.random.default_rng(3)
    lens = rng.integers(16, 513, size=32)
    lens[int(rng.integers(0, 32))] = 4352
    return make_workload("mixed", 32, 12, 2, 128, 64, 1024, lens, seed=3, events=200, append=False, W=68)


def high_occupancy() -> Workload:
    """95 resident sequences, block 16, prompt U{64..2048} + generated
    U{1..256}, a 16384-block pool fragmented by 2000 events; one append and
    one decode step."""
    rng = np.random.default_rng(4)
    lens = rng.integers(64, 2049, size=95) + rng.integers(1, 257, size=95)
    return make_workload("high_occupancy", 95, 12, 2, 128, 16, 16384, lens, seed=4, events=2000, W=144)


def full_step(layers=28, N=2048) -> Workload:
    """A 28-layer decode step: batch 32, lengths U{256..4352}; 16 seeded rows
    share one 640-token prefix through the same 10 physical blocks and hold
    private blocks after it; kv_append then attention in every layer. Tables
    are the same in every layer (a block spans all layers); values are drawn
    per layer."""
    rng = np.random.default_rng(5)
    sharers = np.zeros(32, bool)
    sharers[rng.choice(32, size=16, replace=False)] = True
    lens = np.where(sharers, rng.integers(641, 4353, size=32), rng.integers(256, 4353, size=32))
    return make_workload(
        "full_step", 32, 12, 2, 128, 64, N, lens, seed=5, layers=layers, events=200, W=68,
        shared_prefix_tokens=640, sharers=sharers,
    )


CONFIGS = {
    "tiny": tiny,
    "uniform1024": uniform,
    "uniform4096": uniform4096,
    "mixed": mixed,
    "high_occupancy": high_occupancy,
    "full_step": full_step,
}


def dominant_key(bands, L=16384, seed=41, Hq=12, Hkv=2, D=128, bs=64) -> Workload:
    """Rows whose scores have one dominant key and a long tail a set gap
    below it: row i has length L (the last row L//4 + 1, a ragged length),
    query heads all (a, 0, ..., 0), and K channel 0 chosen so that
    scale * q . k_t = s_top - gap_t, the gaps drawn uniformly from
    bands[i] = (lo, hi) in natural-log units, the dominant key at a seeded
    position. Other K channels, V, and stale slots are N(0,1)."""
    B = len(bands)
    lens = [L] * (B - 1) + [L // 4 + 1]
    N = sum(blocks_for(n, bs) for n in lens) + 4
    w = make_workload("dominant_key", B, Hq, Hkv, D, bs, N, lens, seed, events=10)
    base = w._layer_fn
    a = np.float16(8.0)  # query channel 0
    unit = float(np.float32(w.scale)) * float(a)  # score per unit of K channel 0
    s_top = 32.0

    def fn(layer: int) -> LayerData:
        ld = base(layer)
        rng = np.random.default_rng(seed + 7 + 1000 * layer)
        ld.q[:] = 0
        ld.q[:, :, 0] = a
        for b, (lo, hi) in enumerate(bands):
            n = int(lens[b])
            k_log, v_log = read_row(ld.k_pool, ld.v_pool, w.tables[b], n, bs)
            gaps = rng.uniform(lo, hi, size=(n, Hkv))
            gaps[int(rng.integers(0, n))] = 0.0
            k_log[:, :, 0] = ((s_top - gaps) / unit).astype(np.float16)
            write_row(ld.k_pool, ld.v_pool, w.tables[b], k_log, v_log, bs)
        return ld

    w._layer_fn = fn
    w.name = "dominant_key"
    return w
