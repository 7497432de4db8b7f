"""Input generator and host block pool: page arithmetic, free-list
invariants, and the structure of every workload."""

import json
import os

import numpy as np
import pytest

import workloads as wl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")))


def test_blocks_needed_matches_pages():
    for e in GOLDEN["blocks_needed"]:
        assert wl.blocks_for(e["tokens"], e["block_size"]) == e["blocks"], e["cite"]


def test_whole_block_sharing_matches_pages():
    # Blocks are shared whole or not at all: a prefix shares its full blocks.
    for e in GOLDEN["shared_prefix_tokens"]:
        pool = wl.BlockPool(256)
        nshared = e["prefix"] // e["block_size"]
        shared = pool.alloc(nshared)
        pool.share(shared, 1)
        assert nshared * e["block_size"] == e["shared"], e["cite"]
        assert all(pool.refcount[b] == 2 for b in shared)


def test_internal_fragmentation_bound():
    e = GOLDEN["max_empty_slots_per_sequence"][0]
    bs = e["block_size"]
    worst = max(wl.blocks_for(L, bs) * bs - L for L in range(1, 5000))
    assert worst == e["slots"], e["cite"]


def test_table_bytes_match_pages():
    for e in GOLDEN["block_table_bytes"]:
        entries = wl.blocks_for(e["context_tokens"], e["block_size"])
        assert entries == e["entries_per_row"]
        assert e["rows"] * entries * 4 == e["bytes"], e["cite"]


def test_kv_bytes_per_token_match_pages():
    e = GOLDEN["kv_bytes"]
    per_tok_layer = e["kv_heads"] * e["head_dim"] * e["dtype_bytes"] * 2
    assert per_tok_layer == e["bytes_per_token_per_layer"]
    block_bytes = e["block_size"] * e["layers"] * per_tok_layer
    assert e["pool_bytes"] // block_bytes == e["pool_blocks"], e["cite"]
    waste = e["round_up_tokens"] * e["layers"] * per_tok_layer
    assert abs(waste - e["round_up_bytes_about"]) < 0.05e6
    # The workload's own byte count uses the same per-token figure.
    w = wl.uniform(L=1024)
    assert w.kv_bytes_per_layer() == 32 * 1024 * per_tok_layer


def test_pool_lifo_and_refcounts():
    pool = wl.BlockPool(8, np.arange(8))
    a = pool.alloc(3)
    assert a == [0, 1, 2]
    pool.release(a)
    # LIFO: the last block pushed is the next popped
    assert pool.alloc(1) == [2]
    with pytest.raises(ValueError):
        pool.release([5])  # never allocated
    s = pool.alloc(2)
    pool.share(s, 2)
    pool.release(s)
    pool.release(s)
    assert all(pool.refcount[b] == 1 for b in s)
    pool.release(s)
    assert all(pool.refcount[b] == 0 for b in s)
    with pytest.raises(ValueError):
        pool.release(s)
    with pytest.raises(wl.PoolExhausted):
        pool.alloc(100)


def test_churn_preserves_the_pool():
    rng = np.random.default_rng(0)
    pool = wl.BlockPool(500, rng.permutation(500))
    wl.churn(pool, 2000, rng)
    assert sorted(pool.free) == list(range(500))
    assert np.all(pool.refcount == 0)


@pytest.mark.parametrize("name", ["tiny", "uniform1024", "uniform4096", "mixed", "high_occupancy", "full_step"])
def test_configs_are_valid(name, oracle):
    w = wl.CONFIGS[name]()
    assert w.tables.shape == (w.B, w.W)
    assert w.seq_lens.shape == (w.B,)
    assert oracle.validate(w.tables, w.seq_lens, w.bs, w.N, check_append=w.append) == 0
    for b in range(w.B):
        n = wl.blocks_for(int(w.seq_lens[b]), w.bs)
        assert np.all(w.tables[b, n:] == -1)
        assert np.all(w.tables[b, :n] >= 0)
    # every physical block is held by at most one row, except shared prefix blocks
    held = w.tables[w.tables >= 0]
    ids, counts = np.unique(held, return_counts=True)
    multi = set(ids[counts > 1].tolist())
    assert multi <= set(w.shared_blocks)


def test_config_shapes():
    t = wl.tiny()
    assert (t.B, t.Hq, t.Hkv, t.D, t.bs, t.N, t.W) == (4, 2, 1, 64, 16, 32, 5)
    assert t.seq_lens.tolist() == [5, 16, 33, 70]
    assert t.scale == 0.125
    m = wl.mixed()
    assert (m.B, m.Hq, m.Hkv, m.D, m.bs, m.W) == (32, 12, 2, 128, 64, 68)
    assert int(np.sum(m.seq_lens == 4352)) == 1
    short = m.seq_lens[m.seq_lens != 4352]
    assert len(short) == 31 and short.min() >= 16 and short.max() <= 512
    h = wl.high_occupancy()
    assert h.B == 95 and h.bs == 16 and h.N == 16384 and h.W == 144
    assert h.seq_lens.min() >= 65 and h.seq_lens.max() <= 2304
    f = wl.full_step()
    assert f.layers == 28 and f.B == 32 and len(f.shared_blocks) == 10
    assert int(f.sharers.sum()) == 16
    assert np.all(f.seq_lens[f.sharers] >= 641)
    assert np.all((f.seq_lens >= 256) & (f.seq_lens <= 4352))
    for b in np.flatnonzero(f.sharers):
        assert f.tables[b, :10].tolist() == f.shared_blocks


def test_poison_marks_only_dead_slots():
    w = wl.tiny()
    ld = w.layer(0)
    kp, vp = ld.k_pool.copy(), ld.v_pool.copy()
    wl.poison_stale(kp, vp, w.tables, w.seq_lens, w.bs)
    for b in range(w.B):
        k, v = wl.read_row(kp, vp, w.tables[b], int(w.seq_lens[b]), w.bs)
        assert np.all(np.isfinite(k)) and np.all(np.isfinite(v))
    live = wl.live_slot_mask(w.tables, w.seq_lens, w.bs, w.N)
    assert np.isnan(kp[~live.any(axis=1)]).all()


def test_write_read_roundtrip():
    rng = np.random.default_rng(3)
    k = wl.normal_f16(rng, (100, 2, 64))
    v = wl.normal_f16(rng, (100, 2, 64))
    kp = np.zeros(wl.k_pool_shape(10, 2, 64, 16), np.float16)
    vp = np.zeros(wl.v_pool_shape(10, 2, 64, 16), np.float16)
    row = np.array([9, 3, 0, 7, 1, 5, 2], np.int32)
    wl.write_row(kp, vp, row, k, v, 16)
    k2, v2 = wl.read_row(kp, vp, row, 100, 16)
    assert np.array_equal(k, k2) and np.array_equal(v, v2)
    # channel d of token t sits at K[blk][g][d//8][t%bs][d%8] and V[blk][g][d][t%bs]
    assert kp[0, 1, 5, 32 - 32, 3] == k[32, 1, 43]
    assert vp[0, 1, 43, 0] == v[32, 1, 43]
