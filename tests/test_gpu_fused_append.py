"""GPU parity of paged_decode_attn_append (kv_append and paged_decode_attn in
one launch) through the C ABI.

For every case the fused call must leave the pools bit-identical to the
oracle's kv_append, produce an output bit-identical to the two separate GPU
calls (kv_append, then paged_decode_attn) and within |gpu - ref| <= 2e-3 +
1e-2 |ref| of the oracle's decode after its append. The new token's slot is
poisoned with NaN before the call, so a result that read the pool's old bits
for that token instead of k_new / v_new fails.
"""

import os

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2
NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return torch


@pytest.fixture(scope="module")
def pa(torch):
    import paged_kv_cache_06_amd as pa

    pa.lib()  # raises if the library was not built
    return pa


def say(*a):
    print("[gpu]", *a, flush=True)


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def assert_close(got, ref, what):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not np.any(np.isnan(got)), f"{what}: NaN in output"
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} elements out of tolerance, max abs err {err.max():.3e} "
        f"at {np.unravel_index(err.argmax(), err.shape)}"
    )
    return float(err.max())


def poison_new_slots(k_pool, v_pool, tables, seq_lens, bs):
    """NaN in every appending row's slot L-1 (the bits kv_append overwrites)."""
    W = tables.shape[1]
    D = v_pool.shape[2]
    for b, L in enumerate(seq_lens):
        L = int(L)
        if L < 1 or L > W * bs:
            continue
        blk = int(tables[b, (L - 1) // bs])
        if 0 <= blk < k_pool.shape[0]:
            k_pool[blk, :, :, (L - 1) % bs, :] = np.nan
            v_pool[blk, :, :D, (L - 1) % bs] = np.nan


def check_fused(torch, pa, oracle, w, ld, label, oracle_rows=None):
    """Run the fused call and the two-call path on copies of the same inputs
    and compare both with each other and with the oracle."""
    poison_new_slots(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    tables, lens = dev(torch, w.tables), dev(torch, w.seq_lens)
    q, kn, vn = dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new)
    kp1, vp1 = dev(torch, ld.k_pool), dev(torch, ld.v_pool)
    kp2, vp2 = dev(torch, ld.k_pool), dev(torch, ld.v_pool)
    fused = pa.paged_decode_attn_append(q, kn, vn, kp1, vp1, tables, lens, w.bs, w.scale)
    pa.kv_append(kn, vn, kp2, vp2, tables, lens, w.bs)
    two = pa.paged_decode_attn(q, kp2, vp2, tables, lens, w.bs, w.scale)
    torch.cuda.synchronize()
    fused, two = host(fused), host(two)
    kp, vp = ld.k_pool.copy(), ld.v_pool.copy()
    oracle.kv_append(ld.k_new, ld.v_new, kp, vp, w.tables, w.seq_lens, w.bs)
    assert np.array_equal(host(kp1).view(np.uint16), kp.view(np.uint16)), f"{label}: K pool"
    assert np.array_equal(host(vp1).view(np.uint16), vp.view(np.uint16)), f"{label}: V pool"
    assert np.array_equal(host(kp2).view(np.uint16), kp.view(np.uint16)), f"{label}: K pool, two calls"
    assert np.array_equal(fused.view(np.uint16), two.view(np.uint16)), f"{label}: fused vs two calls"
    rows = np.arange(w.B) if oracle_rows is None else np.asarray(oracle_rows)
    lens_o = np.zeros_like(w.seq_lens)
    lens_o[rows] = w.seq_lens[rows]
    ref, _ = oracle.paged_decode_attn(ld.q, kp, vp, w.tables, lens_o, w.bs, w.scale, nthreads=NTHREADS)
    return assert_close(fused[rows], ref[rows], label)


@pytest.mark.parametrize("name", ["tiny", "uniform1024", "mixed", "high_occupancy", "full_step"])
def test_fused_workloads(torch, pa, oracle, name):
    w = wl.CONFIGS[name]() if name != "full_step" else wl.full_step(layers=1)
    ld = w.layer(0)
    say("fused append+decode", name, "B", w.B, "bs", w.bs)
    e = check_fused(torch, pa, oracle, w, ld, name)
    say("fused", name, "max abs err", e)


EDGE_LENS = [0, 1, 2, 15, 16, 17, 33, 63, 64, 65, 127, 128, 129, 257, 1000, 2049]


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("heads", [(2, 1), (12, 2)])
@pytest.mark.parametrize("D", [64, 128])
def test_fused_edge_lengths(torch, pa, oracle, bs, heads, D):
    Hq, Hkv = heads
    N = sum(wl.blocks_for(L, bs) for L in EDGE_LENS) + 5
    w = wl.make_workload("edge", len(EDGE_LENS), Hq, Hkv, D, bs, N, EDGE_LENS, seed=300 + bs + D + Hq, events=10)
    ld = w.layer(0)
    wl.poison_stale(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    say("fused edge", "bs", bs, "Hq/Hkv", Hq, Hkv, "D", D)
    check_fused(torch, pa, oracle, w, ld, f"fused edge bs={bs} heads={heads} D={D}")


def test_fused_long_rows_split_over_workgroups(torch, pa, oracle):
    # the new token sits in a (row, KV head) whose tiles several workgroups share
    lens = [19200, 1, 4097, 0, 63, 19135]
    N = sum(wl.blocks_for(L, 64) for L in lens) + 8
    w = wl.make_workload("fused long", len(lens), 12, 2, 128, 64, N, lens, seed=31, events=20)
    ld = w.layer(0)
    say("fused long rows")
    check_fused(torch, pa, oracle, w, ld, "fused long rows")


def test_fused_row_past_the_table_is_not_appended(torch, pa, oracle):
    # a length beyond W*block_size: kv_append skips the row and the decode
    # clamps it, in both paths alike; the oracle checks the other rows
    lens = [70, 200, 5]
    w = wl.make_workload("past table", len(lens), 12, 2, 128, 16, 40, lens, seed=32, events=5)
    w.seq_lens[1] = w.W * w.bs + 3
    ld = w.layer(0)
    say("fused, a row past its table")
    check_fused(torch, pa, oracle, w, ld, "row past table", oracle_rows=[0, 2])


def test_fused_rerun_bit_identical(torch, pa):
    w = wl.mixed()
    ld = w.layer(0)
    say("fused rerun determinism, mixed")
    tables, lens = dev(torch, w.tables), dev(torch, w.seq_lens)
    q, kn, vn = dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new)
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)
    outs = []
    for _ in range(3):
        kp, vp = dev(torch, ld.k_pool), dev(torch, ld.v_pool)
        outs.append(host(pa.paged_decode_attn_append(q, kn, vn, kp, vp, tables, lens, w.bs, w.scale, workspace=ws)))
    for o in outs[1:]:
        assert np.array_equal(outs[0].view(np.uint16), o.view(np.uint16))
