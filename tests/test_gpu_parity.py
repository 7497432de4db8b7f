"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* kv_append pools and the paged_gather_kv debug read are bit-identical to
  the oracle's (integer/byte work);
* paged_decode_attn matches the oracle's unrounded fp32 output elementwise
  within |gpu - ref| <= 2e-3 + 1e-2 |ref| (fp16 outputs, fp32 accumulation);
* results are bit-identical across reruns, across relabelling of physical
  blocks, and do not change when every dead slot is NaN;
* all six workloads at full size, every compiled (block_size, head_dim,
  group size), lengths around block and tile edges, zero-length rows, and
  rows long enough to need the split-sequence merge.
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


def upload(torch, w, ld):
    return dict(
        q=dev(torch, ld.q), k_new=dev(torch, ld.k_new), v_new=dev(torch, ld.v_new),
        k_pool=dev(torch, ld.k_pool), v_pool=dev(torch, ld.v_pool),
        tables=dev(torch, w.tables), seq_lens=dev(torch, w.seq_lens),
    )


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


def run_decode(torch, pa, w, t, ws=None):
    out = pa.paged_decode_attn(t["q"], t["k_pool"], t["v_pool"], t["tables"], t["seq_lens"], w.bs, w.scale,
                               workspace=ws)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# kv_append and gather: bit-exact
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["tiny", "mixed", "high_occupancy", "full_step"])
def test_kv_append_bit_exact(torch, pa, oracle, name):
    w = wl.CONFIGS[name]() if name != "full_step" else wl.full_step(layers=1)
    ld = w.layer(0)
    say("kv_append", name, "B", w.B, "bs", w.bs, "N", w.N)
    t = upload(torch, w, ld)
    pa.kv_append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"], t["tables"], t["seq_lens"], w.bs)
    torch.cuda.synchronize()
    kp, vp = ld.k_pool.copy(), ld.v_pool.copy()
    assert oracle.kv_append(ld.k_new, ld.v_new, kp, vp, w.tables, w.seq_lens, w.bs) == 0
    assert np.array_equal(host(t["k_pool"]).view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(host(t["v_pool"]).view(np.uint16), vp.view(np.uint16))


@pytest.mark.parametrize("name", ["tiny", "mixed", "high_occupancy"])
def test_gather_bit_exact(torch, pa, oracle, name):
    w = wl.CONFIGS[name]()
    ld = w.layer(0)
    say("gather", name)
    t = upload(torch, w, ld)
    ko, vo = pa.paged_gather_kv(t["k_pool"], t["v_pool"], t["tables"], t["seq_lens"], w.bs)
    torch.cuda.synchronize()
    rk, rv = oracle.gather_kv(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.Hkv, w.D)
    assert np.array_equal(host(ko).view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(host(vo).view(np.uint16), rv.view(np.uint16))


# ---------------------------------------------------------------------------
# decode attention on the six workloads
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["tiny", "uniform1024", "uniform4096", "mixed", "high_occupancy"])
def test_decode_workloads(torch, pa, oracle, name):
    w = wl.CONFIGS[name]()
    ld = w.layer(0)
    say("decode", name, "B", w.B, "bs", w.bs, "W", w.W, "max L", int(w.seq_lens.max()))
    t = upload(torch, w, ld)
    if w.append:
        pa.kv_append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"], t["tables"], t["seq_lens"], w.bs)
        oracle.kv_append(ld.k_new, ld.v_new, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    out = host(run_decode(torch, pa, w, t))
    ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                      nthreads=NTHREADS)
    e = assert_close(out, ref, name)
    say("decode", name, "max abs err", e)


def test_full_step_28_layers(torch, pa, oracle):
    """kv_append then paged_decode_attn in each of 28 layers; tables are
    shared by every layer, 16 rows share a 640-token prefix."""
    w = wl.full_step()
    tables = dev(torch, w.tables)
    lens = dev(torch, w.seq_lens)
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)
    worst = 0.0
    for layer in range(w.layers):
        ld = w.layer(layer)
        say("full_step layer", layer)
        kp, vp = dev(torch, ld.k_pool), dev(torch, ld.v_pool)
        q, kn, vn = dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new)
        pa.kv_append(kn, vn, kp, vp, tables, lens, w.bs)
        out = pa.paged_decode_attn(q, kp, vp, tables, lens, w.bs, w.scale, workspace=ws)
        torch.cuda.synchronize()
        oracle.kv_append(ld.k_new, ld.v_new, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
        ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                          nthreads=NTHREADS)
        worst = max(worst, assert_close(host(out), ref, f"full_step layer {layer}"))
        # the two rows of a sharing pair read the same 10 prefix blocks
        del kp, vp
    say("full_step max abs err", worst)


# ---------------------------------------------------------------------------
# invariances and robustness
# ---------------------------------------------------------------------------


def test_rerun_bit_identical_and_workspace_reuse(torch, pa):
    w = wl.mixed()
    t = upload(torch, w, w.layer(0))
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)
    say("rerun determinism, mixed")
    a = host(run_decode(torch, pa, w, t, ws))
    for _ in range(3):
        b = host(run_decode(torch, pa, w, t, ws))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_block_relabelling_bit_identical(torch, pa):
    w = wl.mixed()
    ld = w.layer(0)
    say("relabel, mixed")
    base = host(run_decode(torch, pa, w, upload(torch, w, ld)))
    pi = np.random.default_rng(7).permutation(w.N)
    kp = np.empty_like(ld.k_pool)
    vp = np.empty_like(ld.v_pool)
    kp[pi] = ld.k_pool
    vp[pi] = ld.v_pool
    tables = np.where(w.tables >= 0, pi[np.maximum(w.tables, 0)], -1).astype(np.int32)
    t = dict(q=dev(torch, ld.q), k_pool=dev(torch, kp), v_pool=dev(torch, vp), tables=dev(torch, tables),
             seq_lens=dev(torch, w.seq_lens))
    got = host(run_decode(torch, pa, w, t))
    assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


@pytest.mark.parametrize("name", ["tiny", "mixed", "high_occupancy"])
def test_nan_in_dead_slots_changes_nothing(torch, pa, name):
    w = wl.CONFIGS[name]()
    ld = w.layer(0)
    say("nan poison", name)
    base = host(run_decode(torch, pa, w, upload(torch, w, ld)))
    wl.poison_stale(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    tables = w.tables.copy()
    for b in range(w.B):  # unused table entries become garbage too
        tables[b, wl.blocks_for(int(w.seq_lens[b]), w.bs):] = -7
    t = dict(q=dev(torch, ld.q), k_pool=dev(torch, ld.k_pool), v_pool=dev(torch, ld.v_pool),
             tables=dev(torch, tables), seq_lens=dev(torch, w.seq_lens))
    got = host(run_decode(torch, pa, w, t))
    assert np.array_equal(got.view(np.uint16), base.view(np.uint16))


EDGE_LENS = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 1000, 2049]


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("heads", [(2, 1), (12, 2), (8, 8), (4, 1), (16, 2)])
@pytest.mark.parametrize("D", [64, 128])
def test_shapes_and_edge_lengths(torch, pa, oracle, bs, heads, D):
    Hq, Hkv = heads
    lens = [0] + EDGE_LENS
    N = sum(wl.blocks_for(L, bs) for L in lens) + 5
    w = wl.make_workload("edge", len(lens), Hq, Hkv, D, bs, N, lens, seed=100 + bs + D + Hq, events=10)
    ld = w.layer(0)
    say("edge", "bs", bs, "Hq/Hkv", Hq, Hkv, "D", D)
    wl.poison_stale(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    t = upload(torch, w, ld)
    pa.kv_append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"], t["tables"], t["seq_lens"], w.bs)
    oracle.kv_append(ld.k_new, ld.v_new, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    out = host(run_decode(torch, pa, w, t))
    ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                      nthreads=NTHREADS)
    assert np.all(out[0].view(np.uint16) == 0)  # zero-length row
    assert_close(out, ref, f"edge bs={bs} heads={heads} D={D}")


def test_one_very_long_row_uses_many_partitions(torch, pa, oracle):
    # A single 16384-token row: far more tiles than one workgroup takes, so
    # the split-sequence merge runs with many partitions.
    w = wl.make_workload("long", 1, 12, 2, 128, 64, 300, [16384], seed=9, events=30)
    ld = w.layer(0)
    say("long row 16384")
    out = host(run_decode(torch, pa, w, upload(torch, w, ld)))
    ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                      nthreads=NTHREADS)
    assert_close(out, ref, "long row")


def _check_lengths(torch, pa, oracle, lens, bs=64, heads=(12, 2), D=128, seed=11, label=""):
    Hq, Hkv = heads
    N = sum(wl.blocks_for(L, bs) for L in lens) + 8
    w = wl.make_workload(label or "lens", len(lens), Hq, Hkv, D, bs, N, lens, seed=seed, events=20)
    ld = w.layer(0)
    wl.poison_stale(ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs)
    out = host(run_decode(torch, pa, w, upload(torch, w, ld)))
    ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                      nthreads=NTHREADS)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b].view(np.uint16) == 0), f"row {b} has length 0 but a nonzero output"
    return assert_close(out, ref, label)


def test_more_rows_than_one_launch_takes(torch, pa, oracle):
    # 1100 short rows (zero-length ones among them): the host runs the kernel
    # over several row ranges, each with its own slice of every buffer.
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(0, 300, size=1100)]
    lens[0] = lens[517] = lens[1099] = 0
    say("1100 rows")
    _check_lengths(torch, pa, oracle, lens, bs=16, label="1100 rows")


def test_long_rows_share_workgroups_at_the_split_bound(torch, pa, oracle):
    # A table 300 tiles wide: partials per (row, KV head) reach the bound of
    # 64, and long and short rows share workgroup ranges.
    lens = [19200, 1, 4097, 0, 63, 19135]
    say("rows of 19200 tokens")
    _check_lengths(torch, pa, oracle, lens, bs=64, label="split bound")


def test_all_rows_empty(torch, pa, oracle):
    say("all rows empty")
    _check_lengths(torch, pa, oracle, [0, 0, 0, 0, 0], bs=16, heads=(8, 8), D=64, label="empty rows")


def test_one_workspace_for_different_batches(torch, pa, oracle):
    # Arrival counters come back to zero after every call, so one workspace
    # serves batches of different shapes in any order.
    wa = wl.CONFIGS["mixed"]()
    wb = wl.make_workload("other", 7, 12, 2, 128, 64, 200, [5000, 3, 700, 0, 64, 1300, 4097], seed=12, events=10)
    ws = pa.new_workspace(max(wa.B, wb.B), 12, 2, 128, 64, max(wa.W, wb.W))
    res = {}
    for name, w in [("a", wa), ("b", wb), ("a2", wa), ("b2", wb)]:
        ld = w.layer(0)
        res[name] = host(run_decode(torch, pa, w, upload(torch, w, ld), ws=ws))
        say("shared workspace", name)
    for a, b in [("a", "a2"), ("b", "b2")]:
        assert np.array_equal(res[a].view(np.uint16), res[b].view(np.uint16))
    ld = wb.layer(0)
    ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, wb.tables, wb.seq_lens, wb.bs, wb.scale,
                                      nthreads=NTHREADS)
    assert_close(res["b"], ref, "shared workspace")


def test_unsupported_shape_raises(torch, pa):
    q = torch.zeros(2, 12, 128, dtype=torch.float16, device="cuda")
    k = torch.zeros(8, 2, 16, 8, 8, dtype=torch.float16, device="cuda")
    v = torch.zeros(8, 2, 128, 8, dtype=torch.float16, device="cuda")
    t = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    s = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_decode_attn(q, k, v, t, s, 8, 0.1)
    assert e.value.status == 2


def test_workspace_sized_for_long_rows_serves_a_wider_batch(torch, pa, oracle):
    # A workspace sized for 32 rows of a 300-block table (bs 64) also covers a
    # 256-row batch of 4-block tables by size. The counters sit in a region
    # of their own, so the first call's partials cannot land on the second
    # call's counters: both calls, and the first one again, match the oracle.
    ws = pa.new_workspace(32, 12, 2, 128, 64, 300)
    assert pa.paged_decode_workspace_size(256, 12, 2, 128, 64, 4) <= ws.numel()
    rng = np.random.default_rng(31)
    long_lens = [int(x) for x in rng.integers(8000, 19200, size=32)]
    wa = wl.make_workload("long32", 32, 12, 2, 128, 64, sum(wl.blocks_for(L, 64) for L in long_lens) + 8,
                          long_lens, seed=32, events=10)
    wide_lens = [int(x) for x in rng.integers(1, 257, size=256)]
    wb = wl.make_workload("wide256", 256, 12, 2, 128, 64, sum(wl.blocks_for(L, 64) for L in wide_lens) + 8,
                          wide_lens, seed=33, events=10)
    assert wa.W >= 126 and wb.W <= 4
    for name, w in [("long rows", wa), ("wide batch", wb), ("long rows again", wa)]:
        ld = w.layer(0)
        say("workspace reuse", name)
        out = host(run_decode(torch, pa, w, upload(torch, w, ld), ws=ws))
        ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                          nthreads=NTHREADS)
        assert_close(out, ref, f"workspace reuse: {name}")


def test_one_workspace_for_relabelled_blocks_and_other_lengths(torch, pa, oracle):
    # One workspace across calls of the same shapes: the mixed batch, the same
    # lengths with every block relabelled (pools permuted to match), a
    # different length mix, then the first call again. Every output matches
    # the oracle, and the relabelled and repeated calls are bit-identical to
    # the first.
    wa = wl.CONFIGS["mixed"]()
    lda = wa.layer(0)
    perm = np.random.default_rng(61).permutation(wa.N).astype(np.int32)
    tables_b = np.where(wa.tables >= 0, perm[np.maximum(wa.tables, 0)], -1).astype(np.int32)
    kb = np.empty_like(lda.k_pool)
    vb = np.empty_like(lda.v_pool)
    kb[perm] = lda.k_pool
    vb[perm] = lda.v_pool
    wc = wl.make_workload("other_mix", wa.B, 12, 2, 128, 64, wa.N, np.roll(wa.seq_lens, 5), seed=62, events=30,
                          W=wa.W)
    ldc = wc.layer(0)
    ws = pa.new_workspace(wa.B, 12, 2, 128, 64, wa.W)
    cases = [("first", wa.tables, lda.q, lda.k_pool, lda.v_pool, wa.seq_lens),
             ("relabelled", tables_b, lda.q, kb, vb, wa.seq_lens),
             ("other lengths", wc.tables, ldc.q, ldc.k_pool, ldc.v_pool, wc.seq_lens),
             ("first again", wa.tables, lda.q, lda.k_pool, lda.v_pool, wa.seq_lens)]
    outs = {}
    for name, tables, q, kp, vp, lens in cases:
        say("workspace reuse:", name)
        out = pa.paged_decode_attn(dev(torch, q), dev(torch, kp), dev(torch, vp), dev(torch, tables),
                                   dev(torch, lens), 64, wa.scale, workspace=ws)
        torch.cuda.synchronize()
        outs[name] = host(out)
        ref, _ = oracle.paged_decode_attn(q, kp, vp, tables, lens, 64, wa.scale, nthreads=NTHREADS)
        assert_close(outs[name], ref, f"workspace reuse: {name}")
    assert np.array_equal(outs["first"].view(np.uint16), outs["first again"].view(np.uint16))
    assert np.array_equal(outs["first"].view(np.uint16), outs["relabelled"].view(np.uint16))
