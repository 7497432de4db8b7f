"""GPU parity on pools larger than 4 GiB (64-bit block addressing).

Each pool, K and V alike, holds more than 2^32 bytes; half the rows' blocks
are drawn from the pool's last eighth (past byte offset 4 GiB), half from
below it. The pools are
filled with NaN (fp16 0x7e00, E4M3 0x7f) and the blocks in use written from
host data; then a prompt scatter, a fused append + decode step and a block
copy run on them, for fp16 and for E4M3 pools. The oracle runs on a compact
pool holding the same blocks renumbered 0..n-1 (the attention does not depend
on which physical ids a row's blocks have, a pinned property of the oracle):

* the blocks in use read back bit-identical to the oracle's (integer work);
* the attention output within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the oracle.
"""

import os

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2
NTHREADS = min(16, os.cpu_count() or 1)
POOL_BYTES = 5 << 30  # per pool: past 4 GiB
BS, HQ, HKV, D = 64, 12, 2, 128
LENS = [1024, 4352, 1, 0, 65, 64, 300, 2000]  # after this step's append


@pytest.fixture(scope="module")
def torch():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return torch


@pytest.fixture(scope="module")
def pa(torch):
    import paged_kv_cache_06_amd as pa

    pa.lib()
    return pa


def say(*a):
    print("[gpu]", *a, flush=True)


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case(seed, n_big):
    """Compact tables over n blocks (the last one spare, for the copy) and
    the physical id of every compact block in the big pool."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(LENS, np.int32)
    B, W = lens.size, max(wl.blocks_for(L, BS) for L in LENS)
    tables = np.full((B, W), -1, np.int32)
    n = 0
    for b, L in enumerate(LENS):
        k = wl.blocks_for(L, BS)
        tables[b, :k] = np.arange(n, n + k)
        n += k
    n += 1  # the copy's destination
    tail = n_big - n_big // 8  # half the blocks in the pool's last eighth, half below it
    ids = np.concatenate([tail + rng.choice(n_big - tail, size=n // 2, replace=False),
                          rng.choice(tail, size=n - n // 2, replace=False)]).astype(np.int64)
    rng.shuffle(ids)
    big_tables = np.where(tables >= 0, ids[np.maximum(tables, 0)], -1).astype(np.int32)
    prompts = np.maximum(lens - 1, 0).astype(np.int32)
    S = int(prompts.max())
    q = wl.normal_f16(rng, (B, HQ, D))
    kn = wl.normal_f16(rng, (B, HKV, D))
    vn = wl.normal_f16(rng, (B, HKV, D))
    k_src = wl.normal_f16(rng, (B, HKV, S, D))
    v_src = wl.normal_f16(rng, (B, HKV, S, D))
    src_c = np.asarray([tables[1, 5]], np.int32)  # a block of the 4352-token row ...
    dst_c = np.asarray([n - 1], np.int32)  # ... onto the spare block
    return dict(lens=lens, tables=tables, big_tables=big_tables, ids=ids, n=n, prompts=prompts, q=q, kn=kn, vn=vn,
                k_src=k_src, v_src=v_src, src_c=src_c, dst_c=dst_c, scale=float(np.float32(1 / np.sqrt(D))))


def check_out(out, ref, what):
    got = out.astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any(), f"{what}: NaN"
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"{what}: max abs err {err.max():.3e}"


def test_fp16_pool_past_4gib(torch, pa, oracle):
    n_big = POOL_BYTES // (BS * HKV * D * 2)
    c = case(11, n_big)
    rng = np.random.default_rng(12)
    kc = wl.normal_f16(rng, wl.k_pool_shape(c["n"], HKV, D, BS))
    vc = wl.normal_f16(rng, wl.v_pool_shape(c["n"], HKV, D, BS))
    say("fp16 pools of", n_big, "blocks,", 2 * n_big * BS * HKV * D * 2 >> 20, "MiB; max id", int(c["ids"].max()))
    nan = float("nan")
    tk = torch.full(wl.k_pool_shape(n_big, HKV, D, BS), nan, dtype=torch.float16, device="cuda")
    tv = torch.full(wl.v_pool_shape(n_big, HKV, D, BS), nan, dtype=torch.float16, device="cuda")
    ids = torch.from_numpy(c["ids"]).cuda()
    tk.index_copy_(0, ids, dev(torch, kc))
    tv.index_copy_(0, ids, dev(torch, vc))
    tt, tl = dev(torch, c["big_tables"]), dev(torch, c["lens"])
    pa.kv_scatter_prefill(dev(torch, c["k_src"]), dev(torch, c["v_src"]), tk, tv, tt, dev(torch, c["prompts"]), BS)
    out = pa.paged_decode_attn_append(dev(torch, c["q"]), dev(torch, c["kn"]), dev(torch, c["vn"]), tk, tv, tt, tl,
                                      BS, c["scale"])
    pa.kv_copy_blocks(tk, tv, dev(torch, c["ids"][c["src_c"]].astype(np.int32)),
                      dev(torch, c["ids"][c["dst_c"]].astype(np.int32)), BS)
    torch.cuda.synchronize()
    gk, gv = tk.index_select(0, ids).cpu().numpy(), tv.index_select(0, ids).cpu().numpy()
    out = out.cpu().numpy()
    del tk, tv
    torch.cuda.empty_cache()
    assert oracle.kv_scatter_prefill(c["k_src"], c["v_src"], kc, vc, c["tables"], c["prompts"], BS) == 0
    assert oracle.kv_append(c["kn"], c["vn"], kc, vc, c["tables"], c["lens"], BS) == 0
    ref, _ = oracle.paged_decode_attn(c["q"], kc, vc, c["tables"], c["lens"], BS, c["scale"], nthreads=NTHREADS)
    assert oracle.kv_copy_blocks(kc, vc, c["src_c"], c["dst_c"]) == 0
    assert np.array_equal(gk.view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(gv.view(np.uint16), vc.view(np.uint16))
    check_out(out, ref, "fp16 pools past 4 GiB")
    assert np.all(out[3].view(np.uint16) == 0)  # the empty row


def test_fp8_pool_past_4gib(torch, pa, oracle):
    n_big = POOL_BYTES // (BS * HKV * D)
    c = case(13, n_big)
    rng = np.random.default_rng(14)
    kc = wl.fp8_codes(rng, wl.k_pool_shape_fp8(c["n"], HKV, D, BS))
    vc = wl.fp8_codes(rng, wl.v_pool_shape(c["n"], HKV, D, BS))
    ks, vs = 0.05, 0.03
    say("E4M3 pools of", n_big, "blocks,", 2 * n_big * BS * HKV * D >> 20, "MiB; max id", int(c["ids"].max()))
    tk = torch.full(wl.k_pool_shape_fp8(n_big, HKV, D, BS), 0x7F, dtype=torch.uint8, device="cuda")
    tv = torch.full(wl.v_pool_shape(n_big, HKV, D, BS), 0x7F, dtype=torch.uint8, device="cuda")
    ids = torch.from_numpy(c["ids"]).cuda()
    tk.index_copy_(0, ids, dev(torch, kc))
    tv.index_copy_(0, ids, dev(torch, vc))
    tt, tl = dev(torch, c["big_tables"]), dev(torch, c["lens"])
    pa.kv_scatter_prefill_fp8(dev(torch, c["k_src"]), dev(torch, c["v_src"]), tk, tv, tt, dev(torch, c["prompts"]),
                              BS, ks, vs)
    out = pa.paged_decode_attn_append_fp8(dev(torch, c["q"]), dev(torch, c["kn"]), dev(torch, c["vn"]), tk, tv, tt,
                                          tl, BS, c["scale"], ks, vs)
    pa.kv_copy_blocks_fp8(tk, tv, dev(torch, c["ids"][c["src_c"]].astype(np.int32)),
                          dev(torch, c["ids"][c["dst_c"]].astype(np.int32)), BS)
    torch.cuda.synchronize()
    gk, gv = tk.index_select(0, ids).cpu().numpy(), tv.index_select(0, ids).cpu().numpy()
    out = out.cpu().numpy()
    del tk, tv
    torch.cuda.empty_cache()
    assert oracle.kv_scatter_prefill_fp8(c["k_src"], c["v_src"], kc, vc, c["tables"], c["prompts"], BS, ks, vs) == 0
    assert oracle.kv_append_fp8(c["kn"], c["vn"], kc, vc, c["tables"], c["lens"], BS, ks, vs) == 0
    ref, _ = oracle.paged_decode_attn_fp8(c["q"], kc, vc, c["tables"], c["lens"], BS, c["scale"], ks, vs,
                                          nthreads=NTHREADS)
    assert oracle.kv_copy_blocks_fp8(kc, vc, c["src_c"], c["dst_c"]) == 0
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    check_out(out, ref, "E4M3 pools past 4 GiB")
    assert np.all(out[3].view(np.uint16) == 0)  # the empty row
