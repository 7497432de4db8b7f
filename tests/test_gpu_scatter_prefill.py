"""GPU parity of kv_scatter_prefill (post-prefill scatter) through the C ABI.

The pools after the scatter are bit-identical to the oracle's (integer work)
for prompt lengths around block edges, zero and full-width prompts, block
sizes with and without whole 8-slot groups, both head dims, an invalid
block id and a prompt wider than the group. A scatter followed by a decode
step (the fused call) matches the oracle's scatter, append and attention.
The quantizing scatter into E4M3 pools is bit-identical to the oracle's the
same way, and a scatter then a fused E4M3 step matches the oracle.
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

    pa.lib()
    return pa


def say(*a):
    print("[gpu]", *a, flush=True)


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def same(a, b):
    return np.array_equal(np.asarray(a).view(np.uint16), np.asarray(b).view(np.uint16))


PROMPTS = [0, 1, 7, 8, 15, 16, 17, 63, 64, 65, 100, 129, 300]


@pytest.mark.parametrize("bs", [12, 16, 64, 128])
@pytest.mark.parametrize("D", [64, 128])
def test_scatter_prefill_bit_exact(torch, pa, oracle, bs, D):
    Hkv = 2
    S = max(PROMPTS)
    N = sum(wl.blocks_for(P, bs) for P in PROMPTS) + 7
    w = wl.make_workload("prefill", len(PROMPTS), 4, Hkv, D, bs, N, PROMPTS, seed=200 + bs + D, events=20)
    ld = w.layer(0)
    rng = np.random.default_rng(bs * D)
    k_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    v_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    tables = w.tables.copy()
    lens = w.seq_lens.copy()
    tables[9, 0] = N + 3  # an entry outside the pool: that block's tokens are skipped
    lens[3] = S + 1  # wider than the group: the row is skipped
    say("scatter prefill", "bs", bs, "D", D, "rows", w.B, "S", S)
    tk, tv = dev(torch, ld.k_pool), dev(torch, ld.v_pool)
    pa.kv_scatter_prefill(dev(torch, k_src), dev(torch, v_src), tk, tv, dev(torch, tables), dev(torch, lens), bs)
    torch.cuda.synchronize()
    ek, ev = ld.k_pool.copy(), ld.v_pool.copy()
    assert oracle.kv_scatter_prefill(k_src, v_src, ek, ev, tables, lens, bs) == -2
    assert same(host(tk), ek) and same(host(tv), ev)


def test_scatter_then_decode_step(torch, pa, oracle):
    # Qwen shape: the group's prompts scattered, then one fused append + decode
    # at lengths prompt + 1 (the first generated token goes into its slot).
    bs, Hq, Hkv, D = 64, 12, 2, 128
    rng = np.random.default_rng(5)
    prompts = [int(x) for x in rng.integers(16, 1500, size=12)]
    prompts[0] = 64  # the next token opens a fresh block
    lens = [P + 1 for P in prompts]
    S = max(prompts)
    N = sum(wl.blocks_for(L, bs) for L in lens) + 8
    w = wl.make_workload("prefill step", len(lens), Hq, Hkv, D, bs, N, lens, seed=6, events=30)
    ld = w.layer(0)
    k_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    v_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    plen = np.asarray(prompts, np.int32)
    say("scatter then decode", "rows", w.B, "S", S)
    tk, tv = dev(torch, ld.k_pool), dev(torch, ld.v_pool)
    tt, tl = dev(torch, w.tables), dev(torch, w.seq_lens)
    pa.kv_scatter_prefill(dev(torch, k_src), dev(torch, v_src), tk, tv, tt, dev(torch, plen), bs)
    out = pa.paged_decode_attn_append(dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new), tk, tv, tt, tl,
                                      bs, w.scale)
    torch.cuda.synchronize()
    ek, ev = ld.k_pool.copy(), ld.v_pool.copy()
    assert oracle.kv_scatter_prefill(k_src, v_src, ek, ev, w.tables, plen, bs) == 0
    assert oracle.kv_append(ld.k_new, ld.v_new, ek, ev, w.tables, w.seq_lens, bs) == 0
    assert same(host(tk), ek) and same(host(tv), ev)
    ref, _ = oracle.paged_decode_attn(ld.q, ek, ev, w.tables, w.seq_lens, bs, w.scale, nthreads=NTHREADS)
    got = host(out).astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any()
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"max abs err {err.max():.3e}"


@pytest.mark.parametrize("bs", [16, 64, 128])
@pytest.mark.parametrize("D", [64, 128])
def test_scatter_prefill_fp8_bit_exact(torch, pa, oracle, bs, D):
    Hkv = 2
    S = max(PROMPTS)
    N = sum(wl.blocks_for(P, bs) for P in PROMPTS) + 7
    w = wl.make_workload("prefill fp8", len(PROMPTS), 4, Hkv, D, bs, N, PROMPTS, seed=700 + bs + D, events=20)
    rng = np.random.default_rng(bs + D)
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs))
    k_src = (wl.normal_f16(rng, (w.B, Hkv, S, D)).astype(np.float32) * 20).astype(np.float16)  # some saturate
    v_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    tables = w.tables.copy()
    lens = w.seq_lens.copy()
    tables[9, 0] = N + 3  # an entry outside the pool: that block's tokens are skipped
    lens[3] = S + 1  # wider than the group: the row is skipped
    ks, vs = 0.07, 0.4
    say("scatter prefill fp8", "bs", bs, "D", D)
    tk, tv = dev(torch, kp), dev(torch, vp)
    pa.kv_scatter_prefill_fp8(dev(torch, k_src), dev(torch, v_src), tk, tv, dev(torch, tables), dev(torch, lens), bs,
                              ks, vs)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_scatter_prefill_fp8(k_src, v_src, ek, ev, tables, lens, bs, ks, vs) == -2
    assert np.array_equal(host(tk), ek) and np.array_equal(host(tv), ev)


def test_scatter_fp8_then_fused_step(torch, pa, oracle):
    bs, Hq, Hkv, D = 64, 12, 2, 128
    rng = np.random.default_rng(8)
    prompts = [int(x) for x in rng.integers(16, 1500, size=12)]
    prompts[0] = 128  # the next token opens a fresh 128-token tile
    lens = [P + 1 for P in prompts]
    S = max(prompts)
    N = sum(wl.blocks_for(L, bs) for L in lens) + 8
    w = wl.make_workload("prefill step fp8", len(lens), Hq, Hkv, D, bs, N, lens, seed=9, events=30)
    ld = w.layer(0)
    kp = np.zeros(wl.k_pool_shape_fp8(N, Hkv, D, bs), np.uint8)
    vp = np.zeros(wl.v_pool_shape(N, Hkv, D, bs), np.uint8)
    k_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    v_src = wl.normal_f16(rng, (w.B, Hkv, S, D))
    plen = np.asarray(prompts, np.int32)
    ks, vs = 0.03, 0.05
    say("scatter fp8 then fused step", "rows", w.B)
    tk, tv = dev(torch, kp), dev(torch, vp)
    tt, tl = dev(torch, w.tables), dev(torch, w.seq_lens)
    pa.kv_scatter_prefill_fp8(dev(torch, k_src), dev(torch, v_src), tk, tv, tt, dev(torch, plen), bs, ks, vs)
    out = pa.paged_decode_attn_append_fp8(dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new), tk, tv, tt,
                                          tl, bs, w.scale, ks, vs)
    torch.cuda.synchronize()
    assert oracle.kv_scatter_prefill_fp8(k_src, v_src, kp, vp, w.tables, plen, bs, ks, vs) == 0
    assert oracle.kv_append_fp8(ld.k_new, ld.v_new, kp, vp, w.tables, w.seq_lens, bs, ks, vs) == 0
    assert np.array_equal(host(tk), kp) and np.array_equal(host(tv), vp)
    ref, _ = oracle.paged_decode_attn_fp8(ld.q, kp, vp, w.tables, w.seq_lens, bs, w.scale, ks, vs,
                                          nthreads=NTHREADS)
    got = host(out).astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any()
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"max abs err {err.max():.3e}"

