"""GPU parity of kv_copy_blocks (copy-on-write) through the C ABI.

* the pools after the copy are bit-identical to the oracle's block copy
  (integer work), for one layer and for pools with a leading layer dimension;
* pairs naming blocks outside the pool, and a block copied onto itself, are
  skipped as the oracle skips them;
* a decode step whose rows append into a block they share: the host plan
  (paged_kv_cache_06_amd.blocks), the device copies, then the step (fused or
  as two calls) leave the pools bit-identical to the oracle's copy and append,
  and the output within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the oracle's
  attention over the repointed tables;
* the same over E4M3 (FP8) pools: kv_copy_blocks_fp8 bit-identical to the
  oracle's byte copy (one layer and layered pools), and a copy-on-write step
  through the fused E4M3 launch.
"""

import os

import numpy as np
import pytest

import workloads as wl
from paged_kv_cache_06_amd import blocks

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


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_copy_blocks_bit_exact(torch, pa, oracle, bs, D):
    Hkv, N = 2, 96
    rng = np.random.default_rng(100 + bs + D)
    kp = wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))
    vp = wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))
    perm = rng.permutation(N)
    src = np.concatenate([perm[:30], [N, 5, -1]]).astype(np.int32)
    dst = np.concatenate([perm[30:60], [perm[60], 5, perm[61]]]).astype(np.int32)
    say("copy blocks", "bs", bs, "D", D, "pairs", src.size)
    tk, tv = dev(torch, kp), dev(torch, vp)
    pa.kv_copy_blocks(tk, tv, dev(torch, src), dev(torch, dst), bs)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_copy_blocks(ek, ev, src, dst) == -2  # the out-of-range pairs are reported and skipped
    assert same(host(tk), ek) and same(host(tv), ev)


def test_copy_blocks_every_layer(torch, pa, oracle):
    layers, N, Hkv, D, bs = 3, 48, 2, 128, 64
    rng = np.random.default_rng(7)
    kp = np.stack([wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs)) for _ in range(layers)])
    vp = np.stack([wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs)) for _ in range(layers)])
    perm = rng.permutation(N)
    src, dst = perm[:10].astype(np.int32), perm[10:20].astype(np.int32)
    say("copy blocks over", layers, "layers")
    tk, tv = dev(torch, kp), dev(torch, vp)
    pa.kv_copy_blocks(tk, tv, dev(torch, src), dev(torch, dst), bs)
    torch.cuda.synchronize()
    gk, gv = host(tk), host(tv)
    for layer in range(layers):
        ek, ev = kp[layer].copy(), vp[layer].copy()
        assert oracle.kv_copy_blocks(ek, ev, src, dst) == 0
        assert same(gk[layer], ek) and same(gv[layer], ev), f"layer {layer}"


def _cow_case(bs, prefix, writers, other_lens, seed):
    """Rows 0..writers-1 share a prefix whose last block is partly filled and
    each appends into it; the other rows own their blocks."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 12, 2, 128
    lens = [prefix + 1] * writers + list(other_lens)
    B = len(lens)
    N = sum(-(-L // bs) for L in lens) + 16
    order = [int(x) for x in rng.permutation(N)]
    nshared = -(-prefix // bs)
    shared = [order.pop() for _ in range(nshared)]
    W = max(-(-L // bs) for L in lens)
    tables = np.full((B, W), -1, np.int32)
    for b in range(writers):
        tables[b, :nshared] = shared
    for b in range(writers, B):
        for j in range(-(-lens[b] // bs)):
            tables[b, j] = order.pop()
    lens = np.asarray(lens, np.int32)
    q = wl.normal_f16(rng, (B, Hq, D))
    kn = wl.normal_f16(rng, (B, Hkv, D))
    vn = wl.normal_f16(rng, (B, Hkv, D))
    kp = wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))
    vp = wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))
    return tables, lens, N, order, q, kn, vn, kp, vp, float(np.float32(1.0 / np.sqrt(D)))


@pytest.mark.parametrize("bs,prefix", [(16, 40), (64, 100)])
@pytest.mark.parametrize("fused", [True, False])
def test_copy_on_write_then_decode_step(torch, pa, oracle, bs, prefix, fused):
    tables, lens, N, free, q, kn, vn, kp, vp, scale = _cow_case(bs, prefix, 4, [300, 1, 64, 129], seed=bs + prefix)
    rc = blocks.refcounts(tables, lens, bs, N)
    src, dst = blocks.plan_copy_on_write(tables, lens, bs, rc, free)  # tables repointed in place
    assert src.size == 3
    say("copy-on-write step", "bs", bs, "prefix", prefix, "fused", fused, "copies", src.size)
    tk, tv = dev(torch, kp), dev(torch, vp)
    tt, tl = dev(torch, tables), dev(torch, lens)
    pa.kv_copy_blocks(tk, tv, dev(torch, src), dev(torch, dst), bs)
    if fused:
        out = pa.paged_decode_attn_append(dev(torch, q), dev(torch, kn), dev(torch, vn), tk, tv, tt, tl, bs, scale)
    else:
        pa.kv_append(dev(torch, kn), dev(torch, vn), tk, tv, tt, tl, bs)
        out = pa.paged_decode_attn(dev(torch, q), tk, tv, tt, tl, bs, scale)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_copy_blocks(ek, ev, src, dst) == 0
    assert oracle.kv_append(kn, vn, ek, ev, tables, lens, bs) == 0
    assert same(host(tk), ek) and same(host(tv), ev)
    ref, _ = oracle.paged_decode_attn(q, ek, ev, tables, lens, bs, scale, nthreads=NTHREADS)
    got = host(out).astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any()
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"max abs err {err.max():.3e}"


@pytest.mark.parametrize("bs", [16, 64])
def test_copy_blocks_fp8_bit_exact(torch, pa, oracle, bs):
    Hkv, D, N = 2, 128, 80
    rng = np.random.default_rng(300 + bs)
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs))
    perm = rng.permutation(N)
    src = np.concatenate([perm[:25], [N, 7]]).astype(np.int32)
    dst = np.concatenate([perm[25:50], [perm[50], 7]]).astype(np.int32)
    say("copy blocks fp8", "bs", bs, "pairs", src.size)
    tk, tv = dev(torch, kp), dev(torch, vp)
    pa.kv_copy_blocks_fp8(tk, tv, dev(torch, src), dev(torch, dst), bs)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_copy_blocks_fp8(ek, ev, src, dst) == -2
    assert np.array_equal(host(tk), ek) and np.array_equal(host(tv), ev)
    # layered pools: every layer copied
    layers = 3
    kl = np.stack([wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs)) for _ in range(layers)])
    vl = np.stack([wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs)) for _ in range(layers)])
    s2, d2 = perm[:10].astype(np.int32), perm[10:20].astype(np.int32)
    tk, tv = dev(torch, kl), dev(torch, vl)
    pa.kv_copy_blocks_fp8(tk, tv, dev(torch, s2), dev(torch, d2), bs)
    torch.cuda.synchronize()
    gk, gv = host(tk), host(tv)
    for layer in range(layers):
        ek, ev = kl[layer].copy(), vl[layer].copy()
        assert oracle.kv_copy_blocks_fp8(ek, ev, s2, d2) == 0
        assert np.array_equal(gk[layer], ek) and np.array_equal(gv[layer], ev), f"layer {layer}"


def test_copy_on_write_then_fused_fp8_step(torch, pa, oracle):
    bs, prefix = 64, 100
    tables, lens, N, free, q, kn, vn, _, _, scale = _cow_case(bs, prefix, 4, [300, 1, 64, 129], seed=31)
    rng = np.random.default_rng(32)
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, 2, 128, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, 2, 128, bs))
    rc = blocks.refcounts(tables, lens, bs, N)
    src, dst = blocks.plan_copy_on_write(tables, lens, bs, rc, free)
    assert src.size == 3
    ks, vs = 0.125, 0.375
    say("copy-on-write fp8 step", "copies", src.size)
    tk, tv = dev(torch, kp), dev(torch, vp)
    tt, tl = dev(torch, tables), dev(torch, lens)
    pa.kv_copy_blocks_fp8(tk, tv, dev(torch, src), dev(torch, dst), bs)
    out = pa.paged_decode_attn_append_fp8(dev(torch, q), dev(torch, kn), dev(torch, vn), tk, tv, tt, tl, bs, scale,
                                          ks, vs)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_copy_blocks_fp8(ek, ev, src, dst) == 0
    assert oracle.kv_append_fp8(kn, vn, ek, ev, tables, lens, bs, ks, vs) == 0
    assert np.array_equal(host(tk), ek) and np.array_equal(host(tv), ev)
    ref, _ = oracle.paged_decode_attn_fp8(q, ek, ev, tables, lens, bs, scale, ks, vs, nthreads=NTHREADS)
    got = host(out).astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any()
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"max abs err {err.max():.3e}"

