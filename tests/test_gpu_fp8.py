"""GPU parity of the E4M3 (FP8) pool path through the C ABI.

* kv_append_fp8 leaves the pools bit-identical to the oracle's quantizing
  append (integer work): every fp16 bit pattern once (NaN, infinities,
  subnormals, values past 448 * scale, exact ties), and ordinary steps at
  several block sizes, head dims and scales;
* paged_decode_attn_fp8 matches the oracle's attention over the dequantized
  pools within |gpu - ref| <= 2e-3 + 1e-2 |ref| (the fp16 path's bound: codes
  are widened to fp16 exactly and the arithmetic after that is the fp16
  path's, with the two scales folded in), for every compiled (block size,
  head dim, group size), lengths around block and tile edges, zero-length
  rows, NaN codes in every dead slot, and rows split over many partitions;
* an append followed by a decode step on the Qwen2.5-1.5B batch shape;
* the fused step (paged_decode_attn_append_fp8) leaves the pools
  bit-identical to the oracle's append and its output bit-identical to the
  two calls', for new tokens at every position of a 128-token tile's edges.
"""

import os

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2
NTHREADS = min(16, os.cpu_count() or 1)
NAN_CODE = 0x7F


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


def assert_close(got, ref, what):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} out of tolerance, max abs err {err.max():.3e}"


def fp8_case(seed, lens, Hq, Hkv, D, bs, extra_blocks=5):
    rng = np.random.default_rng(seed)
    N = sum(wl.blocks_for(L, bs) for L in lens) + extra_blocks
    w = wl.make_workload("fp8", len(lens), Hq, Hkv, D, bs, N, lens, seed=seed, events=10)
    q = wl.normal_f16(rng, (w.B, Hq, D))
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(N, Hkv, D, bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(N, Hkv, D, bs))
    return w, rng, q, kp, vp


def test_append_fp8_every_half_pattern(torch, pa, oracle):
    # 256 rows x 2 KV heads x 128 channels: K takes every fp16 bit pattern
    # once, V a permutation of them
    B, Hkv, D, bs = 256, 2, 128, 16
    lens = [int(x) for x in np.random.default_rng(1).integers(1, 200, size=B)]
    w, rng, _, kp, vp = fp8_case(90, lens, 2, Hkv, D, bs)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    kn = allbits.reshape(B, Hkv, D).view(np.float16)
    vn = rng.permutation(allbits).reshape(B, Hkv, D).view(np.float16)
    for ks, vs in [(1.0, 1.0), (0.0371, 3.5), (2.0 ** -90, 3.1e25), (float.fromhex("0x1.fffffep95"), 1.7e-27)]:
        say("append fp8, every half pattern, scales", ks, vs)
        tk, tv = dev(torch, kp), dev(torch, vp)
        pa.kv_append_fp8(dev(torch, kn), dev(torch, vn), tk, tv, dev(torch, w.tables), dev(torch, w.seq_lens), bs,
                         ks, vs)
        torch.cuda.synchronize()
        ek, ev = kp.copy(), vp.copy()
        assert oracle.kv_append_fp8(kn, vn, ek, ev, w.tables, w.seq_lens, bs, ks, vs) == 0
        assert np.array_equal(host(tk), ek) and np.array_equal(host(tv), ev)


@pytest.mark.parametrize("bs", [16, 64, 256])
@pytest.mark.parametrize("D", [64, 128])
def test_append_fp8_step(torch, pa, oracle, bs, D):
    lens = [1, 15, 16, 17, 64, 65, 255, 256, 257, 1000]
    w, rng, _, kp, vp = fp8_case(91 + bs + D, lens, 4, 2, D, bs)
    kn = (wl.normal_f16(rng, (w.B, 2, D)).astype(np.float32) * 40).astype(np.float16)  # some saturate
    vn = (wl.normal_f16(rng, (w.B, 2, D)).astype(np.float32) * 1e-3).astype(np.float16)  # many subnormal codes
    seq = w.seq_lens.copy()
    seq[3] = 0  # skipped
    say("append fp8 step", "bs", bs, "D", D)
    tk, tv = dev(torch, kp), dev(torch, vp)
    pa.kv_append_fp8(dev(torch, kn), dev(torch, vn), tk, tv, dev(torch, w.tables), dev(torch, seq), bs, 0.05, 2.0 ** -12)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_append_fp8(kn, vn, ek, ev, w.tables, seq, bs, 0.05, 2.0 ** -12) == 0
    assert np.array_equal(host(tk), ek) and np.array_equal(host(tv), ev)


EDGE_LENS = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 1000, 2049]


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("heads", [(2, 1), (12, 2), (8, 8), (4, 1), (16, 2)])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_fp8_shapes_and_edge_lengths(torch, pa, oracle, bs, heads, D):
    Hq, Hkv = heads
    lens = [0] + EDGE_LENS
    w, rng, q, kp, vp = fp8_case(300 + bs + D + Hq, lens, Hq, Hkv, D, bs)
    wl.poison_stale(kp, vp, w.tables, w.seq_lens, bs, value=NAN_CODE)
    ks, vs = 0.3125, 0.37
    say("decode fp8", "bs", bs, "Hq/Hkv", Hq, Hkv, "D", D)
    out = pa.paged_decode_attn_fp8(dev(torch, q), dev(torch, kp), dev(torch, vp), dev(torch, w.tables),
                                   dev(torch, w.seq_lens), bs, w.scale, ks, vs)
    torch.cuda.synchronize()
    got = host(out)
    ref, _ = oracle.paged_decode_attn_fp8(q, kp, vp, w.tables, w.seq_lens, bs, w.scale, ks, vs, nthreads=NTHREADS)
    assert np.all(got[0].view(np.uint16) == 0)  # the zero-length row
    assert_close(got, ref, f"fp8 bs={bs} heads={heads} D={D}")


def test_decode_fp8_long_rows_split(torch, pa, oracle):
    # rows of 16384 and 6000 tokens next to short ones: many partitions, merged with v_scale applied
    lens = [16384, 3, 6000, 64]
    w, rng, q, kp, vp = fp8_case(400, lens, 12, 2, 128, 64)
    ks, vs = 0.021, 1.7
    say("decode fp8, long rows")
    t = [dev(torch, x) for x in (q, kp, vp, w.tables, w.seq_lens)]
    out = pa.paged_decode_attn_fp8(*t, 64, w.scale, ks, vs)
    torch.cuda.synchronize()
    ref, _ = oracle.paged_decode_attn_fp8(q, kp, vp, w.tables, w.seq_lens, 64, w.scale, ks, vs, nthreads=NTHREADS)
    assert_close(host(out), ref, "fp8 long rows")
    again = pa.paged_decode_attn_fp8(*t, 64, w.scale, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(host(again).view(np.uint16), host(out).view(np.uint16))  # deterministic


@pytest.mark.parametrize("name", ["uniform1024", "uniform4096", "mixed", "high_occupancy"])
def test_fp8_step_on_qwen_batches(torch, pa, oracle, name):
    # the batch shapes of the fp16 benchmarks with E4M3 pools: the step's
    # quantizing append, then the decode
    w = wl.CONFIGS[name]()
    rng = np.random.default_rng(500)
    q = wl.normal_f16(rng, (w.B, w.Hq, w.D))
    kp = wl.fp8_codes(rng, wl.k_pool_shape_fp8(w.N, w.Hkv, w.D, w.bs))
    vp = wl.fp8_codes(rng, wl.v_pool_shape(w.N, w.Hkv, w.D, w.bs))
    kn = wl.normal_f16(rng, (w.B, w.Hkv, w.D))
    vn = wl.normal_f16(rng, (w.B, w.Hkv, w.D))
    ks, vs = 0.25, 0.5
    say("fp8 step on", name)
    tk, tv, tt, tl = dev(torch, kp), dev(torch, vp), dev(torch, w.tables), dev(torch, w.seq_lens)
    pa.kv_append_fp8(dev(torch, kn), dev(torch, vn), tk, tv, tt, tl, w.bs, ks, vs)
    out = pa.paged_decode_attn_fp8(dev(torch, q), tk, tv, tt, tl, w.bs, w.scale, ks, vs)
    torch.cuda.synchronize()
    assert oracle.kv_append_fp8(kn, vn, kp, vp, w.tables, w.seq_lens, w.bs, ks, vs) == 0
    assert np.array_equal(host(tk), kp) and np.array_equal(host(tv), vp)
    ref, _ = oracle.paged_decode_attn_fp8(q, kp, vp, w.tables, w.seq_lens, w.bs, w.scale, ks, vs,
                                          nthreads=NTHREADS)
    assert_close(host(out), ref, f"fp8 step {name}")


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_fused_fp8_step_equals_two_calls(torch, pa, oracle, bs):
    # new tokens at the first, 64th, 65th and last slot of a 128-token tile, a block's edges, and L = 1
    lens = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 4096]
    w, rng, q, kp, vp = fp8_case(600 + bs, lens, 12, 2, 128, bs)
    wl.poison_stale(kp, vp, w.tables, w.seq_lens, bs, value=NAN_CODE)
    kn = (wl.normal_f16(rng, (w.B, 2, 128)).astype(np.float32) * 3).astype(np.float16)
    vn = wl.normal_f16(rng, (w.B, 2, 128))
    ks, vs = 0.0625, 0.19
    say("fused fp8 step", "bs", bs)
    tt, tl, tq, tkn, tvn = (dev(torch, x) for x in (w.tables, w.seq_lens, q, kn, vn))
    fk, fv = dev(torch, kp), dev(torch, vp)
    fused = pa.paged_decode_attn_append_fp8(tq, tkn, tvn, fk, fv, tt, tl, bs, w.scale, ks, vs)
    ck, cv = dev(torch, kp), dev(torch, vp)
    pa.kv_append_fp8(tkn, tvn, ck, cv, tt, tl, bs, ks, vs)
    two = pa.paged_decode_attn_fp8(tq, ck, cv, tt, tl, bs, w.scale, ks, vs)
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    assert oracle.kv_append_fp8(kn, vn, ek, ev, w.tables, w.seq_lens, bs, ks, vs) == 0
    assert np.array_equal(host(fk), ek) and np.array_equal(host(fv), ev)
    assert np.array_equal(host(fused).view(np.uint16), host(two).view(np.uint16))
    ref, _ = oracle.paged_decode_attn_fp8(q, ek, ev, w.tables, w.seq_lens, bs, w.scale, ks, vs, nthreads=NTHREADS)
    assert_close(host(fused), ref, f"fused fp8 step bs={bs}")



def test_fused_fp8_step_more_rows_than_one_launch_takes(torch, pa, oracle):
    # 1100 short rows, some empty: the host runs the kernel over several row
    # ranges, each with its own slice of every buffer (the appends included)
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(0, 300, size=1100)]
    lens[0] = lens[517] = lens[1099] = 0
    w, rng, q, kp, vp = fp8_case(700, lens, 4, 2, 64, 16)
    kn = wl.normal_f16(rng, (w.B, 2, 64))
    vn = wl.normal_f16(rng, (w.B, 2, 64))
    ks, vs = 0.3, 0.6
    say("fused fp8 step, 1100 rows")
    tk, tv = dev(torch, kp), dev(torch, vp)
    out = pa.paged_decode_attn_append_fp8(dev(torch, q), dev(torch, kn), dev(torch, vn), tk, tv, dev(torch, w.tables),
                                          dev(torch, w.seq_lens), 16, w.scale, ks, vs)
    torch.cuda.synchronize()
    assert oracle.kv_append_fp8(kn, vn, kp, vp, w.tables, w.seq_lens, 16, ks, vs) == 0
    assert np.array_equal(host(tk), kp) and np.array_equal(host(tv), vp)
    ref, _ = oracle.paged_decode_attn_fp8(q, kp, vp, w.tables, w.seq_lens, 16, w.scale, ks, vs, nthreads=NTHREADS)
    got = host(out)
    assert np.all(got[[0, 517, 1099]].view(np.uint16) == 0)
    assert_close(got, ref, "fused fp8 step, 1100 rows")
