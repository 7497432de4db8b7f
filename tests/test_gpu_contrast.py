"""GPU parity of the masked-width contrast (paged_decode_attn_masked).

Computed over a fixed width for every row with the positions past each row's
length masked, the result must still be the attention over the row's own
tokens: within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the oracle, zeros for
empty rows, unaffected by NaN in every masked slot, on the contiguous
(identity-table) layout and on shuffled blocks.
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


def identity_tables(B, W):
    return (np.arange(B, dtype=np.int32)[:, None] * W + np.arange(W, dtype=np.int32)[None, :]).astype(np.int32)


def check(out, ref, what):
    got = out.astype(np.float64)
    err = np.abs(got - ref)
    assert not np.isnan(got).any(), f"{what}: NaN"
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"{what}: max abs err {err.max():.3e}"


@pytest.mark.parametrize("layout", ["contiguous", "shuffled"])
def test_masked_width_matches_true_length_attention(torch, pa, oracle, layout):
    rng = np.random.default_rng(41)
    bs, Hq, Hkv, D = 64, 12, 2, 128
    lens = [int(x) for x in rng.integers(16, 513, size=15)] + [0, 1, 4352]
    B = len(lens)
    W = 4352 // bs
    if layout == "contiguous":
        N = B * W
        tables = identity_tables(B, W)
        k_pool = wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))
        v_pool = wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))
        q = wl.normal_f16(rng, (B, Hq, D))
        scale = float(np.float32(1 / np.sqrt(D)))
    else:
        w = wl.make_workload("masked", B, Hq, Hkv, D, bs, B * W, lens, seed=42, events=50, W=W)
        tables = w.tables.copy()
        # the masked width reads W blocks of every non-empty row: give every row a full table
        used = set(int(x) for x in tables[tables >= 0])
        spare = [b for b in range(w.N) if b not in used]
        for b in range(B):
            for j in range(W):
                if tables[b, j] < 0:
                    tables[b, j] = spare.pop()
        ld = w.layer(0)
        k_pool, v_pool, q, scale = ld.k_pool, ld.v_pool, ld.q, w.scale
    lens = np.asarray(lens, np.int32)
    wl.poison_stale(k_pool, v_pool, tables, lens, bs)
    say("masked width", layout, "rows", B, "width", W * bs)
    out = pa.paged_decode_attn_masked(dev(torch, q), dev(torch, k_pool), dev(torch, v_pool), dev(torch, tables),
                                      dev(torch, lens), bs, scale, W * bs)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref, _ = oracle.paged_decode_attn(q, k_pool, v_pool, tables, lens, bs, scale, nthreads=NTHREADS)
    check(out, ref, f"masked width, {layout}")
    assert np.all(out[B - 3].view(np.uint16) == 0)  # the empty row


def test_masked_width_narrower_than_a_row_still_covers_the_row(torch, pa, oracle):
    # rows longer than the width are read at their own length
    w = wl.mixed()
    ld = w.layer(0)
    say("masked width 100 on the mixed batch")
    out = pa.paged_decode_attn_masked(dev(torch, ld.q), dev(torch, ld.k_pool), dev(torch, ld.v_pool),
                                      dev(torch, w.tables), dev(torch, w.seq_lens), w.bs, w.scale, 100)
    torch.cuda.synchronize()
    ref, _ = oracle.paged_decode_attn(ld.q, ld.k_pool, ld.v_pool, w.tables, w.seq_lens, w.bs, w.scale,
                                      nthreads=NTHREADS)
    check(out.cpu().numpy(), ref, "masked width 100")
