"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches) and replayed: every launch only enqueues kernels on the
caller's stream, allocates nothing and sets no memory from the host, and
the workspace's arrival counters come back to zero at the end of every
launch, so replays repeat the eager step exactly.

A three-layer fused step (paged_decode_attn_append per layer) and the same
over E4M3 pools are captured once and replayed three times, with other
eager work on the device between the replays; after every replay the
outputs and pools must be bit-identical to the eager step's (the step's
appends rewrite the same slots with the same values).
"""

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu


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


def same(torch, a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a,
                       b.view(torch.int16) if b.dtype == torch.float16 else b)


def _check_replays(torch, pa, step, init_pools, layers):
    """Run `step` eagerly on fresh copies of the pools, then capture it on
    other fresh copies and replay; compare every replay with the eager run."""
    eager_pools = [[p.clone() for p in lp] for lp in init_pools]
    eager_outs = step(eager_pools)
    torch.cuda.synchronize()
    graph_pools = [[p.clone() for p in lp] for lp in init_pools]
    outs_holder = {}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs_holder["o"] = step(graph_pools)
    filler = torch.randn(1 << 20, device="cuda")
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        for layer in range(layers):
            assert same(torch, outs_holder["o"][layer], eager_outs[layer]), f"replay {r} layer {layer}: output"
            for gp, ep in zip(graph_pools[layer], eager_pools[layer]):
                assert same(torch, gp, ep), f"replay {r} layer {layer}: pool"
        filler.mul_(1.0001).sum().item()  # eager device work and a synchronization between replays
        for o in outs_holder["o"]:
            o.zero_()


def test_fused_step_replays_in_a_graph(torch, pa):
    layers = 3
    w = wl.full_step(layers=layers, N=2048)
    say("graph replay: fused fp16 step,", layers, "layers")
    t, sl = dev(torch, w.tables), dev(torch, w.seq_lens)
    lds = [w.layer(i) for i in range(layers)]
    qs = [(dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new)) for ld in lds]
    init = [[dev(torch, ld.k_pool), dev(torch, ld.v_pool)] for ld in lds]
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)

    def step(pools):
        outs = []
        for layer in range(layers):
            q, kn, vn = qs[layer]
            out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float16, device="cuda")
            pa.paged_decode_attn_append(q, kn, vn, pools[layer][0], pools[layer][1], t, sl, w.bs, w.scale,
                                        out=out, workspace=ws)
            outs.append(out)
        return outs

    _check_replays(torch, pa, step, init, layers)


def test_fused_fp8_step_replays_in_a_graph(torch, pa):
    layers = 3
    w = wl.full_step(layers=layers, N=2048)
    say("graph replay: fused E4M3 step,", layers, "layers")
    rng = np.random.default_rng(77)
    t, sl = dev(torch, w.tables), dev(torch, w.seq_lens)
    lds = [w.layer(i) for i in range(layers)]
    qs = [(dev(torch, ld.q), dev(torch, ld.k_new), dev(torch, ld.v_new)) for ld in lds]
    init = [[dev(torch, wl.fp8_codes(rng, wl.k_pool_shape_fp8(w.N, w.Hkv, w.D, w.bs))),
             dev(torch, wl.fp8_codes(rng, wl.v_pool_shape(w.N, w.Hkv, w.D, w.bs)))] for _ in range(layers)]
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)

    def step(pools):
        outs = []
        for layer in range(layers):
            q, kn, vn = qs[layer]
            out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float16, device="cuda")
            pa.paged_decode_attn_append_fp8(q, kn, vn, pools[layer][0], pools[layer][1], t, sl, w.bs, w.scale,
                                            0.25, 0.5, out=out, workspace=ws)
            outs.append(out)
        return outs

    _check_replays(torch, pa, step, init, layers)
