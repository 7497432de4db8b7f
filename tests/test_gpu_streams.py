"""Calls on a stream other than torch's current one, through the binding.

With `stream=` given and no `out` or workspace, the binding makes the call's
own output and zeroed workspace on that stream: the results must equal
those of the same calls on the current stream, bit for bit (the decode is
deterministic run to run), for the decode, the fused step, the gather and an
E4M3-pool decode, on the mixed batch (Qwen2.5-1.5B shapes).
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


def test_calls_on_a_side_stream_match_the_current_stream(torch, pa):
    w = wl.mixed()
    ld = w.layer(0)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q, kn, vn = d(ld.q), d(ld.k_new), d(ld.v_new)
    kp, vp, tt, tl = d(ld.k_pool), d(ld.v_pool), d(w.tables), d(w.seq_lens)
    rng = np.random.default_rng(3)
    k8 = d(wl.fp8_codes(rng, wl.k_pool_shape_fp8(w.N, w.Hkv, w.D, w.bs)))
    v8 = d(wl.fp8_codes(rng, wl.v_pool_shape(w.N, w.Hkv, w.D, w.bs)))
    kp2, vp2 = kp.clone(), vp.clone()
    say("current stream: decode, fused step, gather, E4M3 decode")
    ref = pa.paged_decode_attn(q, kp, vp, tt, tl, w.bs, w.scale)
    ref_f = pa.paged_decode_attn_append(q, kn, vn, kp2, vp2, tt, tl, w.bs, w.scale)
    ref_g = pa.paged_gather_kv(kp2, vp2, tt, tl, w.bs)
    ref_8 = pa.paged_decode_attn_fp8(q, k8, v8, tt, tl, w.bs, w.scale, 0.1, 0.2)
    torch.cuda.synchronize()
    ref, ref_f, ref_8 = ref.cpu(), ref_f.cpu(), ref_8.cpu()
    ref_g = [t.cpu() for t in ref_g]

    kp3, vp3 = kp.clone(), vp.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("side stream: the same calls")
    out = pa.paged_decode_attn(q, kp, vp, tt, tl, w.bs, w.scale, stream=side)
    out_f = pa.paged_decode_attn_append(q, kn, vn, kp3, vp3, tt, tl, w.bs, w.scale, stream=side)
    out_g = pa.paged_gather_kv(kp3, vp3, tt, tl, w.bs, stream=side)
    out_8 = pa.paged_decode_attn_fp8(q, k8, v8, tt, tl, w.bs, w.scale, 0.1, 0.2, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out_f.cpu().view(torch.int16), ref_f.view(torch.int16))
    assert torch.equal(out_8.cpu().view(torch.int16), ref_8.view(torch.int16))
    assert torch.equal(kp3.cpu().view(torch.int16), kp2.cpu().view(torch.int16))
    assert torch.equal(vp3.cpu().view(torch.int16), vp2.cpu().view(torch.int16))
    for a, b in zip(out_g, ref_g):
        assert torch.equal(a.cpu().view(torch.int16), b.view(torch.int16))
