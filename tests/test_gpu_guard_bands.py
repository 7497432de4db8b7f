"""Writes stay inside their buffers. Every buffer a call may write (out, both
pools, the workspace, the gathered copies) sits between two 4 KiB guard bands
filled with a canary byte; after each entry point runs -- the fp16 and E4M3
decodes, fused, masked and no-workspace forms, the appends, copy-on-write,
the post-prefill scatter and the debug gather -- both bands of every buffer
are unchanged, and after every decode the workspace's arrival counters (its
first MiB) are back at zero. The batch mixes a row long enough to be split
over many partitions with short, ragged and empty rows."""

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

PAD = 4096
CANARY = 0xA5
COUNTER_BYTES = 1 << 20


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


class Guarded:
    """A tensor of `shape` / `dtype` inside a uint8 buffer with PAD canary bytes before and after."""

    def __init__(self, torch, shape, dtype, init=None):
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((self.n + 2 * PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(torch.from_numpy(np.ascontiguousarray(init)).view(dtype).view(shape))

    def intact(self):
        head, tail = self.buf[:PAD], self.buf[PAD + self.n:]
        return bool((head == CANARY).all().item()) and bool((tail == CANARY).all().item())


def _workload():
    lens = [5000, 3, 700, 0, 64, 1300, 4097, 1]
    N = sum(wl.blocks_for(L, 64) for L in lens) + 16
    return wl.make_workload("guards", len(lens), 12, 2, 128, 64, N, lens, seed=51, events=10)


def test_every_entry_point_writes_inside_its_buffers(torch, pa):
    w = _workload()
    ld = w.layer(0)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, kn, vn = d(ld.q), d(ld.k_new), d(ld.v_new)
    tables, lens = d(w.tables), d(w.seq_lens)
    wsn = pa.paged_decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)
    kp = Guarded(torch, ld.k_pool.shape, torch.float16, ld.k_pool)
    vp = Guarded(torch, ld.v_pool.shape, torch.float16, ld.v_pool)
    out = Guarded(torch, (w.B, w.Hq, w.D), torch.float16)
    ws = Guarded(torch, (wsn,), torch.uint8)
    pa.paged_decode_workspace_init(ws.t)
    rng = np.random.default_rng(52)
    k8 = Guarded(torch, wl.k_pool_shape_fp8(w.N, w.Hkv, w.D, w.bs), torch.uint8,
                 wl.fp8_codes(rng, wl.k_pool_shape_fp8(w.N, w.Hkv, w.D, w.bs)))
    v8 = Guarded(torch, wl.v_pool_shape(w.N, w.Hkv, w.D, w.bs), torch.uint8,
                 wl.fp8_codes(rng, wl.v_pool_shape(w.N, w.Hkv, w.D, w.bs)))
    S = 1400
    prompt = d(np.minimum(w.seq_lens, S).astype(np.int32))
    ksrc, vsrc = d(wl.normal_f16(rng, (w.B, w.Hkv, S, w.D))), d(wl.normal_f16(rng, (w.B, w.Hkv, S, w.D)))
    src = d(np.asarray(w.tables[0, :4], np.int32))
    dst = d(np.asarray([w.N - 1, w.N - 2, w.N - 3, w.N - 4], np.int32))
    gk = Guarded(torch, (w.B, w.Hkv, w.W * w.bs, w.D), torch.float16)
    gv = Guarded(torch, (w.B, w.Hkv, w.W * w.bs, w.D), torch.float16)
    buffers = {"k_pool": kp, "v_pool": vp, "out": out, "workspace": ws, "k_pool_fp8": k8, "v_pool_fp8": v8,
               "gather_k": gk, "gather_v": gv}
    calls = [
        ("kv_append", lambda: pa.kv_append(kn, vn, kp.t, vp.t, tables, lens, w.bs)),
        ("paged_decode_attn", lambda: pa.paged_decode_attn(q, kp.t, vp.t, tables, lens, w.bs, w.scale,
                                                           out=out.t, workspace=ws.t)),
        ("paged_decode_attn_append", lambda: pa.paged_decode_attn_append(
            q, kn, vn, kp.t, vp.t, tables, lens, w.bs, w.scale, out=out.t, workspace=ws.t)),
        ("paged_decode_attn_masked", lambda: pa.paged_decode_attn_masked(
            q, kp.t, vp.t, tables, lens, w.bs, w.scale, 1024, out=out.t, workspace=ws.t)),
        ("paged_decode_attn_noalloc", lambda: pa.paged_decode_attn_noalloc(
            q, kp.t, vp.t, tables, lens, w.bs, w.scale, out=out.t)),
        ("kv_append_fp8", lambda: pa.kv_append_fp8(kn, vn, k8.t, v8.t, tables, lens, w.bs, 0.25, 0.5)),
        ("paged_decode_attn_fp8", lambda: pa.paged_decode_attn_fp8(
            q, k8.t, v8.t, tables, lens, w.bs, w.scale, 0.25, 0.5, out=out.t, workspace=ws.t)),
        ("paged_decode_attn_append_fp8", lambda: pa.paged_decode_attn_append_fp8(
            q, kn, vn, k8.t, v8.t, tables, lens, w.bs, w.scale, 0.25, 0.5, out=out.t, workspace=ws.t)),
        ("kv_copy_blocks", lambda: pa.kv_copy_blocks(kp.t, vp.t, src, dst, w.bs)),
        ("kv_copy_blocks_fp8", lambda: pa.kv_copy_blocks_fp8(k8.t, v8.t, src, dst, w.bs)),
        ("kv_scatter_prefill", lambda: pa.kv_scatter_prefill(ksrc, vsrc, kp.t, vp.t, tables, prompt, w.bs)),
        ("kv_scatter_prefill_fp8", lambda: pa.kv_scatter_prefill_fp8(
            ksrc, vsrc, k8.t, v8.t, tables, prompt, w.bs, 0.25, 0.5)),
        ("paged_gather_kv", lambda: pa.paged_gather_kv(kp.t, vp.t, tables, lens, w.bs, k_out=gk.t, v_out=gv.t)),
    ]
    for name, call in calls:
        print("[gpu] guard bands:", name, flush=True)
        call()
        torch.cuda.synchronize()
        bad = [b for b, g in buffers.items() if not g.intact()]
        assert not bad, f"{name} wrote outside {bad}"
        counters = ws.t[:COUNTER_BYTES]
        assert int(counters.count_nonzero().item()) == 0, f"{name} left arrival counters nonzero"
    assert not torch.isnan(out.t.float()).any()
