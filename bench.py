"""Decode-attention throughput of libpagedattn on one MI355X.

A step is one pass of the whole hot path over one batch: kv_append (the
step's new K/V scattered into each row's last block) then paged_decode_attn
(every row's blocks gathered at its own length, grouped-query attention for
one query token), for every layer of the workload. The timed step issues both
as one launch per layer (paged_decode_attn_append); the same step issued as
the two separate calls is timed beside it (`two_call_ms_per_step`).

Default workload: batch 32, Qwen2.5-1.5B attention shape (12 query heads,
2 KV heads, head_dim 128, fp16), block 64, every row at length 1024, blocks
shuffled over a 1024-block pool. Inputs are synthetic N(0,1) fp16 and
resident in HBM before timing starts; R replicas of the pools (distinct
memory, ~1 GiB touched in total) are rotated so consecutive steps stream
from HBM rather than the 256 MB last-level cache.

Output: one JSON line. `value` is algorithmic bytes moved per step (every
row's K and V at its own length, q, out, table entries, lengths, and the
append's reads and writes) divided by the measured time per step. The
`roofline` object reports the decode kernel alone, as the step launches it
(with the append fused in): its algorithmic bytes per launch over its average
duration (`decode_us`), against 8 TB/s. The duration is measured with HIP
events on the launch stream in two ways, each an upper bound on it, and the
smaller is taken: the launches issued eagerly back to back
(`decode_us_eager_back_to_back`, host-bound where the host issues launches
more slowly than the kernel runs) and a HIP graph replay of the step's
launches (`decode_us_graph`, `graph_ms_per_step` over the layers of a step,
which adds the graph's own gaps between kernels). Events bracketing each
single launch give `decode_us_bracketed`. `probe_read` times a plain
streaming read of the same byte count (pa_probe_read, the smaller of the
same two measurements), the ceiling any kernel reading those bytes meets at
that size. `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload, on the host's threads and on one thread.

`graded` (default run only) times the same step on the three workloads
the 70 %-of-peak target is set on -- the mixed batch (31 rows of 16..512
tokens and one of 4,352), uniform batch 32 at 4,096 tokens, and the 28-layer
step -- with `--graded-steps` timed steps each, and reports for each the
decode kernel's duration (the same smaller-of-two upper bounds), its GB/s
and fraction of 8 TB/s over the workload's unique algorithmic bytes, whether
that meets 0.70 and the duration that would, the recorded HBM traffic where
profiles/ holds it for the current kernel code, the same-size streaming
read, and the whole step's rows*layers/s. `--no-graded` skips it.

Other modes (`--op`): fp8 (the step over E4M3 pools), contrast (the mixed
batch paged, contiguous, at masked full width and at block sizes 16..256),
copy_blocks (copy-on-write block copies), scatter_prefill (the post-prefill
scatter, `--kv fp8` for E4M3 pools).

`roofline.traffic` is the decode kernel's HBM bytes per launch from two
rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of this same script with
--copy-calibration, each scaled by what the counter reads for a plain device
copy of known size in the same run. `--pmc-summary FETCH_DIR WRITE_DIR`
turns those runs into profiles/decode_kernel_<workload>_traffic.txt; the
figure is reported only while the kernel source still has the hash recorded
there (code, comments excluded), else null.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
# the sources of the decode kernel: host side and fp16-pool instances, E4M3-pool instances, the kernel itself
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_06_amd", "csrc", f)
               for f in ("pagedattn.hip", "pagedattn_fp8.hip", "decode_kernel.h", "e4m3.h")]
PROFILES = os.path.join(ROOT, "profiles")
DECODE_KERNEL = "decode_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_REPS = 10


def _code_only(text: str) -> str:
    """The source without comments and blank lines (a comment edit does not change the kernel)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def _compile_flags() -> list:
    """The hipcc flags the library is built with (read from the build module's file)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_pa_build", os.path.join(ROOT, "paged_kv_cache_06_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return list(mod.HIPCC_FLAGS)


def kernel_source_hash() -> str:
    """Hash of the decode kernel's code (comments and blank lines aside) and of
    the compiler flags: a change of either voids the committed counter records."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path) as f:
            h.update(_code_only(f.read()).encode())
    h.update(" ".join(_compile_flags()).encode())
    return h.hexdigest()[:16]


def traffic_file(workload: str, fp8: bool = False) -> str:
    return os.path.join(PROFILES, f"decode_kernel{'_fp8' if fp8 else ''}_{workload}_traffic.txt")


def read_traffic(workload: str, fp8: bool = False):
    """HBM bytes per decode launch from the committed counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = traffic_file(workload, fp8)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "-")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_per_dispatch(run_dir: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (summed over the
    dimensions rocprofv3 reports it in)."""
    per = {}
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, r["Dispatch_Id"])
            per.setdefault(key, [r["Kernel_Name"], 0.0])
            per[key][1] += float(r["Counter_Value"])
    out = {}
    for name, v in per.values():
        out.setdefault(name, []).append(v)
    return out


def _median_for(values: dict, needle: str, largest: int = 0, also: str = ""):
    """Median over the dispatches of one kernel (names holding `needle` and
    `also`); with `largest`, over its `largest` biggest readings only (the
    calibration copies, not the small host-device transfers the same copy
    kernel also serves)."""
    got = sorted(v for name, vs in values.items() if needle in name and also in name for v in vs)
    if largest:
        got = got[-largest:]
    if not got:
        raise SystemExit(f"no dispatch of {needle} in the counter output")
    return float(np.median(got)), len(got)


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int, command: str,
                fp8: bool = False) -> str:
    """Summarise two counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    into HBM bytes per decode launch, each counter scaled by its reading for a
    plain copy of copy_bytes (which reads and writes copy_bytes once). With
    fp8, the E4M3-pool instances (the fused fp16 step's otherwise)."""
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    fmt = ", true>" if fp8 else ", false>"
    f_dec, n_f = _median_for(fetch, DECODE_KERNEL, also=fmt)
    w_dec, n_w = _median_for(write, DECODE_KERNEL, also=fmt)
    f_cpy, n_fc = _median_for(fetch, COPY_KERNEL, largest=COPY_REPS)
    w_cpy, n_wc = _median_for(write, COPY_KERNEL, largest=COPY_REPS)
    f_scale = copy_bytes / (f_cpy * 1024.0)
    w_scale = copy_bytes / (w_cpy * 1024.0)
    traffic = f_dec * 1024.0 * f_scale + w_dec * 1024.0 * w_scale
    w = wl.CONFIGS[workload]()
    algo = decode_bytes_fp8(w) if fp8 else decode_bytes(w, unique=True) + append_bytes(w)
    lines = [
        f"# decode_kernel{' (E4M3 pools)' if fp8 else ''} HBM traffic, workload {workload}",
        f"# command: {command}",
        f"workload: {workload}",
        f"kernel_source_sha256_16: {kernel_source_hash()}",
        f"decode_fetch_kib_per_dispatch_median: {f_dec:.1f}  (dispatches: {n_f})",
        f"decode_write_kib_per_dispatch_median: {w_dec:.1f}  (dispatches: {n_w})",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_kib_per_dispatch_median: {f_cpy:.1f}  (dispatches: {n_fc})",
        f"copy_write_kib_per_dispatch_median: {w_cpy:.1f}  (dispatches: {n_wc})",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"traffic_bytes_per_launch: {int(round(traffic))}",
        f"algorithmic_bytes_per_launch: {algo}",
        f"traffic_over_algorithmic: {traffic / algo:.4f}",
    ]
    return "\n".join(lines) + "\n"


def decode_bytes(w: wl.Workload, unique=False) -> int:
    kv = w.unique_kv_bytes_per_layer() if unique else w.kv_bytes_per_layer()
    qo = 2 * w.B * w.Hq * w.D * 2
    table = 4 * int(sum(wl.blocks_for(int(L), w.bs) for L in w.seq_lens))
    return kv + qo + table + 4 * w.B


def append_bytes(w: wl.Workload) -> int:
    rows = int(np.sum(w.seq_lens >= 1))
    return rows * w.Hkv * w.D * 2 * 2 * 2 + rows * 4 + 4 * w.B


def decode_bytes_fp8(w: wl.Workload) -> int:
    """As decode_bytes, with one byte per K/V element."""
    return decode_bytes(w) - w.kv_bytes_per_layer() // 2


def append_bytes_fp8(w: wl.Workload) -> int:
    """The new K/V read as fp16, written as one byte per element, plus lengths and table entries."""
    rows = int(np.sum(w.seq_lens >= 1))
    return rows * w.Hkv * w.D * 2 * (2 + 1) + rows * 4 + 4 * w.B


def bench_fp8(args, torch, pa):
    """The decode step over E4M3 (FP8) pools: one fused launch per layer
    (paged_decode_attn_append_fp8; beside it the same step as kv_append_fp8
    then paged_decode_attn_fp8), on the chosen workload's shapes with
    random E4M3 codes in the pools; beside it the fp16 decode of the same
    shapes (paged_decode_attn) for the ratio. Bytes count one byte per pool
    element."""
    w = wl.CONFIGS[args.config]()
    layers = w.layers
    rng = np.random.default_rng(7)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    tables, lens = dev(w.tables), dev(w.seq_lens)
    touched = decode_bytes_fp8(w) * layers
    R = args.replicas or (1 if layers > 1 else max(1, math.ceil((1 << 30) / touched)))
    ld = w.layer(0)
    base = [dev(ld.q), dev(ld.k_new), dev(ld.v_new),
            dev(wl.fp8_codes(rng, wl.k_pool_shape_fp8(w.N, w.Hkv, w.D, w.bs))),
            dev(wl.fp8_codes(rng, wl.v_pool_shape(w.N, w.Hkv, w.D, w.bs)))]
    sets = [[[t.clone() for t in base] for _ in range(layers)] for _ in range(R)]
    print(f"[fp8] {w.name}: {R} replicas of {layers} layer(s) resident", file=sys.stderr, flush=True)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float16, device="cuda")
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)
    ks, vs = 0.25, 0.5
    torch.cuda.synchronize()

    def step(i):
        for q, kn, vn, kp, vp in sets[i % R]:
            pa.paged_decode_attn_append_fp8(q, kn, vn, kp, vp, tables, lens, w.bs, w.scale, ks, vs, out=out,
                                            workspace=ws)

    def step_two_calls(i):
        for q, kn, vn, kp, vp in sets[i % R]:
            pa.kv_append_fp8(kn, vn, kp, vp, tables, lens, w.bs, ks, vs)
            pa.paged_decode_attn_fp8(q, kp, vp, tables, lens, w.bs, w.scale, ks, vs, out=out, workspace=ws)

    def timed(fn, n):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(n):
            fn(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    def graphed(fn, n):
        """Per-call time of fn(0..n-1) replayed from a HIP graph: kernel
        durations back to back, with no host launch overhead between them."""
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        del graph
        return t0.elapsed_time(t1) / n

    def kernel_ms(fn, n):
        """A kernel's duration: the smaller of two upper bounds (eager back to back, graph replay)."""
        return min(timed(fn, n), graphed(fn, n))

    ms_per_step = timed(step, args.steps)
    two_call_ms = timed(step_two_calls, args.steps)
    dec_ms = kernel_ms(lambda i: pa.paged_decode_attn_fp8(sets[i % R][i % layers][0], sets[i % R][i % layers][3],
                                                       sets[i % R][i % layers][4], tables, lens, w.bs, w.scale, ks,
                                                       vs, out=out, workspace=ws), args.steps)
    app_ms = kernel_ms(lambda i: pa.kv_append_fp8(sets[i % R][i % layers][1], sets[i % R][i % layers][2],
                                               sets[i % R][i % layers][3], sets[i % R][i % layers][4], tables, lens,
                                               w.bs, ks, vs), args.steps)
    print(f"[fp8] step {ms_per_step * 1e3:.2f} us, decode {dec_ms * 1e3:.2f} us, append {app_ms * 1e3:.2f} us",
          file=sys.stderr, flush=True)
    # the fp16 decode on the same shapes (its own pools, the same number of replicas up to ~1 GiB)
    R16 = max(1, min(R, math.ceil((1 << 30) / (decode_bytes(w) * layers))))
    k16 = dev(ld.k_pool)
    v16 = dev(ld.v_pool)
    p16 = [(k16.clone(), v16.clone()) for _ in range(R16)]
    del sets
    f16_ms = kernel_ms(lambda i: pa.paged_decode_attn(base[0], p16[i % R16][0], p16[i % R16][1], tables, lens, w.bs,
                                                   w.scale, out=out, workspace=ws), args.steps)
    probe_us, probe_bytes = probe_read_us(args, torch, pa, decode_bytes_fp8(w), args.steps)
    launch_bytes = decode_bytes_fp8(w) + append_bytes_fp8(w)
    value = launch_bytes * layers / (ms_per_step * 1e-3) / 1e9
    dec_gbs = decode_bytes_fp8(w) / (dec_ms * 1e-3) / 1e9
    line = {
        "metric": "paged decode attention over E4M3 (FP8) KV pools: achieved HBM GB/s of the step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 q/out, e4m3 KV",
        "data": "synthetic (random E4M3 codes, k_scale 0.25, v_scale 0.5)",
        "config": {"workload": w.name, "batch": w.B, "layers": layers, "num_heads": w.Hq, "num_kv_heads": w.Hkv,
                   "head_dim": w.D, "block_size": w.bs, "seq_len_sum": int(w.seq_lens.sum()), "replicas": R},
        "rows_layers_per_s": round(w.B * layers / (ms_per_step * 1e-3), 1),
        "bytes_per_step": launch_bytes * layers,
        "two_call_ms_per_step": round(two_call_ms, 6),
        "decode_us": round(dec_ms * 1e3, 3),
        "append_us": round(app_ms * 1e3, 3),
        "fp16_decode_us": round(f16_ms * 1e3, 3),
        "decode_speedup_vs_fp16": round(f16_ms / dec_ms, 3),
        "probe_read": {"bytes": probe_bytes, "us": round(probe_us, 3),
                       "GBs": round(probe_bytes / (probe_us * 1e-6) / 1e9, 2),
                       "decode_over_probe_time": round(dec_ms * 1e3 / probe_us, 3)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(dec_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(w.name, fp8=True),
            "kernel": "decode_kernel (E4M3 pools)",
            "bytes_per_launch": decode_bytes_fp8(w),
        },
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    copy_calibration(args, torch)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def probe_read_us(args, torch, pa, nbytes, n):
    """Back-to-back launches of the streaming-read probe over nbytes (rounded
    up to 16), rotating replicas of ~1 GiB in total like the decode, issued
    eagerly and replayed from a HIP graph; returns (us per launch, the smaller
    of the two: each is an upper bound on the kernel's duration, the first
    host-bound where launches are issued more slowly than they run, the second
    with the graph's own gaps between kernels), bytes)."""
    nbytes = (nbytes + 15) // 16 * 16
    R = max(1, math.ceil((1 << 30) / nbytes))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    for i in range(max(args.warmup, 1)):
        pa.probe_read(bufs[i % R], sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        pa.probe_read(bufs[i % R], sink)
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / n
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            pa.probe_read(bufs[i % R], sink)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return min(eager, e0.elapsed_time(e1) / n) * 1e3, nbytes


def copy_calibration(args, torch):
    """Plain device copies of a known size after the bench (the counter runs' scale)."""
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()


def bench_copy_blocks(args, torch, pa):
    """kv_copy_blocks alone: `--copy-pairs` random disjoint (src, dst) pairs of
    a Qwen-shaped pool (2 KV heads, head_dim 128, block 64: 32 KiB of K and
    32 KiB of V per block), one layer per call, replicas rotated so the copies
    stream from HBM. Bytes per call: every copied block read once and written
    once."""
    Hkv, D, bs, N = 2, 128, 64, 4096
    n = min(args.copy_pairs, N // 2)
    block_bytes = Hkv * D * bs * 2 * 2  # K and V
    pool_bytes = N * block_bytes
    R = args.replicas or max(1, math.ceil((1 << 30) / pool_bytes))
    rng = np.random.default_rng(17)
    kp0 = torch.from_numpy(wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))).cuda()
    vp0 = torch.from_numpy(wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))).cuda()
    pools = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(R - 1)]
    pairs = []
    for r in range(R):
        perm = rng.permutation(N).astype(np.int32)
        pairs.append((torch.from_numpy(perm[:n].copy()).cuda(), torch.from_numpy(perm[n:2 * n].copy()).cuda()))
    torch.cuda.synchronize()

    def call(i):
        kp, vp = pools[i % R]
        src, dst = pairs[i % R]
        pa.kv_copy_blocks(kp, vp, src, dst, bs)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        call(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    moved = 2 * n * block_bytes
    gbs = moved / (ms * 1e-3) / 1e9
    line = {
        "metric": "kv_copy_blocks (copy-on-write) achieved HBM GB/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": "copy_blocks", "pairs": n, "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "pool_blocks": N, "replicas": R, "bytes_per_call": moved},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "copy_blocks_kernel",
                     "bytes_per_launch": moved},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


def bench_scatter_prefill(args, torch, pa):
    """kv_scatter_prefill alone: a prefill group of 32 prompts of seeded
    U{16..4096} tokens (the pages' range of prompt lengths), left padded to
    4096, Qwen-shaped (2 KV heads, head_dim 128), block 64, scattered into
    shuffled blocks of a 4,096-block pool; replicas rotated. Bytes per call:
    every prompt token's K and V read once and written once. With --kv fp8,
    kv_scatter_prefill_fp8 into E4M3 pools (one byte written per element)."""
    B, Hkv, D, bs, S = 32, 2, 128, 64, 4096
    fp8 = args.kv == "fp8"
    rng = np.random.default_rng(19)
    prompts = rng.integers(16, S + 1, size=B).astype(np.int32)
    w = wl.make_workload("scatter", B, 12, Hkv, D, bs, 4096, prompts, seed=19, events=0, append=False)
    moved = int(prompts.sum()) * Hkv * D * 2 * (2 + (1 if fp8 else 2))
    group_bytes = B * Hkv * S * D * 2 * 2
    R = args.replicas or max(1, math.ceil((1 << 30) / (group_bytes + 4096 * Hkv * D * bs * 2 * 2)))
    ks0 = torch.from_numpy(wl.normal_f16(rng, (B, Hkv, S, D))).cuda()
    vs0 = torch.from_numpy(wl.normal_f16(rng, (B, Hkv, S, D))).cuda()
    if fp8:
        kp0 = torch.zeros(wl.k_pool_shape_fp8(4096, Hkv, D, bs), dtype=torch.uint8, device="cuda")
        vp0 = torch.zeros(wl.v_pool_shape(4096, Hkv, D, bs), dtype=torch.uint8, device="cuda")
    else:
        kp0 = torch.zeros(wl.k_pool_shape(4096, Hkv, D, bs), dtype=torch.float16, device="cuda")
        vp0 = torch.zeros(wl.v_pool_shape(4096, Hkv, D, bs), dtype=torch.float16, device="cuda")
    sets = [(ks0, vs0, kp0, vp0)] + [tuple(t.clone() for t in (ks0, vs0, kp0, vp0)) for _ in range(R - 1)]
    tables = torch.from_numpy(w.tables).cuda()
    plen = torch.from_numpy(prompts).cuda()
    torch.cuda.synchronize()

    def call(i):
        ks, vs, kp, vp = sets[i % R]
        if fp8:
            pa.kv_scatter_prefill_fp8(ks, vs, kp, vp, tables, plen, bs, 0.05, 0.05)
        else:
            pa.kv_scatter_prefill(ks, vs, kp, vp, tables, plen, bs)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        call(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gbs = moved / (ms * 1e-3) / 1e9
    line = {
        "metric": f"kv_scatter_prefill{'_fp8' if fp8 else ''} (post-prefill scatter) achieved HBM GB/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 -> e4m3" if fp8 else "u16",
        "data": "synthetic",
        "config": {"workload": "scatter_prefill", "pool": "e4m3" if fp8 else "f16", "rows": B, "padded_len": S, "prompt_tokens": int(prompts.sum()),
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs, "replicas": R, "bytes_per_call": moved},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "scatter_prefill_fp8_kernel" if fp8 else "scatter_prefill_kernel",
                     "bytes_per_launch": moved},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


def bench_contrast(args, torch, pa):
    """The mixed batch (31 rows of U{16..512} tokens and one of 4,352) decoded
    (a) paged, blocks shuffled through the pool (the normal path); (b) on the
    contiguous layout (identity tables); (c) the way the earlier fixed-width
    engine computed it: every row over the widest row's 4,352 positions,
    masked (paged_decode_attn_masked on the contiguous layout); (d) paged at
    block sizes 16, 32, 64, 128 and 256 with the same lengths. Decode kernel
    duration per call from back-to-back launches; replicas rotated."""
    w0 = wl.mixed()
    lens = w0.seq_lens
    B, Hq, Hkv, D = w0.B, w0.Hq, w0.Hkv, w0.D
    width = int(lens.max())
    kv_true = int(lens.sum()) * Hkv * D * 2 * 2
    rng = np.random.default_rng(23)

    def timed(name, make_call, touched):
        R = min(32, max(1, math.ceil((1 << 30) / touched)))
        first = make_call(None)
        calls = [first] + [make_call(first) for _ in range(R - 1)]
        for i in range(args.warmup):
            calls[i % R]()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            calls[i % R]()
        t1.record()
        torch.cuda.synchronize()
        eager = t0.elapsed_time(t1) / args.steps * 1e3
        # the same calls replayed from a HIP graph; the smaller of the two is
        # taken (each bounds the kernel's duration from above)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                calls[i % R]()
        graph.replay()
        torch.cuda.synchronize()
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        del graph
        us = min(eager, t0.elapsed_time(t1) / args.steps * 1e3)
        print(f"[contrast] {name}: {us:.2f} us per call ({R} replicas; eager {eager:.2f})", file=sys.stderr,
              flush=True)
        return us, R

    def setup(bs, tables, N, width_arg, like=None):
        # random data once per configuration; further replicas are device copies of it
        if like is None:
            q = torch.from_numpy(wl.normal_f16(rng, (B, Hq, D))).cuda()
            kp = torch.from_numpy(wl.normal_f16(rng, wl.k_pool_shape(N, Hkv, D, bs))).cuda()
            vp = torch.from_numpy(wl.normal_f16(rng, wl.v_pool_shape(N, Hkv, D, bs))).cuda()
        else:
            q, kp, vp = (t.clone() for t in like.tensors)
        tt = torch.from_numpy(tables).cuda()
        ll = torch.from_numpy(lens).cuda()
        ws = pa.new_workspace(B, Hq, Hkv, D, bs, tables.shape[1])
        out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
        if width_arg:
            def call():
                pa.paged_decode_attn_masked(q, kp, vp, tt, ll, bs, w0.scale, width_arg, out=out, workspace=ws)
        else:
            def call():
                pa.paged_decode_attn(q, kp, vp, tt, ll, bs, w0.scale, out=out, workspace=ws)
        call.tensors = (q, kp, vp)
        return call

    res = {}
    bs = w0.bs
    W = -(-width // bs)
    ident = (np.arange(B, dtype=np.int32)[:, None] * W + np.arange(W, dtype=np.int32)[None, :]).astype(np.int32)
    res["paged_us"], _ = timed("paged", lambda like: setup(bs, w0.tables, w0.N, 0, like), kv_true)
    res["contiguous_us"], _ = timed("contiguous", lambda like: setup(bs, ident, B * W, 0, like), kv_true)
    res["masked_width_us"], _ = timed("masked width", lambda like: setup(bs, ident, B * W, width, like),
                                      B * width * Hkv * D * 4)
    for b2 in (16, 32, 64, 128, 256):
        nb = int(sum(-(-int(L) // b2) for L in lens))
        w2 = wl.make_workload(f"mixed bs{b2}", B, Hq, Hkv, D, b2, nb + 64, lens, seed=3, events=200, append=False)
        res[f"paged_bs{b2}_us"], _ = timed(f"paged bs {b2}", lambda like: setup(b2, w2.tables, w2.N, 0, like),
                                           kv_true)
    res = {k: round(v, 3) for k, v in res.items()}
    line = {
        "metric": "mixed-batch decode: width and gather contrasts (kernel us per call)",
        "value": res["paged_us"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": False,
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "mixed", "batch": B, "width": width, "true_tokens": int(lens.sum()),
                   "kv_bytes_true": kv_true, "kv_bytes_masked_width": B * width * Hkv * D * 4},
        "contrast": res,
        "width_penalty": round(res["masked_width_us"] / res["contiguous_us"], 2),
        "gather_penalty": round(res["paged_us"] / res["contiguous_us"], 3),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


def measure(args, torch, pa, w, steps, warmup, with_cpu):
    """Time the step on workload w: the fused step and the two-call step back to
    back, a HIP graph replay, per-launch event brackets, a same-size streaming
    read, and (with_cpu) the CPU oracle on a bounded sample."""
    layers = w.layers

    # ---- inputs, resident on the device
    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    tables = dev(w.tables)
    lens = dev(w.seq_lens)
    touched = decode_bytes(w) * layers
    R = args.replicas or (1 if layers > 1 else max(1, math.ceil((1 << 30) / touched)))
    host0 = w.layer(0)
    sets = []  # per replica: list over layers of (q, k_new, v_new, k_pool, v_pool)
    for r in range(R):
        per_layer = []
        for layer in range(layers):
            ld = host0 if layer == 0 else w.layer(layer)
            if r == 0:
                per_layer.append([dev(ld.q), dev(ld.k_new), dev(ld.v_new), dev(ld.k_pool), dev(ld.v_pool)])
            else:
                per_layer.append([t.clone() for t in sets[0][layer]])
        sets.append(per_layer)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float16, device="cuda")
    ws = pa.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.bs, w.W)
    torch.cuda.synchronize()

    def step(i):
        for q, kn, vn, kp, vp in sets[i % R]:
            pa.paged_decode_attn_append(q, kn, vn, kp, vp, tables, lens, w.bs, w.scale, out=out, workspace=ws)

    def step_two_calls(i):
        for q, kn, vn, kp, vp in sets[i % R]:
            pa.kv_append(kn, vn, kp, vp, tables, lens, w.bs)
            pa.paged_decode_attn(q, kp, vp, tables, lens, w.bs, w.scale, out=out, workspace=ws)

    def time_steps(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            fn(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    # ---- whole-step throughput (the two-call form of the same step beside it)
    ms_per_step = time_steps(step)
    two_call_ms_per_step = time_steps(step_two_calls)

    # ---- the same steps replayed from a HIP graph: one capture of G = min(R, K)
    # consecutive steps (through G replicas), replayed until K steps have run
    G = min(R, steps)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(G):
            step(i)
    reps = max(1, math.ceil(steps / G))
    for _ in range(max(1, math.ceil(warmup / G))):
        graph.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(reps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms_per_step = g0.elapsed_time(g1) / (reps * G)
    del graph

    # ---- per-launch durations (events around each launch)
    n_k = max(20, min(steps, 400))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_k)]
    ev_a = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_k)]
    for i in range(n_k):
        q, kn, vn, kp, vp = sets[i % R][i % layers]
        ev_a[i][0].record()
        pa.kv_append(kn, vn, kp, vp, tables, lens, w.bs)
        ev_a[i][1].record()
        ev[i][0].record()
        pa.paged_decode_attn_append(q, kn, vn, kp, vp, tables, lens, w.bs, w.scale, out=out, workspace=ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    app_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_a]))

    # launches back to back on the same stream: the average gap between
    # consecutive completions, i.e. a kernel's duration without launch gaps
    def back_to_back(call):
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record()
        for i in range(n_k):
            call(*sets[i % R][i % layers])
        b1.record()
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / n_k

    dec_b2b_ms = back_to_back(lambda q, kn, vn, kp, vp: pa.paged_decode_attn_append(
        q, kn, vn, kp, vp, tables, lens, w.bs, w.scale, out=out, workspace=ws))
    dec_only_b2b_ms = back_to_back(lambda q, kn, vn, kp, vp: pa.paged_decode_attn(
        q, kp, vp, tables, lens, w.bs, w.scale, out=out, workspace=ws))

    # ---- a plain streaming read of the same byte count (the achievable at this size)
    probe_us, probe_bytes = probe_read_us(args, torch, pa, decode_bytes(w, unique=True) + append_bytes(w), n_k)

    launch_bytes = decode_bytes(w) + append_bytes(w)
    unique_launch_bytes = decode_bytes(w, unique=True) + append_bytes(w)
    step_bytes = launch_bytes * layers
    unique_step_bytes = unique_launch_bytes * layers
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # the kernel's duration per launch: the smaller of two upper bounds, the
    # fused launches issued eagerly back to back (host-bound where the host
    # issues them more slowly than they run) and the graph replay of the same
    # launches (which adds the graph's own gaps between kernels)
    dec_graph_ms = graph_ms_per_step / layers
    dec_kernel_ms = min(dec_b2b_ms, dec_graph_ms)
    dec_gbs = launch_bytes / (dec_kernel_ms * 1e-3) / 1e9
    dec_unique_gbs = unique_launch_bytes / (dec_kernel_ms * 1e-3) / 1e9

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if with_cpu:
        import oracle

        orc = oracle.get()
        threads = min(16, os.cpu_count() or 1)
        kp_h = sets[0][0][3].cpu().numpy()
        vp_h = sets[0][0][4].cpu().numpy()
        q_h, kn_h, vn_h = (sets[0][0][j].cpu().numpy() for j in range(3))
        def sample(nthreads, seconds):
            reps, t_used = 0, 0.0
            start = time.perf_counter()
            while True:
                orc.kv_append(kn_h, vn_h, kp_h, vp_h, w.tables, w.seq_lens, w.bs)
                orc.paged_decode_attn(q_h, kp_h, vp_h, w.tables, w.seq_lens, w.bs, w.scale, nthreads=nthreads)
                reps += 1
                t_used = time.perf_counter() - start
                if t_used + t_used / reps > seconds:  # the next repetition would pass the bound
                    return reps, t_used

        reps, t_used = sample(threads, args.cpu_seconds * 0.75)
        reps1, t_used1 = sample(1, args.cpu_seconds * 0.25)
        per_layer_s = t_used / reps
        cpu = {
            "value": round((decode_bytes(w) + append_bytes(w)) / per_layer_s / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} x (kv_append + paged_decode_attn) of layer 0 of the same workload "
                      f"({w.B} rows), {threads} threads, {t_used:.2f} s",
            "rows_layers_per_s": round(w.B / per_layer_s, 2),
            "single_thread_value": round((decode_bytes(w) + append_bytes(w)) / (t_used1 / reps1) / 1e9, 4),
            "single_thread_sample": f"{reps1} x the same on 1 thread, {t_used1:.2f} s",
            "cpu_model": cpu_model(),
        }

    return dict(w=w, layers=layers, R=R, ms_per_step=ms_per_step, two_call_ms_per_step=two_call_ms_per_step,
                graph_ms_per_step=graph_ms_per_step, dec_kernel_ms=dec_kernel_ms, dec_b2b_ms=dec_b2b_ms,
                dec_graph_ms=dec_graph_ms, dec_ms=dec_ms, dec_only_b2b_ms=dec_only_b2b_ms, app_ms=app_ms,
                probe_us=probe_us, probe_bytes=probe_bytes, launch_bytes=launch_bytes,
                unique_launch_bytes=unique_launch_bytes, step_bytes=step_bytes, unique_step_bytes=unique_step_bytes,
                value=value, dec_gbs=dec_gbs, dec_unique_gbs=dec_unique_gbs, cpu=cpu)


GRADED = ("mixed", "uniform4096", "full_step")
TARGET_FRAC = 0.70


def graded_entry(m):
    """The decode kernel on one workload against the 70 %-of-peak target."""
    w = m["w"]
    frac = m["dec_unique_gbs"] / PEAK_HBM_GBS
    return {
        "decode_us": round(m["dec_kernel_ms"] * 1e3, 3),
        "GBs": round(m["dec_unique_gbs"], 2),
        "frac": round(frac, 4),
        "meets_target": bool(frac >= TARGET_FRAC),
        "target_decode_us": round(m["unique_launch_bytes"] / (TARGET_FRAC * PEAK_HBM_GBS * 1e9) * 1e6, 3),
        "bytes_per_launch": m["unique_launch_bytes"],
        "traffic": read_traffic(w.name),
        "probe_read_us": round(m["probe_us"], 3),
        "decode_over_probe_time": round(m["dec_kernel_ms"] * 1e3 / m["probe_us"], 3),
        "ms_per_step": round(m["ms_per_step"], 6),
        "rows_layers_per_s": round(w.B * m["layers"] / (m["ms_per_step"] * 1e-3), 1),
        "layers": m["layers"],
        "seq_len_sum": int(w.seq_lens.sum()),
    }



def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="uniform1024", choices=sorted(wl.CONFIGS))
    ap.add_argument("--replicas", type=int, default=0, help="pool replicas rotated per step (0 = auto, ~1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the oracle's timed sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help=f"after the bench, run {COPY_REPS} plain device copies of MIB MiB (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 counter runs into profiles/ and exit (no GPU)")
    ap.add_argument("--pmc-copy-mib", type=int, default=256, help="MiB of the calibration copy in those runs")
    ap.add_argument("--pmc-command", default="", help="the commands that made the counter runs (required with --pmc-summary)")
    ap.add_argument("--pmc-fp8", action="store_true", help="--pmc-summary of an --op fp8 run (E4M3-pool kernel)")
    ap.add_argument("--op", default="step", choices=["step", "copy_blocks", "scatter_prefill", "contrast", "fp8"],
                    help="step: the decode step (default); copy_blocks: the copy-on-write block copy alone; "
                         "scatter_prefill: the post-prefill scatter alone; contrast: the mixed batch decoded "
                         "paged, contiguous, at masked full width, and at block sizes 16..256; fp8: the step "
                         "over E4M3 pools on --config's shapes")
    ap.add_argument("--copy-pairs", type=int, default=1024, help="copy_blocks: block pairs per call")
    ap.add_argument("--kv", default="f16", choices=["f16", "fp8"], help="scatter_prefill: pool format")
    ap.add_argument("--no-graded", action="store_true",
                    help="skip the mixed, uniform-4096 and 28-layer workloads timed beside the default one")
    ap.add_argument("--graded-steps", type=int, default=40, help="timed steps of each graded workload")
    return ap.parse_args()


def main():
    args = parse()
    if args.pmc_summary:
        if not args.pmc_command.strip():
            sys.exit("--pmc-summary needs --pmc-command: the record names the counter runs it summarises")
        text = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config, args.pmc_copy_mib << 20,
                           args.pmc_command, fp8=args.pmc_fp8)
        os.makedirs(PROFILES, exist_ok=True)
        with open(traffic_file(args.config, args.pmc_fp8), "w") as f:
            f.write(text)
        print(text, end="")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            f"bench.py measures one GPU only: the decode path has no cross-GPU step here "
            f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import paged_kv_cache_06_amd as pa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.op == "copy_blocks":
        bench_copy_blocks(args, torch, pa)
        return
    if args.op == "scatter_prefill":
        bench_scatter_prefill(args, torch, pa)
        return
    if args.op == "contrast":
        bench_contrast(args, torch, pa)
        return
    if args.op == "fp8":
        bench_fp8(args, torch, pa)
        return
    w = wl.CONFIGS[args.config]()
    m = measure(args, torch, pa, w, args.steps, args.warmup, not args.no_cpu_baseline)
    graded = None
    if not args.no_graded and args.config == "uniform1024":
        graded = {"target_frac": TARGET_FRAC}
        for name in GRADED:
            gm = measure(args, torch, pa, wl.CONFIGS[name](), args.graded_steps, min(args.warmup, 10), False)
            graded[name] = graded_entry(gm)
            del gm
            torch.cuda.empty_cache()
    layers, R = m["layers"], m["R"]
    ms_per_step, two_call_ms_per_step = m["ms_per_step"], m["two_call_ms_per_step"]
    graph_ms_per_step, dec_kernel_ms, dec_b2b_ms = m["graph_ms_per_step"], m["dec_kernel_ms"], m["dec_b2b_ms"]
    dec_graph_ms, dec_ms, dec_only_b2b_ms, app_ms = m["dec_graph_ms"], m["dec_ms"], m["dec_only_b2b_ms"], m["app_ms"]
    probe_us, probe_bytes, step_bytes = m["probe_us"], m["probe_bytes"], m["step_bytes"]
    unique_step_bytes, unique_launch_bytes = m["unique_step_bytes"], m["unique_launch_bytes"]
    value, dec_gbs, dec_unique_gbs, cpu = m["value"], m["dec_gbs"], m["dec_unique_gbs"], m["cpu"]

    cfg = {
        "workload": w.name,
        "batch": w.B,
        "layers": layers,
        "num_heads": w.Hq,
        "num_kv_heads": w.Hkv,
        "head_dim": w.D,
        "block_size": w.bs,
        "max_blocks_per_seq": w.W,
        "pool_blocks": w.N,
        "seq_len_min": int(w.seq_lens.min()),
        "seq_len_max": int(w.seq_lens.max()),
        "seq_len_sum": int(w.seq_lens.sum()),
        "replicas": R,
    }
    line = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) and rows*layers/s at batch 32",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": cfg,
        "pct_of_peak": round(100 * unique_step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "rows_layers_per_s": round(w.B * layers / (ms_per_step * 1e-3), 1),
        "bytes_per_step": step_bytes,
        "unique_bytes_per_step": unique_step_bytes,
        "two_call_ms_per_step": round(two_call_ms_per_step, 6),
        "two_call_value": round(step_bytes / (two_call_ms_per_step * 1e-3) / 1e9, 2),
        "graph_ms_per_step": round(graph_ms_per_step, 6),
        "graph_value": round(step_bytes / (graph_ms_per_step * 1e-3) / 1e9, 2),
        "decode_us": round(dec_kernel_ms * 1e3, 3),
        "decode_us_eager_back_to_back": round(dec_b2b_ms * 1e3, 3),
        "decode_us_graph": round(dec_graph_ms * 1e3, 3),
        "decode_us_bracketed": round(dec_ms * 1e3, 3),
        "decode_without_append_us": round(dec_only_b2b_ms * 1e3, 3),
        "append_us": round(app_ms * 1e3, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(dec_unique_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_unique_gbs / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(w.name),
            "kernel": "decode_kernel",
            "bytes_per_launch": unique_launch_bytes,
            "logical_GBs": round(dec_gbs, 2),
        },
        "probe_read": {"bytes": probe_bytes, "us": round(probe_us, 3),
                       "GBs": round(probe_bytes / (probe_us * 1e-6) / 1e9, 2),
                       "decode_over_probe_time": round(dec_kernel_ms * 1e3 / probe_us, 3)},
        "cpu_baseline": cpu,
        "graded": graded,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    copy_calibration(args, torch)


if __name__ == "__main__":
    main()
