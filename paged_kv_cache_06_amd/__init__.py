"""Python binding of libpagedattn (paged KV-cache decode attention, MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libpagedattn.so`` (built from the sources under ``csrc/`` by ``build.py``).
torch is used for device memory and streams. There is no CPU fallback: if
the library is missing, or a tensor is not on the GPU, the call raises.

Names and argument order follow the C ABI in ``include/pagedattn.h``:

  kv_append(k_new, v_new, k_pool, v_pool, block_tables, seq_lens, block_size)
  paged_decode_attn(q, k_pool, v_pool, block_tables, seq_lens, block_size,
                    scale, out=None, workspace=None)
      (workspace=None: a zeroed workspace kept by the binding per (device,
      stream) and reused by later calls on that stream; calls to be
      captured in a HIP graph should pass their own, made beforehand)
  paged_decode_attn_noalloc(q, k_pool, v_pool, block_tables, seq_lens,
                            block_size, scale, out=None)   (no workspace:
                                                           static scratch)
  paged_decode_attn_append(q, k_new, v_new, k_pool, v_pool, block_tables,
                           seq_lens, block_size, scale, out=None,
                           workspace=None)   (the two calls above, fused)
  kv_copy_blocks(k_pool, v_pool, src, dst, block_size)   (copy-on-write)
  kv_scatter_prefill(k_src, v_src, k_pool, v_pool, block_tables,
                     prompt_lens, block_size)            (after prefill)
  paged_gather_kv(k_pool, v_pool, block_tables, seq_lens, block_size)
  paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                              block_size, max_blocks_per_seq)
  kv_append_fp8(k_new, v_new, k_pool, v_pool, block_tables, seq_lens,
                block_size, k_scale, v_scale)              (E4M3 pools)
  paged_decode_attn_fp8(q, k_pool, v_pool, block_tables, seq_lens,
                        block_size, scale, k_scale, v_scale, out=None,
                        workspace=None)                    (E4M3 pools)
  paged_decode_attn_append_fp8(q, k_new, v_new, k_pool, v_pool, block_tables,
                               seq_lens, block_size, scale, k_scale, v_scale,
                               out=None, workspace=None)  (the two above, fused)
  kv_copy_blocks_fp8(k_pool, v_pool, src, dst, block_size)   (E4M3 pools)
  kv_scatter_prefill_fp8(k_src, v_src, k_pool, v_pool, block_tables,
                         prompt_lens, block_size, k_scale, v_scale)

Pool layouts: k_pool [N][Hkv][D/8][bs][8], v_pool [N][Hkv][D][bs] (fp16);
E4M3 pools (uint8 codes, or torch.float8_e4m3fn): k_pool [N][Hkv][D/16][bs][16],
v_pool [N][Hkv][D][bs].
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_OK = 0
_ERRORS = {1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_HIP", 4: "PA_ERR_WORKSPACE",
           5: "PA_ERR_SCRATCH"}

_lib = None


class PagedAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg}: {_ERRORS.get(status, status)}")
        self.status = status


def lib():
    """Load libpagedattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with paged_kv_cache_06_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.paged_decode_supported.argtypes = [i32] * 4
    L.paged_decode_supported.restype = ctypes.c_int
    L.kv_append.argtypes = [vp] * 6 + [i32] * 6 + [vp]
    L.kv_append.restype = ctypes.c_int
    L.paged_decode_workspace_size.argtypes = [i32] * 6
    L.paged_decode_workspace_size.restype = sz
    L.paged_decode_workspace_init.argtypes = [vp, sz, vp]
    L.paged_decode_workspace_init.restype = ctypes.c_int
    L.paged_decode_attn.argtypes = [vp] * 6 + [i32] * 7 + [ctypes.c_float, vp, sz, vp]
    L.paged_decode_attn.restype = ctypes.c_int
    L.paged_decode_attn_noalloc.argtypes = [vp] * 6 + [i32] * 7 + [ctypes.c_float, vp]
    L.paged_decode_attn_noalloc.restype = ctypes.c_int
    L.paged_decode_attn_append.argtypes = [vp] * 8 + [i32] * 7 + [ctypes.c_float, vp, sz, vp]
    L.paged_decode_attn_masked.argtypes = [vp] * 6 + [i32] * 7 + [ctypes.c_float, i32, vp, sz, vp]
    L.paged_decode_attn_masked.restype = ctypes.c_int
    L.paged_decode_attn_append.restype = ctypes.c_int
    L.kv_copy_blocks.argtypes = [vp] * 4 + [i32] * 6 + [ctypes.c_int64, vp]
    L.kv_copy_blocks.restype = ctypes.c_int
    L.kv_scatter_prefill.argtypes = [vp] * 6 + [i32] * 7 + [vp]
    L.kv_scatter_prefill.restype = ctypes.c_int
    L.kv_scatter_prefill_fp8.argtypes = [vp] * 6 + [i32] * 7 + [ctypes.c_float] * 2 + [vp]
    L.kv_scatter_prefill_fp8.restype = ctypes.c_int
    L.pa_probe_read.argtypes = [vp, sz, vp, i32, vp]
    L.pa_probe_read.restype = ctypes.c_int
    L.kv_copy_blocks_fp8.argtypes = [vp] * 4 + [i32] * 6 + [ctypes.c_int64, vp]
    L.kv_copy_blocks_fp8.restype = ctypes.c_int
    L.kv_append_fp8.argtypes = [vp] * 6 + [i32] * 6 + [ctypes.c_float] * 2 + [vp]
    L.kv_append_fp8.restype = ctypes.c_int
    L.paged_decode_attn_fp8.argtypes = [vp] * 6 + [i32] * 7 + [ctypes.c_float] * 3 + [vp, sz, vp]
    L.paged_decode_attn_fp8.restype = ctypes.c_int
    L.paged_decode_attn_append_fp8.argtypes = [vp] * 8 + [i32] * 7 + [ctypes.c_float] * 3 + [vp, sz, vp]
    L.paged_decode_attn_append_fp8.restype = ctypes.c_int
    L.paged_gather_kv.argtypes = [vp] * 6 + [i32] * 6 + [vp]
    L.paged_gather_kv.restype = ctypes.c_int
    _lib = L
    return L


def _check(status, what):
    if status != PA_OK:
        raise PagedAttnError(status, what)


def _dev(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _pool_dims(k_pool, v_pool, block_size):
    N, Hkv, D8, bs, eight = k_pool.shape
    if eight != 8 or bs != block_size:
        raise ValueError(f"k_pool must be [N][Hkv][D/8][{block_size}][8], got {tuple(k_pool.shape)}")
    D = D8 * 8
    if tuple(v_pool.shape) != (N, Hkv, D, bs):
        raise ValueError(f"v_pool must be {(N, Hkv, D, bs)}, got {tuple(v_pool.shape)}")
    return N, Hkv, D


def paged_decode_supported(num_heads, num_kv_heads, head_dim, block_size) -> bool:
    return bool(lib().paged_decode_supported(num_heads, num_kv_heads, head_dim, block_size))


def kv_append(k_new, v_new, k_pool, v_pool, block_tables, seq_lens, block_size, stream=None):
    """Write k_new / v_new [B][Hkv][D] at position seq_lens[b]-1 of each row."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, W = block_tables.shape
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new / v_new must be [B][Hkv][D]")
    if tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be [B]")
    st = lib().kv_append(
        _dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hkv, D, block_size, W, N, _stream(stream),
    )
    _check(st, "kv_append")


def paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq):
    return int(lib().paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                 max_blocks_per_seq))


def new_workspace(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, device="cuda"):
    """A zeroed workspace (uint8 tensor) of the size paged_decode_attn needs
    (the fill kernel runs on torch's current stream)."""
    n = paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    paged_decode_workspace_init(ws)
    return ws


def paged_decode_workspace_init(workspace, stream=None):
    st = lib().paged_decode_workspace_init(_dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                           _stream(stream))
    _check(st, "paged_decode_workspace_init")


def _on(stream):
    """Context in which a call's own tensors are made: torch's allocator then
    ties their memory to the call's stream (so it is not handed out again
    while the call may still use it) and their fill kernels run on it, ahead
    of the call."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _new_on(stream, shape, dtype, device, zero=False):
    with _on(stream):
        return (torch.zeros if zero else torch.empty)(shape, dtype=dtype, device=device)


# Workspaces the binding keeps for calls made without one: one per (device,
# stream), grown (never shrunk) to the largest size asked for on that stream.
# Calls on one stream run in order, and each leaves the workspace's counters
# at zero, so they can share it; calls on different streams get different
# ones. A replacement is made on the same stream, so torch's allocator does
# not hand the old memory out again while queued calls may still use it.
_ws_cache = {}


def _call_workspace(workspace, B, Hq, Hkv, D, block_size, W, device, stream):
    """The caller's workspace, or the binding's cached one for the call's
    (device, stream), zero-filled on that stream when it is made."""
    if workspace is not None:
        return workspace
    n = paged_decode_workspace_size(B, Hq, Hkv, D, block_size, W)
    dev = torch.device(device)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), s.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < n:
        with torch.cuda.stream(s):
            ws = new_workspace(B, Hq, Hkv, D, block_size, W, device=dev)
        _ws_cache[key] = ws
    return ws


def paged_decode_attn(q, k_pool, v_pool, block_tables, seq_lens, block_size, scale, out=None, workspace=None,
                      stream=None):
    """out [B][Hq][D] fp16 = softmax(scale q k^T) v over each row's own blocks."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the pools")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    if out is None:
        out = _new_on(stream, (B, Hq, D), torch.float16, q.device)
    workspace = _call_workspace(workspace, B, Hq, Hkv, D, block_size, W, q.device, stream)
    st = lib().paged_decode_attn(
        _dev(out, "out", torch.float16, 3), _dev(q, "q", torch.float16, 3),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hq, Hkv, D, block_size, W, N, ctypes.c_float(scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream),
    )
    _check(st, "paged_decode_attn")
    return out


def paged_decode_attn_noalloc(q, k_pool, v_pool, block_tables, seq_lens, block_size, scale, out=None, stream=None):
    """paged_decode_attn with the library's static device scratch as its
    workspace: the C call allocates nothing (pass `out` to allocate nothing
    here either). Calls that overlap on one GPU race on the scratch."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the pools")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    if out is None:
        out = _new_on(stream, (B, Hq, D), torch.float16, q.device)
    st = lib().paged_decode_attn_noalloc(
        _dev(out, "out", torch.float16, 3), _dev(q, "q", torch.float16, 3),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hq, Hkv, D, block_size, W, N, ctypes.c_float(scale), _stream(stream),
    )
    _check(st, "paged_decode_attn_noalloc")
    return out


def paged_decode_attn_masked(q, k_pool, v_pool, block_tables, seq_lens, block_size, scale, width, out=None,
                             workspace=None, stream=None):
    """paged_decode_attn's result computed over `width` tokens of every row,
    positions past each row's length masked (the masked-width contrast)."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the pools")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    if out is None:
        out = _new_on(stream, (B, Hq, D), torch.float16, q.device)
    workspace = _call_workspace(workspace, B, Hq, Hkv, D, block_size, W, q.device, stream)
    st = lib().paged_decode_attn_masked(
        _dev(out, "out", torch.float16, 3), _dev(q, "q", torch.float16, 3),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hq, Hkv, D, block_size, W, N, ctypes.c_float(scale), int(width),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream),
    )
    _check(st, "paged_decode_attn_masked")
    return out


def paged_decode_attn_append(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, block_size, scale, out=None,
                             workspace=None, stream=None):
    """kv_append(k_new, v_new, ...) then paged_decode_attn(q, ...), in one launch."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the pools")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new / v_new must be [B][Hkv][D]")
    if out is None:
        out = _new_on(stream, (B, Hq, D), torch.float16, q.device)
    workspace = _call_workspace(workspace, B, Hq, Hkv, D, block_size, W, q.device, stream)
    st = lib().paged_decode_attn_append(
        _dev(out, "out", torch.float16, 3), _dev(q, "q", torch.float16, 3),
        _dev(k_new, "k_new", torch.float16, 3), _dev(v_new, "v_new", torch.float16, 3),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hq, Hkv, D, block_size, W, N, ctypes.c_float(scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream),
    )
    _check(st, "paged_decode_attn_append")
    return out


def kv_copy_blocks(k_pool, v_pool, src, dst, block_size, stream=None):
    """Block dst[i] <- block src[i] in both pools (copy-on-write); pools of one
    layer ([N][Hkv][D/8][bs][8], [N][Hkv][D][bs]) or of several layers with a
    leading layer dimension, every layer copied."""
    layered = k_pool.dim() == 6
    kp1 = k_pool[0] if layered else k_pool
    vp1 = v_pool[0] if layered else v_pool
    N, Hkv, D = _pool_dims(kp1, vp1, block_size)
    layers = k_pool.shape[0] if layered else 1
    if layered and (v_pool.dim() != 5 or v_pool.shape[0] != layers):
        raise ValueError("k_pool / v_pool must both have the same leading layer dimension")
    if tuple(src.shape) != tuple(dst.shape) or src.dim() != 1:
        raise ValueError("src and dst must be 1-D of the same length")
    st = lib().kv_copy_blocks(
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(src, "src", torch.int32, 1), _dev(dst, "dst", torch.int32, 1),
        src.numel(), Hkv, D, block_size, N, layers, ctypes.c_int64(N * Hkv * D * block_size), _stream(stream),
    )
    _check(st, "kv_copy_blocks")


def kv_scatter_prefill(k_src, v_src, k_pool, v_pool, block_tables, prompt_lens, block_size, stream=None):
    """Row b's prompt KV (the last prompt_lens[b] of the S positions of a
    left-padded prefill group, k_src / v_src [B][Hkv][S][D]) into its blocks,
    padding dropped."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, W = block_tables.shape
    if k_src.dim() != 4 or tuple(k_src.shape[:2]) != (B, Hkv) or k_src.shape[3] != D:
        raise ValueError("k_src must be [B][Hkv][S][D]")
    if tuple(v_src.shape) != tuple(k_src.shape):
        raise ValueError("v_src must have k_src's shape")
    if tuple(prompt_lens.shape) != (B,):
        raise ValueError("prompt_lens must be [B]")
    st = lib().kv_scatter_prefill(
        _dev(k_src, "k_src", torch.float16, 4), _dev(v_src, "v_src", torch.float16, 4),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(prompt_lens, "prompt_lens", torch.int32, 1),
        B, Hkv, D, block_size, W, N, k_src.shape[2], _stream(stream),
    )
    _check(st, "kv_scatter_prefill")


def paged_gather_kv(k_pool, v_pool, block_tables, seq_lens, block_size, k_out=None, v_out=None, stream=None):
    """Debug path: [B][Hkv][W*bs][D] copies of each row's tokens (positions
    past seq_lens[b] are left as they were in k_out / v_out)."""
    N, Hkv, D = _pool_dims(k_pool, v_pool, block_size)
    B, W = block_tables.shape
    shape = (B, Hkv, W * block_size, D)
    if k_out is None:
        k_out = _new_on(stream, shape, torch.float16, k_pool.device, zero=True)
    if v_out is None:
        v_out = _new_on(stream, shape, torch.float16, k_pool.device, zero=True)
    st = lib().paged_gather_kv(
        _dev(k_out, "k_out", torch.float16, 4), _dev(v_out, "v_out", torch.float16, 4),
        _dev(k_pool, "k_pool", torch.float16), _dev(v_pool, "v_pool", torch.float16),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hkv, D, block_size, W, N, _stream(stream),
    )
    _check(st, "paged_gather_kv")
    return k_out, v_out


def _fp8_pool(t, name):
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _dev(t, name, torch.uint8)
    return t


def _pool_dims_fp8(k_pool, v_pool, block_size):
    N, Hkv, D16, bs, sixteen = k_pool.shape
    if sixteen != 16 or bs != block_size:
        raise ValueError(f"k_pool must be [N][Hkv][D/16][{block_size}][16], got {tuple(k_pool.shape)}")
    D = D16 * 16
    if tuple(v_pool.shape) != (N, Hkv, D, bs):
        raise ValueError(f"v_pool must be {(N, Hkv, D, bs)}, got {tuple(v_pool.shape)}")
    return N, Hkv, D


def kv_append_fp8(k_new, v_new, k_pool, v_pool, block_tables, seq_lens, block_size, k_scale, v_scale,
                  stream=None):
    """Quantize k_new / v_new [B][Hkv][D] (fp16) to E4M3 codes of x / scale
    and write them at position seq_lens[b]-1 of each row of the E4M3 pools."""
    k_pool, v_pool = _fp8_pool(k_pool, "k_pool"), _fp8_pool(v_pool, "v_pool")
    N, Hkv, D = _pool_dims_fp8(k_pool, v_pool, block_size)
    B, W = block_tables.shape
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new / v_new must be [B][Hkv][D]")
    if tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be [B]")
    st = lib().kv_append_fp8(
        _dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16),
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hkv, D, block_size, W, N, ctypes.c_float(k_scale), ctypes.c_float(v_scale), _stream(stream),
    )
    _check(st, "kv_append_fp8")


def paged_decode_attn_fp8(q, k_pool, v_pool, block_tables, seq_lens, block_size, scale, k_scale, v_scale,
                          out=None, workspace=None, stream=None):
    """paged_decode_attn over E4M3 pools whose elements are code * k_scale
    (keys) and code * v_scale (values)."""
    k_pool, v_pool = _fp8_pool(k_pool, "k_pool"), _fp8_pool(v_pool, "v_pool")
    N, Hkv, D = _pool_dims_fp8(k_pool, v_pool, block_size)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the pools")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    if out is None:
        out = _new_on(stream, (B, Hq, D), torch.float16, q.device)
    workspace = _call_workspace(workspace, B, Hq, Hkv, D, block_size, W, q.device, stream)
    st = lib().paged_decode_attn_fp8(
        _dev(out, "out", torch.float16, 3), _dev(q, "q", torch.float16, 3),
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hq, Hkv, D, block_size, W, N, ctypes.c_float(scale), ctypes.c_float(k_scale), ctypes.c_float(v_scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream),
    )
    _check(st, "paged_decode_attn_fp8")
    return out


def paged_decode_attn_append_fp8(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, block_size, scale,
                                 k_scale, v_scale, out=None, workspace=None, stream=None):
    """kv_append_fp8 + paged_decode_attn_fp8 in one launch (same results)."""
    k_pool, v_pool = _fp8_pool(k_pool, "k_pool"), _fp8_pool(v_pool, "v_pool")
    N, Hkv, D = _pool_dims_fp8(k_pool, v_pool, block_size)
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the pools")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new / v_new must be [B][Hkv][D]")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    if out is None:
        out = _new_on(stream, (B, Hq, D), torch.float16, q.device)
    workspace = _call_workspace(workspace, B, Hq, Hkv, D, block_size, W, q.device, stream)
    st = lib().paged_decode_attn_append_fp8(
        _dev(out, "out", torch.float16, 3), _dev(q, "q", torch.float16, 3),
        _dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16),
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, Hq, Hkv, D, block_size, W, N, ctypes.c_float(scale), ctypes.c_float(k_scale), ctypes.c_float(v_scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream),
    )
    _check(st, "paged_decode_attn_append_fp8")
    return out


def kv_copy_blocks_fp8(k_pool, v_pool, src, dst, block_size, stream=None):
    """kv_copy_blocks for E4M3 pools ([N][Hkv][D/16][bs][16], [N][Hkv][D][bs]
    bytes, or with a leading layer dimension, every layer copied)."""
    k_pool, v_pool = _fp8_pool(k_pool, "k_pool"), _fp8_pool(v_pool, "v_pool")
    layered = k_pool.dim() == 6
    kp1 = k_pool[0] if layered else k_pool
    vp1 = v_pool[0] if layered else v_pool
    N, Hkv, D = _pool_dims_fp8(kp1, vp1, block_size)
    layers = k_pool.shape[0] if layered else 1
    if layered and (v_pool.dim() != 5 or v_pool.shape[0] != layers):
        raise ValueError("k_pool / v_pool must both have the same leading layer dimension")
    if tuple(src.shape) != tuple(dst.shape) or src.dim() != 1:
        raise ValueError("src and dst must be 1-D of the same length")
    st = lib().kv_copy_blocks_fp8(
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(src, "src", torch.int32, 1), _dev(dst, "dst", torch.int32, 1),
        src.numel(), Hkv, D, block_size, N, layers, ctypes.c_int64(N * Hkv * D * block_size), _stream(stream),
    )
    _check(st, "kv_copy_blocks_fp8")


def kv_scatter_prefill_fp8(k_src, v_src, k_pool, v_pool, block_tables, prompt_lens, block_size, k_scale, v_scale,
                           stream=None):
    """kv_scatter_prefill into E4M3 pools, each element quantized (code of x / scale)."""
    k_pool, v_pool = _fp8_pool(k_pool, "k_pool"), _fp8_pool(v_pool, "v_pool")
    N, Hkv, D = _pool_dims_fp8(k_pool, v_pool, block_size)
    B, Hs, S, Ds = k_src.shape
    if (Hs, Ds) != (Hkv, D) or tuple(v_src.shape) != (B, Hkv, S, D):
        raise ValueError(f"k_src / v_src must be [B][{Hkv}][S][{D}]")
    W = block_tables.shape[1]
    if block_tables.shape[0] != B or tuple(prompt_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][W] and prompt_lens [B]")
    st = lib().kv_scatter_prefill_fp8(
        _dev(k_src, "k_src", torch.float16, 4), _dev(v_src, "v_src", torch.float16, 4),
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(prompt_lens, "prompt_lens", torch.int32, 1),
        B, Hkv, D, block_size, W, N, S, ctypes.c_float(k_scale), ctypes.c_float(v_scale), _stream(stream),
    )
    _check(st, "kv_scatter_prefill_fp8")


def probe_read(buf, sink, num_workgroups=2048, stream=None):
    """Measurement aid: read every byte of `buf` (a contiguous GPU tensor) once
    (pa_probe_read); `sink` is a uint32 GPU tensor of num_workgroups words."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if sink.numel() < num_workgroups:
        raise ValueError("sink must hold num_workgroups words")
    st = lib().pa_probe_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                             _dev(sink, "sink", torch.int32), num_workgroups, _stream(stream))
    _check(st, "pa_probe_read")

