"""CPU oracle for paged decode attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It loads ``liboracle.so`` built from
``oracle.cpp`` with plain ``g++`` (``-O2 -ffp-contract=off``, no fast-math)
and exposes numpy-in / numpy-out wrappers. It shares no code with the HIP
library and imports nothing from the product package.

Pool layout the oracle reads (fp16 bit patterns as uint16):
  K: [N][Hkv][D/8][bs][8]    V: [N][Hkv][D][bs]
FP8 pools (E4M3 codes as uint8):
  K: [N][Hkv][D/16][bs][16]  V: [N][Hkv][D][bs]
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.cpp")
LIB = os.path.join(_HERE, "liboracle.so")

CXXFLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(extra_flags=(), out=LIB) -> str:
    """Compile oracle.cpp into a shared library with g++ and return its path."""
    cmd = ["g++", *CXXFLAGS, *extra_flags, SRC, "-o", out]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _load(path=None):
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB
    if not os.path.exists(p):
        build(out=p)
    lib = ctypes.CDLL(p)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f32p = ctypes.POINTER(ctypes.c_float)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i32 = ctypes.c_int32
    lib.oracle_half_to_float.argtypes = [f32p, u16p, ctypes.c_int64]
    lib.oracle_half_to_float.restype = None
    lib.oracle_float_to_half.argtypes = [u16p, f32p, ctypes.c_int64]
    lib.oracle_float_to_half.restype = None
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32 = ctypes.c_float
    lib.oracle_fp8_to_float.argtypes = [f32p, u8p, ctypes.c_int64]
    lib.oracle_fp8_to_float.restype = None
    lib.oracle_float_to_fp8.argtypes = [u8p, f32p, ctypes.c_int64]
    lib.oracle_float_to_fp8.restype = None
    lib.oracle_quantize_fp8.argtypes = [u8p, u16p, ctypes.c_int64, f32]
    lib.oracle_quantize_fp8.restype = None
    lib.oracle_kv_append_fp8.argtypes = [u16p, u16p, u8p, u8p, i32p, i32p] + [i32] * 6 + [f32, f32]
    lib.oracle_kv_append_fp8.restype = ctypes.c_int
    lib.oracle_paged_decode_attn_fp8.argtypes = [f32p, u16p, u16p, u8p, u8p, i32p, i32p] + [i32] * 7 + [
        f32, f32, f32, i32]
    lib.oracle_paged_decode_attn_fp8.restype = ctypes.c_int
    lib.oracle_kv_scatter_prefill_fp8.argtypes = [u16p, u16p, u8p, u8p, i32p, i32p] + [i32] * 7 + [f32, f32]
    lib.oracle_kv_scatter_prefill_fp8.restype = ctypes.c_int
    lib.oracle_kv_copy_blocks_fp8.argtypes = [u8p, u8p, i32p, i32p] + [i32] * 5
    lib.oracle_kv_copy_blocks_fp8.restype = ctypes.c_int
    lib.oracle_kv_append.argtypes = [u16p, u16p, u16p, u16p, i32p, i32p] + [i32] * 6
    lib.oracle_kv_append.restype = ctypes.c_int
    lib.oracle_kv_copy_blocks.argtypes = [u16p, u16p, i32p, i32p] + [i32] * 5
    lib.oracle_kv_copy_blocks.restype = ctypes.c_int
    lib.oracle_kv_scatter_prefill.argtypes = [u16p, u16p, u16p, u16p, i32p, i32p] + [i32] * 7
    lib.oracle_kv_scatter_prefill.restype = ctypes.c_int
    lib.oracle_gather_kv.argtypes = [u16p, u16p, u16p, u16p, i32p, i32p] + [i32] * 6
    lib.oracle_gather_kv.restype = ctypes.c_int
    lib.oracle_paged_decode_attn.argtypes = [f32p, u16p, u16p, u16p, u16p, i32p, i32p] + [i32] * 7 + [
        ctypes.c_float,
        i32,
    ]
    lib.oracle_paged_decode_attn.restype = ctypes.c_int
    lib.oracle_dense_attn.argtypes = [f32p, u16p, u16p, u16p] + [i32] * 4 + [ctypes.c_float]
    lib.oracle_dense_attn.restype = ctypes.c_int
    lib.oracle_validate.argtypes = [i32p, i32p] + [i32] * 5
    lib.oracle_validate.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


class Oracle:
    """numpy wrappers around one build of the oracle library."""

    def __init__(self, path=None):
        self.lib = _load(path)

    @staticmethod
    def _p(a, ctype):
        assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
        return a.ctypes.data_as(ctypes.POINTER(ctype))

    @staticmethod
    def _bits(a):
        a = np.ascontiguousarray(a)
        return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.uint16, copy=False)

    def half_to_float(self, bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float32)
        self.lib.oracle_half_to_float(self._p(out, ctypes.c_float), self._p(bits, ctypes.c_uint16), bits.size)
        return out

    def float_to_half(self, x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_float_to_half(self._p(out, ctypes.c_uint16), self._p(x, ctypes.c_float), x.size)
        return out

    def fp8_to_float(self, codes):
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape, np.float32)
        self.lib.oracle_fp8_to_float(self._p(out, ctypes.c_float), self._p(codes, ctypes.c_uint8), codes.size)
        return out

    def float_to_fp8(self, x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint8)
        self.lib.oracle_float_to_fp8(self._p(out, ctypes.c_uint8), self._p(x, ctypes.c_float), x.size)
        return out

    def quantize_fp8(self, x, scale):
        """fp16 array -> E4M3 codes of x / scale (uint8, same shape)."""
        bits = self._bits(np.asarray(x, dtype=np.float16))
        out = np.empty(bits.shape, np.uint8)
        self.lib.oracle_quantize_fp8(self._p(out, ctypes.c_uint8), self._p(bits, ctypes.c_uint16), bits.size,
                                     ctypes.c_float(scale))
        return out

    def kv_append_fp8(self, k_new, v_new, k_pool, v_pool, tables, seq_lens, bs, k_scale, v_scale):
        """In-place quantizing append into uint8 pools; returns the C status."""
        B, Hkv, D = k_new.shape
        W = tables.shape[1]
        N = k_pool.shape[0]
        assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
        t = np.ascontiguousarray(tables, dtype=np.int32)
        s = np.ascontiguousarray(seq_lens, dtype=np.int32)
        return self.lib.oracle_kv_append_fp8(
            self._p(self._bits(k_new), ctypes.c_uint16), self._p(self._bits(v_new), ctypes.c_uint16),
            self._p(k_pool, ctypes.c_uint8), self._p(v_pool, ctypes.c_uint8),
            self._p(t, ctypes.c_int32), self._p(s, ctypes.c_int32),
            B, Hkv, D, bs, W, N, ctypes.c_float(k_scale), ctypes.c_float(v_scale),
        )

    def paged_decode_attn_fp8(self, q, k_pool, v_pool, tables, seq_lens, bs, scale, k_scale, v_scale, nthreads=1):
        """FP8 pools (uint8 codes); returns (out_f32 [B][Hq][D], out_f16 [B][Hq][D])."""
        B, Hq, D = q.shape
        Hkv = k_pool.shape[1]
        W = tables.shape[1]
        N = k_pool.shape[0]
        assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
        of = np.empty((B, Hq, D), np.float32)
        oh = np.empty((B, Hq, D), np.uint16)
        t = np.ascontiguousarray(tables, dtype=np.int32)
        s = np.ascontiguousarray(seq_lens, dtype=np.int32)
        rc = self.lib.oracle_paged_decode_attn_fp8(
            self._p(of, ctypes.c_float), self._p(oh, ctypes.c_uint16), self._p(self._bits(q), ctypes.c_uint16),
            self._p(np.ascontiguousarray(k_pool), ctypes.c_uint8), self._p(np.ascontiguousarray(v_pool), ctypes.c_uint8),
            self._p(t, ctypes.c_int32), self._p(s, ctypes.c_int32),
            B, Hq, Hkv, D, bs, W, N,
            ctypes.c_float(scale), ctypes.c_float(k_scale), ctypes.c_float(v_scale), int(nthreads),
        )
        if rc != 0:
            raise ValueError(f"oracle_paged_decode_attn_fp8 failed: {rc}")
        return of, oh.view(np.float16)

    def kv_append(self, k_new, v_new, k_pool, v_pool, tables, seq_lens, bs):
        """In-place append into k_pool / v_pool (fp16 arrays); returns the C status."""
        B, Hkv, D = k_new.shape
        W = tables.shape[1]
        N = k_pool.shape[0]
        kp, vp = k_pool.view(np.uint16), v_pool.view(np.uint16)
        t = np.ascontiguousarray(tables, dtype=np.int32)
        s = np.ascontiguousarray(seq_lens, dtype=np.int32)
        return self.lib.oracle_kv_append(
            self._p(self._bits(k_new), ctypes.c_uint16),
            self._p(self._bits(v_new), ctypes.c_uint16),
            self._p(kp, ctypes.c_uint16),
            self._p(vp, ctypes.c_uint16),
            self._p(t, ctypes.c_int32),
            self._p(s, ctypes.c_int32),
            B, Hkv, D, bs, W, N,
        )

    def kv_copy_blocks(self, k_pool, v_pool, src, dst):
        """In-place: block dst[i] <- block src[i] (K and V), pairs in order; returns the C status."""
        N, Hkv = k_pool.shape[0], k_pool.shape[1]
        D = v_pool.shape[2]
        bs = v_pool.shape[3]
        kp, vp = k_pool.view(np.uint16), v_pool.view(np.uint16)
        s = np.ascontiguousarray(src, dtype=np.int32)
        d = np.ascontiguousarray(dst, dtype=np.int32)
        assert s.shape == d.shape and s.ndim == 1
        return self.lib.oracle_kv_copy_blocks(
            self._p(kp, ctypes.c_uint16), self._p(vp, ctypes.c_uint16),
            self._p(s, ctypes.c_int32), self._p(d, ctypes.c_int32),
            s.size, Hkv, D, bs, N,
        )

    def kv_copy_blocks_fp8(self, k_pool, v_pool, src, dst):
        """In-place on uint8 E4M3 pools ([N][Hkv][D/16][bs][16], [N][Hkv][D][bs]); returns the C status."""
        N, Hkv = k_pool.shape[0], k_pool.shape[1]
        D, bs = v_pool.shape[2], v_pool.shape[3]
        assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
        s = np.ascontiguousarray(src, dtype=np.int32)
        d = np.ascontiguousarray(dst, dtype=np.int32)
        assert s.shape == d.shape and s.ndim == 1
        return self.lib.oracle_kv_copy_blocks_fp8(
            self._p(k_pool, ctypes.c_uint8), self._p(v_pool, ctypes.c_uint8),
            self._p(s, ctypes.c_int32), self._p(d, ctypes.c_int32),
            s.size, Hkv, D, bs, N,
        )

    def kv_scatter_prefill(self, k_src, v_src, k_pool, v_pool, tables, prompt_lens, bs):
        """In-place: row b's prompt (right-aligned in the [B][Hkv][S][D] group) into its blocks."""
        B, Hkv, S, D = k_src.shape
        W = tables.shape[1]
        N = k_pool.shape[0]
        kp, vp = k_pool.view(np.uint16), v_pool.view(np.uint16)
        t = np.ascontiguousarray(tables, dtype=np.int32)
        p = np.ascontiguousarray(prompt_lens, dtype=np.int32)
        return self.lib.oracle_kv_scatter_prefill(
            self._p(self._bits(k_src), ctypes.c_uint16), self._p(self._bits(v_src), ctypes.c_uint16),
            self._p(kp, ctypes.c_uint16), self._p(vp, ctypes.c_uint16),
            self._p(t, ctypes.c_int32), self._p(p, ctypes.c_int32),
            B, Hkv, D, bs, W, N, S,
        )

    def kv_scatter_prefill_fp8(self, k_src, v_src, k_pool, v_pool, tables, prompt_lens, bs, k_scale, v_scale):
        """In-place: row b's prompt (right-aligned in the [B][Hkv][S][D] group), quantized, into E4M3 blocks."""
        B, Hkv, S, D = k_src.shape
        W = tables.shape[1]
        N = k_pool.shape[0]
        assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
        t = np.ascontiguousarray(tables, dtype=np.int32)
        p = np.ascontiguousarray(prompt_lens, dtype=np.int32)
        return self.lib.oracle_kv_scatter_prefill_fp8(
            self._p(self._bits(k_src), ctypes.c_uint16), self._p(self._bits(v_src), ctypes.c_uint16),
            self._p(k_pool, ctypes.c_uint8), self._p(v_pool, ctypes.c_uint8),
            self._p(t, ctypes.c_int32), self._p(p, ctypes.c_int32),
            B, Hkv, D, bs, W, N, S, ctypes.c_float(k_scale), ctypes.c_float(v_scale),
        )

    def gather_kv(self, k_pool, v_pool, tables, seq_lens, bs, Hkv, D, fill=0):
        B, W = tables.shape
        N = k_pool.shape[0]
        cap = W * bs
        ko = np.full((B, Hkv, cap, D), fill, np.uint16)
        vo = np.full((B, Hkv, cap, D), fill, np.uint16)
        t = np.ascontiguousarray(tables, dtype=np.int32)
        s = np.ascontiguousarray(seq_lens, dtype=np.int32)
        rc = self.lib.oracle_gather_kv(
            self._p(ko, ctypes.c_uint16),
            self._p(vo, ctypes.c_uint16),
            self._p(self._bits(k_pool), ctypes.c_uint16),
            self._p(self._bits(v_pool), ctypes.c_uint16),
            self._p(t, ctypes.c_int32),
            self._p(s, ctypes.c_int32),
            B, Hkv, D, bs, W, N,
        )
        if rc != 0:
            raise ValueError(f"oracle_gather_kv failed: {rc}")
        return ko.view(np.float16), vo.view(np.float16)

    def paged_decode_attn(self, q, k_pool, v_pool, tables, seq_lens, bs, scale, nthreads=1):
        """Returns (out_f32 [B][Hq][D], out_f16 [B][Hq][D])."""
        B, Hq, D = q.shape
        Hkv = k_pool.shape[1]
        W = tables.shape[1]
        N = k_pool.shape[0]
        of = np.empty((B, Hq, D), np.float32)
        oh = np.empty((B, Hq, D), np.uint16)
        t = np.ascontiguousarray(tables, dtype=np.int32)
        s = np.ascontiguousarray(seq_lens, dtype=np.int32)
        rc = self.lib.oracle_paged_decode_attn(
            self._p(of, ctypes.c_float),
            self._p(oh, ctypes.c_uint16),
            self._p(self._bits(q), ctypes.c_uint16),
            self._p(self._bits(k_pool), ctypes.c_uint16),
            self._p(self._bits(v_pool), ctypes.c_uint16),
            self._p(t, ctypes.c_int32),
            self._p(s, ctypes.c_int32),
            B, Hq, Hkv, D, bs, W, N,
            ctypes.c_float(scale), int(nthreads),
        )
        if rc != 0:
            raise ValueError(f"oracle_paged_decode_attn failed: {rc}")
        return of, oh.view(np.float16)

    def dense_attn(self, q_row, k, v, scale):
        """q_row [Hq][D], k/v [L][Hkv][D] (fp16) -> [Hq][D] fp32."""
        Hq, D = q_row.shape
        L, Hkv, _ = k.shape
        out = np.empty((Hq, D), np.float32)
        rc = self.lib.oracle_dense_attn(
            self._p(out, ctypes.c_float),
            self._p(self._bits(q_row), ctypes.c_uint16),
            self._p(self._bits(k), ctypes.c_uint16),
            self._p(self._bits(v), ctypes.c_uint16),
            L, Hq, Hkv, D, ctypes.c_float(scale),
        )
        if rc != 0:
            raise ValueError(f"oracle_dense_attn failed: {rc}")
        return out

    def validate(self, tables, seq_lens, bs, N, check_append=True):
        t = np.ascontiguousarray(tables, dtype=np.int32)
        s = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, W = t.shape
        return self.lib.oracle_validate(
            self._p(t, ctypes.c_int32), self._p(s, ctypes.c_int32), B, bs, W, N, int(bool(check_append))
        )


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
