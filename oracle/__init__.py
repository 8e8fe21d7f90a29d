"""CPU oracle for paged verify attention (fp64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg use it. It is never imported by the GPU library, and it
imports nothing from it. The arithmetic lives in ``pa_oracle.c``; this module
only builds that file with gcc and marshals numpy arrays into it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "pa_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
             "-Wno-unused-parameter"]


def compile_source(src: str, lib: str) -> str:
    """Compile one oracle source file into a shared library (plain -O2)."""
    tmp = lib + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"])
    os.replace(tmp, lib)
    return lib


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def default_threads() -> int:
    try:
        return max(1, min(len(os.sched_getaffinity(0)), 16))
    except AttributeError:  # pragma: no cover
        return max(1, min(os.cpu_count() or 1, 16))


def _np(t, dtype):
    """A contiguous numpy array of ``dtype`` from a CPU tensor or an array
    (same-size dtypes are reinterpreted bit for bit, others converted)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        import torch  # only when tensors come in

        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        elif t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        a = t.numpy()
    else:
        a = np.asarray(t)
    if a.dtype.itemsize == np.dtype(dtype).itemsize and a.dtype.kind in "iuf" and \
            np.dtype(dtype).kind in "iu" and a.dtype.kind in "iu":
        a = a.view(dtype)
    elif a.dtype != np.dtype(dtype):
        a = a.astype(dtype)
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """A loaded oracle library (the shipped one, or a test's own build)."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.pa_oracle_verify.argtypes = [
            i32, i32, i32, i32, P, P, P, P, P, P, i32, P, P, P, i32, P, i32,
            ctypes.c_double, P, P, P, i32]
        lib.pa_oracle_verify.restype = i32
        lib.pa_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.pa_oracle_e4m3_to_double.restype = ctypes.c_double
        lib.pa_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.pa_oracle_bf16_to_double.restype = ctypes.c_double
        lib.pa_oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.pa_oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.pa_oracle_kv_append.argtypes = [i32, i32, i32, P, P, P, P, P, i32, i32, i32, P, P, P, P]
        lib.pa_oracle_kv_append.restype = i32
        lib.pa_oracle_greedy_verdict.argtypes = [i32, P, i32, ctypes.c_int64, P, i32, P, P, P, P]
        lib.pa_oracle_greedy_verdict.restype = i32
        self.lib = lib

    def e4m3_to_double(self, code: int) -> float:
        return self.lib.pa_oracle_e4m3_to_double(code)

    def bf16_to_double(self, bits: int) -> float:
        return self.lib.pa_oracle_bf16_to_double(bits)

    def verify_arrays(self, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      ctx_lens, q_lens, window, q_bits, k_pool, v_pool, kv_fp8: bool,
                      k_scales, v_scales, block_table, sinks, sinks_mode: int,
                      softmax_scale: float, unit_mask=None,
                      threads: Optional[int] = None):
        """Run the oracle on raw arrays. bf16 data are uint16 bit patterns, FP8
        pools uint8 codes. Returns (out [T][Hq][D], lse [T][Hq]) as float64;
        rows of (sequence, head) units left out by ``unit_mask`` stay NaN."""
        ctx = _np(ctx_lens, np.int32)
        ql = _np(q_lens, np.int32)
        win = _np(window, np.int32)
        B = int(ctx.shape[0])
        T = int(ql.sum())
        Hq, D = num_q_heads, head_dim
        qa = _np(q_bits, np.uint16)
        pool_dt = np.uint8 if kv_fp8 else np.uint16
        ka = _np(k_pool, pool_dt)
        va = _np(v_pool, pool_dt)
        ks = _np(k_scales, np.float32)
        vs = _np(v_scales, np.float32)
        bt = _np(block_table, np.int32)
        sk = _np(sinks, np.float32)
        um = _np(unit_mask, np.uint8)
        out = np.full((T, Hq, D), np.nan, dtype=np.float64)
        lse = np.full((T, Hq), np.nan, dtype=np.float64)
        rc = self.lib.pa_oracle_verify(
            B, Hq, num_kv_heads, D, _ptr(ctx), _ptr(ql), _ptr(win), _ptr(qa), _ptr(ka),
            _ptr(va), int(kv_fp8), _ptr(ks), _ptr(vs), _ptr(bt), int(bt.shape[1]),
            _ptr(sk), int(sinks_mode), float(softmax_scale), _ptr(um), _ptr(out),
            _ptr(lse), int(threads or default_threads()))
        if rc != 0:
            raise ValueError(f"oracle rejected its arguments (code {rc})")
        return out, lse

    def e4m3_encode(self, v: float) -> int:
        """Nearest e4m3 code to fp32 value v (|v| <= 448), ties to even."""
        return self.lib.pa_oracle_e4m3_encode(v)

    def kv_append_arrays(self, *, num_kv_heads: int, head_dim: int, ctx_lens, q_lens,
                         k_new_bits, v_new_bits, block_table, kv_fp8: bool, k_pool, v_pool,
                         k_scales=None, v_scales=None):
        """Paged KV append on host arrays, in place: the new rows (uint16 bf16
        bits, [T][Hkv][D]) go into the pools (uint16 bf16 bits, or uint8 e4m3
        codes with float32 scales). Pools and scales must be C-contiguous
        numpy arrays; they are modified."""
        ctx = _np(ctx_lens, np.int32)
        ql = _np(q_lens, np.int32)
        kn = _np(k_new_bits, np.uint16)
        vn = _np(v_new_bits, np.uint16)
        bt = _np(block_table, np.int32)
        for a in (k_pool, v_pool) + ((k_scales, v_scales) if kv_fp8 else ()):
            if not (isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"]):
                raise ValueError("pools and scales must be C-contiguous numpy arrays")
        rc = self.lib.pa_oracle_kv_append(
            int(ctx.shape[0]), num_kv_heads, head_dim, _ptr(ctx), _ptr(ql), _ptr(kn), _ptr(vn),
            _ptr(bt), int(bt.shape[1]), int(k_pool.shape[0]), int(kv_fp8), _ptr(k_pool),
            _ptr(v_pool), _ptr(k_scales) if kv_fp8 else None,
            _ptr(v_scales) if kv_fp8 else None)
        if rc != 0:
            raise ValueError(f"oracle rejected its arguments (code {rc})")

    def greedy_verdict_arrays(self, *, q_lens, logits, input_ids, out_ids=None, accepted=None,
                              next_ids=None):
        """Greedy verify verdict on host arrays. logits: [T][V] float32, or
        uint16 bf16 bits. Returns (out_ids [T], accepted [B], next_ids [B])
        int32; entries of padded slots keep the values of the arrays passed
        in (default -7)."""
        ql = _np(q_lens, np.int32)
        lg = np.ascontiguousarray(logits)
        if lg.dtype == np.float32:
            bf = 0
        elif lg.dtype == np.uint16:
            bf = 1
        else:
            raise ValueError("logits must be float32 or uint16 bf16 bits")
        T, V = lg.shape
        ids = _np(input_ids, np.int32)
        B = int(ql.shape[0])
        out = np.full(T, -7, np.int32) if out_ids is None else out_ids
        acc = np.full(B, -7, np.int32) if accepted is None else accepted
        nxt = np.full(B, -7, np.int32) if next_ids is None else next_ids
        rc = self.lib.pa_oracle_greedy_verdict(B, _ptr(ql), V, V, _ptr(lg), bf, _ptr(ids),
                                               _ptr(out), _ptr(acc), _ptr(nxt))
        if rc != 0:
            raise ValueError(f"oracle rejected its arguments (code {rc})")
        return out, acc, nxt

    def verify(self, wl, unit_mask=None, threads: Optional[int] = None):
        """Oracle output for a ``workloads.Workload`` whose tensors are on the CPU."""
        return self.verify_arrays(
            num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
            head_dim=wl.head_dim, ctx_lens=wl.ctx_lens, q_lens=wl.q_lens,
            window=wl.window, q_bits=wl.q, k_pool=wl.k_pool, v_pool=wl.v_pool,
            kv_fp8=(wl.kv_dtype == "fp8"), k_scales=wl.k_scales, v_scales=wl.v_scales,
            block_table=wl.block_table, sinks=wl.sinks, sinks_mode=wl.sinks_mode,
            softmax_scale=wl.softmax_scale, unit_mask=unit_mask, threads=threads)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def verify(wl, unit_mask=None, threads: Optional[int] = None):
    return default().verify(wl, unit_mask=unit_mask, threads=threads)


def e4m3_to_double(code: int) -> float:
    return default().e4m3_to_double(code)


def bf16_to_double(bits: int) -> float:
    return default().bf16_to_double(bits)


def e4m3_encode(v: float) -> int:
    return default().e4m3_encode(v)
