"""Paged verify attention for MI355X: a thin binding over libpa_verify.so.

The names mirror the C ABI in include/pa_verify.h (pa_plan, pa_decode_verify,
pa_decode_verify_dev, pa_decode_verify_fused, pa_decode_verify_noalloc,
pa_kv_append, pa_verify_greedy, pa_free, pa_last_error, pa_plan_info,
pa_plan_items, pa_set_partition_events, pa_set_workgroup_stamps,
pa_stream_floor). This module only
marshals arguments: torch tensors
are passed as raw device pointers and torch's current stream as the HIP
stream. Every step of the computation runs in the library's HIP kernels;
there is no other path, and loading fails loudly if the library is missing.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libpa_verify.so")

PA_OK, PA_E_INVALID, PA_E_UNSUPPORTED, PA_E_HIP, PA_E_NOMEM = 0, 1, 2, 3, 4
PA_BF16, PA_FP8_E4M3, PA_FP32 = 0, 1, 2
ITEM_FIELDS = 7  # int32 per work item from pa_plan_items
STATUS_NAMES = {0: "PA_OK", 1: "PA_E_INVALID", 2: "PA_E_UNSUPPORTED", 3: "PA_E_HIP",
                4: "PA_E_NOMEM"}
EXPORTED = ("pa_plan", "pa_decode_verify", "pa_decode_verify_dev", "pa_decode_verify_fused",
            "pa_decode_verify_noalloc", "pa_kv_append", "pa_verify_greedy", "pa_free",
            "pa_last_error", "pa_plan_info", "pa_plan_items", "pa_set_partition_events",
            "pa_set_workgroup_stamps", "pa_stream_floor")


class PaShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("q_dtype", ctypes.c_int),
        ("kv_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int),
        ("softmax_scale", ctypes.c_float),
        ("partition_tokens", ctypes.c_int32),
        ("sinks_mode", ctypes.c_int32),
        ("lengths_are_bounds", ctypes.c_int32),
    ]


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """Load libpa_verify.so (built by paged_kv_cache_verify_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(f"{LIBRARY} is missing: run paged_kv_cache_verify_amd.build.build()")
        lib = ctypes.CDLL(LIBRARY)
        P = ctypes.c_void_p
        I32P = ctypes.POINTER(ctypes.c_int32)
        lib.pa_plan.argtypes = [ctypes.POINTER(PaShape), I32P, I32P, I32P, ctypes.c_int,
                                ctypes.POINTER(P)]
        lib.pa_plan.restype = ctypes.c_int
        lib.pa_decode_verify.argtypes = [P, P, P, P, P, P, P, P, P, P]
        lib.pa_decode_verify.restype = ctypes.c_int
        lib.pa_decode_verify_dev.argtypes = [P, P, P, P, P, P, P, P, P, P, P]
        lib.pa_decode_verify_dev.restype = ctypes.c_int
        lib.pa_decode_verify_fused.argtypes = [P, P, P, P, P, P, P, P, P, P, P]
        lib.pa_decode_verify_fused.restype = ctypes.c_int
        lib.pa_decode_verify_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P]
        lib.pa_decode_verify_noalloc.restype = ctypes.c_int
        lib.pa_kv_append.argtypes = [P, P, P, P, P, P, P, P, P]
        lib.pa_kv_append.restype = ctypes.c_int
        lib.pa_verify_greedy.argtypes = [P, P, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, P,
                                         P, P, P, P]
        lib.pa_verify_greedy.restype = ctypes.c_int
        lib.pa_free.argtypes = [P]
        lib.pa_free.restype = None
        lib.pa_last_error.argtypes = []
        lib.pa_last_error.restype = ctypes.c_char_p
        lib.pa_plan_info.argtypes = [P, ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_int64), I32P, I32P]
        lib.pa_plan_info.restype = ctypes.c_int
        lib.pa_plan_items.argtypes = [P, I32P, ctypes.c_int32]
        lib.pa_plan_items.restype = ctypes.c_int
        lib.pa_set_partition_events.argtypes = [P, P, P]
        lib.pa_set_partition_events.restype = ctypes.c_int
        lib.pa_set_workgroup_stamps.argtypes = [P, P, ctypes.c_int64]
        lib.pa_set_workgroup_stamps.restype = ctypes.c_int
        lib.pa_stream_floor.argtypes = [P, P, P, P, P, P, P]
        lib.pa_stream_floor.restype = ctypes.c_int
        _lib = lib
    return _lib


def pa_last_error() -> str:
    return library().pa_last_error().decode()


def _check(status: int) -> None:
    if status != PA_OK:
        raise PaError(status, pa_last_error())


def _i32_array(vals: Optional[Sequence[int]]):
    if vals is None:
        return None
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * len(vals))(*vals)


def make_shape(*, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
               max_blocks_per_seq, kv_dtype="bf16", out_dtype="bf16", softmax_scale,
               partition_tokens=0, sinks_mode=0, block_size=16, q_dtype="bf16",
               lengths_are_bounds=0) -> PaShape:
    dt = {"bf16": PA_BF16, "fp8": PA_FP8_E4M3, "fp32": PA_FP32}
    return PaShape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, dt[q_dtype], dt[kv_dtype], dt[out_dtype],
                   float(softmax_scale), partition_tokens, sinks_mode, lengths_are_bounds)


class Plan:
    """An owned pa_plan_t*; freed by pa_free on close() or garbage collection."""

    def __init__(self, handle: int, shape: PaShape, device: int):
        self.handle = ctypes.c_void_p(handle)
        self.shape = shape
        self.device = device
        self._events = None

    def close(self) -> None:
        if self.handle is not None and self.handle.value:
            library().pa_free(self.handle)
        self.handle = None

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass

    def info(self) -> dict:
        kv = ctypes.c_int64()
        scr = ctypes.c_int64()
        n = ctypes.c_int32()
        p = ctypes.c_int32()
        _check(library().pa_plan_info(self.handle, ctypes.byref(kv), ctypes.byref(scr),
                                      ctypes.byref(n), ctypes.byref(p)))
        return {"kv_bytes": kv.value, "scratch_bytes": scr.value, "work_items": n.value,
                "partition_tokens": p.value}

    def items(self):
        """The work list: (sequence, kv head, first key, end key, slot,
        first packed row, packed rows) per item."""
        n = self.info()["work_items"]
        buf = (ctypes.c_int32 * (ITEM_FIELDS * max(n, 1)))()
        _check(library().pa_plan_items(self.handle, buf, n))
        return [tuple(buf[ITEM_FIELDS * i:ITEM_FIELDS * (i + 1)]) for i in range(n)]


def pa_plan(shape: PaShape, context_lens: Sequence[int], query_lens: Sequence[int],
            window: Optional[Sequence[int]] = None, device: int = 0) -> Plan:
    """Validate and plan (see pa_plan in include/pa_verify.h). device=-1 plans
    on the host only."""
    out = ctypes.c_void_p()
    st = library().pa_plan(ctypes.byref(shape), _i32_array(context_lens),
                           _i32_array(query_lens), _i32_array(window), device,
                           ctypes.byref(out))
    _check(st)
    return Plan(out.value, shape, device)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("the library takes device tensors")
    if not t.is_contiguous():
        raise ValueError("the library takes contiguous tensors")
    return t.data_ptr()


def _stream_handle(stream):
    import torch  # torch provides the device memory and the stream

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def pa_decode_verify(plan: Plan, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks,
                     out, stream=None) -> None:
    """Enqueue one call on `stream` (default: torch's current stream)."""
    _check(library().pa_decode_verify(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                      _ptr(block_table), _ptr(k_scales), _ptr(v_scales),
                                      _ptr(sinks), _ptr(out), _stream_handle(stream)))


def pa_decode_verify_dev(plan: Plan, context_lens_dev, q, k_pool, v_pool, block_table, k_scales,
                         v_scales, sinks, out, stream=None) -> None:
    """pa_decode_verify with the lengths read from a device int32 [B] tensor
    (the plan's lengths are upper bounds)."""
    _check(library().pa_decode_verify_dev(plan.handle, _ptr(context_lens_dev), _ptr(q),
                                          _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                          _ptr(k_scales), _ptr(v_scales), _ptr(sinks), _ptr(out),
                                          _stream_handle(stream)))


def pa_decode_verify_fused(plan: Plan, context_lens_dev, q, k_pool, v_pool, block_table,
                           k_scales, v_scales, sinks, out, stream=None) -> None:
    """The call as a single launch whose split items merge their partials
    themselves; context_lens_dev is a device int32 [B] tensor of lengths
    (the plan's are then upper bounds) or None for the plan's own."""
    _check(library().pa_decode_verify_fused(plan.handle, _ptr(context_lens_dev), _ptr(q),
                                            _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                            _ptr(k_scales), _ptr(v_scales), _ptr(sinks),
                                            _ptr(out), _stream_handle(stream)))


def pa_decode_verify_noalloc(plan: Plan, q, k_pool, v_pool, block_table, k_scales, v_scales,
                             sinks, out, stream=None) -> None:
    """pa_decode_verify with the work list and partials in the library's
    static scratch (no allocation; host-only plans accepted). Calls that
    overlap on one device race on that scratch."""
    _check(library().pa_decode_verify_noalloc(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                              _ptr(block_table), _ptr(k_scales), _ptr(v_scales),
                                              _ptr(sinks), _ptr(out), _stream_handle(stream)))


def pa_kv_append(plan: Plan, k_new, v_new, block_table, k_pool, v_pool, k_scales=None,
                 v_scales=None, stream=None) -> None:
    """Store the plan's new tokens ([T][Hkv][D] bf16 K and V rows) into the
    pools, quantising to e4m3 with per-token scales for FP8 KV (see
    pa_kv_append in include/pa_verify.h). Enqueued on `stream`."""
    _check(library().pa_kv_append(plan.handle, _ptr(k_new), _ptr(v_new), _ptr(block_table),
                                  _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales),
                                  _stream_handle(stream)))


def pa_verify_greedy(plan: Plan, logits, input_ids, out_ids, accepted, next_ids,
                     stream=None) -> None:
    """Greedy verify verdict (see pa_verify_greedy in include/pa_verify.h):
    logits [T][V] (bf16 or float32; a row may be a strided view with unit
    last stride), input_ids [T] int32 -> out_ids [T], accepted [B],
    next_ids [B] int32."""
    import torch

    dt = {torch.bfloat16: PA_BF16, torch.float32: PA_FP32}.get(logits.dtype)
    if dt is None:
        raise ValueError("logits must be bfloat16 or float32")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [T][V] with unit stride along V")
    if not logits.is_cuda:
        raise ValueError("the library takes device tensors")
    _check(library().pa_verify_greedy(plan.handle, ctypes.c_void_p(logits.data_ptr()), dt,
                                      logits.shape[1], logits.stride(0), _ptr(input_ids),
                                      _ptr(out_ids), _ptr(accepted), _ptr(next_ids),
                                      _stream_handle(stream)))


def pa_stream_floor(plan: Plan, k_pool, v_pool, block_table, k_scales=None, v_scales=None,
                    stream=None) -> None:
    """Measurement: read the plan's KV bytes with the partition kernel's
    loads and compute nothing (see pa_stream_floor in include/pa_verify.h)."""
    _check(library().pa_stream_floor(plan.handle, _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                     _ptr(k_scales), _ptr(v_scales), _stream_handle(stream)))


def pa_free(plan: Plan) -> None:
    plan.close()


def pa_set_workgroup_stamps(plan: Plan, stamps=None) -> None:
    """Attach a device int64 tensor of at least 8 x work_items stamps (or None
    to stop); see pa_set_workgroup_stamps in include/pa_verify.h."""
    import torch

    if stamps is not None and stamps.dtype != torch.int64:
        raise ValueError("stamps must be an int64 tensor")
    cap = 0 if stamps is None else stamps.numel()
    _check(library().pa_set_workgroup_stamps(plan.handle, _ptr(stamps), cap))
    plan._stamps = stamps


def pa_set_partition_events(plan: Plan, before=None, after=None) -> None:
    """Attach torch.cuda.Event handles to the partition kernel's launch, which
    then takes its start and end timestamps (or stop, with None)."""
    for ev in (before, after):
        if ev is not None and not ev.cuda_event:
            ev.record()  # torch creates its HIP event on the first record
    b = ctypes.c_void_p(before.cuda_event) if before is not None else None
    a = ctypes.c_void_p(after.cuda_event) if after is not None else None
    plan._events = (before, after)
    _check(library().pa_set_partition_events(plan.handle, b, a))


# ---------------------------------------------------------------------------
# Convenience for callers holding a workloads.Workload-like object.
# ---------------------------------------------------------------------------

def plan_for(wl, device: int = 0, partition_tokens: Optional[int] = None) -> Plan:
    shape = make_shape(
        num_seqs=wl.num_seqs, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
        head_dim=wl.head_dim, num_blocks=wl.num_blocks,
        max_blocks_per_seq=wl.max_blocks_per_seq, kv_dtype=wl.kv_dtype,
        out_dtype=wl.out_dtype, softmax_scale=wl.softmax_scale,
        partition_tokens=wl.partition_tokens if partition_tokens is None else partition_tokens,
        sinks_mode=wl.sinks_mode)
    win = None if wl.window is None else wl.window.tolist()
    return pa_plan(shape, wl.ctx_lens.tolist(), wl.q_lens.tolist(), win, device)


def run(plan: Plan, wl, out=None, stream=None):
    """One call on a workload whose tensors are on the plan's device."""
    import torch

    if out is None:
        dt = torch.float32 if wl.out_dtype == "fp32" else torch.bfloat16
        out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=dt,
                          device=wl.q.device)
    pa_decode_verify(plan, wl.q, wl.k_pool, wl.v_pool, wl.block_table, wl.k_scales,
                     wl.v_scales, wl.sinks, out, stream)
    return out
