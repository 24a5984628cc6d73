"""ctypes binding of libpkc (include/pkc.h), with the same call names.

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
Importing this module loads ``libpkc.so`` and raises ImportError when the
library has not been built (there is no fallback).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkc.so")

MAX_LEVELS = 8
PLAN_MAGIC = 0x504B4331

STATUS = {0: "PKC_OK", 1: "PKC_ERR_INVALID_ARG", 2: "PKC_ERR_UNSUPPORTED",
          3: "PKC_ERR_WORKSPACE_TOO_SMALL", 4: "PKC_ERR_PLAN_MISMATCH", 5: "PKC_ERR_HIP",
          6: "PKC_ERR_INTERNAL"}
F32, F16, BF16 = 0, 1, 2
_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

# Kernel kinds of the timing interface.
KIND_DECODE, KIND_PREFIX, KIND_MERGE_PLAN, KIND_MERGE = 0, 1, 2, 3


class PkcError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class PlanParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_ctas", ctypes.c_int32),
                ("level_ctas", ctypes.c_int32), ("level_tile_q", ctypes.c_int32),
                ("chunk_align", ctypes.c_int32), ("enable_split", ctypes.c_int32),
                ("alpha", ctypes.c_int64), ("beta", ctypes.c_int64), ("decode_waves", ctypes.c_int32),
                ("level_write_through", ctypes.c_int32), ("level_streams", ctypes.c_int32),
                ("contraction", ctypes.c_int32), ("defer_upload", ctypes.c_int32)]


class LevelHost(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("qo_indptr", ctypes.POINTER(ctypes.c_int32)),
                ("kv_lens", ctypes.POINTER(ctypes.c_int32)), ("causal", ctypes.c_int32)]


class LevelDev(ctypes.Structure):
    _fields_ = [("kv_page_indptr", ctypes.c_void_p), ("kv_page_indices", ctypes.c_void_p),
                ("num_page_indices", ctypes.c_int32)]


_L8 = ctypes.c_int32 * MAX_LEVELS
_O8 = ctypes.c_int64 * MAX_LEVELS


class PlanInfo(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("batch", ctypes.c_int32),
                ("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_levels", ctypes.c_int32), ("num_ctas", ctypes.c_int32),
                ("level_ctas", ctypes.c_int32), ("dec_items", ctypes.c_int32),
                ("dec_slots", ctypes.c_int32), ("dec_kv_chunk", ctypes.c_int32),
                ("dec_waves", ctypes.c_int32),
                ("lvl_groups", _L8), ("lvl_tile_q", _L8), ("lvl_items", _L8),
                ("lvl_kv_chunk", _L8), ("lvl_row_base", _L8),
                ("dec_row_base", ctypes.c_int32), ("state_rows", ctypes.c_int32),
                ("merge_entries", ctypes.c_int32), ("num_merge", ctypes.c_int32),
                ("off_dec_indptr", ctypes.c_int64), ("off_dec_items", ctypes.c_int64),
                ("off_lvl_indptr", _O8), ("off_lvl_items", _O8),
                ("off_merge_ptr", ctypes.c_int64), ("off_merge_rows", ctypes.c_int64),
                ("off_req_flags", ctypes.c_int64), ("off_req_levels", ctypes.c_int64),
                ("int_bytes", ctypes.c_int64),
                ("off_state_o", ctypes.c_int64), ("off_state_lse", ctypes.c_int64),
                ("dev_bytes", ctypes.c_int64), ("dev_ws", ctypes.c_uint64), ("lvl_causal", _L8),
                ("lvl_write_through", ctypes.c_int32), ("lvl_streams", ctypes.c_int32),
                ("dec_contraction", ctypes.c_int32), ("off_counters", ctypes.c_int64),
                ("host_src", ctypes.c_uint64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes) for every function declared in include/pkc.h
SIGNATURES = {
    "pkc_status_string": (ctypes.c_char_p, [_I32]),
    "pkc_last_error": (ctypes.c_char_p, []),
    "pkc_version": (ctypes.c_char_p, []),
    "pkc_abi_struct_sizes": (None, [ctypes.POINTER(_SZ)] * 4),
    "pkc_device_info": (_I32, [_I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32), ctypes.POINTER(_I64)]),
    "pkc_plan_buffer_sizes": (_I32, [ctypes.POINTER(PlanParams), ctypes.POINTER(LevelHost), _I32,
                                     ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "pkc_plan": (_I32, [ctypes.POINTER(PlanParams), ctypes.POINTER(_I32), ctypes.POINTER(LevelHost),
                        _I32, _P, _SZ, _P, _SZ, _P, ctypes.POINTER(PlanInfo)]),
    "pkc_plan_host": (_I32, [ctypes.POINTER(PlanParams), ctypes.POINTER(_I32),
                             ctypes.POINTER(LevelHost), _I32, _P, _SZ, ctypes.POINTER(PlanInfo)]),
    "pkc_batch_decode_paged": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _I64, _P, _I32, _P, _P,
                                      _I32, _I32, _I32, _I32, _I32, _I32, _F, _P, _P, _P, _SZ, _P]),
    "pkc_batch_decode_paged_noalloc": (_I32, [ctypes.POINTER(PlanInfo), _P, _SZ, _P, _P, _P, _I64, _P, _I32,
                                              _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _F, _P, _P, _P]),
    "pkc_prefix_attention": (_I32, [ctypes.POINTER(PlanInfo), _I32, _P, _P, _P, _I64,
                                    ctypes.POINTER(LevelDev), _I32, _I32, _I32, _I32, _I32, _I32,
                                    _F, _P, _I32, _P, _P, _SZ, _P]),
    "pkc_merge_states": (_I32, [_P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _P, _P]),
    "pkc_merge_state_inplace": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P]),
    "pkc_cascade_decode": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _I64,
                                  ctypes.POINTER(LevelDev), _I32, _P, _I32, _P, _I32, _I32, _I32,
                                  _I32, _I32, _I32, _F, _P, _P, _P, _SZ, _P]),
    "pkc_validate_block_table": (_I32, [ctypes.POINTER(_I32), _I32, ctypes.POINTER(_I32),
                                        ctypes.POINTER(_I32), _I32, _I32, _I64]),
    "pkc_debug_gather_rows": (_I32, [_P, _I32, _P, _P, _I32, _I32, _I64, _P, _I32, _P]),
    "pkc_debug_cta_trace": (_I32, [ctypes.POINTER(PlanInfo), _I32, _P, _P, _I64, _I32, _P]),
    "pkc_timing_enable": (_I32, [_I32]),
    "pkc_timing_reset": (_I32, []),
    "pkc_timing_read": (_I32, [_I32, ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double)]),
    "pkc_read_stream_probe": (_I32, [_P, _I64, _P, _I64, _P]),
    "pkc_append_kv": (_I32, [_P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "pkc_append_kv_ragged": (_I32, [_P, _P, _I64, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32,
                                    _I32, _I32, _P]),
    "pkc_batch_decode_paged_fp8": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _F, _F, _I64, _P, _I32,
                                          _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _F, _P, _P, _P,
                                          _SZ, _P]),
    "pkc_prefix_attention_fp8": (_I32, [ctypes.POINTER(PlanInfo), _I32, _P, _P, _P, _F, _F, _I64,
                                        ctypes.POINTER(LevelDev), _I32, _I32, _I32, _I32, _I32, _I32,
                                        _F, _P, _I32, _P, _P, _SZ, _P]),
    "pkc_batch_prefill_paged": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _I64, _P, _I32, _P, _P, _I32,
                                       _I32, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _P, _SZ, _P]),
    "pkc_batch_prefill_paged_tree": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _I64, _P, _I32, _P, _P, _P,
                                            _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F, _P, _P,
                                            _P, _SZ, _P]),
    "pkc_batch_prefill_paged_fp8": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _F, _F, _I64, _P, _I32, _P,
                                           _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _P,
                                           _P, _SZ, _P]),
    "pkc_cascade_decode_fp8": (_I32, [ctypes.POINTER(PlanInfo), _P, _P, _P, _F, _F, _I64,
                                      ctypes.POINTER(LevelDev), _I32, _P, _I32, _P, _I32, _I32, _I32,
                                      _I32, _I32, _I32, _F, _P, _P, _P, _SZ, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cascade_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    sizes = [_SZ() for _ in range(4)]
    lib.pkc_abi_struct_sizes(*[ctypes.byref(s) for s in sizes])
    want = [ctypes.sizeof(PlanParams), ctypes.sizeof(LevelHost), ctypes.sizeof(LevelDev),
            ctypes.sizeof(PlanInfo)]
    if [s.value for s in sizes] != want:
        raise ImportError(f"ABI struct size mismatch: library {[s.value for s in sizes]} vs binding {want}")
    return lib


lib = _load()


def _check(status):
    if status != 0:
        raise PkcError(status, lib.pkc_last_error().decode())


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DTYPES:
        raise PkcError(2, f"unsupported dtype {dt}")
    return _DTYPES[dt]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32_array(values):
    arr = (ctypes.c_int32 * max(1, len(values)))(*[int(v) for v in values])
    return arr


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_contiguous():
        raise PkcError(1, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PkcError(1, f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise PkcError(1, f"{name} must be on {device}")


def version() -> str:
    return lib.pkc_version().decode()


def device_info(device: int = 0):
    cus, ws, lds = _I32(), _I32(), _I64()
    _check(lib.pkc_device_info(device, ctypes.byref(cus), ctypes.byref(ws), ctypes.byref(lds)))
    return {"num_cus": cus.value, "wave_size": ws.value, "lds_bytes_per_block": lds.value}


def make_params(batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_ctas=0, level_ctas=0,
                level_tile_q=0, chunk_align=1, enable_split=True, alpha=1, beta=1,
                decode_waves=0, level_write_through=False, level_streams=0,
                contraction=0, defer_upload=False) -> PlanParams:
    return PlanParams(batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_ctas, level_ctas,
                      level_tile_q, chunk_align, 1 if enable_split else 0, alpha, beta, decode_waves,
                      1 if level_write_through else 0, level_streams, contraction,
                      1 if defer_upload else 0)


class HostLevels:
    """Host level descriptors (pkc_level_host) marshalled once; pass the object itself to
    plan / plan_buffer_sizes / Workspace in place of the list of dicts to skip the conversion
    (a serving loop plans every step with the same level shapes)."""

    def __init__(self, levels: Sequence[dict]):
        self.keep = []
        self.arr = (LevelHost * max(1, len(levels)))()
        for i, lv in enumerate(levels):
            qi = _i32_array(lv["qo_indptr"])
            kl = _i32_array(lv["kv_lens"]) if lv.get("kv_lens") is not None else None
            self.keep += [qi, kl]
            self.arr[i].num_groups = len(lv["qo_indptr"]) - 1
            self.arr[i].qo_indptr = ctypes.cast(qi, ctypes.POINTER(ctypes.c_int32))
            self.arr[i].kv_lens = ctypes.cast(kl, ctypes.POINTER(ctypes.c_int32)) if kl is not None else None
            self.arr[i].causal = 1 if lv.get("causal") else 0
        self.n = len(levels)


def plan_buffer_sizes(params: PlanParams, levels: Sequence[dict] = ()):
    lv = _levels_arg(levels)
    hb, db = _SZ(), _SZ()
    _check(lib.pkc_plan_buffer_sizes(ctypes.byref(params), lv.arr, lv.n, ctypes.byref(hb), ctypes.byref(db)))
    return hb.value, db.value


class Workspace:
    """Caller-owned buffers of a plan: a pinned host buffer and a device workspace, sized from
    the library's upper bounds so their addresses stay fixed across steps."""

    def __init__(self, params: PlanParams, levels: Sequence[dict] = (), device="cuda"):
        hb, db = plan_buffer_sizes(params, levels)
        self.host = torch.empty(max(hb, 16), dtype=torch.uint8, pin_memory=True)
        self.device = torch.empty(max(db, 256), dtype=torch.uint8, device=device)


def _lens_arg(kv_lens):
    """kv_lens as a C int32 pointer: an int32 CPU tensor is passed as it is (no copy), anything
    else is converted."""
    if isinstance(kv_lens, torch.Tensor):
        if kv_lens.dtype != torch.int32 or kv_lens.device.type != "cpu" or not kv_lens.is_contiguous():
            raise PkcError(1, "kv_lens tensor must be contiguous int32 on the CPU")
        return ctypes.cast(kv_lens.data_ptr(), ctypes.POINTER(ctypes.c_int32))
    return _i32_array(list(kv_lens))


def _levels_arg(levels):
    return levels if isinstance(levels, HostLevels) else HostLevels(levels)


def plan(params: PlanParams, kv_lens, levels: Sequence[dict] = (), workspace: Workspace = None,
         device="cuda") -> PlanInfo:
    """pkc_plan: build the plan on the CPU and enqueue its copy on the current stream (with
    params.defer_upload, enqueue nothing: the run calls bring the plan over from the workspace's
    pinned host buffer, which must then stay untouched until they complete).
    kv_lens: a sequence of ints or an int32 CPU tensor; levels: dicts or a HostLevels."""
    if workspace is None:
        raise PkcError(1, "plan needs a Workspace")
    kl = _lens_arg(kv_lens)
    lv = _levels_arg(levels)
    info = PlanInfo()
    _check(lib.pkc_plan(ctypes.byref(params), kl, lv.arr, lv.n, _ptr(workspace.host),
                        workspace.host.numel(), _ptr(workspace.device), workspace.device.numel(),
                        _stream(workspace.device.device), ctypes.byref(info)))
    info._workspace = workspace
    return info


def plan_host(params: PlanParams, kv_lens, levels: Sequence[dict] = (), host_buf: torch.Tensor = None):
    """pkc_plan_host: the same plan with no HIP call.  Returns (PlanInfo, host buffer)."""
    hb, _ = plan_buffer_sizes(params, levels)
    if host_buf is None:
        host_buf = torch.zeros(max(hb, 16), dtype=torch.uint8)
    kl = _lens_arg(kv_lens)
    lv = _levels_arg(levels)
    info = PlanInfo()
    _check(lib.pkc_plan_host(ctypes.byref(params), kl, lv.arr, lv.n, _ptr(host_buf), host_buf.numel(),
                             ctypes.byref(info)))
    return info, host_buf


def _ws_of(plan_info: Optional[PlanInfo]):
    if plan_info is None:
        return None, 0
    ws = getattr(plan_info, "_workspace", None)
    if ws is None:
        raise PkcError(1, "plan has no device workspace (built with plan_host?)")
    return _ptr(ws.device), ws.device.numel()


def batch_decode_paged(q, k_pool, v_pool, block_table, cache_seqlens, kv_start=None, sm_scale=None,
                       plan_info: Optional[PlanInfo] = None, out=None, lse=None):
    """pkc_batch_decode_paged.  q [B, Hq, D]; pools [N, P, Hkv, D]; block_table int32 [B, M];
    cache_seqlens int32 [B].  Returns (o [B, Hq, D] in q's dtype, lse fp32 [B, Hq])."""
    B, Hq, D = q.shape
    N, P, Hkv, D2 = k_pool.shape
    dev = q.device
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, n, q.dtype, dev)
    _need(block_table, "block_table", torch.int32, dev)
    if cache_seqlens is not None:
        _need(cache_seqlens, "cache_seqlens", torch.int32, dev)
    if kv_start is not None:
        _need(kv_start, "kv_start", torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_batch_decode_paged(ctypes.byref(plan_info) if plan_info is not None else None,
                                      _ptr(q), _ptr(k_pool), _ptr(v_pool), N, _ptr(block_table),
                                      block_table.shape[1], _ptr(cache_seqlens), _ptr(kv_start),
                                      B, Hq, Hkv, D, P, dtype_code(q.dtype), scale, _ptr(out),
                                      _ptr(lse), ws, wsn, _stream(dev)))
    return out, lse


def batch_decode_paged_noalloc(plan_info: PlanInfo, plan_host_buf, q, k_pool, v_pool, block_table,
                               cache_seqlens, kv_start=None, sm_scale=None, out=None, lse=None):
    """pkc_batch_decode_paged_noalloc: split-KV decode from a host-built plan (plan_host) whose
    workspace is the library's fixed device array.  Returns (o, lse); with ``out`` and ``lse``
    given, nothing is allocated on the device."""
    B, Hq, D = q.shape
    N, P, Hkv, D2 = k_pool.shape
    dev = q.device
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, n, q.dtype, dev)
    _need(block_table, "block_table", torch.int32, dev)
    if kv_start is not None:
        _need(kv_start, "kv_start", torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    _check(lib.pkc_batch_decode_paged_noalloc(ctypes.byref(plan_info), _ptr(plan_host_buf), plan_host_buf.numel(),
                                              _ptr(q), _ptr(k_pool), _ptr(v_pool), N, _ptr(block_table),
                                              block_table.shape[1], _ptr(cache_seqlens), _ptr(kv_start),
                                              B, Hq, Hkv, D, P, dtype_code(q.dtype), scale, _ptr(out),
                                              _ptr(lse), _stream(dev)))
    return out, lse


NOALLOC_SCRATCH_BYTES = 32 << 20


def append_kv(k_new, v_new, k_pool, v_pool, block_table, cache_seqlens, new_seqlens=None):
    """pkc_append_kv: write each request's new token rows (k_new / v_new [B, Hkv, D]) at
    position cache_seqlens[b] of its block-table row, in place.  Returns the new lengths
    (new_seqlens, allocated when None; pass cache_seqlens itself to update it in place)."""
    B, Hkv, D = k_new.shape
    N, P, Hkv2, D2 = k_pool.shape
    dev = k_pool.device
    if (Hkv, D) != (Hkv2, D2) or tuple(v_new.shape) != tuple(k_new.shape) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise PkcError(1, "append_kv: shape mismatch")
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, n, k_pool.dtype, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev)
    if new_seqlens is None:
        new_seqlens = torch.empty_like(cache_seqlens)
    _check(lib.pkc_append_kv(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), N, _ptr(block_table),
                             block_table.shape[1], _ptr(cache_seqlens), _ptr(new_seqlens), B, Hkv, D, P,
                             dtype_code(k_pool.dtype), _stream(dev)))
    return new_seqlens



def append_kv_ragged(k_new, v_new, new_indptr, k_pool, v_pool, block_table, cache_seqlens,
                     new_seqlens=None):
    """pkc_append_kv_ragged: request b's new rows k_new / v_new[new_indptr[b] .. new_indptr[b+1])
    ([total_new, Hkv, D]) go to positions cache_seqlens[b] + i of its block-table row, in place.
    new_indptr and cache_seqlens are int32 device tensors.  Returns the new lengths (allocated
    when None; must not be cache_seqlens)."""
    T, Hkv, D = k_new.shape
    N, P, Hkv2, D2 = k_pool.shape
    dev = k_pool.device
    if (Hkv, D) != (Hkv2, D2) or tuple(v_new.shape) != tuple(k_new.shape) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise PkcError(1, "append_kv_ragged: shape mismatch")
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, n, k_pool.dtype, dev)
    for t, n in ((block_table, "block_table"), (cache_seqlens, "cache_seqlens"), (new_indptr, "new_indptr")):
        _need(t, n, torch.int32, dev)
    B = cache_seqlens.numel()
    if new_indptr.numel() != B + 1:
        raise PkcError(1, "append_kv_ragged: new_indptr must have batch + 1 entries")
    if new_seqlens is None:
        new_seqlens = torch.empty_like(cache_seqlens)
    _check(lib.pkc_append_kv_ragged(_ptr(k_new), _ptr(v_new), T, _ptr(new_indptr), _ptr(k_pool), _ptr(v_pool),
                                    N, _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
                                    _ptr(new_seqlens), B, Hkv, D, P, dtype_code(k_pool.dtype), _stream(dev)))
    return new_seqlens


def batch_decode_paged_fp8(q, k_pool, v_pool, block_table, cache_seqlens, k_scale=1.0, v_scale=1.0,
                           kv_start=None, sm_scale=None, plan_info: Optional[PlanInfo] = None,
                           out=None, lse=None):
    """pkc_batch_decode_paged_fp8.  k_pool / v_pool: OCP FP8 E4M3 pools [N, P, Hkv, D]
    (torch.float8_e4m3fn, or uint8 holding the codes); q fp16 / bf16 [B, Hq, D].  Returns
    (o in q's dtype, lse fp32)."""
    B, Hq, D = q.shape
    N, P, Hkv, D2 = k_pool.shape
    dev = q.device
    _check_fp8_pools(q, k_pool, v_pool)
    _need(q, "q", q.dtype, dev)
    _need(block_table, "block_table", torch.int32, dev)
    if cache_seqlens is not None:
        _need(cache_seqlens, "cache_seqlens", torch.int32, dev)
    if kv_start is not None:
        _need(kv_start, "kv_start", torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_batch_decode_paged_fp8(ctypes.byref(plan_info) if plan_info is not None else None,
                                          _ptr(q), _ptr(k_pool), _ptr(v_pool), float(k_scale),
                                          float(v_scale), N, _ptr(block_table), block_table.shape[1],
                                          _ptr(cache_seqlens), _ptr(kv_start), B, Hq, Hkv, D, P,
                                          dtype_code(q.dtype), scale, _ptr(out), _ptr(lse), ws, wsn,
                                          _stream(dev)))
    return out, lse


def level_dev(level: dict, device="cuda"):
    """Device page arrays of one cascade level (returns LevelDev plus the tensors it points to)."""
    indptr = torch.tensor(level["kv_page_indptr"], dtype=torch.int32, device=device)
    indices = torch.tensor(list(level["kv_page_indices"]) or [0], dtype=torch.int32, device=device)
    return LevelDev(indptr.data_ptr(), indices.data_ptr(), len(level["kv_page_indices"])), (indptr, indices)


def prefix_attention(plan_info: PlanInfo, level: int, q, k_pool, v_pool, lvl_dev: LevelDev,
                     sm_scale=None, o_dtype=torch.float32, out=None, lse=None):
    """pkc_prefix_attention: state of every request over its group's KV run at one level."""
    B, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    if out is None:
        out = torch.empty(B, Hq, D, dtype=o_dtype, device=dev)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_prefix_attention(ctypes.byref(plan_info), level, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                    N, ctypes.byref(lvl_dev), B, Hq, Hkv, D, P, dtype_code(q.dtype),
                                    scale, _ptr(out), dtype_code(out.dtype), _ptr(lse), ws, wsn,
                                    _stream(dev)))
    return out, lse


def merge_states(o_states, lse_states, indptr=None, indices=None, states_per_output=None,
                 num_outputs=None, out_dtype=None, out=None, lse=None):
    """pkc_merge_states.  o_states [S, H, D], lse_states [S, H].  With indptr (int32 device
    [n+1]) output i merges states indices[indptr[i]:indptr[i+1]] (or that range itself);
    without it output i merges states i*S' .. i*S'+S'-1, S' = states_per_output."""
    S, H, D = o_states.shape
    dev = o_states.device
    _need(o_states, "o_states", device=dev)
    _need(lse_states, "lse_states", torch.float32, dev)
    if indptr is not None:
        n = indptr.numel() - 1 if num_outputs is None else num_outputs
        spo = 0
    else:
        spo = int(states_per_output)
        n = (S // spo if spo else 0) if num_outputs is None else num_outputs
    odt = o_states.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(n, H, D, dtype=odt, device=dev)
    if lse is None:
        lse = torch.empty(n, H, dtype=torch.float32, device=dev)
    _check(lib.pkc_merge_states(_ptr(o_states), dtype_code(o_states.dtype), _ptr(lse_states), S,
                                _ptr(indptr), _ptr(indices), n, spo, H, D, _ptr(out),
                                dtype_code(out.dtype), _ptr(lse), _stream(dev)))
    return out, lse


def merge_state_inplace(o_a, lse_a, o_b, lse_b):
    """pkc_merge_state_inplace: (o_a, lse_a) <- (o_a, lse_a) merged with (o_b, lse_b)."""
    R, H, D = o_a.shape
    _check(lib.pkc_merge_state_inplace(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), R, H, D,
                                       dtype_code(o_a.dtype), _stream(o_a.device)))
    return o_a, lse_a


def cascade_decode(plan_info: PlanInfo, q, k_pool, v_pool, lvl_devs: Sequence[LevelDev], block_table,
                   suffix_seqlens, sm_scale=None, out=None, lse=None):
    """pkc_cascade_decode: levels (MFMA prefix kernels), suffix decode, then one merge."""
    B, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    arr = (LevelDev * max(1, len(lvl_devs)))(*lvl_devs)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_cascade_decode(ctypes.byref(plan_info), _ptr(q), _ptr(k_pool), _ptr(v_pool), N,
                                  arr, len(lvl_devs), _ptr(block_table), block_table.shape[1],
                                  _ptr(suffix_seqlens), B, Hq, Hkv, D, P, dtype_code(q.dtype), scale,
                                  _ptr(out), _ptr(lse), ws, wsn, _stream(dev)))
    return out, lse


def _check_fp8_pools(q, k_pool, v_pool):
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise PkcError(1, "q must be fp16 or bf16")
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, n, None, q.device)
        if t.element_size() != 1:
            raise PkcError(1, f"{n} must hold one-byte FP8 codes")


def prefix_attention_fp8(plan_info: PlanInfo, level: int, q, k_pool, v_pool, lvl_dev: LevelDev,
                         k_scale=1.0, v_scale=1.0, sm_scale=None, o_dtype=torch.float32, out=None,
                         lse=None):
    """pkc_prefix_attention_fp8: prefix_attention over OCP FP8 E4M3 pools (float8_e4m3fn or
    uint8 codes) with per-pool scales; q fp16 / bf16."""
    B, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    _check_fp8_pools(q, k_pool, v_pool)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=o_dtype, device=dev)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_prefix_attention_fp8(ctypes.byref(plan_info), level, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        float(k_scale), float(v_scale), N, ctypes.byref(lvl_dev), B, Hq, Hkv,
                                        D, P, dtype_code(q.dtype), scale, _ptr(out), dtype_code(out.dtype),
                                        _ptr(lse), ws, wsn, _stream(dev)))
    return out, lse


def cascade_decode_fp8(plan_info: PlanInfo, q, k_pool, v_pool, lvl_devs: Sequence[LevelDev], block_table,
                       suffix_seqlens, k_scale=1.0, v_scale=1.0, sm_scale=None, out=None, lse=None):
    """pkc_cascade_decode_fp8: cascade_decode over OCP FP8 E4M3 pools with per-pool scales;
    q and o fp16 / bf16."""
    B, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    _check_fp8_pools(q, k_pool, v_pool)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    arr = (LevelDev * max(1, len(lvl_devs)))(*lvl_devs)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_cascade_decode_fp8(ctypes.byref(plan_info), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                      float(k_scale), float(v_scale), N, arr, len(lvl_devs), _ptr(block_table),
                                      block_table.shape[1], _ptr(suffix_seqlens), B, Hq, Hkv, D, P,
                                      dtype_code(q.dtype), scale, _ptr(out), _ptr(lse), ws, wsn, _stream(dev)))
    return out, lse


def prefill_plan(qo_lens, kv_lens, num_qo_heads, num_kv_heads, head_dim, page_size, level_ctas=0,
                 level_tile_q=0, enable_split=True, alpha=1, beta=1, causal=True,
                 workspace: Workspace = None, write_through=True, defer_upload=False):
    """Plan of a batch prefill: every query row is one plan request (batch = total_q, no own
    KV) and one level whose groups are the requests (qo_indptr = cumulative query lengths,
    kv_lens; causal: tiles weighed by the KV their last query sees).  level_ctas = 0 takes
    8 x floor(compute units / Hkv): a prefill level has many tiles per workgroup, and several
    rounds of 4-wave workgroups balance them better than the one 8-wave workgroup per
    compute unit that suits a decode step's level (causal 8 x 2048 at 32 heads: 585 against
    700-760 us).  write_through: query tiles whose KV is a single chunk write their final
    output from the level kernel, and only the other rows go through the merge pass.  Returns
    (plan_info, workspace, qo_indptr list)."""
    if level_ctas == 0:
        level_ctas = 8 * max(1, device_info(torch.cuda.current_device())["num_cus"] // int(num_kv_heads))
    qo_lens = [int(x) for x in qo_lens]
    qo_indptr = [0]
    for n in qo_lens:
        qo_indptr.append(qo_indptr[-1] + n)
    total_q = qo_indptr[-1]
    params = make_params(total_q, num_qo_heads, num_kv_heads, head_dim, page_size, num_ctas=1,
                         level_ctas=level_ctas, level_tile_q=level_tile_q, enable_split=enable_split,
                         alpha=alpha, beta=beta, level_write_through=write_through,
                         defer_upload=defer_upload)
    levels = [{"qo_indptr": qo_indptr, "kv_lens": [int(x) for x in kv_lens], "causal": bool(causal)}]
    if workspace is None:
        workspace = Workspace(params, levels)
    info = plan(params, [0] * total_q, levels, workspace=workspace)
    return info, workspace, qo_indptr


def batch_prefill_paged(plan_info: PlanInfo, q, k_pool, v_pool, block_table, qo_indptr, kv_lens, causal=True,
                        sm_scale=None, out=None, lse=None):
    """pkc_batch_prefill_paged: ragged queries q [total_q, Hq, D] (rows qo_indptr[b] ..
    qo_indptr[b+1]-1 belong to request b) over the requests' block-table rows of kv_lens[b]
    tokens; qo_indptr / kv_lens are int32 device tensors.  Returns (o, lse)."""
    T, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    B = block_table.shape[0]
    for t, n in ((block_table, "block_table"), (qo_indptr, "qo_indptr"), (kv_lens, "kv_lens")):
        _need(t, n, torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_batch_prefill_paged(ctypes.byref(plan_info), _ptr(q), _ptr(k_pool), _ptr(v_pool), N,
                                       _ptr(block_table), block_table.shape[1], _ptr(qo_indptr), _ptr(kv_lens),
                                       B, T, Hq, Hkv, D, P, dtype_code(q.dtype), scale, 1 if causal else 0,
                                       _ptr(out), _ptr(lse), ws, wsn, _stream(dev)))
    return out, lse


def batch_prefill_paged_tree(plan_info: PlanInfo, q, k_pool, v_pool, block_table, qo_indptr, kv_lens,
                             tree_mask, mask_indptr, sm_scale=None, out=None, lse=None):
    """pkc_batch_prefill_paged_tree: causal ragged queries with per-request tree masks
    (tree_mask: uint8 device tensor holding every request's l_q x l_q byte matrix, request b's
    at byte mask_indptr[b]; mask_indptr: int32 device tensor [num_requests])."""
    T, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    B = block_table.shape[0]
    for t, n in ((block_table, "block_table"), (qo_indptr, "qo_indptr"), (kv_lens, "kv_lens"),
                 (mask_indptr, "mask_indptr")):
        _need(t, n, torch.int32, dev)
    _need(tree_mask, "tree_mask", torch.uint8, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_batch_prefill_paged_tree(ctypes.byref(plan_info), _ptr(q), _ptr(k_pool), _ptr(v_pool), N,
                                            _ptr(block_table), block_table.shape[1], _ptr(qo_indptr),
                                            _ptr(kv_lens), _ptr(tree_mask), _ptr(mask_indptr), tree_mask.numel(),
                                            B, T, Hq, Hkv, D, P, dtype_code(q.dtype), scale, _ptr(out), _ptr(lse),
                                            ws, wsn, _stream(dev)))
    return out, lse


def batch_prefill_paged_fp8(plan_info: PlanInfo, q, k_pool, v_pool, block_table, qo_indptr, kv_lens,
                            k_scale=1.0, v_scale=1.0, causal=True, sm_scale=None, out=None, lse=None):
    """pkc_batch_prefill_paged_fp8: batch_prefill_paged over OCP FP8 E4M3 pools (float8_e4m3fn
    or uint8 codes) with per-pool scales; q and o fp16 / bf16."""
    T, Hq, D = q.shape
    N, P, Hkv, _ = k_pool.shape
    dev = q.device
    B = block_table.shape[0]
    _check_fp8_pools(q, k_pool, v_pool)
    for t, n in ((block_table, "block_table"), (qo_indptr, "qo_indptr"), (kv_lens, "kv_lens")):
        _need(t, n, torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    ws, wsn = _ws_of(plan_info)
    _check(lib.pkc_batch_prefill_paged_fp8(ctypes.byref(plan_info), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                           float(k_scale), float(v_scale), N, _ptr(block_table),
                                           block_table.shape[1], _ptr(qo_indptr), _ptr(kv_lens), B, T, Hq, Hkv,
                                           D, P, dtype_code(q.dtype), scale, 1 if causal else 0, _ptr(out),
                                           _ptr(lse), ws, wsn, _stream(dev)))
    return out, lse


def validate_block_table(block_table, cache_seqlens, page_size, num_pages, kv_start=None):
    """pkc_validate_block_table on host copies."""
    bt = block_table.detach().to("cpu", torch.int32).contiguous()
    sl = cache_seqlens.detach().to("cpu", torch.int32).contiguous()
    ks = kv_start.detach().to("cpu", torch.int32).contiguous() if kv_start is not None else None
    P32 = ctypes.POINTER(ctypes.c_int32)
    _check(lib.pkc_validate_block_table(ctypes.cast(bt.data_ptr(), P32), bt.shape[1],
                                        ctypes.cast(sl.data_ptr(), P32),
                                        ctypes.cast(ks.data_ptr(), P32) if ks is not None else None,
                                        bt.shape[0], page_size, num_pages))


def debug_gather_rows(block_table, cache_seqlens, page_size, num_pages, max_tokens, kv_start=None):
    B = block_table.shape[0]
    out = torch.empty(B, max_tokens, dtype=torch.int32, device=block_table.device)
    _check(lib.pkc_debug_gather_rows(_ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
                                     _ptr(kv_start), B, page_size, num_pages, _ptr(out), max_tokens,
                                     _stream(block_table.device)))
    return out


def debug_cta_trace(plan_info: PlanInfo, stage: int, max_items_per_cta: int):
    ws = plan_info._workspace
    ctas = plan_info.num_ctas if stage == plan_info.num_levels else plan_info.level_ctas
    out = torch.empty(ctas * max_items_per_cta * 8, dtype=torch.int32, device=ws.device.device)
    _check(lib.pkc_debug_cta_trace(ctypes.byref(plan_info), stage, _ptr(ws.device), _ptr(out), out.numel(),
                                   max_items_per_cta, _stream(ws.device.device)))
    return out.view(ctas, max_items_per_cta, 8)


def timing_enable(on=True):
    _check(lib.pkc_timing_enable(1 if on else 0))


def timing_reset():
    _check(lib.pkc_timing_reset())


def timing_read(kind):
    n, ms = _I64(), ctypes.c_double()
    _check(lib.pkc_timing_read(kind, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def read_stream_probe(buf: torch.Tensor, sink: torch.Tensor = None):
    """pkc_read_stream_probe: one nontemporal read pass over `buf` (a device tensor whose byte
    size is a multiple of 1 MiB), on torch's current stream.  Returns the sink tensor."""
    nbytes = buf.numel() * buf.element_size()
    n = nbytes // (1 << 20) * 256
    if sink is None:
        sink = torch.empty(max(n, 1), dtype=torch.int32, device=buf.device)
    _check(lib.pkc_read_stream_probe(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(buf.device)))
    return sink


def read_plan_arrays(info: PlanInfo, host_buf: torch.Tensor):
    """Decode the integer plan arrays from a host buffer (layout documented in pkc.h) into
    Python lists: per stage the CTA item lists, merge rows per request and write-through
    flags.  Used by the plan parity tests."""
    buf = host_buf.numpy().view("int32") if host_buf.dtype == torch.uint8 else host_buf.numpy()

    def ints(off, n):
        return buf[off // 4: off // 4 + n].tolist()

    def stage(off_indptr, off_items, ctas):
        indptr = ints(off_indptr, ctas + 1)
        items = ints(off_items, 8 * indptr[-1])
        recs = [items[8 * k: 8 * k + 8] for k in range(indptr[-1])]
        return [recs[indptr[c]:indptr[c + 1]] for c in range(ctas)]

    out = {"levels": [], "decode": stage(info.off_dec_indptr, info.off_dec_items, info.num_ctas)}
    for l in range(info.num_levels):
        out["levels"].append(stage(info.off_lvl_indptr[l], info.off_lvl_items[l], info.level_ctas))
    nl2 = info.num_levels + 2
    mptr = ints(info.off_merge_ptr, info.batch * nl2)
    rows = ints(info.off_merge_rows, info.merge_entries)
    out["merge_ptr"] = [mptr[b * nl2:(b + 1) * nl2] for b in range(info.batch)]
    out["merge_rows"] = rows
    out["req_flags"] = ints(info.off_req_flags, info.batch)
    rl = ints(info.off_req_levels, info.batch * info.num_levels * 2)
    out["req_levels"] = [[tuple(rl[(b * info.num_levels + l) * 2:(b * info.num_levels + l) * 2 + 2])
                          for l in range(info.num_levels)] for b in range(info.batch)]
    return out
