"""Python binding of libdeft (ctypes).  Argument marshalling only.

Every function has the name of the C entry point it wraps (include/deft.h)
and does nothing but convert arguments: torch tensors become device pointers,
numpy arrays become host pointers, the torch stream becomes a hipStream_t.
All computation happens inside libdeft.so.  A failing call raises DeftError
with the library's code and message.  Since the C ABI sees bare pointers,
the wrappers of the attention calls first check each tensor's dtype, shape
and size against the plan and the descriptor (DeftError with
DEFT_ERR_INVALID_ARGUMENT), so a mis-shaped tensor never reaches a kernel.

torch is imported before the library is loaded so that the process holds one
HIP runtime (torch's), which libdeft then binds to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

# DEFT_LIB_PATH names another build of the library (the host-only sanitizer
# build of the planner, in the CPU tests).
LIB_PATH = os.environ.get("DEFT_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libdeft.so")

DEFT_OK = 0
DEFT_ERR_INVALID_ARGUMENT = -1
DEFT_ERR_INVALID_TREE = -2
DEFT_ERR_UNSUPPORTED = -3
DEFT_ERR_HIP = -4
DEFT_ERR_NO_MEMORY = -5
DEFT_DTYPE_F32 = 0
DEFT_DTYPE_BF16 = 1
DEFT_PARTIAL_F32 = 0
DEFT_PARTIAL_BF16_NORM = 1

EXPORTED_SYMBOLS = (
    "deft_plan_create", "deft_plan_create_query_centric", "deft_plan_create_node_chunks",
    "deft_plan_create_multi_token", "deft_plan_destroy", "deft_plan_export", "deft_plan_device_bytes",
    "deft_plan_upload", "deft_tree_attention", "deft_tree_attention_fused", "deft_partial_attention",
    "deft_lse_merge", "deft_last_error", "deft_tree_attention_noalloc", "deft_plan_status",
    "deft_plan_auto_chunk_tokens",
)
DEFT_NOALLOC_SCRATCH_BYTES = 64 << 20

_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


class DeftError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdeft error {code}: {msg}")
        self.code = code


class deft_plan_view(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_nodes", "num_queries", "chunk_tokens", "total_tokens", "num_chunks", "num_slots",
        "mask_words")] + [
        ("node_start", _I32P), ("flat_node_order", _I32P), ("node_flat_start", _I32P),
        ("flat_to_logical", _I32P), ("chunk_start", _I32P), ("group_offsets", _I32P),
        ("slot_query", _I32P), ("slot_mask", ctypes.POINTER(ctypes.c_uint32)),
        ("chunk_full", ctypes.POINTER(ctypes.c_uint8)), ("query_slot_offsets", _I32P),
        ("query_slots", _I32P)]


class deft_attn_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dtype", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages", "f32_partials")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdeft.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m tree_structured_decode_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    L.deft_plan_create.argtypes = [_I32P, _I32P, ctypes.c_int32, _I32P, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.POINTER(_P)]
    L.deft_plan_create_query_centric.argtypes = L.deft_plan_create.argtypes
    L.deft_plan_create_node_chunks.argtypes = L.deft_plan_create.argtypes
    L.deft_plan_create_multi_token.argtypes = [
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(_P)]
    L.deft_plan_destroy.argtypes = [_P]
    L.deft_plan_destroy.restype = None
    L.deft_plan_export.argtypes = [_P, ctypes.POINTER(deft_plan_view)]
    L.deft_plan_device_bytes.argtypes = [_P, ctypes.POINTER(deft_attn_desc),
                                         ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.deft_plan_upload.argtypes = [_P, ctypes.POINTER(deft_attn_desc), _P, ctypes.c_size_t, _P]
    L.deft_tree_attention.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.POINTER(deft_attn_desc),
                                      _P, ctypes.c_size_t, _P]
    L.deft_tree_attention_fused.argtypes = L.deft_tree_attention.argtypes
    L.deft_tree_attention_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.POINTER(deft_attn_desc), _P]
    L.deft_plan_status.argtypes = [_P, _P]
    L.deft_plan_auto_chunk_tokens.argtypes = [_I32P, _I32P, ctypes.c_int32, _I32P, _I32P, ctypes.c_int32,
                                              ctypes.POINTER(deft_attn_desc), ctypes.c_int32, _I32P]
    L.deft_partial_attention.argtypes = [_P, _P, _P, _P, _P, ctypes.POINTER(deft_attn_desc),
                                         _P, _P, _P, ctypes.c_int32, _P]
    L.deft_lse_merge.argtypes = [_P, ctypes.POINTER(deft_attn_desc), _P, _P, _P, ctypes.c_int32,
                                 _P, _P]
    L.deft_last_error.restype = ctypes.c_char_p
    for name in ("deft_plan_create", "deft_plan_create_query_centric", "deft_plan_create_node_chunks",
                 "deft_plan_create_multi_token", "deft_plan_export",
                 "deft_plan_device_bytes", "deft_plan_upload",
                 "deft_tree_attention", "deft_tree_attention_fused", "deft_tree_attention_noalloc",
                 "deft_partial_attention", "deft_lse_merge", "deft_plan_status",
                 "deft_plan_auto_chunk_tokens"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def deft_last_error() -> str:
    return lib().deft_last_error().decode()


def _check(rc: int):
    if rc != DEFT_OK:
        raise DeftError(rc, deft_last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _dev(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class Plan:
    """Owns a deft_plan* and frees it on garbage collection.  Also keeps the
    sizes the tensor checks need: queries, slots and logical tokens."""

    def __init__(self, handle: ctypes.c_void_p, logical_tokens: int):
        self.handle = handle
        v = deft_plan_view()
        _check(lib().deft_plan_export(handle, ctypes.byref(v)))
        self.num_queries, self.num_slots = int(v.num_queries), int(v.num_slots)
        self.logical_tokens = int(logical_tokens)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.deft_plan_destroy(self.handle)
            self.handle = None


def deft_plan_create(parents, seg_lens, query_nodes, chunk_tokens: int) -> Plan:
    p, s, q = _i32(parents), _i32(seg_lens), _i32(query_nodes)
    h = _P()
    _check(lib().deft_plan_create(_ptr_i32(p), _ptr_i32(s), int(p.shape[0]), _ptr_i32(q),
                                  int(q.shape[0]), int(chunk_tokens), ctypes.byref(h)))
    return Plan(h, int(s.sum(dtype=np.int64)))


def deft_plan_create_query_centric(parents, seg_lens, query_nodes, chunk_tokens: int) -> Plan:
    p, s, q = _i32(parents), _i32(seg_lens), _i32(query_nodes)
    h = _P()
    _check(lib().deft_plan_create_query_centric(_ptr_i32(p), _ptr_i32(s), int(p.shape[0]), _ptr_i32(q),
                                                int(q.shape[0]), int(chunk_tokens), ctypes.byref(h)))
    return Plan(h, int(s.sum(dtype=np.int64)))


def deft_plan_create_node_chunks(parents, seg_lens, query_nodes, chunk_tokens: int) -> Plan:
    p, s, q = _i32(parents), _i32(seg_lens), _i32(query_nodes)
    h = _P()
    _check(lib().deft_plan_create_node_chunks(_ptr_i32(p), _ptr_i32(s), int(p.shape[0]), _ptr_i32(q),
                                              int(q.shape[0]), int(chunk_tokens), ctypes.byref(h)))
    return Plan(h, int(s.sum(dtype=np.int64)))


def deft_plan_create_multi_token(parents, seg_lens, query_nodes, query_lens, chunk_tokens: int) -> Plan:
    """query_lens None passes NULL (every query sees its whole node)."""
    p, s, q = _i32(parents), _i32(seg_lens), _i32(query_nodes)
    ql = None if query_lens is None else _i32(query_lens)
    if ql is not None and ql.shape[0] != q.shape[0]:
        raise ValueError("query_lens needs one entry per query")
    h = _P()
    _check(lib().deft_plan_create_multi_token(_ptr_i32(p), _ptr_i32(s), int(p.shape[0]), _ptr_i32(q),
                                              None if ql is None else _ptr_i32(ql), int(q.shape[0]),
                                              int(chunk_tokens), ctypes.byref(h)))
    return Plan(h, int(s.sum(dtype=np.int64)))


def deft_plan_auto_chunk_tokens(parents, seg_lens, query_nodes, desc, num_cus: int = 0,
                                query_lens=None) -> int:
    """The library's chunk size for this tree and attention shape (see deft.h)."""
    p, s, q = _i32(parents), _i32(seg_lens), _i32(query_nodes)
    ql = None if query_lens is None else _i32(query_lens)
    if ql is not None and ql.shape[0] != q.shape[0]:
        raise ValueError("query_lens needs one entry per query")
    out = ctypes.c_int32()
    _check(lib().deft_plan_auto_chunk_tokens(_ptr_i32(p), _ptr_i32(s), int(p.shape[0]), _ptr_i32(q),
                                             None if ql is None else _ptr_i32(ql), int(q.shape[0]),
                                             ctypes.byref(desc), int(num_cus), ctypes.byref(out)))
    return int(out.value)


def deft_plan_destroy(plan: Plan):
    if plan.handle:
        lib().deft_plan_destroy(plan.handle)
        plan.handle = None


def deft_plan_export(plan: Plan) -> dict:
    """Copies of the plan's arrays, keyed as in deft_plan_view."""
    v = deft_plan_view()
    _check(lib().deft_plan_export(plan.handle, ctypes.byref(v)))

    def arr(ptr, n, dt):
        if n == 0:
            return np.zeros(0, dtype=dt)
        return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dt, copy=True)

    n, nq, t, nc, s, w = v.num_nodes, v.num_queries, v.total_tokens, v.num_chunks, v.num_slots, v.mask_words
    return {
        "num_nodes": n, "num_queries": nq, "chunk_tokens": v.chunk_tokens, "total_tokens": t,
        "num_chunks": nc, "num_slots": s, "mask_words": w,
        "node_start": arr(v.node_start, n, np.int32),
        "flat_node_order": arr(v.flat_node_order, n, np.int32),
        "node_flat_start": arr(v.node_flat_start, n, np.int32),
        "flat_to_logical": arr(v.flat_to_logical, t, np.int32),
        "chunk_start": arr(v.chunk_start, nc + 1, np.int32),
        "group_offsets": arr(v.group_offsets, nc + 1, np.int32),
        "slot_query": arr(v.slot_query, s, np.int32),
        "slot_mask": arr(v.slot_mask, s * w, np.uint32).reshape(s, w),
        "chunk_full": arr(v.chunk_full, nc, np.uint8),
        "query_slot_offsets": arr(v.query_slot_offsets, nq + 1, np.int32),
        "query_slots": arr(v.query_slots, s, np.int32),
    }


def make_desc(dtype: torch.dtype, num_q_heads: int, num_kv_heads: int, head_dim: int,
              num_pages: int, page_size: int = 16, f32_partials: bool = False) -> deft_attn_desc:
    """f32_partials: fp32 unnormalised per-slot partials in the workspace for
    bf16 inputs too (the default keeps bf16 O / l for bf16 inputs)."""
    code = {torch.float32: DEFT_DTYPE_F32, torch.bfloat16: DEFT_DTYPE_BF16}.get(dtype, 99)
    return deft_attn_desc(code, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, int(f32_partials))


def deft_plan_device_bytes(plan: Plan, desc: deft_attn_desc):
    pb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().deft_plan_device_bytes(plan.handle, ctypes.byref(desc), ctypes.byref(pb), ctypes.byref(wb)))
    return pb.value, wb.value


def deft_plan_upload(plan: Plan, desc: deft_attn_desc, dev_plan: torch.Tensor, stream=None):
    _check(lib().deft_plan_upload(plan.handle, ctypes.byref(desc), _dev(dev_plan),
                                  dev_plan.numel() * dev_plan.element_size(), _stream(stream)))
    plan.dev_plan = dev_plan          # keep the device image alive with the plan


def deft_plan_status(plan: Plan, stream=None):
    """Raises DeftError(DEFT_ERR_HIP) if a kernel's bounded wait gave up since
    the last check (synchronises the stream)."""
    _check(lib().deft_plan_status(plan.handle, _stream(stream)))


_DTYPES = {DEFT_DTYPE_F32: torch.float32, DEFT_DTYPE_BF16: torch.bfloat16}


def _expect(t, what, dtype, shape=None, min_numel=None, min_rows=None):
    """shape: the exact shape, or with min_rows the shape after the first
    dimension, which then needs at least min_rows entries."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        bad = True
    else:
        if shape is not None and min_rows is not None:
            ok_shape = t.dim() == len(shape) + 1 and t.shape[0] >= min_rows and tuple(t.shape[1:]) == tuple(shape)
        else:
            ok_shape = shape is None or tuple(t.shape) == tuple(shape)
        bad = t.dtype != dtype or not ok_shape or (min_numel is not None and t.numel() < min_numel)
    if bad:
        want = f"{dtype}" + (f" of shape {tuple(shape)}" if shape is not None and min_rows is None else "") + \
            (f" of shape (>= {min_rows}, {', '.join(map(str, shape))})" if min_rows is not None else "") + \
            (f" with at least {min_numel} elements" if min_numel is not None else "")
        got = f"{t.dtype} of shape {tuple(t.shape)}" if isinstance(t, torch.Tensor) else type(t).__name__
        raise DeftError(DEFT_ERR_INVALID_ARGUMENT, f"{what}: expected {want}, got {got}")


def _check_inputs(plan: Plan, desc, q=None, k_cache=None, v_cache=None, block_table=None, out=None):
    dt = _DTYPES.get(desc.dtype)
    if dt is None:
        return                                   # the library reports the unsupported dtype
    nq, hq, hkv, d = plan.num_queries, desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    _expect(q, "q", dt, (nq, hq, d))
    _expect(out, "out", dt, (nq, hq, d))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):    # pages [num_pages, page, Hkv, d]
        _expect(t, name, dt, (desc.page_size, hkv, d), min_rows=desc.num_pages)
    _expect(block_table, "block_table", torch.int32,
            min_numel=-(-plan.logical_tokens // max(desc.page_size, 1)))


def _check_partials(plan: Plan, desc, fmt, part_o, part_m, part_l):
    if fmt not in (DEFT_PARTIAL_F32, DEFT_PARTIAL_BF16_NORM):
        return                                   # the library reports the format
    s, hq, d = plan.num_slots, desc.num_q_heads, desc.head_dim
    odt = torch.bfloat16 if fmt == DEFT_PARTIAL_BF16_NORM else torch.float32
    _expect(part_o, "part_o", odt, (s, hq, d))
    _expect(part_m, "part_m", torch.float32, (s, hq))
    _expect(part_l, "part_l", torch.float32, (s, hq))


def deft_tree_attention(q, k_cache, v_cache, block_table, plan: Plan, out, desc, workspace, stream=None):
    _check_inputs(plan, desc, q, k_cache, v_cache, block_table, out)
    _check(lib().deft_tree_attention(_dev(q), _dev(k_cache), _dev(v_cache), _dev(block_table),
                                     plan.handle, _dev(out), ctypes.byref(desc), _dev(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def deft_tree_attention_fused(q, k_cache, v_cache, block_table, plan: Plan, out, desc, workspace,
                              stream=None):
    _check_inputs(plan, desc, q, k_cache, v_cache, block_table, out)
    _check(lib().deft_tree_attention_fused(_dev(q), _dev(k_cache), _dev(v_cache), _dev(block_table),
                                           plan.handle, _dev(out), ctypes.byref(desc), _dev(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))


def deft_tree_attention_noalloc(q, k_cache, v_cache, block_table, plan: Plan, out, desc, stream=None):
    _check_inputs(plan, desc, q, k_cache, v_cache, block_table, out)
    _check(lib().deft_tree_attention_noalloc(_dev(q), _dev(k_cache), _dev(v_cache), _dev(block_table),
                                             plan.handle, _dev(out), ctypes.byref(desc), _stream(stream)))


def deft_partial_attention(q, k_cache, v_cache, block_table, plan: Plan, desc, part_o, part_m,
                           part_l, partial_format=DEFT_PARTIAL_F32, stream=None):
    _check_inputs(plan, desc, q, k_cache, v_cache, block_table)
    _check_partials(plan, desc, partial_format, part_o, part_m, part_l)
    _check(lib().deft_partial_attention(_dev(q), _dev(k_cache), _dev(v_cache), _dev(block_table),
                                        plan.handle, ctypes.byref(desc), _dev(part_o), _dev(part_m),
                                        _dev(part_l), int(partial_format), _stream(stream)))


def deft_lse_merge(plan: Plan, desc, part_o, part_m, part_l, out, partial_format=DEFT_PARTIAL_F32,
                   stream=None):
    _check_inputs(plan, desc, out=out)
    _check_partials(plan, desc, partial_format, part_o, part_m, part_l)
    _check(lib().deft_lse_merge(plan.handle, ctypes.byref(desc), _dev(part_o), _dev(part_m),
                                _dev(part_l), int(partial_format), _dev(out), _stream(stream)))
