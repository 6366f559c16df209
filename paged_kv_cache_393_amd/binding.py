"""ctypes binding of libpagedattn.so (C-ABI in include/paged_attn.h).

Argument marshalling only: torch tensors are checked for dtype/shape/device
and passed as raw device pointers with sizes; every step of the decode runs
in the library's HIP kernels.  There is no fallback: if the library is
missing or a call fails, this module raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "paged_attn.h")
WRITE_HEADER = os.path.join(os.path.dirname(_HERE), "include", "paged_kv_write.h")
EVICT_HEADER = os.path.join(os.path.dirname(_HERE), "include", "paged_kv_evict.h")
PREFILL_HEADER = os.path.join(os.path.dirname(_HERE), "include", "paged_prefill.h")

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_SHAPE = -2
PA_ERR_UNSUPPORTED = -3
PA_ERR_WORKSPACE = -4
PA_ERR_LAUNCH = -5
PA_ERR_ALIGNMENT = -6
PA_ERR_SCRATCH = -7


class PaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "max_blocks_per_seq", "num_blocks", "split_tokens")]


class PaWriteShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "num_kv_heads", "head_dim", "block_size", "num_blocks", "key_stride",
        "value_stride")]


class PaScoreShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_kv_heads", "head_dim", "block_size", "max_blocks_per_seq", "num_blocks")]


class PaPrefillShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "max_blocks_per_seq",
        "num_blocks", "max_q_len")]


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"paged_attn error {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    SP = ctypes.POINTER(PaShape)
    lib.paged_attn_plan.argtypes = [SP, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.paged_attn_plan.restype = ctypes.c_int
    lib.paged_attn_workspace_bytes.argtypes = [SP]
    lib.paged_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.paged_attn_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, SP, P, ctypes.c_size_t, P]
    lib.paged_attn_decode.restype = ctypes.c_int
    lib.paged_attn_decode_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, SP, P]
    lib.paged_attn_decode_noalloc.restype = ctypes.c_int
    lib.paged_attn_decode_int8.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P, SP, P,
                                           ctypes.c_size_t, P]
    lib.paged_attn_decode_int8.restype = ctypes.c_int
    WP = ctypes.POINTER(PaWriteShape)
    lib.paged_kv_write.argtypes = [P, P, P, P, P, WP, P]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_kv_write_int8.argtypes = [P, P, P, P, P, P, P, WP, P]
    lib.paged_kv_write_int8.restype = ctypes.c_int
    lib.paged_attn_decode_fp8.argtypes = [P, P, P, P, P, ctypes.c_float, P, SP, P,
                                          ctypes.c_size_t, P]
    lib.paged_attn_decode_fp8.restype = ctypes.c_int
    lib.paged_kv_write_fp8.argtypes = [P, P, P, P, P, WP, P]
    lib.paged_kv_write_fp8.restype = ctypes.c_int
    CP = ctypes.POINTER(PaScoreShape)
    lib.paged_kv_token_scores.argtypes = [P, P, P, P, P, P, CP, P]
    lib.paged_kv_token_scores.restype = ctypes.c_int
    lib.paged_kv_token_scores_int8.argtypes = [P, P, P, P, P, P, P, P, CP, P]
    lib.paged_kv_token_scores_int8.restype = ctypes.c_int
    lib.paged_kv_token_scores_fp8.argtypes = [P, P, P, P, P, P, CP, P]
    lib.paged_kv_token_scores_fp8.restype = ctypes.c_int
    lib.paged_kv_evict_lowest_block.argtypes = [P, P, P, P, P, CP, P]
    lib.paged_kv_evict_lowest_block.restype = ctypes.c_int
    lib.paged_attn_check_tables.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, P, P]
    lib.paged_attn_check_tables.restype = ctypes.c_int
    lib.paged_kv_compress_workspace_bytes.argtypes = [CP, ctypes.c_int32]
    lib.paged_kv_compress_workspace_bytes.restype = ctypes.c_size_t
    lib.paged_kv_compress_prefill.argtypes = [P, P, P, P, P, ctypes.c_int32, CP, P, ctypes.c_size_t, P]
    lib.paged_kv_compress_prefill.restype = ctypes.c_int
    lib.paged_kv_compress_prefill_int8.argtypes = [P, P, P, P, P, P, P, ctypes.c_int32, CP, P,
                                                   ctypes.c_size_t, P]
    lib.paged_kv_compress_prefill_int8.restype = ctypes.c_int
    lib.paged_kv_compress_prefill_fp8.argtypes = [P, P, P, P, P, ctypes.c_int32, CP, P, ctypes.c_size_t, P]
    lib.paged_kv_compress_prefill_fp8.restype = ctypes.c_int
    lib.paged_attn_prefill.argtypes = [P, P, P, P, P, P, ctypes.c_float, P,
                                       ctypes.POINTER(PaPrefillShape), P]
    lib.paged_attn_prefill.restype = ctypes.c_int
    lib.paged_attn_prefill_int8.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                            ctypes.POINTER(PaPrefillShape), P]
    lib.paged_attn_prefill_int8.restype = ctypes.c_int
    lib.paged_attn_prefill_fp8.argtypes = [P, P, P, P, P, P, ctypes.c_float, P,
                                           ctypes.POINTER(PaPrefillShape), P]
    lib.paged_attn_prefill_fp8.restype = ctypes.c_int
    PS = ctypes.POINTER(PaPrefillShape)
    lib.paged_attn_prefill_plan.argtypes = [PS, ctypes.POINTER(ctypes.c_int32)]
    lib.paged_attn_prefill_plan.restype = ctypes.c_int
    lib.paged_attn_prefill_workspace_bytes.argtypes = [PS, ctypes.c_int32]
    lib.paged_attn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.paged_attn_prefill_split.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, PS, ctypes.c_int32,
                                             P, ctypes.c_size_t, P]
    lib.paged_attn_prefill_split.restype = ctypes.c_int
    lib.paged_attn_prefill_split_int8.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_float, P, PS,
                                                  ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.paged_attn_prefill_split_int8.restype = ctypes.c_int
    lib.paged_attn_prefill_split_fp8.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, PS,
                                                 ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.paged_attn_prefill_split_fp8.restype = ctypes.c_int
    lib.paged_attn_strerror.argtypes = [ctypes.c_int]
    lib.paged_attn_strerror.restype = ctypes.c_char_p
    lib.paged_attn_abi_version.argtypes = []
    lib.paged_attn_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions the library's headers (include/paged_attn.h,
    include/paged_kv_write.h, include/paged_kv_evict.h, include/paged_prefill.h)
    declare."""
    names = set()
    for h in (HEADER, WRITE_HEADER, EVICT_HEADER, PREFILL_HEADER):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b((?:paged_attn|paged_kv)_\w+)\s*\(", text))
    return sorted(names)


def strerror(code: int) -> str:
    return load().paged_attn_strerror(code).decode()


def _check(rc: int):
    if rc != PA_OK:
        raise PagedAttnError(rc, strerror(rc))


def make_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
               num_blocks, split_tokens=0) -> PaShape:
    return PaShape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                   max_blocks_per_seq, num_blocks, split_tokens)


def plan(shape: PaShape):
    st = ctypes.c_int32()
    ms = ctypes.c_int32()
    _check(load().paged_attn_plan(ctypes.byref(shape), ctypes.byref(st), ctypes.byref(ms)))
    return st.value, ms.value


def workspace_bytes(shape: PaShape) -> int:
    return int(load().paged_attn_workspace_bytes(ctypes.byref(shape)))


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _on(stream):
    """Context for the tensors a wrapper allocates for a call on `stream`:
    made under it, they belong to that stream, so the caching allocator does
    not hand their memory to other work before the call's kernels are done,
    and a fill that initialises one runs on that stream, before the call."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def shape_of(q, k_cache, block_tables, split_tokens=0) -> PaShape:
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim of q and cache differ")
    return make_shape(S, Hq, Hkv, D, bs, block_tables.shape[1], NB, split_tokens)


def _validate(q, k_cache, v_cache, block_tables, context_lens, kv_dtype):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("context_lens", context_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bf16")
    if k_cache.dtype != kv_dtype or v_cache.dtype != kv_dtype:
        raise TypeError(f"cache must be {kv_dtype}")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")


def _check_out(out, q):
    """A caller's `out` must be a contiguous fp32 device tensor shaped like q:
    the kernels write q's row count times Hq x D floats into it."""
    if out is not None and (not out.is_cuda or out.dtype != torch.float32 or
                            tuple(out.shape) != tuple(q.shape) or not out.is_contiguous()):
        raise ValueError("out must be a contiguous fp32 device tensor shaped like q")


def alloc_workspace(shape: PaShape, device) -> torch.Tensor:
    """Scratch workspace for decode calls of `shape` (no initialisation needed)."""
    n = workspace_bytes(shape)
    if n <= 0:
        raise PagedAttnError(PA_ERR_SHAPE, "no workspace size for this shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out=None,
           split_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
    """out fp32 [S, Hq, D] = paged_attn_decode(...) on the current (or given) stream."""
    _validate(q, k_cache, v_cache, block_tables, context_lens, torch.bfloat16)
    shape = shape_of(q, k_cache, block_tables, split_tokens)
    _check_out(out, q)
    with _on(stream):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(shape, q.device)
    ws_n = workspace.numel() if workspace is not None else 0
    rc = load().paged_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                  _ptr(context_lens), ctypes.c_float(scale), _ptr(out),
                                  ctypes.byref(shape), _ptr(workspace), ctypes.c_size_t(ws_n),
                                  _stream_handle(stream))
    _check(rc)
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
                   split_tokens: int = 0, stream=None) -> torch.Tensor:
    """paged_attn_decode_noalloc: the bf16 decode with its partial results in
    the library's static device scratch; `out` fp32 [S, Hq, D] is the caller's
    and nothing is allocated."""
    _validate(q, k_cache, v_cache, block_tables, context_lens, torch.bfloat16)
    if out is None:
        raise ValueError("out must be a contiguous fp32 device tensor shaped like q")
    _check_out(out, q)
    shape = shape_of(q, k_cache, block_tables, split_tokens)
    _check(load().paged_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(block_tables), _ptr(context_lens),
                                            ctypes.c_float(scale), _ptr(out), ctypes.byref(shape),
                                            _stream_handle(stream)))
    return out


def decode_int8(q, k_cache, v_cache, k_scales, v_scales, block_tables, context_lens,
                scale: float, out=None, split_tokens: int = 0, workspace=None,
                stream=None) -> torch.Tensor:
    """out fp32 [S, Hq, D] = paged_attn_decode_int8(...)."""
    _validate(q, k_cache, v_cache, block_tables, context_lens, torch.int8)
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 device tensor")
        if tuple(t.shape) != tuple(k_cache.shape[:3]):
            raise ValueError(f"{name} must be [num_blocks, block_size, num_kv_heads]")
    shape = shape_of(q, k_cache, block_tables, split_tokens)
    _check_out(out, q)
    with _on(stream):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(shape, q.device)
    ws_n = workspace.numel() if workspace is not None else 0
    rc = load().paged_attn_decode_int8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales),
                                       _ptr(v_scales), _ptr(block_tables), _ptr(context_lens),
                                       ctypes.c_float(scale), _ptr(out), ctypes.byref(shape),
                                       _ptr(workspace), ctypes.c_size_t(ws_n),
                                       _stream_handle(stream))
    _check(rc)
    return out


FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale: float, out=None,
               split_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
    """out fp32 [S, Hq, D] = paged_attn_decode_fp8(...): the cache holds FP8 E4M3
    codes (a float8_e4m3fn or uint8 tensor)."""
    if k_cache.dtype not in FP8_DTYPES or v_cache.dtype != k_cache.dtype:
        raise TypeError("fp8 cache must be float8_e4m3fn (or uint8 codes)")
    _validate(q, k_cache, v_cache, block_tables, context_lens, k_cache.dtype)
    shape = shape_of(q, k_cache, block_tables, split_tokens)
    _check_out(out, q)
    with _on(stream):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(shape, q.device)
    rc = load().paged_attn_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                      _ptr(context_lens), ctypes.c_float(scale), _ptr(out),
                                      ctypes.byref(shape), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel()), _stream_handle(stream))
    _check(rc)
    return out


def decode_views(views: dict, out=None, split_tokens: int = 0, workspace=None, stream=None):
    """Decode one layer given the per-layer views of the input generator."""
    if views["k_cache"].dtype in FP8_DTYPES:
        return decode_fp8(views["q"], views["k_cache"], views["v_cache"], views["block_tables"],
                          views["context_lens"], views["scale"], out=out,
                          split_tokens=split_tokens, workspace=workspace, stream=stream)
    if "k_scales" in views:
        return decode_int8(views["q"], views["k_cache"], views["v_cache"], views["k_scales"],
                           views["v_scales"], views["block_tables"], views["context_lens"],
                           views["scale"], out=out, split_tokens=split_tokens,
                           workspace=workspace, stream=stream)
    return decode(views["q"], views["k_cache"], views["v_cache"], views["block_tables"],
                  views["context_lens"], views["scale"], out=out, split_tokens=split_tokens,
                  workspace=workspace, stream=stream)


def write_shape(key, k_cache, num_blocks=None) -> PaWriteShape:
    """Shape record of a write of `key` [T, Hkv, d] (rows may be strided) into `k_cache`."""
    T, Hkv, D = key.shape
    NB, bs, Hkv2, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D):
        raise ValueError("key and cache disagree on kv heads / head_dim")
    return PaWriteShape(T, Hkv, D, bs, NB if num_blocks is None else num_blocks, 0, 0)


def _validate_write(key, value, slot_mapping, k_cache, v_cache, kv_dtype):
    for name, t in (("key", key), ("value", value), ("slot_mapping", slot_mapping),
                    ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    for name, t in (("key", key), ("value", value)):
        if t.dtype != torch.bfloat16 or t.dim() != 3:
            raise TypeError(f"{name} must be bf16 [T, Hkv, d]")
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name}: each token's [Hkv, d] rows must be contiguous")
    if value.shape != key.shape:
        raise ValueError("key and value shapes differ")
    if slot_mapping.dtype != torch.int32 or tuple(slot_mapping.shape) != (key.shape[0],):
        raise TypeError("slot_mapping must be int32 [T]")
    if not slot_mapping.is_contiguous() or not k_cache.is_contiguous() or \
            not v_cache.is_contiguous():
        raise ValueError("slot_mapping and the caches must be contiguous")
    if k_cache.dtype != kv_dtype or v_cache.dtype != kv_dtype or k_cache.shape != v_cache.shape:
        raise TypeError(f"caches must be two {kv_dtype} tensors of one shape")


def _write_shape_strided(key, value, k_cache):
    sh = write_shape(key, k_cache)
    sh.key_stride = key.stride(0) if key.shape[0] > 1 else 0
    sh.value_stride = value.stride(0) if value.shape[0] > 1 else 0
    return sh


def kv_write(key, value, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """paged_kv_write: store token t's K/V rows at slot slot_mapping[t] (bf16 cache)."""
    _validate_write(key, value, slot_mapping, k_cache, v_cache, torch.bfloat16)
    sh = _write_shape_strided(key, value, k_cache)
    _check(load().paged_kv_write(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache),
                                 _ptr(v_cache), ctypes.byref(sh), _stream_handle(stream)))


def kv_write_int8(key, value, slot_mapping, k_cache, v_cache, k_scales, v_scales,
                  stream=None) -> None:
    """paged_kv_write_int8: quantize token t's K/V rows and store them at slot_mapping[t]."""
    _validate_write(key, value, slot_mapping, k_cache, v_cache, torch.int8)
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 device tensor")
        if tuple(t.shape) != tuple(k_cache.shape[:3]):
            raise ValueError(f"{name} must be [num_blocks, block_size, num_kv_heads]")
    sh = _write_shape_strided(key, value, k_cache)
    _check(load().paged_kv_write_int8(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache),
                                      _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
                                      ctypes.byref(sh), _stream_handle(stream)))


def kv_write_fp8(key, value, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """paged_kv_write_fp8: cast token t's K/V rows to FP8 E4M3 and store them at
    slot_mapping[t] (cache: float8_e4m3fn or uint8 codes)."""
    if k_cache.dtype not in FP8_DTYPES:
        raise TypeError("fp8 cache must be float8_e4m3fn (or uint8 codes)")
    _validate_write(key, value, slot_mapping, k_cache, v_cache, k_cache.dtype)
    sh = _write_shape_strided(key, value, k_cache)
    _check(load().paged_kv_write_fp8(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache),
                                     _ptr(v_cache), ctypes.byref(sh), _stream_handle(stream)))


def kv_write_inputs(inp: dict, stream=None) -> None:
    """Run the write of a make_write_inputs() dict (bf16, int8 or fp8 cache)."""
    if inp["k_cache"].dtype in FP8_DTYPES:
        kv_write_fp8(inp["key"], inp["value"], inp["slots"], inp["k_cache"], inp["v_cache"],
                     stream=stream)
        return
    if "k_scales" in inp:
        kv_write_int8(inp["key"], inp["value"], inp["slots"], inp["k_cache"], inp["v_cache"],
                      inp["k_scales"], inp["v_scales"], stream=stream)
    else:
        kv_write(inp["key"], inp["value"], inp["slots"], inp["k_cache"], inp["v_cache"],
                 stream=stream)


def score_shape(k_cache, block_tables) -> PaScoreShape:
    NB, bs, Hkv, D = k_cache.shape
    S, MB = block_tables.shape
    return PaScoreShape(S, Hkv, D, bs, MB, NB)


def token_scores(views: dict, scores=None, token_begin=None, stream=None) -> torch.Tensor:
    """PagedEviction importances ||V|| / ||K|| of the tokens of per-layer views
    (bf16, int8 or fp8 cache), stored per token slot: fp32 [num_blocks,
    block_size].  A new `scores` tensor is filled with NaN first; slots of no
    scored token keep what `scores` held."""
    kc, vc = views["k_cache"], views["v_cache"]
    bt, cl = views["block_tables"], views["context_lens"]
    for name, t in (("k_cache", kc), ("v_cache", vc), ("block_tables", bt), ("context_lens", cl)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if bt.dtype != torch.int32 or cl.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    NB, bs = kc.shape[0], kc.shape[1]
    if scores is None:
        with _on(stream):
            scores = torch.full((NB, bs), float("nan"), dtype=torch.float32, device=kc.device)
    if scores.dtype != torch.float32 or tuple(scores.shape) != (NB, bs) or not scores.is_contiguous():
        raise ValueError("scores must be contiguous fp32 [num_blocks, block_size]")
    if token_begin is not None and (token_begin.dtype != torch.int32 or not token_begin.is_cuda):
        raise TypeError("token_begin must be an int32 device tensor")
    sh = score_shape(kc, bt)
    L = load()
    tb = _ptr(token_begin)
    if kc.dtype in FP8_DTYPES:
        rc = L.paged_kv_token_scores_fp8(_ptr(kc), _ptr(vc), _ptr(bt), tb, _ptr(cl), _ptr(scores),
                                         ctypes.byref(sh), _stream_handle(stream))
    elif "k_scales" in views:
        rc = L.paged_kv_token_scores_int8(_ptr(kc), _ptr(vc), _ptr(views["k_scales"]),
                                          _ptr(views["v_scales"]), _ptr(bt), tb, _ptr(cl),
                                          _ptr(scores), ctypes.byref(sh), _stream_handle(stream))
    else:
        if kc.dtype != torch.bfloat16:
            raise TypeError("cache must be bf16, int8 (with scales) or fp8")
        rc = L.paged_kv_token_scores(_ptr(kc), _ptr(vc), _ptr(bt), tb, _ptr(cl), _ptr(scores),
                                     ctypes.byref(sh), _stream_handle(stream))
    _check(rc)
    return scores


def evict_lowest_block(scores, block_tables, context_lens, evict_mask, evicted=None,
                       stream=None) -> torch.Tensor:
    """paged_kv_evict_lowest_block: for every masked sequence evict its full
    block of lowest mean importance (block_tables and context_lens updated in
    place); returns evicted int32 [S] (the freed physical block, or -1)."""
    S, MB = block_tables.shape
    NB, bs = scores.shape
    for name, t, dt in (("scores", scores, torch.float32), ("block_tables", block_tables, torch.int32),
                        ("context_lens", context_lens, torch.int32),
                        ("evict_mask", evict_mask, torch.int32)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt:
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    if tuple(context_lens.shape) != (S,) or tuple(evict_mask.shape) != (S,):
        raise ValueError("context_lens and evict_mask must be [S]")
    if evicted is None:
        with _on(stream):
            evicted = torch.empty(S, dtype=torch.int32, device=scores.device)
    sh = PaScoreShape(S, 1, 64, bs, MB, NB)     # heads / head_dim are not used here
    _check(load().paged_kv_evict_lowest_block(_ptr(scores), _ptr(block_tables), _ptr(context_lens),
                                              _ptr(evict_mask), _ptr(evicted), ctypes.byref(sh),
                                              _stream_handle(stream)))
    return evicted


def check_tables(block_tables, context_lens, num_blocks: int, block_size: int, stream=None):
    """paged_attn_check_tables: (number of sequences breaking the caller
    contract, lowest such sequence or -1), checked on the device."""
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    S, MB = block_tables.shape
    if tuple(context_lens.shape) != (S,):
        raise ValueError("context_lens must be [num_seqs]")
    with _on(stream):
        res = torch.empty(2, dtype=torch.int32, device=block_tables.device)
        _check(load().paged_attn_check_tables(_ptr(block_tables), _ptr(context_lens), S, MB,
                                              int(block_size), int(num_blocks), _ptr(res),
                                              _stream_handle(stream)))
        r = res.cpu().tolist()   # copied on the call's stream, after the check
    return r[0], r[1]


def compress_workspace_bytes(k_cache, block_tables, budget: int) -> int:
    return int(load().paged_kv_compress_workspace_bytes(ctypes.byref(score_shape(k_cache, block_tables)),
                                                        int(budget)))


def compress_prefill(views: dict, scores, budget: int, workspace=None, stream=None) -> None:
    """paged_kv_compress_prefill*: every sequence longer than `budget` keeps
    its `budget` most important tokens (scores fp32 [num_blocks, block_size]),
    in order, at positions 0 .. budget-1; the cache, its int8 scales, the
    scores and context_lens are updated in place."""
    kc, vc = views["k_cache"], views["v_cache"]
    bt, cl = views["block_tables"], views["context_lens"]
    for name, t in (("k_cache", kc), ("v_cache", vc), ("block_tables", bt), ("context_lens", cl),
                    ("scores", scores)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if bt.dtype != torch.int32 or cl.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    NB, bs = kc.shape[0], kc.shape[1]
    if scores.dtype != torch.float32 or tuple(scores.shape) != (NB, bs):
        raise ValueError("scores must be fp32 [num_blocks, block_size]")
    if tuple(cl.shape) != (bt.shape[0],):
        raise ValueError("context_lens must be [num_seqs]")
    sh = score_shape(kc, bt)
    L = load()
    need = int(L.paged_kv_compress_workspace_bytes(ctypes.byref(sh), int(budget)))
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=kc.device)
    st = _stream_handle(stream)
    ws, wsb = _ptr(workspace), workspace.numel() * workspace.element_size()
    if kc.dtype in FP8_DTYPES:
        rc = L.paged_kv_compress_prefill_fp8(_ptr(kc), _ptr(vc), _ptr(scores), _ptr(bt), _ptr(cl),
                                             int(budget), ctypes.byref(sh), ws, wsb, st)
    elif "k_scales" in views:
        rc = L.paged_kv_compress_prefill_int8(_ptr(kc), _ptr(vc), _ptr(views["k_scales"]),
                                              _ptr(views["v_scales"]), _ptr(scores), _ptr(bt),
                                              _ptr(cl), int(budget), ctypes.byref(sh), ws, wsb, st)
    else:
        if kc.dtype != torch.bfloat16:
            raise TypeError("cache must be bf16, int8 (with scales) or fp8")
        rc = L.paged_kv_compress_prefill(_ptr(kc), _ptr(vc), _ptr(scores), _ptr(bt), _ptr(cl),
                                         int(budget), ctypes.byref(sh), ws, wsb, st)
    _check(rc)


def _prefill_shape(q, k_cache, v_cache, block_tables, context_lens, q_offsets, max_q_len,
                   cache_dtypes, scales=()):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("context_lens", context_lens),
                    ("q_offsets", q_offsets)) + tuple(scales):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bf16")
    if k_cache.dtype not in cache_dtypes or v_cache.dtype not in cache_dtypes:
        raise TypeError(f"the cache must be one of {cache_dtypes}")
    if k_cache.shape != v_cache.shape or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q / cache shapes disagree")
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens),
                    ("q_offsets", q_offsets)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    for name, t in scales:
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(k_cache.shape[:3]):
            raise ValueError(f"{name} must be fp32 [NB, bs, Hkv]")
    S, MB = block_tables.shape
    if tuple(q_offsets.shape) != (S + 1,) or tuple(context_lens.shape) != (S,):
        raise ValueError("q_offsets must be [S + 1] and context_lens [S]")
    NB, bs, Hkv, D = k_cache.shape
    return PaPrefillShape(S, q.shape[1], Hkv, D, bs, MB, NB, int(max_q_len))


def prefill_plan(shape: PaPrefillShape) -> int:
    """paged_attn_prefill_plan: a key_splits for `shape` on the current device."""
    k = ctypes.c_int32()
    _check(load().paged_attn_prefill_plan(ctypes.byref(shape), ctypes.byref(k)))
    return k.value


def prefill_workspace_bytes(shape: PaPrefillShape, key_splits: int) -> int:
    return int(load().paged_attn_prefill_workspace_bytes(ctypes.byref(shape), int(key_splits)))


def alloc_prefill_workspace(shape: PaPrefillShape, key_splits: int, device) -> Optional[torch.Tensor]:
    """Workspace of a key-split prefill call (None when key_splits == 1)."""
    if int(key_splits) == 1:
        return None
    n = prefill_workspace_bytes(shape, key_splits)
    if n <= 0:
        raise PagedAttnError(PA_ERR_SHAPE, "no prefill workspace size for this shape / key_splits")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _prefill_call(fn_plain, fn_split, lead, sh, key_splits, workspace, q, out, scale, stream):
    """One prefill call: the plain entry point for key_splits == 1, else the
    key-split one with `workspace` (allocated on `stream` when None)."""
    _check_out(out, q)
    with _on(stream):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if int(key_splits) != 1 and workspace is None:
            workspace = alloc_prefill_workspace(sh, key_splits, q.device)
    tail = (ctypes.c_float(scale), _ptr(out), ctypes.byref(sh))
    if int(key_splits) == 1:
        rc = fn_plain(*lead, *tail, _stream_handle(stream))
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        rc = fn_split(*lead, *tail, int(key_splits), _ptr(workspace),
                      ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                      _stream_handle(stream))
    _check(rc)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, q_offsets, scale: float,
            max_q_len: int, out=None, stream=None, key_splits: int = 1,
            workspace=None) -> torch.Tensor:
    """out fp32 [q_offsets[-1], Hq, D] = paged_attn_prefill(...): every sequence's
    last (q_offsets[s+1] - q_offsets[s]) context tokens attend causally over
    the paged bf16 cache.  max_q_len bounds the query tokens of any sequence.
    key_splits > 1: paged_attn_prefill_split, each row tile's keys over that
    many workgroups (workspace: alloc_prefill_workspace, or made here)."""
    sh = _prefill_shape(q, k_cache, v_cache, block_tables, context_lens, q_offsets, max_q_len,
                        (torch.bfloat16,))
    L = load()
    lead = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
            _ptr(q_offsets))
    return _prefill_call(L.paged_attn_prefill, L.paged_attn_prefill_split, lead, sh, key_splits,
                         workspace, q, out, scale, stream)


def prefill_int8(q, k_cache, v_cache, k_scales, v_scales, block_tables, context_lens, q_offsets,
                 scale: float, max_q_len: int, out=None, stream=None, key_splits: int = 1,
                 workspace=None) -> torch.Tensor:
    """paged_attn_prefill_int8: prefill over an int8 cache with fp32 scales [NB, bs, Hkv]."""
    sh = _prefill_shape(q, k_cache, v_cache, block_tables, context_lens, q_offsets, max_q_len,
                        (torch.int8,), (("k_scales", k_scales), ("v_scales", v_scales)))
    L = load()
    lead = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
            _ptr(block_tables), _ptr(context_lens), _ptr(q_offsets))
    return _prefill_call(L.paged_attn_prefill_int8, L.paged_attn_prefill_split_int8, lead, sh,
                         key_splits, workspace, q, out, scale, stream)


def prefill_fp8(q, k_cache, v_cache, block_tables, context_lens, q_offsets, scale: float,
                max_q_len: int, out=None, stream=None, key_splits: int = 1,
                workspace=None) -> torch.Tensor:
    """paged_attn_prefill_fp8: prefill over an FP8 E4M3 cache (float8_e4m3fn or uint8 codes)."""
    sh = _prefill_shape(q, k_cache, v_cache, block_tables, context_lens, q_offsets, max_q_len,
                        FP8_DTYPES)
    L = load()
    lead = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
            _ptr(q_offsets))
    return _prefill_call(L.paged_attn_prefill_fp8, L.paged_attn_prefill_split_fp8, lead, sh,
                         key_splits, workspace, q, out, scale, stream)


def prefill_shape_of(views, q, q_offsets, max_q_len: int) -> PaPrefillShape:
    """The pa_prefill_shape of a prefill call over the input generator's views."""
    return _prefill_shape(q, views["k_cache"], views["v_cache"], views["block_tables"],
                          views["context_lens"], q_offsets, max_q_len,
                          (views["k_cache"].dtype,))


def prefill_views(views, q, q_offsets, max_q_len: int, out=None, stream=None, scale=None,
                  key_splits: int = 1, workspace=None):
    """Prefill of query tokens q [q_offsets[-1], Hq, D] over the per-layer
    views of the input generator, whatever the cache kind."""
    sc = views["scale"] if scale is None else scale
    args = (views["block_tables"], views["context_lens"], q_offsets, sc, max_q_len)
    kw = dict(out=out, stream=stream, key_splits=key_splits, workspace=workspace)
    if views["k_cache"].dtype in FP8_DTYPES:
        return prefill_fp8(q, views["k_cache"], views["v_cache"], *args, **kw)
    if "k_scales" in views:
        return prefill_int8(q, views["k_cache"], views["v_cache"], views["k_scales"],
                            views["v_scales"], *args, **kw)
    return prefill(q, views["k_cache"], views["v_cache"], *args, **kw)
