"""fp64 CPU oracle for PagedAttention decode and the KV write path -- TEST
INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's ``cpu_baseline`` leg may
import this package.  It shares no code with the HIP library or with the
product package: the arithmetic lives in ``oracle.c`` (plain C, fp64,
OpenMP over (sequence, query head) rows) and this module only marshals numpy
arrays through ctypes.

Every function here cites the passage it follows in ``oracle.c``'s header:
the ybb.press page "LLM 推理 KV Cache 内存管理深度工程实践" sections 2.2
(paged attention forward), 2.1 (BlockTable.append_slot: a token's global
slot address block * block_size + offset), 6.1 (INT8 KV quantization, and the
cast of the cache to FP8 E4M3) and 6.2 (GQA sharing), the blog.hotdry.top page
"KV缓存内存布局优化：分页策略、量化压缩与动态驱逐的工程实践", section
"PagedEviction 块级驱逐机制" (token importance ||V||/||K||, lowest-mean full
block evicted), the ybb.press page's section 7.3 and the t6page page's
section "Chunked prefill：让 prefill 不阻塞 decode" (a prompt's prefill in
512-token chunks, each chunk's queries attending causally over the paged
cache),
and the t6page "KV cache" page, section "PagedAttention 的算子" (softmax after
merging all blocks).

Pins: every function is pinned by the CPU tests (``tests/test_oracle_pins.py``)
against closed forms, invariants and a library routine (torch SDPA in fp64);
none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCE = os.path.join(_HERE, "oracle.c")


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (strict IEEE, no contraction)."""
    import subprocess

    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", SOURCE, "-o", LIB_PATH + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class OracleLib:
    """ctypes handle on one build of oracle.c (the default build, or a test's own)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"oracle library missing: {path} (run __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        i64 = ctypes.c_int64
        lib.oracle_paged_decode_bf16.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                                 i64, ctypes.c_float, P]
        lib.oracle_paged_decode_bf16.restype = i32
        lib.oracle_paged_decode_int8.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                                 i32, i64, ctypes.c_float, P]
        lib.oracle_paged_decode_int8.restype = i32
        lib.oracle_quantize_int8_rows.argtypes = [P, i64, i32, P, P]
        lib.oracle_quantize_int8_rows.restype = None
        lib.oracle_kv_write_bf16.argtypes = [P, P, P, i32, i32, i32, i64, i64, P, P, i32, i64]
        lib.oracle_kv_write_bf16.restype = i32
        lib.oracle_kv_write_int8.argtypes = [P, P, P, i32, i32, i32, i64, i64, P, P, P, P, i32,
                                             i64]
        lib.oracle_kv_write_int8.restype = i32
        lib.oracle_paged_decode_fp8.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                                i64, ctypes.c_float, P]
        lib.oracle_paged_decode_fp8.restype = i32
        lib.oracle_kv_write_fp8.argtypes = [P, P, P, i32, i32, i32, i64, i64, P, P, i32, i64]
        lib.oracle_kv_write_fp8.restype = i32
        lib.oracle_fp8_e4m3_decode_array.argtypes = [P, i64, P]
        lib.oracle_fp8_e4m3_decode_array.restype = None
        lib.oracle_fp8_e4m3_encode_array.argtypes = [P, i64, P]
        lib.oracle_fp8_e4m3_encode_array.restype = None
        for name, cache_args in (("oracle_token_scores_bf16", [P, P]),
                                 ("oracle_token_scores_int8", [P, P, P, P]),
                                 ("oracle_token_scores_fp8", [P, P])):
            fn = getattr(lib, name)
            fn.argtypes = cache_args + [P, P, P, i32, i32, i32, i32, i32, i64, P]
            fn.restype = i32
        lib.oracle_evict_lowest_block.argtypes = [P, P, P, P, P, i32, i32, i32, i64]
        lib.oracle_evict_lowest_block.restype = i32
        lib.oracle_compress_prefill.argtypes = [P, P, i64, P, P, i32, P, P, P, i32, i32, i32, i64,
                                                i32]
        lib.oracle_compress_prefill.restype = i32
        lib.oracle_paged_prefill_bf16.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                                  i64, ctypes.c_float, P]
        lib.oracle_paged_prefill_bf16.restype = i32
        lib.oracle_paged_prefill_int8.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                                  i32, i64, ctypes.c_float, P]
        lib.oracle_paged_prefill_int8.restype = i32
        lib.oracle_paged_prefill_fp8.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                                 i64, ctypes.c_float, P]
        lib.oracle_paged_prefill_fp8.restype = i32
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib
        self.path = path


_default = None


def _load() -> "ctypes.CDLL":
    global _default
    if _default is None:
        _default = OracleLib(LIB_PATH)
    return _default.lib


def build_to(path: str, source_text: str) -> str:
    """Compile a given oracle source text into `path` (used by mutation tests)."""
    import subprocess
    import tempfile

    with tempfile.NamedTemporaryFile("w", suffix=".c", delete=False) as f:
        f.write(source_text)
        src = f.name
    try:
        subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fPIC", "-shared", src, "-o", path, "-lm"])
    finally:
        os.unlink(src)
    return path


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def _check_shapes(q, k, block_tables, context_lens):
    S, Hq, D = q.shape
    NB, BS, Hkv, D2 = k.shape
    if D2 != D:
        raise ValueError("head_dim mismatch between q and the cache")
    if block_tables.ndim != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    return S, Hq, Hkv, D, BS, block_tables.shape[1], NB


def paged_decode_bf16(q_bits, k_bits, v_bits, block_tables, context_lens, scale,
                      lib: "OracleLib | None" = None) -> np.ndarray:
    """out[s,h,:] (float64) for a bf16 cache given as raw uint16 bit patterns."""
    q_bits = _c(q_bits, np.uint16)
    k_bits = _c(k_bits, np.uint16)
    v_bits = _c(v_bits, np.uint16)
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    if v_bits.shape != k_bits.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    S, Hq, Hkv, D, BS, MB, NB = _check_shapes(q_bits, k_bits, bt, cl)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_paged_decode_bf16(_ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(bt),
                                    _ptr(cl), S, Hq, Hkv, D, BS, MB, NB,
                                    ctypes.c_float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def paged_decode_int8(q_bits, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                      scale, lib: "OracleLib | None" = None) -> np.ndarray:
    """out[s,h,:] (float64) for an int8 cache with fp32 per-(slot, kv head) scales."""
    q_bits = _c(q_bits, np.uint16)
    k_codes = _c(k_codes, np.int8)
    v_codes = _c(v_codes, np.int8)
    k_scales = _c(k_scales, np.float32)
    v_scales = _c(v_scales, np.float32)
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    S, Hq, Hkv, D, BS, MB, NB = _check_shapes(q_bits, k_codes, bt, cl)
    if v_codes.shape != k_codes.shape or k_scales.shape != (NB, BS, Hkv) or \
            v_scales.shape != (NB, BS, Hkv):
        raise ValueError("int8 cache / scale shapes disagree")
    out = np.zeros((S, Hq, D), dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_paged_decode_int8(_ptr(q_bits), _ptr(k_codes), _ptr(v_codes),
                                    _ptr(k_scales), _ptr(v_scales), _ptr(bt), _ptr(cl),
                                    S, Hq, Hkv, D, BS, MB, NB, ctypes.c_float(scale),
                                    _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def paged_decode_fp8(q_bits, k_codes, v_codes, block_tables, context_lens, scale,
                     lib: "OracleLib | None" = None) -> np.ndarray:
    """out[s,h,:] (float64) for an FP8 E4M3 cache given as uint8 codes."""
    q_bits = _c(q_bits, np.uint16)
    k_codes = _c(k_codes, np.uint8)
    v_codes = _c(v_codes, np.uint8)
    bt = _c(block_tables, np.int32)
    cl = _c(context_lens, np.int32)
    if v_codes.shape != k_codes.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    S, Hq, Hkv, D, BS, MB, NB = _check_shapes(q_bits, k_codes, bt, cl)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_paged_decode_fp8(_ptr(q_bits), _ptr(k_codes), _ptr(v_codes), _ptr(bt), _ptr(cl),
                                   S, Hq, Hkv, D, BS, MB, NB, ctypes.c_float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def fp8_e4m3_decode(codes, lib: "OracleLib | None" = None) -> np.ndarray:
    """float64 values of E4M3 codes (uint8, any shape)."""
    codes = _c(codes, np.uint8)
    out = np.zeros(codes.shape, dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    L.oracle_fp8_e4m3_decode_array(_ptr(codes), codes.size, _ptr(out))
    return out


def fp8_e4m3_encode(x, lib: "OracleLib | None" = None) -> np.ndarray:
    """uint8 E4M3 codes of float64 values x (any shape): the cast to float8_e4m3fn."""
    x = _c(x, np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    L = lib.lib if lib is not None else _load()
    L.oracle_fp8_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def quantize_int8_rows(x, lib: "OracleLib | None" = None) -> tuple[np.ndarray, np.ndarray]:
    """(codes int8 [..., D], scales fp32 [...]) for fp32 rows x [..., D]."""
    x = _c(x, np.float32)
    D = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.zeros(x.shape[:-1], dtype=np.float32)
    L = lib.lib if lib is not None else _load()
    L.oracle_quantize_int8_rows(_ptr(x), rows, D, _ptr(codes), _ptr(scales))
    return codes, scales


def slot_of(block_table_row, pos: int, block_size: int) -> int:
    """Global slot address of logical token `pos` of a sequence whose logical
    blocks map to block_table_row (ybb.press page, section 2.1: append_slot
    hands out last_block * block_size + used_slots)."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


def _write_args(key_bits, value_bits, slots):
    key_bits = _c(key_bits, np.uint16)
    value_bits = _c(value_bits, np.uint16)
    slots = _c(slots, np.int32)
    if key_bits.ndim != 3 or value_bits.shape != key_bits.shape or slots.shape != key_bits.shape[:1]:
        raise ValueError("key / value must be [T, Hkv, D] and slots [T]")
    return key_bits, value_bits, slots


def kv_write_bf16(key_bits, value_bits, slots, k_cache_bits, v_cache_bits,
                  lib: "OracleLib | None" = None):
    """(k_cache, v_cache) after storing token t's rows at slot slots[t] (copies;
    the inputs are not modified).  bf16 as raw uint16 bits; caches
    [NB, BS, Hkv, D]; a negative slot writes nothing."""
    key_bits, value_bits, slots = _write_args(key_bits, value_bits, slots)
    kc = np.array(_c(k_cache_bits, np.uint16), copy=True)
    vc = np.array(_c(v_cache_bits, np.uint16), copy=True)
    T, Hkv, D = key_bits.shape
    NB, BS, Hkv2, D2 = kc.shape
    if (Hkv2, D2) != (Hkv, D) or vc.shape != kc.shape:
        raise ValueError("cache shape disagrees with key / value")
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_kv_write_bf16(_ptr(key_bits), _ptr(value_bits), _ptr(slots), T, Hkv, D,
                                Hkv * D, Hkv * D, _ptr(kc), _ptr(vc), BS, NB)
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return kc, vc


def kv_write_int8(key_bits, value_bits, slots, k_codes, v_codes, k_scales, v_scales,
                  lib: "OracleLib | None" = None):
    """(k_codes, v_codes, k_scales, v_scales) after quantizing and storing token
    t's rows at slot slots[t] (copies).  Codes int8 [NB, BS, Hkv, D], scales
    fp32 [NB, BS, Hkv]."""
    key_bits, value_bits, slots = _write_args(key_bits, value_bits, slots)
    kc = np.array(_c(k_codes, np.int8), copy=True)
    vc = np.array(_c(v_codes, np.int8), copy=True)
    ks = np.array(_c(k_scales, np.float32), copy=True)
    vs = np.array(_c(v_scales, np.float32), copy=True)
    T, Hkv, D = key_bits.shape
    NB, BS, Hkv2, D2 = kc.shape
    if (Hkv2, D2) != (Hkv, D) or vc.shape != kc.shape or ks.shape != (NB, BS, Hkv) or \
            vs.shape != ks.shape:
        raise ValueError("cache / scale shapes disagree with key / value")
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_kv_write_int8(_ptr(key_bits), _ptr(value_bits), _ptr(slots), T, Hkv, D,
                                Hkv * D, Hkv * D, _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), BS, NB)
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return kc, vc, ks, vs


def kv_write_fp8(key_bits, value_bits, slots, k_codes, v_codes, lib: "OracleLib | None" = None):
    """(k_codes, v_codes) after casting token t's rows to FP8 E4M3 and storing
    them at slot slots[t] (copies).  Codes uint8 [NB, BS, Hkv, D]."""
    key_bits, value_bits, slots = _write_args(key_bits, value_bits, slots)
    kc = np.array(_c(k_codes, np.uint8), copy=True)
    vc = np.array(_c(v_codes, np.uint8), copy=True)
    T, Hkv, D = key_bits.shape
    NB, BS, Hkv2, D2 = kc.shape
    if (Hkv2, D2) != (Hkv, D) or vc.shape != kc.shape:
        raise ValueError("cache shape disagrees with key / value")
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_kv_write_fp8(_ptr(key_bits), _ptr(value_bits), _ptr(slots), T, Hkv, D,
                               Hkv * D, Hkv * D, _ptr(kc), _ptr(vc), BS, NB)
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return kc, vc


def token_scores(views, token_begin=None, lib: "OracleLib | None" = None):
    """PagedEviction importances ||V_t|| / ||K_t|| kept per token slot:
    float64 [NB, BS] (NaN where no scored token lives) for per-layer views
    (bf16, int8 or fp8 cache)."""
    import torch

    bt = _c(views["block_tables"].cpu().numpy(), np.int32)
    cl = _c(views["context_lens"].cpu().numpy(), np.int32)
    kc, vc = views["k_cache"].cpu(), views["v_cache"].cpu()
    NB, BS, Hkv, D = kc.shape
    S, MB = bt.shape
    out = np.full((NB, BS), np.nan, dtype=np.float64)
    tb = None if token_begin is None else _c(np.asarray(token_begin, dtype=np.int32), np.int32)
    tbp = _ptr(tb) if tb is not None else None
    L = lib.lib if lib is not None else _load()
    if kc.dtype == torch.float8_e4m3fn:
        k8 = _c(kc.view(torch.uint8).numpy(), np.uint8)
        v8 = _c(vc.view(torch.uint8).numpy(), np.uint8)
        rc = L.oracle_token_scores_fp8(_ptr(k8), _ptr(v8), _ptr(bt), tbp, _ptr(cl), S, Hkv, D, BS,
                                       MB, NB, _ptr(out))
    elif "k_scales" in views:
        k8 = _c(kc.numpy(), np.int8)
        v8 = _c(vc.numpy(), np.int8)
        ks = _c(views["k_scales"].cpu().numpy(), np.float32)
        vs = _c(views["v_scales"].cpu().numpy(), np.float32)
        rc = L.oracle_token_scores_int8(_ptr(k8), _ptr(v8), _ptr(ks), _ptr(vs), _ptr(bt), tbp,
                                        _ptr(cl), S, Hkv, D, BS, MB, NB, _ptr(out))
    else:
        kb = _c(kc.contiguous().view(torch.int16).numpy().view(np.uint16), np.uint16)
        vb = _c(vc.contiguous().view(torch.int16).numpy().view(np.uint16), np.uint16)
        rc = L.oracle_token_scores_bf16(_ptr(kb), _ptr(vb), _ptr(bt), tbp, _ptr(cl), S, Hkv, D, BS,
                                        MB, NB, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def evict_lowest_block(scores, block_tables, context_lens, evict_mask,
                       lib: "OracleLib | None" = None):
    """Decode-phase PagedEviction on copies: returns (block_tables,
    context_lens, evicted) after evicting, for every masked sequence, its full
    block of lowest mean importance.  scores: float32 per-slot [NB, BS]."""
    as_i32 = lambda a: np.asarray(a, dtype=np.int32) if isinstance(a, (list, tuple)) else a
    sc = _c(scores, np.float32)
    NB, BS = sc.shape
    bt = np.array(_c(as_i32(block_tables), np.int32), copy=True)
    cl = np.array(_c(as_i32(context_lens), np.int32), copy=True)
    mask = _c(np.asarray(evict_mask, dtype=np.int32), np.int32)
    S, MB = bt.shape
    ev = np.zeros(S, dtype=np.int32)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_evict_lowest_block(_ptr(sc), _ptr(bt), _ptr(cl), _ptr(mask), _ptr(ev), S, MB,
                                     BS, NB)
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return bt, cl, ev


def compress_prefill(views, scores, budget: int, lib: "OracleLib | None" = None):
    """Prefill-phase PagedEviction on copies: for every sequence whose context
    exceeds `budget`, keep the `budget` most important tokens (NaN first, then
    higher importance, then earlier position), in order, at logical positions
    0 .. budget-1.  views: per-layer views (bf16, int8 or fp8 cache); scores:
    float32 per-slot importances [NB, BS].  Returns a dict of host arrays:
    k_cache / v_cache (the cache's raw bytes, [NB, BS, Hkv, D * elem] uint8),
    k_scales / v_scales (int8 only), scores, context_lens."""
    import torch

    kc, vc = views["k_cache"].detach().cpu().contiguous(), views["v_cache"].detach().cpu().contiguous()
    NB, BS, Hkv, D = kc.shape
    kb = np.array(kc.view(torch.uint8).numpy(), copy=True).reshape(NB, BS, Hkv, -1)
    vb = np.array(vc.view(torch.uint8).numpy(), copy=True).reshape(NB, BS, Hkv, -1)
    row_bytes = Hkv * kb.shape[-1]
    sc = np.array(_c(scores, np.float32), copy=True)
    bt = _c(views["block_tables"].cpu().numpy(), np.int32)
    cl = np.array(_c(views["context_lens"].cpu().numpy(), np.int32), copy=True)
    S, MB = bt.shape
    out = {"k_cache": kb, "v_cache": vb, "scores": sc, "context_lens": cl}
    ksp = vsp = None
    if "k_scales" in views:
        out["k_scales"] = np.array(_c(views["k_scales"].cpu().numpy(), np.float32), copy=True)
        out["v_scales"] = np.array(_c(views["v_scales"].cpu().numpy(), np.float32), copy=True)
        ksp, vsp = _ptr(out["k_scales"]), _ptr(out["v_scales"])
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_compress_prefill(_ptr(kb), _ptr(vb), row_bytes, ksp, vsp, Hkv, _ptr(sc),
                                   _ptr(bt), _ptr(cl), S, MB, BS, NB, int(budget))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def paged_prefill_bf16(q_bits, k_bits, v_bits, block_tables, context_lens, q_offsets, scale,
                       lib: "OracleLib | None" = None) -> np.ndarray:
    """out [q_offsets[-1], Hq, D] (float64): chunked-prefill attention, every
    sequence's last n_q context tokens as causal queries (bf16 cache)."""
    as_i32 = lambda a: np.asarray(a, dtype=np.int32) if isinstance(a, (list, tuple)) else a
    q_bits = _c(q_bits, np.uint16)
    k_bits = _c(k_bits, np.uint16)
    v_bits = _c(v_bits, np.uint16)
    bt = _c(block_tables, np.int32)
    cl = _c(as_i32(context_lens), np.int32)
    qo = _c(as_i32(q_offsets), np.int32)
    Nq, Hq, D = q_bits.shape
    NB, BS, Hkv, D2 = k_bits.shape
    S, MB = bt.shape
    if D2 != D or v_bits.shape != k_bits.shape or cl.shape != (S,) or qo.shape != (S + 1,) or \
            int(qo[-1]) != Nq:
        raise ValueError("shapes disagree")
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_paged_prefill_bf16(_ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(bt), _ptr(cl),
                                     _ptr(qo), S, Hq, Hkv, D, BS, MB, NB, ctypes.c_float(scale),
                                     _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def _prefill_checked(q_bits, k, v, block_tables, context_lens, q_offsets):
    as_i32 = lambda a: np.asarray(a, dtype=np.int32) if isinstance(a, (list, tuple)) else a
    bt = _c(block_tables, np.int32)
    cl = _c(as_i32(context_lens), np.int32)
    qo = _c(as_i32(q_offsets), np.int32)
    Nq, Hq, D = q_bits.shape
    NB, BS, Hkv, D2 = k.shape
    S, MB = bt.shape
    if D2 != D or v.shape != k.shape or cl.shape != (S,) or qo.shape != (S + 1,) or \
            int(qo[-1]) != Nq:
        raise ValueError("shapes disagree")
    return bt, cl, qo, (Nq, Hq, D, NB, BS, Hkv, S, MB)


def paged_prefill_int8(q_bits, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                       q_offsets, scale, lib: "OracleLib | None" = None) -> np.ndarray:
    """The chunked prefill of paged_prefill_bf16 over an int8 cache: element =
    code * scale of its (slot, kv head); scales fp32 [NB, BS, Hkv]."""
    q_bits = _c(q_bits, np.uint16)
    k_codes = _c(k_codes, np.int8)
    v_codes = _c(v_codes, np.int8)
    ks = _c(k_scales, np.float32)
    vs = _c(v_scales, np.float32)
    bt, cl, qo, (Nq, Hq, D, NB, BS, Hkv, S, MB) = _prefill_checked(q_bits, k_codes, v_codes,
                                                                   block_tables, context_lens,
                                                                   q_offsets)
    if ks.shape != (NB, BS, Hkv) or vs.shape != (NB, BS, Hkv):
        raise ValueError("scales must be [NB, BS, Hkv]")
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_paged_prefill_int8(_ptr(q_bits), _ptr(k_codes), _ptr(v_codes), _ptr(ks), _ptr(vs),
                                     _ptr(bt), _ptr(cl), _ptr(qo), S, Hq, Hkv, D, BS, MB, NB,
                                     ctypes.c_float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def paged_prefill_fp8(q_bits, k_codes, v_codes, block_tables, context_lens, q_offsets, scale,
                      lib: "OracleLib | None" = None) -> np.ndarray:
    """The chunked prefill of paged_prefill_bf16 over an FP8 E4M3 cache (uint8 codes)."""
    q_bits = _c(q_bits, np.uint16)
    k_codes = _c(k_codes, np.uint8)
    v_codes = _c(v_codes, np.uint8)
    bt, cl, qo, (Nq, Hq, D, NB, BS, Hkv, S, MB) = _prefill_checked(q_bits, k_codes, v_codes,
                                                                   block_tables, context_lens,
                                                                   q_offsets)
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    L = lib.lib if lib is not None else _load()
    rc = L.oracle_paged_prefill_fp8(_ptr(q_bits), _ptr(k_codes), _ptr(v_codes), _ptr(bt), _ptr(cl),
                                    _ptr(qo), S, Hq, Hkv, D, BS, MB, NB, ctypes.c_float(scale),
                                    _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out
