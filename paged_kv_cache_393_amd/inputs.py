"""Seeded synthetic inputs for PagedAttention decode.

This module only builds inputs: context lengths, shuffled block pools, block
tables and random q / K / V (and the int8 codes + scales of the int8 cache).
It holds none of the decode arithmetic, and both the HIP path and the fp64
oracle consume exactly the bits it produces.

Workloads (names say what they are; shapes follow the pages):
  * ``tiny``: 4 sequences with contexts {1, 17, 100, 250}, 8 q / 2 kv heads,
    head_dim 64, block_size 16, a 64-block pool, permuted tables.
  * ``llama3_8b``: one Llama-3-8B-shaped layer (32 q / 8 kv heads, d 128 --
    t6page "KV cache" page, Llama 3 8B configuration), batch 64, contexts
    uniform in [512, 4096], block_size 16 (the default the pages recommend),
    pool sized to fit.
  * ``long_context``: batch 4 x 131072 tokens, 32/8/128, block_size 16,
    512-token context partitions.
  * ``nano_vllm_70b``: the layered nano-vLLM cache [2, 4 layers, blocks, 256,
    8, 128] (nano-vLLM page, physical layout section; 256-token default
    blocks), 64 q / 8 kv heads (G = 8, the Llama-2-70B grouping on the
    ybb.press page, section 6.2), batch 32, contexts uniform in [2048, 32768].
  * ``int8_llama3_8b``: 32/8/128, block_size 16, batch 128, contexts uniform in
    [1024, 8192], K/V int8 with one fp32 scale per (token, kv head) from
    N(0,1) source data.
  * ``fp8_llama3_8b``: the same shapes with the K/V cache in FP8 E4M3.

New tokens for the KV write path (``make_new_tokens``, ``draw_slots``): key
and value rows fp32 N(0, 1) rounded to bf16, and distinct destination slots
drawn as a seeded random permutation of the pool's slots, optionally with a
seeded fraction of tokens given no slot (-1).

Recipe (the same for every workload):
  * context lengths: integer-uniform in [lo, hi] inclusive from a CPU
    ``torch.Generator`` seeded with the workload seed (or the fixed list);
  * pool: exactly sum_s ceil(ctx_s / block_size) blocks unless the workload
    fixes the pool size; physical ids are a seeded random permutation of the
    pool, handed out in logical order (sequence 0 first); table entries past a
    sequence's last block are 0;
  * q, K, V: fp32 N(0, 1) from a generator on the target device seeded with
    the workload seed, rounded to bf16 (round-to-nearest-even);
  * fp8 cache: fp32 N(0, 1) cast to float8_e4m3fn by torch (the cast of the
    ybb.press page, section 6.1), no scale;
  * int8 cache: fp32 N(0, 1) source rows of head_dim, one row per (token slot,
    kv head), turned into codes and scales by the symmetric amax/127 recipe
    of the ybb.press page, section 6.1 (round half to even, zero rows get
    scale 0).  This is input synthesis: the decode oracle only ever sees the
    resulting codes and scales.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seed: int
    ctx_fixed: Optional[Sequence[int]] = None
    ctx_range: Optional[tuple] = None          # (lo, hi) inclusive
    num_blocks: Optional[int] = None           # None: exactly what the contexts need
    max_blocks_per_seq: Optional[int] = None   # None: ceil(max possible ctx / block_size)
    num_layers: int = 1                        # > 1: layered [2, L, NB, bs, Hkv, d] cache
    kv_dtype: str = "bf16"                     # "bf16", "int8" or "fp8"
    split_tokens: int = 0                      # 0: let the library choose

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_ctx(self) -> int:
        if self.ctx_fixed is not None:
            return max(self.ctx_fixed)
        return self.ctx_range[1]


WORKLOADS = {
    "tiny": Workload("tiny", 4, 8, 2, 64, 16, seed=1, ctx_fixed=(1, 17, 100, 250),
                     num_blocks=64, max_blocks_per_seq=16),
    "llama3_8b": Workload("llama3_8b", 64, 32, 8, 128, 16, seed=2, ctx_range=(512, 4096)),
    "long_context": Workload("long_context", 4, 32, 8, 128, 16, seed=3,
                             ctx_fixed=(131072,) * 4, split_tokens=512),
    "nano_vllm_70b": Workload("nano_vllm_70b", 32, 64, 8, 128, 256, seed=4,
                              ctx_range=(2048, 32768), num_layers=4),
    "int8_llama3_8b": Workload("int8_llama3_8b", 128, 32, 8, 128, 16, seed=5,
                               ctx_range=(1024, 8192), kv_dtype="int8"),
    "fp8_llama3_8b": Workload("fp8_llama3_8b", 128, 32, 8, 128, 16, seed=9,
                              ctx_range=(1024, 8192), kv_dtype="fp8"),
    # One tensor-parallel rank's share of the llama3_8b batch at TP = 8: one kv
    # head and its 4 query heads per rank, the same sequences and lengths.
    "llama3_8b_tp8": Workload("llama3_8b_tp8", 64, 4, 1, 128, 16, seed=2, ctx_range=(512, 4096)),
}


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of `wl` with some fields replaced (smaller batches for tests, ...)."""
    return dataclasses.replace(wl, **changes)


def draw_context_lens(wl: Workload) -> torch.Tensor:
    g = torch.Generator().manual_seed(wl.seed)
    if wl.ctx_fixed is not None:
        if len(wl.ctx_fixed) != wl.num_seqs:
            raise ValueError("ctx_fixed must list one length per sequence")
        return torch.tensor(list(wl.ctx_fixed), dtype=torch.int32)
    lo, hi = wl.ctx_range
    return torch.randint(lo, hi + 1, (wl.num_seqs,), generator=g, dtype=torch.int64).to(torch.int32)


def build_block_tables(wl: Workload, context_lens: torch.Tensor):
    """(block_tables int32 [S, MB], num_blocks) -- seeded shuffled pool, logical order."""
    bs = wl.block_size
    nblk = [(int(c) + bs - 1) // bs for c in context_lens.tolist()]
    used = sum(nblk)
    NB = wl.num_blocks if wl.num_blocks is not None else max(used, 1)
    if used > NB:
        raise ValueError(f"pool of {NB} blocks cannot hold {used}")
    MB = wl.max_blocks_per_seq or max(1, (wl.max_ctx + bs - 1) // bs)
    g = torch.Generator().manual_seed(wl.seed * 7919 + 17)
    perm = torch.randperm(NB, generator=g).to(torch.int32)
    tables = torch.zeros((wl.num_seqs, MB), dtype=torch.int32)
    pos = 0
    for s, n in enumerate(nblk):
        if n > MB:
            raise ValueError("context longer than max_blocks_per_seq * block_size")
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    return tables, NB


def _fill_normal_bf16(t: torch.Tensor, gen: torch.Generator, chunk_elems: int = 1 << 27):
    flat = t.view(-1)
    for start in range(0, flat.numel(), chunk_elems):
        n = min(chunk_elems, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=gen, device=t.device,
                                            dtype=torch.float32).to(torch.bfloat16)


def _fill_normal_fp8(t: torch.Tensor, gen: torch.Generator, chunk_elems: int = 1 << 27):
    flat = t.view(-1)
    for start in range(0, flat.numel(), chunk_elems):
        n = min(chunk_elems, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=gen, device=t.device,
                                            dtype=torch.float32).to(torch.float8_e4m3fn)


def synth_int8_rows(x: torch.Tensor):
    """Codes + scales for fp32 rows x [..., d] by the symmetric amax/127 recipe."""
    amax = x.abs().amax(dim=-1)
    scale = amax / 127.0
    safe = torch.where(scale == 0, torch.ones_like(scale), scale)
    codes = torch.round(x / safe.unsqueeze(-1))
    codes = torch.where(scale.unsqueeze(-1) == 0, torch.zeros_like(codes), codes)
    return codes.clamp_(-127, 127).to(torch.int8), scale


def _fill_int8(codes: torch.Tensor, scales: torch.Tensor, gen: torch.Generator,
               chunk_rows: int = 1 << 20):
    d = codes.shape[-1]
    c2 = codes.view(-1, d)
    s1 = scales.view(-1)
    for start in range(0, c2.shape[0], chunk_rows):
        n = min(chunk_rows, c2.shape[0] - start)
        x = torch.randn((n, d), generator=gen, device=codes.device, dtype=torch.float32)
        c, s = synth_int8_rows(x)
        c2[start:start + n] = c
        s1[start:start + n] = s


def make_inputs(wl: Workload, device="cpu") -> dict:
    """All inputs of one decode call (per layer for layered caches), seeded by wl.seed.

    Keys: ``q`` bf16 [L, S, Hq, d] (L = num_layers), ``block_tables`` int32
    [S, MB], ``context_lens`` int32 [S], ``num_blocks``, ``scale`` (python
    float, 1/sqrt(d)), and either ``kv`` bf16 (or float8_e4m3fn) [2, L, NB,
    bs, Hkv, d] or
    ``kv_codes`` int8 [2, L, NB, bs, Hkv, d] + ``kv_scales`` fp32
    [2, L, NB, bs, Hkv].  Use :func:`layer_views` for per-layer tensors.
    """
    device = torch.device(device)
    ctx = draw_context_lens(wl)
    tables, NB = build_block_tables(wl, ctx)
    L = wl.num_layers
    gen = torch.Generator(device=device).manual_seed(wl.seed)
    q = torch.empty((L, wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                    device=device)
    _fill_normal_bf16(q, gen)
    shape = (2, L, NB, wl.block_size, wl.num_kv_heads, wl.head_dim)
    out = {
        "workload": wl,
        "q": q,
        "block_tables": tables.to(device),
        "context_lens": ctx.to(device),
        "num_blocks": NB,
        "scale": 1.0 / math.sqrt(wl.head_dim),
    }
    if wl.kv_dtype == "bf16":
        kv = torch.empty(shape, dtype=torch.bfloat16, device=device)
        _fill_normal_bf16(kv, gen)
        out["kv"] = kv
    elif wl.kv_dtype == "int8":
        codes = torch.empty(shape, dtype=torch.int8, device=device)
        scales = torch.empty(shape[:-1], dtype=torch.float32, device=device)
        _fill_int8(codes, scales, gen)
        out["kv_codes"] = codes
        out["kv_scales"] = scales
    elif wl.kv_dtype == "fp8":
        kv = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
        _fill_normal_fp8(kv, gen)
        out["kv"] = kv
    else:
        raise ValueError(f"unknown kv dtype {wl.kv_dtype}")
    return out


def layer_views(inp: dict, layer: int = 0) -> dict:
    """Per-layer q / K / V (and scales) views of a make_inputs() result."""
    v = {"q": inp["q"][layer], "block_tables": inp["block_tables"],
         "context_lens": inp["context_lens"], "scale": inp["scale"]}
    if "kv" in inp:
        v["k_cache"] = inp["kv"][0, layer]
        v["v_cache"] = inp["kv"][1, layer]
    else:
        v["k_cache"] = inp["kv_codes"][0, layer]
        v["v_cache"] = inp["kv_codes"][1, layer]
        v["k_scales"] = inp["kv_scales"][0, layer]
        v["v_scales"] = inp["kv_scales"][1, layer]
    return v


def select_sequences(views: dict, seq_ids: Sequence[int], block_size: int) -> dict:
    """A smaller, self-contained problem holding only the sequences `seq_ids`.

    The physical blocks those sequences use are copied out in table order and
    the table is relabelled to the compacted pool (a bijective relabelling of
    block ids; the blocks' contents are untouched).  Everything is returned on
    the CPU, ready for a host-side reference.
    """
    seq_ids = list(seq_ids)
    ctx = views["context_lens"].cpu()[seq_ids]
    tables = views["block_tables"].cpu()[seq_ids]
    nblk = [(int(c) + block_size - 1) // block_size for c in ctx.tolist()]
    phys = []
    new_tables = torch.zeros((len(seq_ids), max(1, max(nblk) if nblk else 1)), dtype=torch.int32)
    for i, n in enumerate(nblk):
        ids = tables[i, :n].tolist()
        new_tables[i, :n] = torch.arange(len(phys), len(phys) + n, dtype=torch.int32)
        phys.extend(ids)
    if not phys:
        phys = [0]
    idx = torch.tensor(phys, dtype=torch.int64, device=views["k_cache"].device)

    def pick(t):   # float8 tensors are gathered as their bytes
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).index_select(0, idx).cpu().view(torch.float8_e4m3fn)
        return t.index_select(0, idx).cpu()

    out = {"q": views["q"][seq_ids].cpu(), "block_tables": new_tables, "context_lens": ctx,
           "scale": views["scale"], "k_cache": pick(views["k_cache"]),
           "v_cache": pick(views["v_cache"])}
    if "k_scales" in views:
        out["k_scales"] = views["k_scales"].index_select(0, idx).cpu()
        out["v_scales"] = views["v_scales"].index_select(0, idx).cpu()
    return out


def make_new_tokens(num_tokens: int, num_kv_heads: int, head_dim: int, seed: int,
                    device="cpu", token_stride: Optional[int] = None):
    """(key, value) bf16 [T, Hkv, d] for T new tokens: fp32 N(0, 1) rounded to bf16.

    With token_stride (elements, >= Hkv * d) the rows are views into a wider
    buffer, as when K and V are slices of a fused projection output."""
    device = torch.device(device)
    row = num_kv_heads * head_dim
    stride = token_stride or row
    if stride < row:
        raise ValueError("token_stride smaller than a token's row")
    gen = torch.Generator(device=device).manual_seed(seed * 104729 + 3)
    buf = torch.empty((2, max(num_tokens, 1), stride), dtype=torch.bfloat16, device=device)
    _fill_normal_bf16(buf, gen)
    key = buf[0, :num_tokens, :row].unflatten(-1, (num_kv_heads, head_dim))
    value = buf[1, :num_tokens, :row].unflatten(-1, (num_kv_heads, head_dim))
    return key, value


def draw_slots(num_tokens: int, num_slots: int, seed: int, pad_fraction: float = 0.0):
    """int32 [T]: distinct token slots drawn at random from [0, num_slots), a
    seeded fraction of them replaced by -1 (tokens without a slot)."""
    if num_tokens > num_slots:
        raise ValueError("more tokens than slots")
    g = torch.Generator().manual_seed(seed * 15485863 + 11)
    slots = torch.randperm(num_slots, generator=g)[:num_tokens].to(torch.int32)
    if pad_fraction > 0 and num_tokens > 0:
        pad = torch.rand(num_tokens, generator=g) < pad_fraction
        slots[pad] = -1
    return slots


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    """Chunked prefill: sequence s has context ctx[s] whose last n_q[s] tokens
    are the chunk's queries (their K/V already in the cache)."""
    name: str
    ctx: tuple
    n_q: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seed: int
    kv_dtype: str = "bf16"


PREFILL_WORKLOADS = {
    # The eight 512-token chunks of a 4096-token prompt of one Llama-3-8B-shaped
    # layer (32 q / 8 kv heads, d 128, block_size 16) in one batch: chunk k
    # attends over 512 (k + 1) tokens.
    "prefill_llama3_8b": PrefillWorkload("prefill_llama3_8b", tuple(512 * (k + 1) for k in range(8)),
                                         (512,) * 8, 32, 8, 128, 16, seed=10),
    # The same batch over int8 (per-token scales) and FP8 E4M3 caches.
    "prefill_int8_llama3_8b": PrefillWorkload("prefill_int8_llama3_8b",
                                              tuple(512 * (k + 1) for k in range(8)), (512,) * 8,
                                              32, 8, 128, 16, seed=11, kv_dtype="int8"),
    "prefill_fp8_llama3_8b": PrefillWorkload("prefill_fp8_llama3_8b",
                                             tuple(512 * (k + 1) for k in range(8)), (512,) * 8,
                                             32, 8, 128, 16, seed=12, kv_dtype="fp8"),
}


def _sarathi_contexts(num_seqs: int, lo: int, hi: int, seed: int) -> tuple:
    g = torch.Generator().manual_seed(seed)
    return tuple(int(c) for c in torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist())


# A chunked-prefill serving batch: one prefill chunk plus every running
# decode (t6page "KV cache" page, chunked-prefill section; ybb.press page,
# section 7.3): sequence 0's last 512 context tokens are the chunk, the other
# 63 sequences decode one token each; Llama-3-8B layer shape, contexts
# uniform in [512, 4096] as in the decode batch.
PREFILL_WORKLOADS["sarathi_llama3_8b"] = PrefillWorkload(
    "sarathi_llama3_8b", _sarathi_contexts(64, 512, 4096, seed=13), (512,) + (1,) * 63,
    32, 8, 128, 16, seed=13)


def make_prefill_inputs(pw: PrefillWorkload, device="cpu") -> dict:
    """Cache, tables and lengths as make_inputs (seeded, shuffled pool), plus
    the chunk queries q bf16 [sum n_q, Hq, d] (fp32 N(0,1) rounded) and
    q_offsets int32 [S + 1]."""
    wl = Workload(pw.name, len(pw.ctx), pw.num_q_heads, pw.num_kv_heads, pw.head_dim,
                  pw.block_size, seed=pw.seed, ctx_fixed=pw.ctx, kv_dtype=pw.kv_dtype)
    inp = make_inputs(wl, device)
    views = layer_views(inp, 0)
    nq = torch.tensor((0,) + tuple(pw.n_q), dtype=torch.int64)
    q_off = torch.cumsum(nq, 0).to(torch.int32)
    gen = torch.Generator(device=torch.device(device)).manual_seed(pw.seed * 31 + 7)
    q = torch.empty((int(q_off[-1]), pw.num_q_heads, pw.head_dim), dtype=torch.bfloat16,
                    device=device)
    _fill_normal_bf16(q, gen)
    views.update(q=q, q_offsets=q_off.to(device), max_q_len=max(pw.n_q))
    return views


@dataclasses.dataclass(frozen=True)
class WriteWorkload:
    """A KV write: num_tokens new tokens stored into a pool of num_blocks blocks."""
    name: str
    num_tokens: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seed: int
    kv_dtype: str = "bf16"
    pad_fraction: float = 0.0


WRITE_WORKLOADS = {
    # A 16384-token prefill chunk of one Llama-3-8B-shaped layer (8 kv heads,
    # d 128, block_size 16) filling a 1024-block pool: every slot written once,
    # in a random order of slots.
    "kv_write_llama3_8b": WriteWorkload("kv_write_llama3_8b", 16384, 8, 128, 16, 1024, seed=6),
    "kv_write_int8_llama3_8b": WriteWorkload("kv_write_int8_llama3_8b", 16384, 8, 128, 16, 1024,
                                             seed=7, kv_dtype="int8"),
    "kv_write_fp8_llama3_8b": WriteWorkload("kv_write_fp8_llama3_8b", 16384, 8, 128, 16, 1024,
                                            seed=8, kv_dtype="fp8"),
}


def make_write_inputs(ww: WriteWorkload, device="cpu") -> dict:
    """key / value bf16 [T, Hkv, d], slots int32 [T] (a seeded random choice of
    distinct pool slots) and the destination caches (bf16 zeros, or int8 zeros
    with zero scales) of a write workload."""
    device = torch.device(device)
    key, value = make_new_tokens(ww.num_tokens, ww.num_kv_heads, ww.head_dim, ww.seed, device)
    slots = draw_slots(ww.num_tokens, ww.num_blocks * ww.block_size, ww.seed, ww.pad_fraction)
    shape = (ww.num_blocks, ww.block_size, ww.num_kv_heads, ww.head_dim)
    out = {"workload": ww, "key": key, "value": value, "slots": slots.to(device)}
    if ww.kv_dtype == "bf16":
        out["k_cache"] = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        out["v_cache"] = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    elif ww.kv_dtype == "fp8":
        out["k_cache"] = torch.zeros(shape, dtype=torch.float8_e4m3fn, device=device)
        out["v_cache"] = torch.zeros(shape, dtype=torch.float8_e4m3fn, device=device)
    elif ww.kv_dtype == "int8":
        out["k_cache"] = torch.zeros(shape, dtype=torch.int8, device=device)
        out["v_cache"] = torch.zeros(shape, dtype=torch.int8, device=device)
        out["k_scales"] = torch.zeros(shape[:3], dtype=torch.float32, device=device)
        out["v_scales"] = torch.zeros(shape[:3], dtype=torch.float32, device=device)
    else:
        raise ValueError(f"unknown kv dtype {ww.kv_dtype}")
    return out


def bf16_bits(t: torch.Tensor):
    """Raw uint16 bit patterns (numpy) of a bf16 tensor."""
    import numpy as np

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
