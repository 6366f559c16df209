"""Byte and flop accounting for PagedAttention decode.

KV bytes per token follow the formula of the t6page "KV cache" page (equation
kv-per-token): 2 (K and V) x layers x kv heads x head_dim x bytes per element;
that page works it out as 131,072 B/token for Llama 3 8B (equation
kv-llama3-8b) and tabulates 1K / 4K / 32K / 128K contexts.

Algorithmic bytes of ONE decode call (one layer) are what the operation must
move at least once: every valid K and V element (plus the int8 scales), q,
out, the valid block-table entries and the context lengths.  Split partials
are overhead and are not counted.
"""
from __future__ import annotations

from typing import Iterable


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       bytes_per_elem: int = 2) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * bytes_per_elem


def decode_bytes(context_lens: Iterable[int], num_q_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, kv_dtype: str = "bf16") -> int:
    ctx = [int(c) for c in context_lens]
    tokens = sum(ctx)
    if kv_dtype == "bf16":
        kv = tokens * kv_bytes_per_token(1, num_kv_heads, head_dim, 2)
    elif kv_dtype == "int8":
        kv = tokens * (kv_bytes_per_token(1, num_kv_heads, head_dim, 1) + 2 * num_kv_heads * 4)
    elif kv_dtype == "fp8":
        kv = tokens * kv_bytes_per_token(1, num_kv_heads, head_dim, 1)
    else:
        raise ValueError(kv_dtype)
    S = len(ctx)
    q = S * num_q_heads * head_dim * 2
    out = S * num_q_heads * head_dim * 4
    tables = sum((c + block_size - 1) // block_size for c in ctx) * 4
    return kv + q + out + tables + S * 4


def decode_flops(context_lens: Iterable[int], num_q_heads: int, head_dim: int) -> int:
    """QK and PV multiply-adds (2 flops each) over every (query head, context token)."""
    return 4 * head_dim * num_q_heads * sum(int(c) for c in context_lens)


def write_bytes(num_tokens: int, num_written: int, num_kv_heads: int, head_dim: int,
                kv_dtype: str = "bf16") -> int:
    """Algorithmic bytes of one KV write call: the slot of every token, the K
    and V rows (bf16) of the tokens that have a slot, and what lands in the
    cache -- the same rows in bf16, int8 codes plus one fp32 scale per row, or
    FP8 codes."""
    rows = 2 * num_written * num_kv_heads           # K and V rows moved
    read = num_tokens * 4 + rows * head_dim * 2
    if kv_dtype == "bf16":
        written = rows * head_dim * 2
    elif kv_dtype == "int8":
        written = rows * (head_dim + 4)
    elif kv_dtype == "fp8":
        written = rows * head_dim
    else:
        raise ValueError(kv_dtype)
    return read + written


def score_bytes(context_lens: Iterable[int], num_kv_heads: int, head_dim: int, block_size: int,
                kv_dtype: str = "bf16") -> int:
    """Algorithmic bytes of one PagedEviction scoring call over whole contexts:
    every token's K and V rows (plus int8 scales), its fp32 score, the valid
    block-table entries and the context lengths."""
    ctx = [int(c) for c in context_lens]
    tokens = sum(ctx)
    elem = 2 if kv_dtype == "bf16" else 1
    per_token = 2 * num_kv_heads * head_dim * elem + 4
    if kv_dtype == "int8":
        per_token += 2 * num_kv_heads * 4
    tables = sum((c + block_size - 1) // block_size for c in ctx) * 4
    return tokens * per_token + tables + 4 * len(ctx)


def prefill_flops(context_lens: Iterable[int], n_q: Iterable[int], num_q_heads: int,
                  head_dim: int) -> int:
    """QK and PV multiply-adds (2 flops each) of causal chunked prefill: the
    query at position p of a sequence attends to p + 1 tokens."""
    total = 0
    for c, nq in zip(context_lens, n_q):
        c, nq = int(c), int(nq)
        # sum over positions p = c - nq .. c - 1 of (p + 1)
        total += nq * (2 * c - nq + 1) // 2
    return 4 * head_dim * num_q_heads * total


def prefill_bytes(context_lens: Iterable[int], n_q: Iterable[int], num_q_heads: int,
                  num_kv_heads: int, head_dim: int, block_size: int, kv_dtype: str = "bf16") -> int:
    """Bytes one chunked-prefill call must move at least once: each context's
    K and V (2, or 1 byte a code, + two fp32 scales a token and kv head for
    int8), the queries (bf16) and outputs (fp32), the table entries."""
    ctx = [int(c) for c in context_lens]
    nq = [int(n) for n in n_q]
    elem = 2 if kv_dtype == "bf16" else 1
    kv = sum(ctx) * 2 * num_kv_heads * (head_dim * elem + (4 if kv_dtype == "int8" else 0))
    qo = sum(nq) * num_q_heads * head_dim * (2 + 4)
    tables = sum((c + block_size - 1) // block_size for c in ctx) * 4
    return kv + qo + tables + 8 * len(ctx) + 4


def compress_moved_tokens(logical_scores, budget: int) -> int:
    """Kept tokens that change position in a prefill-phase compression (the
    rows the move kernel reads and writes), from each sequence's importances
    in logical order: the budget highest-ranked tokens (NaN first, then
    larger, then earlier) in position order, minus those already in place."""
    import numpy as np

    moved = 0
    for vals in logical_scores:
        vals = np.asarray(vals, dtype=np.float32)
        n = len(vals)
        if n <= budget:
            continue
        nan = np.isnan(vals)
        key = np.where(nan, 0.0, vals).astype(np.float64)
        order = np.lexsort((np.arange(n), -key, ~nan))
        kept = np.sort(order[:budget])
        moved += int(np.count_nonzero(kept != np.arange(budget)))
    return moved


def compress_bytes(context_lens: Iterable[int], budget: int, moved: int, num_kv_heads: int,
                   head_dim: int, block_size: int, kv_dtype: str = "bf16") -> int:
    """Algorithmic bytes of one prefill-phase compression call: the context
    lengths (read, and written where a sequence is compressed); for each
    compressed sequence its valid table entries and its importances (read
    once); each moved token's K and V rows, int8 scales and importance (read
    and written).  The kept-position list in the workspace is not counted."""
    ctx = [int(c) for c in context_lens]
    over = [c for c in ctx if c > budget]
    elem = 2 if kv_dtype == "bf16" else 1
    row = 2 * num_kv_heads * head_dim * elem + 4
    if kv_dtype == "int8":
        row += 2 * num_kv_heads * 4
    tables = sum((c + block_size - 1) // block_size for c in over) * 4
    return 4 * len(ctx) + 4 * len(over) + tables + 4 * sum(over) + 2 * moved * row
