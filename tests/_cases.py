"""Test helpers: small seeded cases, poisoning of padding, host-side references.

Builds on the seeded generators of ``paged_kv_cache_393_amd.inputs`` (which
hold no decode arithmetic) and on the fp64 oracle.  Nothing here runs on the
GPU except copies.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_cache_393_amd import inputs as I


def make_case(S, Hq, Hkv, D, bs, ctx, NB=None, MB=None, seed=0, kv_dtype="bf16",
              device="cpu", split_tokens=0):
    """(workload, per-layer views) of a single-layer case with fixed context lengths."""
    ctx = tuple(int(c) for c in ctx)
    if MB is None:
        MB = max(1, (max(ctx) + bs - 1) // bs) if ctx else 1
    wl = I.Workload("case", S, Hq, Hkv, D, bs, seed=seed, ctx_fixed=ctx, num_blocks=NB,
                    max_blocks_per_seq=MB, kv_dtype=kv_dtype, split_tokens=split_tokens)
    inp = I.make_inputs(wl, device)
    return wl, I.layer_views(inp, 0)


def oracle_out(views) -> np.ndarray:
    """fp64 oracle output for per-layer views (any device; copied to host)."""
    q = I.bf16_bits(views["q"])
    bt = views["block_tables"].cpu().numpy()
    cl = views["context_lens"].cpu().numpy()
    if views["k_cache"].dtype == torch.float8_e4m3fn:
        return oracle.paged_decode_fp8(q, fp8_codes(views["k_cache"]), fp8_codes(views["v_cache"]),
                                       bt, cl, views["scale"])
    if "k_scales" in views:
        return oracle.paged_decode_int8(q, views["k_cache"].cpu().numpy(),
                                        views["v_cache"].cpu().numpy(),
                                        views["k_scales"].cpu().numpy(),
                                        views["v_scales"].cpu().numpy(), bt, cl, views["scale"])
    return oracle.paged_decode_bf16(q, I.bf16_bits(views["k_cache"]), I.bf16_bits(views["v_cache"]),
                                    bt, cl, views["scale"])


def fp8_codes(t: torch.Tensor) -> np.ndarray:
    """uint8 codes (numpy) of a float8_e4m3fn tensor."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def used_blocks(views, bs):
    used = set()
    bt = views["block_tables"].cpu()
    for s, c in enumerate(views["context_lens"].cpu().tolist()):
        n = (c + bs - 1) // bs
        used.update(bt[s, :n].tolist())
    return used


def poison(views, bs, value=float("nan"), table_pad=-1):
    """Fill every slot the decode must not read: tail slots of each last block,
    unreferenced pool blocks, and table entries past each sequence's last block.
    Works in place on the views' storage; returns the views."""
    kc, vc = views["k_cache"], views["v_cache"]
    NB = kc.shape[0]
    bt = views["block_tables"]
    ctx = views["context_lens"].cpu().tolist()
    int8 = kc.dtype == torch.int8
    fill = -128 if int8 else value
    if kc.dtype == torch.float8_e4m3fn:
        fill = float("nan")
    bt_cpu = bt.cpu()
    for s, c in enumerate(ctx):
        n = (c + bs - 1) // bs
        if n > 0 and c % bs:
            b = int(bt_cpu[s, n - 1])
            kc[b, c % bs:] = fill
            vc[b, c % bs:] = fill
            if int8:
                views["k_scales"][b, c % bs:] = float("nan")
                views["v_scales"][b, c % bs:] = float("nan")
        bt_cpu[s, n:] = table_pad
    used = used_blocks(views, bs)
    bt.copy_(bt_cpu)
    for b in range(NB):
        if b not in used:
            kc[b] = fill
            vc[b] = fill
            if int8:
                views["k_scales"][b] = float("nan")
                views["v_scales"][b] = float("nan")
    return views


def gathered(views, bs, s):
    """Contiguous fp64 K, V [Hkv, n, D] of sequence s, gathered by numpy indexing."""
    n = int(views["context_lens"][s])
    bt = views["block_tables"].cpu().numpy()[s]
    t = np.arange(n)
    phys = bt[t // bs]
    slot = t % bs
    if "k_scales" in views:
        k = views["k_cache"].cpu().numpy().astype(np.float64) * \
            views["k_scales"].cpu().numpy().astype(np.float64)[..., None]
        v = views["v_cache"].cpu().numpy().astype(np.float64) * \
            views["v_scales"].cpu().numpy().astype(np.float64)[..., None]
    else:
        k = views["k_cache"].cpu().to(torch.float64).numpy()
        v = views["v_cache"].cpu().to(torch.float64).numpy()
    K = k[phys, slot]            # [n, Hkv, D]
    V = v[phys, slot]
    return np.ascontiguousarray(K.transpose(1, 0, 2)), np.ascontiguousarray(V.transpose(1, 0, 2))


def sdpa_reference(views, bs) -> np.ndarray:
    """Brute force: gather each sequence contiguously, then torch SDPA (fp64, CPU, GQA)."""
    q = views["q"].cpu().to(torch.float64)
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, D))
    for s in range(S):
        n = int(views["context_lens"][s])
        if n == 0:
            continue
        K, V = gathered(views, bs, s)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[s][None, :, None, :], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
            scale=float(np.float32(views["scale"])), enable_gqa=True)
        out[s] = o[0, :, 0, :].numpy()
    return out


def prefill_oracle(views, q, q_offsets, scale=None):
    """fp64 oracle chunked prefill for the cache kind of the views (any device)."""
    qb = I.bf16_bits(q)
    bt = views["block_tables"].cpu().numpy()
    cl = views["context_lens"].cpu().numpy()
    qo = np.asarray(q_offsets.cpu().numpy() if isinstance(q_offsets, torch.Tensor) else q_offsets,
                    dtype=np.int32)
    sc = views["scale"] if scale is None else scale
    if "k_scales" in views:
        return oracle.paged_prefill_int8(qb, views["k_cache"].cpu().numpy(), views["v_cache"].cpu().numpy(),
                                         views["k_scales"].cpu().numpy(), views["v_scales"].cpu().numpy(),
                                         bt, cl, qo, sc)
    if views["k_cache"].dtype == torch.float8_e4m3fn:
        return oracle.paged_prefill_fp8(qb, fp8_codes(views["k_cache"]), fp8_codes(views["v_cache"]),
                                        bt, cl, qo, sc)
    return oracle.paged_prefill_bf16(qb, I.bf16_bits(views["k_cache"]), I.bf16_bits(views["v_cache"]),
                                     bt, cl, qo, sc)
