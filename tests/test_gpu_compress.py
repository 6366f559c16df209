"""GPU parity of PagedEviction's prefill phase (paged_kv_compress_prefill*)
through the C-ABI against the oracle.

Compression is integer and byte work decided from the given fp32 importances:
the whole pool (K and V bytes, int8 scales, importances) and the context
lengths must be bit-identical to the oracle's on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_393_amd import binding as B
from paged_kv_cache_393_amd import inputs as I
from tests import _cases as C

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _raw(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.uint8).numpy().reshape(t.shape[0], t.shape[1], t.shape[2], -1)


def tie_heavy_scores(v, seed, nan_fraction=0.02, levels=8.0):
    """GPU importances of the cache, rounded to a few levels (many ties), with
    some NaN and -0 entries."""
    sc = B.token_scores(v)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(seed)
    host = sc.cpu()
    host = torch.round(host * levels) / levels
    u = torch.rand(host.shape, generator=g)
    host[u < nan_fraction] = float("nan")
    host[(u >= nan_fraction) & (u < 2 * nan_fraction)] = -0.0
    return host.to(DEV)


def check(v, scores, budget):
    """Run the GPU compression on v (in place) and compare with the oracle."""
    ref = oracle.compress_prefill(v, scores.cpu().numpy(), budget)
    B.compress_prefill(v, scores, budget)
    torch.cuda.synchronize()
    assert np.array_equal(v["context_lens"].cpu().numpy(), ref["context_lens"])
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), ref["scores"].view(np.uint32))
    assert np.array_equal(_raw(v["k_cache"]), ref["k_cache"]), "K bytes differ"
    assert np.array_equal(_raw(v["v_cache"]), ref["v_cache"]), "V bytes differ"
    if "k_scales" in v:
        assert np.array_equal(v["k_scales"].cpu().numpy().view(np.uint32),
                              ref["k_scales"].view(np.uint32))
        assert np.array_equal(v["v_scales"].cpu().numpy().view(np.uint32),
                              ref["v_scales"].view(np.uint32))


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("D,Hkv,bs", [(64, 2, 16), (128, 8, 16), (128, 3, 32), (64, 1, 256)])
def test_compress_matches_oracle(kv, D, Hkv, bs):
    ctx = (0, 1, 40, 300, 777, 1500, 64, 2049)
    note(f"compress kv={kv} D={D} Hkv={Hkv} bs={bs} ctx={ctx}")
    _, v = C.make_case(len(ctx), Hkv, Hkv, D, bs, ctx=ctx, seed=300 + D + Hkv + bs, kv_dtype=kv,
                       device=DEV)
    check(v, tie_heavy_scores(v, seed=bs + D), budget=100)


@pytest.mark.parametrize("budget", [0, 1, 15, 16, 17, 300, 5000])
def test_compress_budgets(budget):
    ctx = (10, 16, 17, 301, 1024, 3000)
    note(f"compress budget={budget} ctx={ctx}")
    _, v = C.make_case(len(ctx), 8, 2, 128, 16, ctx=ctx, seed=400 + budget, device=DEV)
    check(v, tie_heavy_scores(v, seed=budget, nan_fraction=0.05, levels=2.0), budget)


def test_compress_equal_scores_keep_the_prefix_and_move_nothing():
    ctx = (200, 513)
    note(f"compress equal scores ctx={ctx}")
    _, v = C.make_case(2, 8, 2, 128, 16, ctx=ctx, seed=410, device=DEV)
    k0, v0 = _raw(v["k_cache"]), _raw(v["v_cache"])
    sc = torch.ones(v["k_cache"].shape[:2], dtype=torch.float32, device=DEV)
    check(v, sc, budget=64)
    assert np.array_equal(_raw(v["k_cache"]), k0) and np.array_equal(_raw(v["v_cache"]), v0)


def test_compress_all_nan_and_newest_first():
    ctx = (300, 129)
    note(f"compress all-NaN / rising scores ctx={ctx}")
    _, v = C.make_case(2, 4, 1, 64, 16, ctx=ctx, seed=411, device=DEV)
    check(v, torch.full(v["k_cache"].shape[:2], float("nan"), device=DEV), budget=50)
    _, v = C.make_case(2, 4, 1, 64, 16, ctx=ctx, seed=412, kv_dtype="int8", device=DEV)
    NB, bs = v["k_cache"].shape[:2]
    sc = np.zeros((NB, bs), np.float32)
    bt = v["block_tables"].cpu().numpy()
    for s, n in enumerate(ctx):
        for t in range(n):
            sc[bt[s, t // bs], t % bs] = t          # newest most important: every kept row moves
    check(v, torch.from_numpy(sc).to(DEV), budget=50)


def test_compress_long_context_keys_outside_lds():
    ctx = (20000, 13000, 12288)
    note(f"compress long contexts ctx={ctx}")
    _, v = C.make_case(3, 4, 2, 64, 16, ctx=ctx, seed=413, device=DEV)
    check(v, tie_heavy_scores(v, seed=413, levels=32.0), budget=5000)


@pytest.mark.parametrize("budget", [1, 4095, 4096, 4097, 12289, 20000])
def test_compress_split_select_ties_across_chunks(budget):
    # Contexts longer than 12288 tokens select over 4096-token chunks: few
    # score levels make the tied key span many chunks, and the budgets put the
    # cut inside, at and around chunk boundaries.
    ctx = (30000, 12289, 16385, 5, 8192)
    note(f"compress split select budget={budget} ctx={ctx}")
    _, v = C.make_case(len(ctx), 2, 1, 64, 16, ctx=ctx, seed=415 + budget, device=DEV)
    check(v, tie_heavy_scores(v, seed=budget, nan_fraction=0.01, levels=2.0), budget)


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_compress_split_select_quantized_caches(kv):
    ctx = (20000, 13001, 4000)
    note(f"compress split select kv={kv} ctx={ctx}")
    _, v = C.make_case(len(ctx), 4, 2, 128, 16, ctx=ctx, seed=416, kv_dtype=kv, device=DEV)
    check(v, tie_heavy_scores(v, seed=416, levels=16.0), budget=4097)


def test_compress_long_context_full_size():
    # The bench's long-context workload: four 131072-token sequences to 1024.
    wl = I.WORKLOADS["long_context"]
    note(f"compress full size {wl.name} budget 1024")
    v = I.layer_views(I.make_inputs(wl, DEV), 0)
    check(v, B.token_scores(v), budget=1024)


def test_compress_twice_then_decode_matches_oracle_decode():
    ctx = (900, 333, 2000)
    note(f"compress twice then decode ctx={ctx}")
    _, v = C.make_case(3, 32, 8, 128, 16, ctx=ctx, seed=414, device=DEV)
    sc = tie_heavy_scores(v, seed=414, nan_fraction=0.0, levels=1024.0)
    check(v, sc, budget=500)
    check(v, sc, budget=300)
    out = B.decode_views(v)
    torch.cuda.synchronize()
    ref = C.oracle_out(v)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    assert err <= 2e-3, err


def test_compress_full_size_llama3_8b_batch():
    wl = I.WORKLOADS["llama3_8b"]
    note(f"compress full size {wl.name} budget 1024")
    v = I.layer_views(I.make_inputs(wl, DEV), 0)
    check(v, B.token_scores(v), budget=1024)
