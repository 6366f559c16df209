"""GPU parity of the key-split chunked prefill (paged_attn_prefill_split*)
through the C-ABI against the fp64 oracle, at the decode's bar (max |gpu -
oracle| <= 2e-3, per-row max err / max |oracle| <= 1e-2).  Each row tile's
key tiles are cut into min(K, tiles) runs over separate workgroups whose
partial sums a merge kernel combines, so the cases below put run boundaries
inside contexts of every length class: shorter than K tiles (fewer runs, or
one run written directly beside merged row tiles in the same call), long
contexts whose block-table window starts mid-table, running maxima that move
between runs, the bf16 second pass in some runs only, and every cache kind.
Bit-exact: a poisoned workspace, repeated calls, a side stream, a loose
max_q_len.  Also here, split and unsplit: the three dispatch orders (up to 64
sequences ranked per wave, up to 2048 through LDS, beyond that by index), the
full-size 8-chunk batch and serving chunk, and the wrappers' checks on a
caller's out.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_393_amd import binding as B
from paged_kv_cache_393_amd import inputs as I
from tests import _cases as C
from tests.test_gpu_parity import assert_parity
from tests.test_gpu_prefill import make_kind

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_split(v, q, q_off, key_splits, max_q=None, scale=None, workspace=None):
    out = B.prefill_views(v, q, q_off.to(DEV), max_q or int((q_off[1:] - q_off[:-1]).max()),
                          scale=scale, key_splits=key_splits, workspace=workspace)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("key_splits", [2, 3, 7, 64])
def test_split_prefill_against_oracle(kind, D, key_splits):
    # contexts from one token to 2012 (63 tiles): with 64 pieces every tile of
    # the long rows is its own run; short rows get fewer runs or one
    note(f"split prefill {kind} D={D} K={key_splits}")
    ctx = (1, 17, 100, 300, 513, 64, 2012)
    nq = [1, 17, 33, 128, 200, 1, 512]
    v, q, q_off = make_kind(ctx, nq, 32, 8, D, 16, 600 + D + key_splits, kind)
    assert_parity(run_split(v, q, q_off, key_splits), C.prefill_oracle(v, q, q_off),
                  f"split {kind} K={key_splits}")


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (12, 2), (32, 1)])
@pytest.mark.parametrize("bs", [16, 256])
def test_split_prefill_group_sizes_and_block_sizes(kind, Hq, Hkv, bs):
    note(f"split prefill {kind} Hq={Hq} Hkv={Hkv} bs={bs}")
    ctx = (40, 700, 1300, 96)
    nq = [40, 300, 77, 1]
    v, q, q_off = make_kind(ctx, nq, Hq, Hkv, 128, bs, 610 + Hq + Hkv + bs, kind)
    assert_parity(run_split(v, q, q_off, 4), C.prefill_oracle(v, q, q_off), f"split {kind} groups")


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_split_prefill_mixed_batch_with_empty_sequences(kind):
    # a chunk, decodes, a sequence with no queries and an empty context in one
    # call; row tiles with one run (short contexts) write out directly while
    # the chunk's are merged
    note(f"split prefill {kind} mixed batch")
    ctx = (2012, 37, 900, 5, 0, 128, 31)
    nq = [512, 1, 1, 0, 0, 1, 31]
    v, q, q_off = make_kind(ctx, nq, 32, 8, 128, 16, 620, kind)
    assert_parity(run_split(v, q, q_off, 5), C.prefill_oracle(v, q, q_off), f"split {kind} mixed")


@pytest.mark.parametrize("bs", [16, 4096])
@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_split_prefill_long_context_window_starts_mid_table(bs, kind):
    # 30000 tokens at block size 16: runs start hundreds of blocks into the
    # table, and each run's 64-entry window slides from there
    note(f"split prefill {kind} long context bs={bs}")
    ctx = (30000, 1500, 7)
    v, q, q_off = make_kind(ctx, [96, 1, 7], 8, 2, 128, bs, 621, kind)
    assert_parity(run_split(v, q, q_off, 9), C.prefill_oracle(v, q, q_off), f"split long {kind} bs {bs}")


@pytest.mark.parametrize("D", [64, 128])
def test_split_prefill_running_max_differs_between_runs(D):
    # Keys growing block by block: each run ends with a different running
    # max (late runs' maxima are far above early ones'), so the merge's
    # rescaling of every run is exercised, with early runs' weights underflowing.
    note(f"split prefill growing keys D={D}")
    bs = 16
    ctx = (1000, 333, 64)
    v, q, q_off = make_kind(ctx, [200, 333, 64], 8, 2, D, bs, 622 + D, "bf16")
    k = v["k_cache"].float()
    bt = v["block_tables"].cpu()
    for s_, c in enumerate(ctx):
        for j in range((c + bs - 1) // bs):
            k[int(bt[s_, j])] *= 0.5 + 0.75 * j
    v["k_cache"].copy_(k.to(torch.bfloat16))
    assert_parity(run_split(v, q, q_off, 6), C.prefill_oracle(v, q, q_off), "split growing keys")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.6])
def test_split_prefill_any_scale(scale):
    note(f"split prefill scale={scale}")
    ctx = (40, 700, 129)
    v, q, q_off = make_kind(ctx, [40, 300, 65], 16, 4, 128, 16, 623, "bf16")
    assert_parity(run_split(v, q, q_off, 3, scale=scale), C.prefill_oracle(v, q, q_off, scale=scale),
                  f"split scale {scale}")


@pytest.mark.parametrize("D", [64, 128])
def test_split_prefill_int8_second_pass_in_some_runs(D):
    # int8 V scales of 600 (past the fast range) on tokens 100..139 of
    # sequence 1, kv head 0: only the runs holding those tiles take the
    # second pass (bf16 codes, the weights times the whole scales); the merge
    # combines them with fast runs.  Large outputs compared in units of the
    # largest V.
    note(f"split prefill int8 second pass in some runs, D={D}")
    ctx, nq = (300, 700, 90), [50, 300, 90]
    v, q, q_off = make_kind(ctx, nq, 8, 2, D, 16, 627 + D, "int8")
    bt = v["block_tables"].cpu()
    for t in range(100, 140):
        v["v_scales"][int(bt[1, t // 16]), t % 16, 0] = 600.0
    got = run_split(v, q, q_off, 5).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    unit = np.where(np.abs(ref).max(axis=-1, keepdims=True) > 8.0, 127.0 * 600.0, 1.0)
    assert (unit > 1).any() and (unit == 1).any()
    assert_parity(torch.from_numpy(got / unit), ref / unit, "split int8 V x 600")


def test_split_prefill_bf16_second_pass_in_some_runs():
    # V x 2^16 on tokens 100..139 of sequence 1, kv head 0: only the runs
    # holding those tiles take the bf16 second pass; the merge combines them
    # with fp16 runs.  Large outputs compared in units of 2^16.
    note("split prefill bf16 V partly x 2^16")
    ctx, nq = (300, 700, 90), [50, 300, 90]
    v, q, q_off = make_kind(ctx, nq, 8, 2, 128, 16, 624, "bf16")
    bt = v["block_tables"].cpu()
    for t in range(100, 140):
        b = int(bt[1, t // 16])
        v["v_cache"][b, t % 16, 0] *= 65536.0
    got = run_split(v, q, q_off, 5).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    unit = np.where(np.abs(ref).max(axis=-1, keepdims=True) > 64.0, 65536.0, 1.0)
    assert (unit > 1).any() and (unit == 1).any()
    assert_parity(torch.from_numpy(got / unit), ref / unit, "split V partly x 2^16")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_split_prefill_poisoned_workspace_and_repeat_bit_identical(kind):
    # The workspace needs no initialisation: NaN-filled or reused, the output
    # is the same to the bit; a repeated call too.
    note(f"split prefill {kind} workspace poison")
    ctx = (17, 300, 1513)
    nq = [17, 40, 500]
    v, q, q_off = make_kind(ctx, nq, 8, 2, 128, 16, 625, kind)
    sh = B.prefill_shape_of(v, q, q_off.to(DEV), 500)
    ws = B.alloc_prefill_workspace(sh, 4, DEV)
    ws.zero_()
    a = run_split(v, q, q_off, 4, workspace=ws).clone()
    ws.view(torch.float32).fill_(float("nan"))
    b = run_split(v, q, q_off, 4, workspace=ws)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    c = run_split(v, q, q_off, 4, workspace=ws)
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    assert_parity(a, C.prefill_oracle(v, q, q_off), f"split {kind} poisoned workspace")


def test_split_prefill_one_piece_is_the_unsplit_call():
    # key_splits = 1 takes the unsplit kernel: bit-identical to paged_attn_prefill
    note("split prefill K=1")
    ctx = (300, 1200)
    v, q, q_off = make_kind(ctx, [64, 512], 32, 8, 128, 16, 626, "bf16")
    a = run_split(v, q, q_off, 1).clone()
    b = B.prefill(q, v["k_cache"], v["v_cache"], v["block_tables"], v["context_lens"], q_off.to(DEV),
                  v["scale"], 512)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_prefill_plan_covers_the_compute_units():
    note("prefill plan")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pw = I.PREFILL_WORKLOADS["sarathi_llama3_8b"]
    # the serving batch's chunk alone: 1 sequence x 8 kv heads x 8 row tiles
    sh = B.PaPrefillShape(1, pw.num_q_heads, pw.num_kv_heads, pw.head_dim, pw.block_size,
                          4096 // pw.block_size, 1 << 14, 512)
    k = B.prefill_plan(sh)
    units = 1 * pw.num_kv_heads * 8
    assert k == -(-cus // units), (k, cus)
    # enough units already: no split
    sh8 = B.PaPrefillShape(64, pw.num_q_heads, pw.num_kv_heads, pw.head_dim, pw.block_size,
                           4096 // pw.block_size, 1 << 14, 512)
    assert B.prefill_plan(sh8) == 1
    # a short table caps the pieces at 4 tiles each: 256 tokens = 8 tiles -> 2
    short = B.PaPrefillShape(1, 8, 8, 128, 16, 16, 64, 8)
    assert B.prefill_plan(short) == 2


def test_full_size_serving_chunk_key_split():
    # The serving batch's chunk (512 queries over a 1485-token context, the
    # Llama-3-8B shape) with the plan's key split, as the bench times it;
    # every output row against the oracle.
    import bench

    note("full-size serving chunk, key split")
    pw = I.PREFILL_WORKLOADS["sarathi_llama3_8b"]
    inp = I.make_prefill_inputs(pw, DEV)
    sp = bench.split_decode_batch(pw, inp, None, DEV)
    ch = sp["chunks"]
    k = B.prefill_plan(B.prefill_shape_of(ch, ch["q"], ch["q_offsets"], ch["max_q_len"]))
    assert k > 1
    B.prefill_views(ch, ch["q"], ch["q_offsets"], ch["max_q_len"], out=sp["chunk_out"],
                    key_splits=k)
    torch.cuda.synchronize()
    r = C.prefill_oracle(ch, ch["q"], ch["q_offsets"].cpu())
    assert_parity(sp["chunk_out"], r, f"serving chunk, key split {k}")


def test_split_prefill_on_a_side_stream():
    # With stream= a non-current stream, the wrapper allocates out and the
    # workspace for that stream: allocator churn on the current stream while
    # the side stream runs cannot reuse them.  Every result equals the call
    # on the current stream bit for bit and passes against the oracle.
    note("split prefill side stream")
    ctx = (1513, 300)
    v, q, q_off = make_kind(ctx, [512, 64], 32, 8, 128, 16, 627, "bf16")
    main = run_split(v, q, q_off, 4).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(B.prefill_views(v, q, q_off.to(DEV), 512, stream=side, key_splits=4))
        junk = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
        junk.fill_(0x7F)
        del junk
    side.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int32), main.view(torch.int32))
    assert_parity(outs[0], C.prefill_oracle(v, q, q_off), "split side stream")


def test_wrappers_reject_a_caller_out_that_does_not_fit():
    # A caller's out must be a contiguous fp32 device tensor shaped like q:
    # anything else raises before a kernel could write past it.
    note("out validation")
    v, q, q_off = make_kind((300, 40), [64, 40], 8, 2, 128, 16, 628, "bf16")
    bad = [torch.empty(q.shape[0] - 1, *q.shape[1:], dtype=torch.float32, device=DEV),
           torch.empty(q.shape, dtype=torch.bfloat16, device=DEV),
           torch.empty(q.shape[0], q.shape[1], 2 * q.shape[2], dtype=torch.float32, device=DEV)[..., ::2],
           torch.empty(q.shape, dtype=torch.float32)]
    for o in bad:
        for ks in (1, 3):
            with pytest.raises(ValueError):
                B.prefill_views(v, q, q_off.to(DEV), 64, out=o, key_splits=ks)
    # the decode of the same two sequences, one query each
    dv = dict(v, q=q[:2].contiguous())
    bad_d = [torch.empty(1, *q.shape[1:], dtype=torch.float32, device=DEV),
             torch.empty(2, *q.shape[1:], dtype=torch.bfloat16, device=DEV),
             torch.empty(2, q.shape[1], 2 * q.shape[2], dtype=torch.float32, device=DEV)[..., ::2],
             torch.empty(2, *q.shape[1:], dtype=torch.float32)]
    for o in bad_d:
        with pytest.raises(ValueError):
            B.decode_views(dv, out=o)
    torch.cuda.synchronize()


def test_full_size_eight_chunk_batch_key_split():
    # The 8-chunk prefill batch at full size with two runs per row tile (the
    # plan keeps it unsplit: 512 workgroups already cover the GPU); every
    # query of every chunk against the oracle.
    note("full-size prefill, 8 chunks, key split 2")
    pw = I.PREFILL_WORKLOADS["prefill_llama3_8b"]
    inp = I.make_prefill_inputs(pw, DEV)
    out = B.prefill_views(inp, inp["q"], inp["q_offsets"], inp["max_q_len"], key_splits=2)
    torch.cuda.synchronize()
    assert_parity(out, C.prefill_oracle(inp, inp["q"], inp["q_offsets"]), "prefill_llama3_8b key split 2")


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("key_splits", [1, 3])
def test_prefill_more_than_64_sequences(kind, key_splits):
    # Batches of more than 64 sequences take the dispatch ranking through LDS
    # (up to 64, each wave ranks alone): 100 sequences of mixed chunks,
    # decodes, empty query sets and an empty context, unsplit and key-split.
    note(f"prefill {kind} 100 sequences K={key_splits}")
    rng = np.random.default_rng(640 + key_splits)
    ctx = [int(c) for c in rng.integers(1, 700, size=100)]
    ctx[7] = 0
    nq = [0 if c == 0 else int(min(c, rng.choice([1, 1, 1, 5, 40, 130])) ) for c in ctx]
    nq[11] = 0
    v, q, q_off = make_kind(tuple(ctx), nq, 8, 2, 128, 16, 641 + key_splits, kind)
    assert_parity(run_split(v, q, q_off, key_splits), C.prefill_oracle(v, q, q_off),
                  f"{kind} 100 sequences K={key_splits}")


def test_split_prefill_loose_max_q_len_bit_identical():
    # A max_q_len above every sequence's query count adds row tiles that
    # exit (in the prefill and the merge): the output is the same to the bit.
    note("split prefill loose max_q_len")
    v, q, q_off = make_kind((300, 1300), [64, 512], 16, 4, 128, 16, 629, "bf16")
    a = run_split(v, q, q_off, 4).clone()
    b = run_split(v, q, q_off, 4, max_q=2048)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("key_splits", [1, 2])
def test_prefill_more_than_2048_sequences_keep_index_order(key_splits):
    # Past 2048 sequences the dispatch order is the index order (no ranking):
    # 2100 short sequences, one to three queries each.
    note(f"prefill 2100 sequences K={key_splits}")
    rng = np.random.default_rng(650)
    ctx = [int(c) for c in rng.integers(1, 70, size=2100)]
    nq = [int(min(c, rng.integers(1, 4))) for c in ctx]
    v, q, q_off = make_kind(tuple(ctx), nq, 8, 2, 64, 16, 651, "bf16")
    assert_parity(run_split(v, q, q_off, key_splits), C.prefill_oracle(v, q, q_off),
                  f"2100 sequences K={key_splits}")
