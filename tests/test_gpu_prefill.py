"""GPU parity of paged chunked-prefill attention (paged_attn_prefill) through the
C-ABI against the fp64 oracle, with the decode's bar: max |gpu - oracle| <=
2e-3 over all elements and, per (query token, head) row, max err / max |oracle|
<= 1e-2.  bf16 and FP8 caches: V enters the second matrix product as fp16
(exact for bf16 values below 2^16 and every E4M3 value) and the softmax
weights as fp16 (2^-11 relative rounding, the row sums adding the same
rounded weights); a bf16 V beyond fp16 sends the workgroup to a second pass
with bf16 V and the weights split exactly into a bf16 pair.  int8: the codes
times the power of two of their V scale as fp16, the weights times the
scale's mantissa as fp16, and the row sums adding each rounded weight over
that mantissa; a V scale outside 2^-14 .. 2^9 (and not 0) sends the
workgroup to a second pass with the weights times the whole scales as a bf16
pair (exact to 2^-17).  Checked below up to 4096 tokens.  Bit-exact: padding
poison, loose max_q_len.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_393_amd import binding as B
from paged_kv_cache_393_amd import inputs as I
from tests import _cases as C
from tests.test_gpu_parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def make(ctx, nq, Hq, Hkv, D, bs, seed):
    NB = sum((c + bs - 1) // bs for c in ctx) + 3
    _, v = C.make_case(len(ctx), Hq, Hkv, D, bs, ctx=ctx, NB=NB, seed=seed, device=DEV)
    q_off = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32)
    gen = torch.Generator(device=DEV).manual_seed(seed + 1)
    q = torch.randn(int(q_off[-1]), Hq, D, generator=gen, device=DEV).to(torch.bfloat16)
    return v, q, q_off


def run(v, q, q_off, max_q=None, scale=None):
    out = B.prefill(q, v["k_cache"], v["v_cache"], v["block_tables"], v["context_lens"],
                    q_off.to(DEV), v["scale"] if scale is None else scale,
                    max_q or int((q_off[1:] - q_off[:-1]).max()))
    torch.cuda.synchronize()
    return out


def ref(v, q, q_off, scale=None):
    return oracle.paged_prefill_bf16(I.bf16_bits(q), I.bf16_bits(v["k_cache"]),
                                     I.bf16_bits(v["v_cache"]), v["block_tables"].cpu().numpy(),
                                     v["context_lens"].cpu().numpy(), q_off.numpy(),
                                     v["scale"] if scale is None else scale)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (12, 2), (32, 8), (32, 1)])
@pytest.mark.parametrize("bs", [16, 256])
def test_prefill_chunk_shapes(D, Hq, Hkv, bs):
    note(f"prefill D={D} Hq={Hq} Hkv={Hkv} bs={bs}")
    ctx = (1, 17, 100, 300, 513, 64)
    nq = [1, 17, 33, 128, 200, 1]
    v, q, q_off = make(ctx, nq, Hq, Hkv, D, bs, seed=500 + D + Hq + Hkv + bs)
    assert_parity(run(v, q, q_off), ref(v, q, q_off), "prefill")


def test_prefill_single_queries_match_decode_output():
    note("prefill n_q=1 vs decode")
    ctx = (1, 17, 100, 250, 4000)
    v, q, q_off = make(ctx, [1] * 5, 32, 8, 128, 16, seed=510)
    got = run(v, q, q_off)
    r = ref(v, q, q_off)
    assert_parity(got, r, "prefill as decode")
    dec = B.decode_views(dict(v, q=q))
    torch.cuda.synchronize()
    assert_parity(dec, r, "decode")


def test_prefill_mixed_chunk_and_decodes_and_empty():
    # One 512-token chunk after a 1500-token prefix, decodes, and a sequence
    # with no query tokens, in one call.
    note("prefill mixed batch")
    ctx = (2012, 37, 900, 5, 128)
    nq = [512, 1, 1, 0, 1]
    v, q, q_off = make(ctx, nq, 32, 8, 128, 16, seed=511)
    assert_parity(run(v, q, q_off), ref(v, q, q_off), "mixed")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.6])
def test_prefill_any_scale(scale):
    # A negative scale flips every score (the kernel negates q and uses
    # |scale|); scale 0 gives every visible token the same weight; 0.6 makes
    # the weights peaked.
    note(f"prefill scale={scale}")
    ctx = (40, 700, 129)
    v, q, q_off = make(ctx, [40, 300, 65], 16, 4, 128, 16, seed=514)
    assert_parity(run(v, q, q_off, scale=scale), ref(v, q, q_off, scale=scale), f"scale {scale}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_growing_keys_move_the_running_max(D):
    # Keys whose magnitude grows block after block along each context: the
    # scores of later tiles exceed the running max by many powers of two, so
    # the accumulators are rescaled again and again (and the first tiles'
    # weights underflow to 0), in both causal and unmasked tiles.
    note(f"prefill growing keys D={D}")
    bs = 16
    ctx = (1000, 333, 64)
    v, q, q_off = make(ctx, [200, 333, 64], 8, 2, D, bs, seed=515 + D)
    k = v["k_cache"].float()
    bt = v["block_tables"].cpu()
    for s_, c in enumerate(ctx):
        for j in range((c + bs - 1) // bs):
            k[int(bt[s_, j])] *= 0.5 + 0.75 * j
    v["k_cache"].copy_(k.to(torch.bfloat16))
    assert_parity(run(v, q, q_off), ref(v, q, q_off), "growing keys")


@pytest.mark.parametrize("bs", [16, 4096])
def test_prefill_long_context_many_table_windows(bs):
    # A 30000-token context at block size 16 is 1875 blocks: the kernel's
    # 64-entry block-table window slides about 30 times (and the last chunk
    # tile crosses a slide); block size 4096 puts a whole tile in one block.
    note(f"prefill long context bs={bs}")
    ctx = (30000, 1500, 7)
    v, q, q_off = make(ctx, [96, 1, 7], 8, 2, 128, bs, seed=516)
    assert_parity(run(v, q, q_off), ref(v, q, q_off), f"long context bs {bs}")


def test_prefill_poisoned_padding_bit_identical():
    note("prefill poison")
    for bs in (16, 256):
        ctx = (17, 300, 513)
        v, q, q_off = make(ctx, [17, 40, 100], 8, 2, 128, bs, seed=512)
        clean = run(v, q, q_off).clone()
        C.poison(v, bs, value=float("nan"), table_pad=-1)
        assert torch.equal(run(v, q, q_off).view(torch.int32), clean.view(torch.int32)), bs


def test_prefill_max_q_len_larger_than_needed_is_harmless():
    note("prefill loose max_q_len")
    v, q, q_off = make((300, 40), [64, 40], 16, 4, 128, 16, seed=513)
    a = run(v, q, q_off).clone()
    b = run(v, q, q_off, max_q=4096)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_full_size_prefill_workload_every_chunk():
    # The bench's workload at full size, same launch as the bench; the oracle
    # checks every query of all eight chunks, every head.
    note("full-size prefill, all chunks")
    pw = I.PREFILL_WORKLOADS["prefill_llama3_8b"]
    inp = I.make_prefill_inputs(pw, DEV)
    out = B.prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                    inp["context_lens"], inp["q_offsets"], inp["scale"], inp["max_q_len"])
    torch.cuda.synchronize()
    r = C.prefill_oracle(inp, inp["q"], inp["q_offsets"])
    assert_parity(out, r, "prefill_llama3_8b")


def test_full_size_serving_batch_one_call_and_split():
    # One 512-token chunk and 63 decodes over the Llama-3-8B decode shapes, as
    # the bench times it: in one paged_attn_prefill call, and as the chunk
    # through paged_attn_prefill plus the decodes through paged_attn_decode;
    # every output row against the oracle.
    import bench

    note("full-size serving batch (1 chunk + 63 decodes)")
    pw = I.PREFILL_WORKLOADS["sarathi_llama3_8b"]
    inp = I.make_prefill_inputs(pw, DEV)
    out = B.prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                    inp["context_lens"], inp["q_offsets"], inp["scale"], inp["max_q_len"])
    torch.cuda.synchronize()
    r = C.prefill_oracle(inp, inp["q"], inp["q_offsets"])
    assert_parity(out, r, "serving batch, one call")
    sp = bench.split_decode_batch(pw, inp, None, DEV)
    B.prefill_views(sp["chunks"], sp["chunks"]["q"], sp["chunks"]["q_offsets"],
                    sp["chunks"]["max_q_len"], out=sp["chunk_out"])
    B.decode_views(sp["decodes"], out=sp["decode_out"], workspace=sp["ws"])
    torch.cuda.synchronize()
    assert_parity(sp["chunk_out"], r[sp["rows_c"].cpu().numpy()], "serving batch, chunk call")
    assert_parity(sp["decode_out"], r[sp["rows_d"].cpu().numpy()], "serving batch, decode call")


# ---- int8 (per-token scales) and FP8 E4M3 caches: the same bar against the
# oracle over the codes' exact values.

def make_kind(ctx, nq, Hq, Hkv, D, bs, seed, kind):
    NB = sum((c + bs - 1) // bs for c in ctx) + 3
    _, v = C.make_case(len(ctx), Hq, Hkv, D, bs, ctx=ctx, NB=NB, seed=seed, device=DEV,
                       kv_dtype=kind)
    q_off = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32)
    gen = torch.Generator(device=DEV).manual_seed(seed + 1)
    q = torch.randn(int(q_off[-1]), Hq, D, generator=gen, device=DEV).to(torch.bfloat16)
    return v, q, q_off


def run_kind(v, q, q_off, max_q=None):
    out = B.prefill_views(v, q, q_off.to(DEV), max_q or int((q_off[1:] - q_off[:-1]).max()))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (12, 2), (32, 8)])
@pytest.mark.parametrize("bs", [16, 256])
def test_quantized_prefill_chunk_shapes(kind, D, Hq, Hkv, bs):
    note(f"prefill {kind} D={D} Hq={Hq} Hkv={Hkv} bs={bs}")
    ctx = (1, 17, 100, 300, 513, 64)
    nq = [1, 17, 33, 128, 200, 1]
    v, q, q_off = make_kind(ctx, nq, Hq, Hkv, D, bs, 520 + D + Hq + bs, kind)
    assert_parity(run_kind(v, q, q_off), C.prefill_oracle(v, q, q_off), f"prefill {kind}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantized_prefill_single_queries_match_decode(kind):
    note(f"prefill {kind} n_q=1 vs decode")
    ctx = (1, 17, 100, 250, 4000)
    v, q, q_off = make_kind(ctx, [1] * 5, 32, 8, 128, 16, 521, kind)
    got = run_kind(v, q, q_off)
    r = C.prefill_oracle(v, q, q_off)
    assert_parity(got, r, f"prefill {kind} as decode")
    dec = B.decode_views(dict(v, q=q))
    torch.cuda.synchronize()
    assert_parity(dec, r, f"decode {kind}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantized_prefill_long_context_and_loose_max_q_len(kind):
    note(f"prefill {kind} long context")
    ctx = (30000, 1500, 7)
    v, q, q_off = make_kind(ctx, [96, 1, 7], 8, 2, 128, 16, 522, kind)
    a = run_kind(v, q, q_off)
    assert_parity(a, C.prefill_oracle(v, q, q_off), f"long context {kind}")
    a = a.clone()
    assert torch.equal(run_kind(v, q, q_off, max_q=4096).view(torch.int32), a.view(torch.int32))


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantized_prefill_poisoned_padding_bit_identical(kind):
    note(f"prefill {kind} poison")
    for bs in (16, 256):
        ctx = (17, 300, 513)
        v, q, q_off = make_kind(ctx, [17, 40, 100], 8, 2, 128, bs, 523, kind)
        clean = run_kind(v, q, q_off).clone()
        C.poison(v, bs, table_pad=-1)
        assert torch.equal(run_kind(v, q, q_off).view(torch.int32), clean.view(torch.int32)), bs


@pytest.mark.parametrize("wl", ["prefill_int8_llama3_8b", "prefill_fp8_llama3_8b"])
def test_full_size_quantized_prefill_workload_every_chunk(wl):
    # The bench's workloads at full size, same launch as the bench; the oracle
    # checks every query of all eight chunks.
    note(f"full-size {wl}, all chunks")
    pw = I.PREFILL_WORKLOADS[wl]
    inp = I.make_prefill_inputs(pw, DEV)
    out = B.prefill_views(inp, inp["q"], inp["q_offsets"], inp["max_q_len"])
    torch.cuda.synchronize()
    r = C.prefill_oracle(inp, inp["q"], inp["q_offsets"])
    assert_parity(out, r, wl)


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("qmul", [4.0, 64.0])
def test_prefill_large_scores_every_cache_kind(kind, qmul):
    # Scores of tens to hundreds (log2 units): rows close to one-hot, where
    # the rounding of the dominant weight would show, and most weights far
    # below the running max.
    note(f"prefill {kind} q x {qmul}")
    ctx = (40, 300, 1100)
    v, q, q_off = make_kind(ctx, [40, 77, 300], 8, 2, 128, 16, 530, kind)
    q = (q.float() * qmul).to(torch.bfloat16)
    assert_parity(run_kind(v, q, q_off), C.prefill_oracle(v, q, q_off), f"{kind} q x {qmul}")


def _nan_at(v, kind, s, t, g, bs):
    """Make V of token t of sequence s, kv head g, non-finite (NaN)."""
    bt = v["block_tables"].cpu()
    b, r = int(bt[s, t // bs]), t % bs
    if kind == "int8":
        v["v_scales"][b, r, g] = float("nan")
    elif kind == "fp8":
        v["v_cache"].view(torch.uint8)[b, r, g, 5] = 0x7F
    else:
        v["v_cache"][b, r, g, 5] = float("nan")


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_prefill_nonfinite_value_inside_the_context(kind):
    # A NaN in V of token t (kv head 1; int8: its scale, so the whole row):
    # every query that sees t has NaN exactly where the definition puts it
    # (the oracle's NaN elements) and the oracle's values elsewhere; queries
    # more than one 32-token tile before t's tile, and the other group, are
    # untouched.  (The 32 rows of a wave -- up to 32 query tokens -- multiply
    # every tile the wave takes, so queries that share a wave with one that
    # reaches t's tile may get a zero weight times NaN: not checked.)
    note(f"prefill {kind} NaN inside the context")
    ctx, nq = (700,), [400]
    Hq, Hkv, D, bs = 8, 2, 128, 16
    v, q, q_off = make_kind(ctx, nq, Hq, Hkv, D, bs, 531, kind)
    t, g = 555, 1
    _nan_at(v, kind, 0, t, g, bs)
    got = run_kind(v, q, q_off).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    pos = ctx[0] - nq[0] + np.arange(nq[0])
    G = Hq // Hkv
    sees = pos >= t
    nan_ref = np.isnan(ref)
    assert nan_ref[sees][:, g * G:(g + 1) * G].any() and not nan_ref[~sees].any()
    assert np.array_equal(np.isnan(got[sees]), nan_ref[sees])
    fin = ~nan_ref & sees[:, None, None]
    assert np.abs(got[fin] - ref[fin]).max() <= 2e-3
    before = pos < (t // 32 - 1) * 32
    assert before.sum() > 100
    assert_parity(torch.from_numpy(got[before]), ref[before], f"{kind} before the NaN tile")
    other = slice(0, g * G)
    assert_parity(torch.from_numpy(np.ascontiguousarray(got[:, other])), np.ascontiguousarray(ref[:, other]),
                  f"{kind} other group")


def test_prefill_bf16_values_past_fp16_range():
    # bf16 V beyond fp16's range (the FP8 path's fp16 tiles would not hold
    # it): the bf16 path keeps such values exact to the bar (compared in units
    # of the scale where the outputs are that big).
    note("prefill bf16 V x 2^16")
    ctx, nq = (300, 700, 90), [50, 300, 90]
    v, q, q_off = make_kind(ctx, nq, 8, 2, 128, 16, 532, "bf16")
    clean = C.prefill_oracle(v, q, q_off)
    # (a) the whole cache times 2^16 (exact in bf16): the outputs are 2^16
    # times the unscaled oracle's
    v_big = dict(v, v_cache=v["v_cache"] * 65536.0)
    got = run_kind(v_big, q, q_off)
    assert_parity(got / 65536.0, clean, "V x 2^16")
    # (b) tokens 100..139 of sequence 1, kv head 0, times 2^16: tiles mixing
    # large and ordinary values; rows whose outputs are large compared in
    # units of 2^16
    bt = v["block_tables"].cpu()
    for t in range(100, 140):
        b = int(bt[1, t // 16])
        v["v_cache"][b, t % 16, 0] *= 65536.0
    got = run_kind(v, q, q_off).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    unit = np.where(np.abs(ref).max(axis=-1, keepdims=True) > 64.0, 65536.0, 1.0)
    assert (unit > 1).any() and (unit == 1).any()
    assert_parity(torch.from_numpy(got / unit), ref / unit, "V partly x 2^16")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_bf16_values_past_fp16_range_in_some_dims(D):
    # Large values (x 2^16) in dims 40..47 only, of tokens 200..263 of
    # sequence 0, kv head 1: in those tiles the 32 dims holding them are
    # staged as bf16 while the tile's other dims stay fp16, and one weighted
    # sum mixes both.  Rows whose outputs are large are compared in units of
    # 2^16.
    note(f"prefill bf16 V x 2^16 in dims 40..47, D={D}")
    ctx, nq = (500, 333), [260, 333]
    v, q, q_off = make_kind(ctx, nq, 8, 2, D, 16, 534 + D, "bf16")
    bt = v["block_tables"].cpu()
    for t in range(200, 264):
        b = int(bt[0, t // 16])
        v["v_cache"][b, t % 16, 1, 40:48] *= 65536.0
    got = run_kind(v, q, q_off).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    unit = np.where(np.abs(ref).max(axis=-1, keepdims=True) > 64.0, 65536.0, 1.0)
    assert (unit > 1).any() and (unit == 1).any()
    assert_parity(torch.from_numpy(got / unit), ref / unit, "V dims 40..47 x 2^16")


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_prefill_workgroups_of_one_to_seven_tiles(kind):
    # Sequences whose workgroups walk 1 .. 7 tiles of 32 tokens: even and odd
    # counts, so the cache kinds staged in segments of several tiles (bf16
    # four, FP8 two) end on a short segment as well as on a whole one.
    note(f"prefill {kind} workgroups of 1..7 tiles")
    ctx = (32, 64, 96, 128, 160, 192, 224, 33, 65, 97)
    nq = [32, 32, 32, 32, 32, 32, 32, 1, 33, 5]
    v, q, q_off = make_kind(ctx, nq, 8, 2, 128, 16, 538, kind)
    assert_parity(run_kind(v, q, q_off), C.prefill_oracle(v, q, q_off), f"{kind} 1..7 tiles")


def _set_v_scales(v, s, tokens, g, value, bs):
    """int8 V scale of the given tokens of sequence s, kv head g."""
    bt = v["block_tables"].cpu()
    for t in tokens:
        v["v_scales"][int(bt[s, t // bs]), t % bs, g] = value


def _weighted_abs_units(v, q, q_off):
    """Per output row, max over dims of sum_t p_t |V_t| (the oracle on |codes|
    and |scales|), at least 1: the size of the values a row's weights take.
    The fp16 weights' rounding moves each output by a fraction of it."""
    ab = C.prefill_oracle(dict(v, v_cache=v["v_cache"].abs(), v_scales=v["v_scales"].abs()), q, q_off)
    return np.maximum(np.abs(ab).max(axis=-1, keepdims=True), 1.0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case,value", [("zero", 0.0), ("huge", 600.0), ("tiny", 1e-6),
                                        ("negative", -0.03), ("large_fast", 1.5), ("small_fast", 1e-4)])
def test_int8_prefill_v_scales_at_and_past_the_fast_range(case, value, D):
    # The int8 prefill takes V scales s = m 2^e with s = 0 or 2^-14 <= s < 2^9
    # in its fast mode (codes times 2^e as fp16, the weights times m); a
    # workgroup that meets any other scale (huge, tiny, negative) runs again
    # with the codes as bf16 and the weights times the whole scales as a
    # bf16 pair.  Tokens 100..139 of sequence 1, kv head 0, take the scale.
    # Compared in units of sum_t p_t |V_t| where that exceeds 1.
    note(f"prefill int8 V scales {case} = {value}, D={D}")
    ctx, nq = (300, 700, 90), [50, 300, 90]
    v, q, q_off = make_kind(ctx, nq, 8, 2, D, 16, 536 + D, "int8")
    _set_v_scales(v, 1, range(100, 140), 0, value, 16)
    got = run_kind(v, q, q_off).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    unit = _weighted_abs_units(v, q, q_off)
    if abs(value) >= 1.0:
        assert (unit > 8).any()
    assert_parity(torch.from_numpy(got / unit), ref / unit, f"int8 V scales {case}")


def test_int8_prefill_every_scale_in_the_fast_range():
    # V scales spread over the whole fast range, 2^-14 .. 2^9 (below), one
    # exponent per 16-token block, so every weight takes a different mantissa
    # and the fp16 V tiles hold codes times 2^-14 .. 2^8.  Compared in units
    # of sum_t p_t |V_t| where that exceeds 1.
    note("prefill int8 V scales 2^-14 .. 2^9")
    ctx, nq = (700, 333), [300, 333]
    bs = 16
    v, q, q_off = make_kind(ctx, nq, 8, 2, 128, bs, 537, "int8")
    gen = torch.Generator().manual_seed(537)
    nb = v["v_scales"].shape[0]
    e = torch.randint(-14, 9, (nb, 1, 1), generator=gen).float()
    m = 1.0 + torch.rand((nb, bs, v["v_scales"].shape[2]), generator=gen) * 0.999
    v["v_scales"].copy_((m * torch.exp2(e)).to(v["v_scales"].device))
    got = run_kind(v, q, q_off).double().cpu().numpy()
    ref = C.prefill_oracle(v, q, q_off)
    unit = _weighted_abs_units(v, q, q_off)
    assert (unit > 1000).any()
    assert_parity(torch.from_numpy(got / unit), ref / unit, "int8 V scales 2^-14 .. 2^9")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("bs", [16, 256])
def test_quantized_prefill_mixed_chunk_decodes_empty(kind, bs):
    # A 512-token chunk after a 1500-token prefix, decodes, a sequence with
    # no query tokens, and an empty context with none, in one call.
    note(f"prefill {kind} mixed batch bs={bs}")
    ctx = (2012, 37, 900, 5, 0, 128)
    nq = [512, 1, 1, 0, 0, 1]
    v, q, q_off = make_kind(ctx, nq, 32, 8, 128, bs, 533 + bs, kind)
    assert_parity(run_kind(v, q, q_off), C.prefill_oracle(v, q, q_off), f"{kind} mixed")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantized_prefill_any_scale(kind):
    note(f"prefill {kind} scales")
    ctx = (40, 300, 700)
    v, q, q_off = make_kind(ctx, [40, 77, 200], 8, 2, 128, 16, 534, kind)
    for scale in (-0.09, 0.0, 0.6):
        out = B.prefill_views(v, q, q_off.to(DEV), 200, scale=scale)
        torch.cuda.synchronize()
        assert_parity(out, C.prefill_oracle(v, q, q_off, scale=scale), f"{kind} scale {scale}")
