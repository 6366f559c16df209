"""GPU parity: the HIP path through the C-ABI against the fp64 oracle.

Bar (floating point): max |gpu - oracle| <= 2e-3 over all elements AND, per
(sequence, head) row, max |gpu - oracle| / max |oracle| <= 1e-2; rows whose
oracle output is exactly zero (empty context) must be exactly zero.
Bit-exact checks: padding poison, identity vs permuted tables, run-to-run
reproducibility, context length 1.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_393_amd import binding as B
from paged_kv_cache_393_amd import inputs as I
from tests import _cases as C

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
MAX_ROW_REL = 1e-2
DEV = "cuda:0"


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def assert_parity(got: torch.Tensor, ref: np.ndarray, what=""):
    g = got.double().cpu().numpy()
    assert g.shape == ref.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    row_inf = np.abs(ref).max(axis=-1)
    row_err = err.max(axis=-1)
    zero = row_inf == 0
    assert np.all(g[zero] == 0), f"{what}: empty-context rows not zero"
    max_abs = float(err.max()) if err.size else 0.0
    rel = float((row_err[~zero] / row_inf[~zero]).max()) if np.any(~zero) else 0.0
    assert max_abs <= MAX_ABS, f"{what}: max abs err {max_abs:.3e}"
    assert rel <= MAX_ROW_REL, f"{what}: max row rel err {rel:.3e}"
    return max_abs, rel


def run(views, split_tokens=0):
    out = B.decode_views(views, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out


def test_tiny_workload_all_partitions():
    wl = I.WORKLOADS["tiny"]
    v = I.layer_views(I.make_inputs(wl, DEV), 0)
    ref = C.oracle_out(v)
    for st in (0, 16, 32, 64, 128, 256):
        note(f"tiny split_tokens={st}")
        assert_parity(run(v, st), ref, f"tiny split={st}")


EDGE_CTX = (0, 1, 15, 16, 17, 511, 512, 513)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (16, 2), (32, 1)])
@pytest.mark.parametrize("bs", [16, 32, 256])
def test_edge_contexts(kv, D, Hq, Hkv, bs):
    note(f"edge kv={kv} D={D} Hq={Hq} Hkv={Hkv} bs={bs}")
    ctx = EDGE_CTX
    NB = sum((c + bs - 1) // bs for c in ctx) + 5
    _, v = C.make_case(len(ctx), Hq, Hkv, D, bs, ctx=ctx, NB=NB, seed=100 + D + Hq + bs,
                       kv_dtype=kv, device=DEV)
    ref = C.oracle_out(v)
    for st in (0, 16, 128, 512):
        assert_parity(run(v, st), ref, f"split={st}")


@pytest.mark.parametrize("Hq,Hkv", [(6, 1), (24, 2), (12, 4), (64, 8), (40, 8)])
def test_group_sizes_not_powers_of_two_and_large(Hq, Hkv):
    note(f"groups Hq={Hq} Hkv={Hkv}")
    ctx = (300, 47, 1000)
    _, v = C.make_case(3, Hq, Hkv, 128, 16, ctx=ctx, NB=100, seed=7 + Hq, device=DEV)
    ref = C.oracle_out(v)
    assert_parity(run(v, 0), ref, "auto")
    assert_parity(run(v, 256), ref, "split 256")


def test_batches_beyond_the_lds_prefix():
    # More than 2048 sequences: each workgroup finds its item's first sequence
    # by a running scan over the context lengths instead of the LDS prefix.
    rng = np.random.default_rng(60)
    ctx = tuple(int(x) for x in rng.integers(0, 60, 3000))
    note(f"3000 sequences, ctx 0..59")
    _, v = C.make_case(len(ctx), 8, 2, 64, 16, ctx=ctx, seed=60, device=DEV)
    ref = C.oracle_out(v)
    for st in (0, 16, 64):
        assert_parity(run(v, st), ref, f"split={st}")


def test_context_one_is_exactly_v():
    note("ctx=1 exact")
    _, v = C.make_case(3, 8, 2, 128, 16, ctx=(1, 1, 1), NB=9, seed=31, device=DEV)
    out = run(v).cpu()
    for s in range(3):
        b = int(v["block_tables"][s, 0])
        for h in range(8):
            assert torch.equal(out[s, h], v["v_cache"][b, 0, h // 4].float().cpu())


def test_gqa_mapping_constant_values():
    note("gqa mapping")
    _, v = C.make_case(2, 16, 4, 64, 16, ctx=(70, 9), seed=32, device=DEV)
    for g in range(4):
        v["v_cache"][:, :, g, :] = float(g + 1)
    out = run(v).cpu()
    # Not bit-exact: the softmax weights enter the PV product as a bf16 pair
    # (high part + remainder, exact to 2^-17 relative) and sum(p*c)/sum(p) is
    # rounded in fp32, so the result is c within a few 2^-17 c.  A wrong
    # head->kv-head map (h % G instead of h / G) is off by at least 1.
    for h in range(16):
        assert torch.allclose(out[:, h], torch.full_like(out[:, h], float(h // 4 + 1)),
                              rtol=0, atol=1e-4), h


def test_uniform_keys_mean_of_values():
    note("uniform keys")
    _, v = C.make_case(2, 8, 2, 128, 16, ctx=(1500, 33), seed=33, device=DEV)
    v["k_cache"].copy_(v["k_cache"][0:1, 0:1].expand_as(v["k_cache"]))
    ref = C.oracle_out(v)
    for st in (0, 512):
        assert_parity(run(v, st), ref, f"uniform split={st}")


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_poisoned_padding_bit_identical(kv):
    note(f"poison {kv}")
    for bs in (16, 256):
        ctx = (1, 17, 100, 250, 513)
        NB = sum((c + bs - 1) // bs for c in ctx) + 7
        _, v = C.make_case(len(ctx), 8, 2, 128, bs, ctx=ctx, NB=NB, seed=34, kv_dtype=kv,
                           device=DEV)
        for st in (0, 64):
            clean = run(v, st).clone()
            for fill in (float("nan"), float("inf"), -float("inf"), 1e30):
                w = {k: (t.clone() if torch.is_tensor(t) else t) for k, t in v.items()}
                C.poison(w, bs, value=fill, table_pad=-1 if fill != 1e30 else 2 ** 30)
                got = run(w, st)
                assert torch.equal(got.view(torch.int32), clean.view(torch.int32)), (bs, st, fill)


def test_identity_vs_permuted_tables_bit_identical():
    note("identity vs permuted")
    _, v = C.make_case(3, 32, 8, 128, 16, ctx=(777, 16, 2049), seed=35, device=DEV)
    a = run(v, 0).clone()
    bt = v["block_tables"].cpu()
    nblk = [(c + 15) // 16 for c in v["context_lens"].cpu().tolist()]
    order = [int(bt[s, j]) for s, n in enumerate(nblk) for j in range(n)]
    idx = torch.tensor(order, device=DEV)
    k2 = v["k_cache"].index_select(0, idx).contiguous()
    v2 = v["v_cache"].index_select(0, idx).contiguous()
    ident = torch.zeros_like(bt)
    pos = 0
    for s, n in enumerate(nblk):
        ident[s, :n] = torch.arange(pos, pos + n)
        pos += n
    w = dict(v, k_cache=k2, v_cache=v2, block_tables=ident.to(DEV))
    assert torch.equal(run(w, 0).view(torch.int32), a.view(torch.int32))


def test_split_vs_unsplit_and_reproducible():
    note("split vs unsplit")
    _, v = C.make_case(2, 32, 8, 128, 16, ctx=(8192, 5000), seed=36, device=DEV)
    ref = C.oracle_out(v)
    whole = run(v, 8192).clone()
    for st in (16, 512, 1024):
        part = run(v, st)
        assert_parity(part, ref, f"split={st}")
        assert float((part - whole).abs().max()) <= 1e-5
        again = run(v, st)
        assert torch.equal(again.view(torch.int32), part.view(torch.int32))
    assert_parity(whole, ref, "unsplit")


def test_workspace_reused_across_calls_and_shapes():
    # One workspace serves a sequence of calls of different shapes and item
    # sizes (no state carries over between calls): each result is
    # bit-identical to a run with a fresh workspace.
    note("workspace reuse")
    cases = [C.make_case(5, 32, 8, 128, 16, ctx=(3000, 17, 0, 900, 1), seed=40, device=DEV)[1],
             C.make_case(3, 8, 2, 64, 16, ctx=(250, 1000, 33), seed=41, device=DEV)[1],
             C.make_case(4, 16, 2, 128, 256, ctx=(5000, 257, 4096, 2), seed=42, kv_dtype="int8",
                         device=DEV)[1]]
    splits = (0, 16, 512)
    fresh = {(i, st): run(v, st).clone() for i, v in enumerate(cases) for st in splits}
    need = max(B.workspace_bytes(B.shape_of(v["q"], v["k_cache"], v["block_tables"], st))
               for v in cases for st in splits)
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)   # garbage-filled
    for rep in range(2):
        for i, v in enumerate(cases):
            for st in splits:
                got = B.decode_views(v, split_tokens=st, workspace=ws)
                torch.cuda.synchronize()
                assert torch.equal(got.view(torch.int32), fresh[(i, st)].view(torch.int32)), (rep, i, st)


def test_decode_and_table_check_on_a_side_stream():
    # With stream= a non-current stream, the wrapper allocates out and the
    # workspace for that stream: allocator churn on the current stream while
    # the side stream runs cannot reuse them.  Every result equals a decode on
    # the current stream bit for bit and passes against the oracle.
    note("side stream")
    _, v = C.make_case(5, 32, 8, 128, 16, ctx=(3000, 17, 0, 900, 1), seed=45, device=DEV)
    ref = C.oracle_out(v)
    main = run(v, 0).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(B.decode_views(v, stream=side))
        junk = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
        junk.fill_(0x7F)
        del junk
    side.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int32), main.view(torch.int32))
    assert_parity(outs[0], ref, "side stream")
    n_bad, first = B.check_tables(v["block_tables"], v["context_lens"], v["k_cache"].shape[0], 16,
                                  stream=side)
    assert (n_bad, first) == (0, -1)


def test_large_scores_stable():
    note("large scores")
    _, v = C.make_case(2, 8, 2, 128, 16, ctx=(600, 31), seed=37, device=DEV)
    v["q"] = (v["q"].float() * 64).to(torch.bfloat16)
    ref = C.oracle_out(v)
    for st in (0, 128):
        assert_parity(run(v, st), ref, f"large split={st}")


def test_int8_lossless_values_match_bf16_path():
    note("int8 lossless vs bf16")
    _, vb = C.make_case(3, 32, 8, 128, 16, ctx=(100, 513, 40), seed=38, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(9)
    kc = torch.randint(-127, 128, vb["k_cache"].shape, generator=gen, device=DEV)
    vc = torch.randint(-127, 128, vb["v_cache"].shape, generator=gen, device=DEV)
    kc[..., 5] = 127
    vc[..., 9] = -127
    vb["k_cache"] = (kc.double() * 2.0 ** -5).to(torch.bfloat16)
    vb["v_cache"] = (vc.double() * 2.0 ** -5).to(torch.bfloat16)
    ones = torch.full(vb["k_cache"].shape[:3], 2.0 ** -5, device=DEV)
    vi = dict(vb, k_cache=kc.to(torch.int8), v_cache=vc.to(torch.int8), k_scales=ones,
              v_scales=ones.clone())
    ref = C.oracle_out(vb)
    assert np.array_equal(ref, C.oracle_out(vi))
    assert_parity(run(vb), ref, "bf16")
    assert_parity(run(vi), ref, "int8")


def test_fp8_path_matches_bf16_path_on_the_same_values():
    # Every E4M3 value is a bf16 value and the kernel decodes the codes
    # exactly, so an fp8 cache and a bf16 cache holding the decoded values give
    # the same result up to fp32 summation order: the two layouts feed the QK
    # products' dims to the matrix cores in a different order (16 vs 8
    # elements per 16-byte load).
    note("fp8 vs bf16 same values")
    for bs, ctx in ((16, (100, 513, 40, 1)), (256, (3000, 257, 16))):
        NB = sum((c + bs - 1) // bs for c in ctx) + 2
        _, v8 = C.make_case(len(ctx), 32, 8, 128, bs, ctx=ctx, NB=NB, seed=39, kv_dtype="fp8",
                            device=DEV)
        vb = dict(v8, k_cache=v8["k_cache"].to(torch.bfloat16),
                  v_cache=v8["v_cache"].to(torch.bfloat16))
        ref = C.oracle_out(v8)
        for st in (0, 64):
            a, b = run(v8, st).clone(), run(vb, st)
            assert float((a - b).abs().max()) <= 1e-5, (bs, st)
            assert_parity(a, ref, f"fp8 bs={bs} split={st}")
            assert_parity(b, ref, f"bf16 bs={bs} split={st}")


def test_fp8_nan_code_reaches_only_its_output_elements():
    # A NaN code in V at one valid (token, kv head, dim) makes exactly that dim
    # of that kv head's query heads NaN (as in the definition); every other
    # output element keeps its bits.
    note("fp8 nan locality")
    _, v = C.make_case(2, 8, 2, 64, 16, ctx=(40, 70), seed=44, kv_dtype="fp8", device=DEV)
    clean = run(v).clone()
    b = int(v["block_tables"][1, 1])
    v["v_cache"].view(torch.uint8)[b, 3, 1, 10] = 0x7F      # token 19 of sequence 1
    got = run(v)
    nan = torch.isnan(got)
    expect = torch.zeros_like(nan)
    expect[1, 4:8, 10] = True                               # heads 4..7 use kv head 1
    assert torch.equal(nan, expect)
    assert torch.equal(got[~expect].view(torch.int32), clean[~expect].view(torch.int32))


# Full-size workloads in the launch configuration the bench times: every
# sequence, every head and, for the layered 70B-shaped cache, every layer is
# compared with the oracle.
FULL = ["tiny", "llama3_8b", "long_context", "nano_vllm_70b", "int8_llama3_8b",
        "fp8_llama3_8b", "llama3_8b_tp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workloads_every_sequence_and_layer(name):
    wl = I.WORKLOADS[name]
    inp = I.make_inputs(wl, DEV)
    for l in range(wl.num_layers):
        note(f"full {name} layer {l}")
        v = I.layer_views(inp, l)
        out = B.decode_views(v, split_tokens=wl.split_tokens)
        torch.cuda.synchronize()
        ref = C.oracle_out(v)
        assert_parity(out, ref, f"{name} layer {l}")
        del v, out, ref
    del inp
    torch.cuda.empty_cache()
