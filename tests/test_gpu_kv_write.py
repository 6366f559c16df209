"""GPU parity of the KV write path (paged_kv_write, paged_kv_write_int8)
through the C-ABI against the oracle.

The write is integer / byte work: the whole caches (and, for int8, codes and
scales) must be bit-identical to the oracle's.  Then a write followed by a
decode must pass the decode's floating-point bar against the oracle.
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


def _pool(NB, bs, Hkv, D, seed, kv_dtype):
    gen = torch.Generator().manual_seed(seed)
    if kv_dtype == "bf16":
        kc = torch.randn(NB, bs, Hkv, D, generator=gen).to(torch.bfloat16)
        vc = torch.randn(NB, bs, Hkv, D, generator=gen).to(torch.bfloat16)
        return kc, vc, None, None
    kc = torch.randint(-127, 128, (NB, bs, Hkv, D), generator=gen).to(torch.int8)
    vc = torch.randint(-127, 128, (NB, bs, Hkv, D), generator=gen).to(torch.int8)
    ks = torch.rand(NB, bs, Hkv, generator=gen)
    vs = torch.rand(NB, bs, Hkv, generator=gen)
    return kc, vc, ks, vs


def _bits(t):
    return I.bf16_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def check_write(T, Hkv, D, bs, NB, kv_dtype, seed, pad=0.2, token_stride=None, slots=None):
    kc, vc, ks, vs = _pool(NB, bs, Hkv, D, seed, kv_dtype)
    key, value = I.make_new_tokens(T, Hkv, D, seed=seed, device=DEV, token_stride=token_stride)
    if slots is None:
        slots = I.draw_slots(T, NB * bs, seed=seed, pad_fraction=pad)
    kb, vb = I.bf16_bits(key), I.bf16_bits(value)
    sl = slots.numpy()
    g_kc, g_vc = kc.to(DEV), vc.to(DEV)
    s_dev = slots.to(DEV)
    if kv_dtype == "bf16":
        B.kv_write(key, value, s_dev, g_kc, g_vc)
        torch.cuda.synchronize()
        rk, rv = oracle.kv_write_bf16(kb, vb, sl, _bits(kc), _bits(vc))
        assert np.array_equal(_bits(g_kc), rk), "k_cache differs"
        assert np.array_equal(_bits(g_vc), rv), "v_cache differs"
    else:
        g_ks, g_vs = ks.to(DEV), vs.to(DEV)
        B.kv_write_int8(key, value, s_dev, g_kc, g_vc, g_ks, g_vs)
        torch.cuda.synchronize()
        rk, rv, rks, rvs = oracle.kv_write_int8(kb, vb, sl, kc.numpy(), vc.numpy(), ks.numpy(),
                                                vs.numpy())
        assert np.array_equal(g_kc.cpu().numpy(), rk), "k codes differ"
        assert np.array_equal(g_vc.cpu().numpy(), rv), "v codes differ"
        assert np.array_equal(g_ks.cpu().numpy().view(np.uint32), rks.view(np.uint32)), \
            "k scales differ"
        assert np.array_equal(g_vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32)), \
            "v scales differ"


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hkv", [1, 3, 8])
@pytest.mark.parametrize("T", [0, 1, 5, 37, 300])
def test_write_bit_exact(kv, D, Hkv, T):
    note(f"write kv={kv} D={D} Hkv={Hkv} T={T}")
    bs = 16
    NB = max(1, (T + bs - 1) // bs) + 3
    check_write(T, Hkv, D, bs, NB, kv, seed=200 + T + D + Hkv)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_write_strided_rows_of_a_fused_projection(kv):
    # K and V as slices of a [T, (Hq + 2 Hkv) * d]-wide buffer.
    note(f"write strided kv={kv}")
    Hkv, D = 8, 128
    check_write(77, Hkv, D, 16, 10, kv, seed=210, token_stride=(32 + 16) * D)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_write_block_size_256_and_all_slots(kv):
    note(f"write bs=256 full pool kv={kv}")
    NB, bs = 3, 256
    check_write(NB * bs, 2, 64, bs, NB, kv, seed=211, pad=0.0)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_write_skips_slots_out_of_range(kv):
    note(f"write out-of-range slots kv={kv}")
    NB, bs, Hkv, D = 4, 16, 2, 128
    slots = torch.tensor([3, NB * bs, -1, NB * bs + 1000, 2 ** 31 - 1, 0], dtype=torch.int32)
    kc, vc, ks, vs = _pool(NB, bs, Hkv, D, 212, kv)
    key, value = I.make_new_tokens(len(slots), Hkv, D, seed=212, device=DEV)
    g = [t.to(DEV) for t in (kc, vc) + ((ks, vs) if kv == "int8" else ())]
    if kv == "bf16":
        B.kv_write(key, value, slots.to(DEV), *g)
    else:
        B.kv_write_int8(key, value, slots.to(DEV), *g)
    torch.cuda.synchronize()
    keep = torch.ones(NB * bs, dtype=torch.bool)
    keep[[3, 0]] = False
    for before, after in zip((kc, vc) + ((ks, vs) if kv == "int8" else ()), g):
        b = before.reshape(NB * bs, -1)[keep]
        a = after.cpu().reshape(NB * bs, -1)[keep]
        assert torch.equal(b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32),
                           a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32))
    # the valid ones were written like the oracle does
    sl = np.array([3, 0], dtype=np.int32)
    kb, vb = I.bf16_bits(key)[[0, 5]], I.bf16_bits(value)[[0, 5]]
    if kv == "bf16":
        rk, _ = oracle.kv_write_bf16(kb, vb, sl, _bits(kc), _bits(vc))
        assert np.array_equal(_bits(g[0]), rk)
    else:
        rk, _, rks, _ = oracle.kv_write_int8(kb, vb, sl, kc.numpy(), vc.numpy(), ks.numpy(),
                                             vs.numpy())
        assert np.array_equal(g[0].cpu().numpy(), rk) and np.array_equal(g[2].cpu().numpy(), rks)


def test_int8_write_zero_and_tiny_rows():
    # A row of zeros gets scale 0 and codes 0; a row of tiny values still gets
    # codes +-127 at its maximum.
    note("int8 write zero / tiny rows")
    NB, bs, Hkv, D, T = 2, 16, 2, 128, 4
    kc, vc, ks, vs = _pool(NB, bs, Hkv, D, 213, "int8")
    key, value = I.make_new_tokens(T, Hkv, D, seed=213, device=DEV)
    key[0].zero_()
    value[1, 1].zero_()
    key[2] = key[2] * 1e-30
    slots = torch.tensor([0, 5, 17, 30], dtype=torch.int32)
    g = [t.to(DEV) for t in (kc, vc, ks, vs)]
    B.kv_write_int8(key, value, slots.to(DEV), *g)
    torch.cuda.synchronize()
    rk, rv, rks, rvs = oracle.kv_write_int8(I.bf16_bits(key), I.bf16_bits(value), slots.numpy(),
                                            kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy())
    assert np.array_equal(g[0].cpu().numpy(), rk) and np.array_equal(g[1].cpu().numpy(), rv)
    assert np.array_equal(g[2].cpu().numpy(), rks) and np.array_equal(g[3].cpu().numpy(), rvs)
    assert rks.reshape(-1, Hkv)[0, 0] == 0.0 and np.all(rk.reshape(-1, Hkv, D)[0] == 0)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_write_then_decode(kv):
    # One decode step end to end: each sequence's new token is stored at the
    # slot its block table gives position ctx, then decode runs over ctx + 1
    # tokens -- against the oracle doing the same two steps.
    note(f"write then decode kv={kv}")
    ctx = (0, 15, 16, 100, 511, 2000)
    bs, Hq, Hkv, D = 16, 32, 8, 128
    full = tuple(c + 1 for c in ctx)
    NB = sum((c + bs - 1) // bs for c in full) + 2
    _, v = C.make_case(len(ctx), Hq, Hkv, D, bs, ctx=full, NB=NB, seed=214, kv_dtype=kv,
                       device=DEV)
    key, value = I.make_new_tokens(len(ctx), Hkv, D, seed=214, device=DEV)
    bt = v["block_tables"].cpu().numpy()
    slots = np.array([oracle.slot_of(bt[s], c, bs) for s, c in enumerate(ctx)], dtype=np.int32)
    host = {k: (t.cpu() if torch.is_tensor(t) else t) for k, t in v.items()}
    if kv == "bf16":
        B.kv_write(key, value, torch.from_numpy(slots).to(DEV), v["k_cache"], v["v_cache"])
        rk, rv = oracle.kv_write_bf16(I.bf16_bits(key), I.bf16_bits(value), slots,
                                      I.bf16_bits(host["k_cache"]), I.bf16_bits(host["v_cache"]))
        host["k_cache"] = torch.from_numpy(rk.view(np.int16)).view(torch.bfloat16)
        host["v_cache"] = torch.from_numpy(rv.view(np.int16)).view(torch.bfloat16)
    else:
        B.kv_write_int8(key, value, torch.from_numpy(slots).to(DEV), v["k_cache"], v["v_cache"],
                        v["k_scales"], v["v_scales"])
        rk, rv, rks, rvs = oracle.kv_write_int8(
            I.bf16_bits(key), I.bf16_bits(value), slots, host["k_cache"].numpy(),
            host["v_cache"].numpy(), host["k_scales"].numpy(), host["v_scales"].numpy())
        host.update(k_cache=torch.from_numpy(rk), v_cache=torch.from_numpy(rv),
                    k_scales=torch.from_numpy(rks), v_scales=torch.from_numpy(rvs))
    out = B.decode_views(v)
    torch.cuda.synchronize()
    assert_parity(out, C.oracle_out(host), f"write+decode {kv}")


@pytest.mark.parametrize("name", ["kv_write_llama3_8b", "kv_write_int8_llama3_8b"])
def test_full_size_write_workload_bit_exact(name):
    # The bench's write workloads at full size, same launch as the bench.
    note(f"full-size write workload {name}")
    ww = I.WRITE_WORKLOADS[name]
    inp = I.make_write_inputs(ww, DEV)
    before = {k: t.cpu() for k, t in inp.items() if torch.is_tensor(t)}
    B.kv_write_inputs(inp)
    torch.cuda.synchronize()
    kb, vb, sl = I.bf16_bits(before["key"]), I.bf16_bits(before["value"]), before["slots"].numpy()
    if ww.kv_dtype == "bf16":
        rk, rv = oracle.kv_write_bf16(kb, vb, sl, I.bf16_bits(before["k_cache"]),
                                      I.bf16_bits(before["v_cache"]))
        assert np.array_equal(I.bf16_bits(inp["k_cache"]), rk)
        assert np.array_equal(I.bf16_bits(inp["v_cache"]), rv)
    else:
        rk, rv, rks, rvs = oracle.kv_write_int8(kb, vb, sl, before["k_cache"].numpy(),
                                                before["v_cache"].numpy(),
                                                before["k_scales"].numpy(),
                                                before["v_scales"].numpy())
        assert np.array_equal(inp["k_cache"].cpu().numpy(), rk)
        assert np.array_equal(inp["v_cache"].cpu().numpy(), rv)
        assert np.array_equal(inp["k_scales"].cpu().numpy(), rks)
        assert np.array_equal(inp["v_scales"].cpu().numpy(), rvs)


def _dense_bf16_rows(amaxes, D):
    """Rows of D bf16 values: for each row maximum a, element 0 is a and the
    others run through EVERY bf16 value x with a/512 <= |x| <= a (both signs),
    so every quotient x / (a / 127) that can round to a non-zero code occurs."""
    allbf = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    rows = []
    for a in amaxes:
        xs = allbf[(allbf <= a) & (allbf >= a / 512)]
        xs = np.concatenate([xs, -xs])
        for start in range(0, xs.size, D - 1):
            chunk = xs[start:start + D - 1]
            row = np.zeros(D, dtype=np.float32)
            row[0] = a
            row[1:1 + chunk.size] = chunk
            rows.append(row)
    return torch.from_numpy(np.stack(rows)).to(torch.bfloat16)


def test_int8_write_every_bf16_value_for_many_scales():
    # The kernel forms x / scale by a reciprocal multiply where that provably
    # gives the same rounded code and by IEEE division near half-integers;
    # over all bf16 inputs of 48 rows maxima (powers of two, whose quotients
    # hit half-integers exactly, and random ones) the codes must be the
    # oracle's, which always divides.
    note("int8 write exhaustive bf16 quotients")
    gen = torch.Generator().manual_seed(215)
    pow2 = [2.0 ** e for e in range(-20, 21, 4)]
    rand = (torch.rand(37, generator=gen, dtype=torch.float64) * 60 - 30).exp2().tolist()
    amaxes = [float(torch.tensor(a).to(torch.bfloat16)) for a in pow2 + rand]
    D, Hkv = 128, 1
    rows = _dense_bf16_rows(amaxes, D)
    T = rows.shape[0]
    key = rows.reshape(T, Hkv, D).to(DEV)
    value = (-rows).flip(0).reshape(T, Hkv, D).contiguous().to(DEV)
    NB, bs = (T + 15) // 16, 16
    slots = torch.randperm(NB * bs, generator=gen)[:T].to(torch.int32)
    kc = torch.zeros(NB, bs, Hkv, D, dtype=torch.int8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros(NB, bs, Hkv, dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    B.kv_write_int8(key, value, slots.to(DEV), kc, vc, ks, vs)
    torch.cuda.synchronize()
    z8 = np.zeros((NB, bs, Hkv, D), dtype=np.int8)
    zs = np.zeros((NB, bs, Hkv), dtype=np.float32)
    rk, rv, rks, rvs = oracle.kv_write_int8(I.bf16_bits(key), I.bf16_bits(value), slots.numpy(),
                                            z8, z8, zs, zs)
    for got, ref, what in ((kc, rk, "k codes"), (vc, rv, "v codes"), (ks, rks, "k scales"),
                           (vs, rvs, "v scales")):
        g = got.cpu().numpy()
        assert np.array_equal(g.view(np.uint8), ref.view(np.uint8)), \
            f"{what}: {int((g != ref).sum())} of {g.size} differ"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hkv", [1, 3, 8])
@pytest.mark.parametrize("T", [0, 1, 37, 300])
def test_fp8_write_bit_exact(D, Hkv, T):
    note(f"fp8 write D={D} Hkv={Hkv} T={T}")
    bs = 16
    NB = max(1, (T + bs - 1) // bs) + 3
    check_fp8_write(T, Hkv, D, bs, NB, seed=300 + T + D + Hkv)


def check_fp8_write(T, Hkv, D, bs, NB, seed, pad=0.2, token_stride=None, key=None, value=None,
                    slots=None):
    gen = torch.Generator().manual_seed(seed)
    kc = torch.randint(0, 256, (NB, bs, Hkv, D), generator=gen, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, (NB, bs, Hkv, D), generator=gen, dtype=torch.int32).to(torch.uint8)
    if key is None:
        key, value = I.make_new_tokens(T, Hkv, D, seed=seed, device=DEV, token_stride=token_stride)
    if slots is None:
        slots = I.draw_slots(T, NB * bs, seed=seed, pad_fraction=pad)
    g_kc = kc.to(DEV).view(torch.float8_e4m3fn)
    g_vc = vc.to(DEV).view(torch.float8_e4m3fn)
    B.kv_write_fp8(key, value, slots.to(DEV), g_kc, g_vc)
    torch.cuda.synchronize()
    # the kernel skips slots past the pool (a caller error the oracle rejects):
    # for the oracle they are tokens without a slot
    sl = slots.numpy().copy()
    sl[sl >= NB * bs] = -1
    rk, rv = oracle.kv_write_fp8(I.bf16_bits(key), I.bf16_bits(value), sl, kc.numpy(), vc.numpy())
    gk, gv = C.fp8_codes(g_kc), C.fp8_codes(g_vc)
    assert np.array_equal(gk, rk), f"k codes: {int((gk != rk).sum())} differ"
    assert np.array_equal(gv, rv), f"v codes: {int((gv != rv).sum())} differ"


def test_fp8_write_every_bf16_value():
    # All 65536 bf16 bit patterns (zeros, subnormals, the 448/464 boundary,
    # infinities, NaNs of both signs) go through the kernel's cast: every code
    # must be the oracle's, i.e. torch's float8_e4m3fn cast.
    note("fp8 write exhaustive bf16")
    D, Hkv = 128, 1
    T = 65536 // D
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    key = bits.reshape(T, Hkv, D).to(DEV)
    value = bits.flip(0).reshape(T, Hkv, D).contiguous().to(DEV)
    NB, bs = T // 16, 16
    slots = torch.randperm(NB * bs, generator=torch.Generator().manual_seed(301)).to(torch.int32)
    check_fp8_write(T, Hkv, D, bs, NB, seed=301, key=key, value=value, slots=slots)


def test_fp8_write_strided_and_out_of_range():
    note("fp8 write strided / out of range")
    check_fp8_write(77, 8, 128, 16, 10, seed=302, token_stride=(32 + 16) * 128)
    NB, bs = 4, 16
    key, value = I.make_new_tokens(4, 2, 64, seed=303, device=DEV)
    slots = torch.tensor([3, NB * bs, -1, 0], dtype=torch.int32)
    check_fp8_write(4, 2, 64, bs, NB, seed=303, key=key, value=value, slots=slots)


def test_fp8_write_then_decode():
    note("fp8 write then decode")
    ctx = (0, 15, 16, 100, 511, 2000)
    bs, Hq, Hkv, D = 16, 32, 8, 128
    full = tuple(c + 1 for c in ctx)
    NB = sum((c + bs - 1) // bs for c in full) + 2
    _, v = C.make_case(len(ctx), Hq, Hkv, D, bs, ctx=full, NB=NB, seed=304, kv_dtype="fp8",
                       device=DEV)
    key, value = I.make_new_tokens(len(ctx), Hkv, D, seed=304, device=DEV)
    bt = v["block_tables"].cpu().numpy()
    slots = np.array([oracle.slot_of(bt[s], c, bs) for s, c in enumerate(ctx)], dtype=np.int32)
    host = {k: (t.cpu() if torch.is_tensor(t) else t) for k, t in v.items()}
    B.kv_write_fp8(key, value, torch.from_numpy(slots).to(DEV), v["k_cache"], v["v_cache"])
    rk, rv = oracle.kv_write_fp8(I.bf16_bits(key), I.bf16_bits(value), slots,
                                 C.fp8_codes(host["k_cache"]), C.fp8_codes(host["v_cache"]))
    host["k_cache"] = torch.from_numpy(rk).view(torch.float8_e4m3fn)
    host["v_cache"] = torch.from_numpy(rv).view(torch.float8_e4m3fn)
    out = B.decode_views(v)
    torch.cuda.synchronize()
    assert_parity(out, C.oracle_out(host), "fp8 write+decode")


def test_full_size_fp8_write_workload_every_token():
    # The bench's fp8 write workload at full size, same launch as the bench;
    # the oracle casts every token (its brute-force nearest-code search runs
    # on 16 token ranges at once: ctypes releases the GIL).
    from concurrent.futures import ThreadPoolExecutor

    note("full-size fp8 write workload")
    ww = I.WRITE_WORKLOADS["kv_write_fp8_llama3_8b"]
    inp = I.make_write_inputs(ww, DEV)
    B.kv_write_inputs(inp)
    torch.cuda.synchronize()
    slots_all = inp["slots"].cpu().numpy()
    kb_all, vb_all = I.bf16_bits(inp["key"].cpu()), I.bf16_bits(inp["value"].cpu())
    shape = tuple(inp["k_cache"].shape)
    gk = C.fp8_codes(inp["k_cache"]).reshape(-1, ww.num_kv_heads, ww.head_dim)
    gv = C.fp8_codes(inp["v_cache"]).reshape(-1, ww.num_kv_heads, ww.head_dim)

    def one(lo_hi):
        lo, hi = lo_hi
        z = np.zeros(shape, dtype=np.uint8)
        sl = slots_all[lo:hi]
        rk, rv = oracle.kv_write_fp8(kb_all[lo:hi], vb_all[lo:hi], sl, z, z)
        rk = rk.reshape(-1, ww.num_kv_heads, ww.head_dim)
        rv = rv.reshape(-1, ww.num_kv_heads, ww.head_dim)
        sl = sl[sl >= 0]
        return bool(np.array_equal(gk[sl], rk[sl]) and np.array_equal(gv[sl], rv[sl]))

    T = ww.num_tokens
    ranges = [(i * T // 16, (i + 1) * T // 16) for i in range(16)]
    with ThreadPoolExecutor(16) as ex:
        ok = list(ex.map(one, ranges))
    assert all(ok), ok
