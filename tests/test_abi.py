"""CPU tests of the C-ABI: the library loads, exports what the header declares,
and rejects bad arguments on the host (no GPU call is made on these paths)."""
import ctypes

import pytest

from paged_kv_cache_393_amd import binding as B

DECLARED = {"paged_attn_plan", "paged_attn_workspace_bytes", "paged_attn_decode",
            "paged_attn_decode_int8", "paged_attn_strerror", "paged_attn_abi_version",
            "paged_kv_write", "paged_kv_write_int8", "paged_attn_decode_fp8", "paged_kv_write_fp8",
            "paged_kv_token_scores", "paged_kv_token_scores_int8", "paged_kv_token_scores_fp8",
            "paged_kv_evict_lowest_block", "paged_attn_prefill", "paged_attn_prefill_int8",
            "paged_attn_prefill_fp8", "paged_kv_compress_workspace_bytes",
            "paged_kv_compress_prefill", "paged_kv_compress_prefill_int8",
            "paged_kv_compress_prefill_fp8", "paged_attn_check_tables",
            "paged_attn_decode_noalloc", "paged_attn_prefill_plan",
            "paged_attn_prefill_workspace_bytes", "paged_attn_prefill_split",
            "paged_attn_prefill_split_int8", "paged_attn_prefill_split_fp8"}


def lib():
    return B.load()


def test_header_declares_the_expected_entry_points():
    assert set(B.header_functions()) == DECLARED


def test_library_exports_every_declared_symbol():
    L = lib()
    for name in B.header_functions():
        assert hasattr(L, name), name


def test_probe_library_exports_its_header():
    import re

    from paged_kv_cache_393_amd import probe

    text = re.sub(r"/\*.*?\*/", "", open(probe.HEADER).read(), flags=re.S)
    names = set(re.findall(r"\b(pa_probe_\w+)\s*\(", text))
    assert names == {"pa_probe_read", "pa_probe_copy"}
    L = probe.load()
    for n in names:
        assert hasattr(L, n), n


def test_probe_rejects_bad_arguments_on_the_host():
    from paged_kv_cache_393_amd import probe

    L = probe.load()
    fake = ctypes.c_void_p(0x100000)
    assert L.pa_probe_read(None, 1024, fake, None) == -1
    assert L.pa_probe_read(fake, 1000, fake, None) == -1           # not a multiple of 16
    assert L.pa_probe_read(ctypes.c_void_p(0x100008), 1024, fake, None) == -1
    assert L.pa_probe_copy(fake, None, 1024, None) == -1
    assert L.pa_probe_copy(fake, fake, 0, None) == -1


def test_abi_version_and_strerror():
    assert lib().paged_attn_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert isinstance(B.strerror(code), str) and B.strerror(code)


def shape(**kw):
    base = dict(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                max_blocks_per_seq=16, num_blocks=64, split_tokens=0)
    base.update(kw)
    return B.make_shape(**base)


FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first


def call(sh, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, out=FAKE, ws=None, ws_n=0):
    return lib().paged_attn_decode(q, k, v, bt, cl, ctypes.c_float(0.125), out, ctypes.byref(sh),
                                   ws or ctypes.c_void_p(0), ctypes.c_size_t(ws_n), None)


def call_int8(sh, ks=FAKE, vs=FAKE):
    return lib().paged_attn_decode_int8(FAKE, FAKE, FAKE, ks, vs, FAKE, FAKE,
                                        ctypes.c_float(0.125), FAKE, ctypes.byref(sh),
                                        ctypes.c_void_p(0), ctypes.c_size_t(0), None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=6, num_kv_heads=4), B.PA_ERR_SHAPE),
    (dict(num_q_heads=0), B.PA_ERR_SHAPE),
    (dict(num_kv_heads=0), B.PA_ERR_SHAPE),
    (dict(num_seqs=-1), B.PA_ERR_SHAPE),
    (dict(max_blocks_per_seq=0), B.PA_ERR_SHAPE),
    (dict(num_blocks=0), B.PA_ERR_SHAPE),
    (dict(split_tokens=24), B.PA_ERR_SHAPE),
    (dict(split_tokens=-16), B.PA_ERR_SHAPE),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(head_dim=256), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=8), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=48), B.PA_ERR_UNSUPPORTED),
])
def test_shape_errors(kw, code):
    assert call(shape(**kw)) == code


def call_fp8(sh, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, out=FAKE, ws=None, ws_n=0):
    return lib().paged_attn_decode_fp8(q, k, v, bt, cl, ctypes.c_float(0.125), out,
                                       ctypes.byref(sh), ws or ctypes.c_void_p(0),
                                       ctypes.c_size_t(ws_n), None)


def test_fp8_decode_argument_errors():
    assert call_fp8(shape(num_q_heads=6, num_kv_heads=4)) == B.PA_ERR_SHAPE
    assert call_fp8(shape(head_dim=96)) == B.PA_ERR_UNSUPPORTED
    assert call_fp8(shape(num_seqs=0)) == B.PA_OK
    for name in ("q", "k", "v", "bt", "cl", "out"):
        assert call_fp8(shape(), **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    assert call_fp8(shape(), k=ctypes.c_void_p(0x100008)) == B.PA_ERR_ALIGNMENT
    assert call_fp8(shape()) == B.PA_ERR_WORKSPACE


def test_null_pointers():
    sh = shape()
    for name in ("q", "k", "v", "bt", "cl", "out"):
        assert call(sh, **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    assert call_int8(shape(), ks=ctypes.c_void_p(0)) == B.PA_ERR_NULL
    assert call_int8(shape(), vs=ctypes.c_void_p(0)) == B.PA_ERR_NULL


def test_misaligned_pointers():
    bad = ctypes.c_void_p(0x100008)
    for name in ("q", "k", "v", "out"):
        assert call(shape(), **{name: bad}) == B.PA_ERR_ALIGNMENT, name


def test_workspace_always_required():
    # Partial results of split sequences and their counters live in the workspace.
    for st in (0, 64):
        sh = shape(split_tokens=st)
        need = B.workspace_bytes(sh)
        assert need > 0
        assert call(sh) == B.PA_ERR_WORKSPACE
        assert call(sh, ws=FAKE, ws_n=need - 1) == B.PA_ERR_WORKSPACE


def test_plan_fixed_items():
    sh = shape(split_tokens=64)           # 4 sequences x 16 tiles in items of 4 tiles
    assert B.plan(sh) == (64, 16)
    need = B.workspace_bytes(sh)
    # records: 1 unit group x (S + items) pieces x 4 waves x G heads x (D + 2) floats, + counters
    expect = ((1 * (4 + 16) * 4 * 4 * (64 + 2) * 4 + 255) // 256) * 256 + 256
    assert need == expect, (need, expect)


def test_plan_balanced_is_device_independent():
    sh = shape()
    assert B.plan(sh) == (0, 4096)
    assert B.workspace_bytes(sh) == ((1 * (4 + 4096) * 4 * 4 * 66 * 4 + 255) // 256) * 256 + 256


def test_zero_sequences_is_a_no_op():
    assert call(shape(num_seqs=0)) == B.PA_OK


def test_plan_long_context():
    sh = shape(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
               max_blocks_per_seq=8192, num_blocks=32768, split_tokens=512)
    assert B.plan(sh) == (512, 4 * 131072 // 512)
    pieces = 4 + 1024
    assert B.workspace_bytes(sh) == ((2 * pieces * 4 * 4 * 130 * 4 + 255) // 256) * 256 + 256


# ---- KV write path (include/paged_kv_write.h) ----

def wshape(**kw):
    base = dict(num_tokens=8, num_kv_heads=2, head_dim=128, block_size=16, num_blocks=4,
                key_stride=0, value_stride=0)
    base.update(kw)
    return B.PaWriteShape(*[base[n] for n, _ in B.PaWriteShape._fields_])


def wcall(sh, key=FAKE, value=FAKE, slots=FAKE, kc=FAKE, vc=FAKE):
    return lib().paged_kv_write(key, value, slots, kc, vc, ctypes.byref(sh), None)


def wcall_int8(sh, key=FAKE, value=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE):
    return lib().paged_kv_write_int8(key, value, slots, kc, vc, ks, vs, ctypes.byref(sh), None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_tokens=-1), B.PA_ERR_SHAPE),
    (dict(num_kv_heads=0), B.PA_ERR_SHAPE),
    (dict(block_size=0), B.PA_ERR_SHAPE),
    (dict(num_blocks=0), B.PA_ERR_SHAPE),
    (dict(key_stride=-8), B.PA_ERR_SHAPE),
    (dict(key_stride=128), B.PA_ERR_SHAPE),          # below one token's 2 x 128 row
    (dict(value_stride=200), B.PA_ERR_SHAPE),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(num_tokens=1 << 24, num_kv_heads=8), B.PA_ERR_UNSUPPORTED),
    (dict(key_stride=260), B.PA_ERR_ALIGNMENT),      # not a multiple of 8 elements
])
def test_write_shape_errors(kw, code):
    assert wcall(wshape(**kw)) == code
    assert wcall_int8(wshape(**kw)) == code


def test_write_null_and_alignment():
    sh = wshape()
    assert lib().paged_kv_write(FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == B.PA_ERR_NULL
    for name in ("key", "value", "slots", "kc", "vc"):
        assert wcall(sh, **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
        assert wcall_int8(sh, **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    for name in ("ks", "vs"):
        assert wcall_int8(sh, **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    for name in ("key", "value", "kc", "vc"):
        assert wcall(sh, **{name: ctypes.c_void_p(0x100008)}) == B.PA_ERR_ALIGNMENT, name
    # int8 caches need 8-byte, scales 4-byte alignment
    assert wcall_int8(sh, kc=ctypes.c_void_p(0x100004)) == B.PA_ERR_ALIGNMENT
    assert wcall_int8(sh, vs=ctypes.c_void_p(0x100002)) == B.PA_ERR_ALIGNMENT


def test_fp8_write_argument_errors():
    L = lib()
    sh = wshape()
    assert L.paged_kv_write_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(wshape(head_dim=96)),
                                None) == B.PA_ERR_UNSUPPORTED
    assert L.paged_kv_write_fp8(FAKE, FAKE, ctypes.c_void_p(0), FAKE, FAKE, ctypes.byref(sh),
                                None) == B.PA_ERR_NULL
    assert L.paged_kv_write_fp8(FAKE, FAKE, FAKE, ctypes.c_void_p(0x100004), FAKE,
                                ctypes.byref(sh), None) == B.PA_ERR_ALIGNMENT
    assert L.paged_kv_write_fp8(None, None, None, None, None, ctypes.byref(wshape(num_tokens=0)),
                                None) == B.PA_OK


def test_write_zero_tokens_is_a_no_op():
    assert wcall(wshape(num_tokens=0)) == B.PA_OK
    assert wcall_int8(wshape(num_tokens=0)) == B.PA_OK


# ---- PagedEviction (include/paged_kv_evict.h) ----

def sshape(**kw):
    base = dict(num_seqs=2, num_kv_heads=2, head_dim=128, block_size=16, max_blocks_per_seq=8,
                num_blocks=16)
    base.update(kw)
    return B.PaScoreShape(*[base[n] for n, _ in B.PaScoreShape._fields_])


def scall(sh, k=FAKE, v=FAKE, bt=FAKE, tb=None, cl=FAKE, sc=FAKE):
    return lib().paged_kv_token_scores(k, v, bt, tb, cl, sc, ctypes.byref(sh), None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_seqs=-1), B.PA_ERR_SHAPE),
    (dict(num_kv_heads=0), B.PA_ERR_SHAPE),
    (dict(block_size=0), B.PA_ERR_SHAPE),
    (dict(max_blocks_per_seq=0), B.PA_ERR_SHAPE),
    (dict(num_blocks=0), B.PA_ERR_SHAPE),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=8192), B.PA_ERR_UNSUPPORTED),
    (dict(num_seqs=70000), B.PA_ERR_UNSUPPORTED),
])
def test_score_shape_errors(kw, code):
    assert scall(sshape(**kw)) == code
    L = lib()
    assert L.paged_kv_evict_lowest_block(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sshape(**kw)),
                                         None) == code


def test_score_and_evict_null_alignment_and_empty():
    L = lib()
    for name in ("k", "v", "bt", "cl", "sc"):
        assert scall(sshape(), **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    assert scall(sshape(), k=ctypes.c_void_p(0x100008)) == B.PA_ERR_ALIGNMENT
    assert scall(sshape(), sc=ctypes.c_void_p(0x100002)) == B.PA_ERR_ALIGNMENT
    assert L.paged_kv_token_scores_int8(FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE,
                                        ctypes.byref(sshape()), None) == B.PA_ERR_NULL
    assert L.paged_kv_token_scores_fp8(FAKE, ctypes.c_void_p(0x100004), FAKE, None, FAKE, FAKE,
                                       ctypes.byref(sshape()), None) == B.PA_ERR_ALIGNMENT
    assert scall(sshape(num_seqs=0), k=None, v=None, bt=None, cl=None, sc=None) == B.PA_OK
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        assert L.paged_kv_evict_lowest_block(*args, ctypes.byref(sshape()), None) == B.PA_ERR_NULL
    assert L.paged_kv_evict_lowest_block(None, None, None, None, None,
                                         ctypes.byref(sshape(num_seqs=0)), None) == B.PA_OK


def test_check_tables_host_errors():
    L = lib()
    assert L.paged_attn_check_tables(FAKE, FAKE, -1, 4, 16, 8, FAKE, None) == B.PA_ERR_SHAPE
    assert L.paged_attn_check_tables(FAKE, FAKE, 2, 0, 16, 8, FAKE, None) == B.PA_ERR_SHAPE
    assert L.paged_attn_check_tables(FAKE, FAKE, 2, 4, 0, 8, FAKE, None) == B.PA_ERR_SHAPE
    assert L.paged_attn_check_tables(FAKE, FAKE, 2, 4, 16, 0, FAKE, None) == B.PA_ERR_SHAPE
    assert L.paged_attn_check_tables(FAKE, FAKE, 2, 4, 16, 8, None, None) == B.PA_ERR_NULL
    assert L.paged_attn_check_tables(None, FAKE, 2, 4, 16, 8, FAKE, None) == B.PA_ERR_NULL
    assert L.paged_attn_check_tables(FAKE, None, 2, 4, 16, 8, FAKE, None) == B.PA_ERR_NULL


# ---- prefill-phase compression (include/paged_kv_evict.h) ----

def ccall(sh, budget=8, k=FAKE, v=FAKE, sc=FAKE, bt=FAKE, cl=FAKE, ws=FAKE, wsb=1 << 20):
    return lib().paged_kv_compress_prefill(k, v, sc, bt, cl, budget, ctypes.byref(sh), ws, wsb, None)


def test_compress_workspace_size():
    L = lib()
    assert L.paged_kv_compress_workspace_bytes(ctypes.byref(sshape(num_seqs=3)), 100) == 1280 + 256
    assert L.paged_kv_compress_workspace_bytes(ctypes.byref(sshape(num_seqs=3)), 0) == 256
    assert L.paged_kv_compress_workspace_bytes(ctypes.byref(sshape()), -1) == 0
    # contexts longer than the LDS key buffer (12288) split the selection into
    # 4096-token chunks (4 here): a key row per sequence, first-digit histograms
    # per chunk, two digit histograms per sequence, three states per sequence
    # and last-digit counts per chunk, each part rounded up to 256 bytes
    long = sshape(num_seqs=2, max_blocks_per_seq=1000, block_size=16)
    r = lambda b: (b + 255) // 256 * 256
    split = r(2 * 16000 * 4) + r(2 * 4 * 256 * 4) + r(2 * 512 * 4) + r(3 * 2 * 2 * 4) + r(2 * 4 * 257 * 4)
    assert L.paged_kv_compress_workspace_bytes(ctypes.byref(long), 100) == 1024 + 256 + split


@pytest.mark.parametrize("kw,code", [
    (dict(num_seqs=-1), B.PA_ERR_SHAPE),
    (dict(num_kv_heads=0), B.PA_ERR_SHAPE),
    (dict(block_size=0), B.PA_ERR_SHAPE),
    (dict(max_blocks_per_seq=0), B.PA_ERR_SHAPE),
    (dict(num_blocks=0), B.PA_ERR_SHAPE),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=8192), B.PA_ERR_UNSUPPORTED),
    (dict(num_seqs=70000), B.PA_ERR_UNSUPPORTED),
])
def test_compress_shape_errors(kw, code):
    assert ccall(sshape(**kw)) == code


def test_compress_host_checks():
    L = lib()
    assert ccall(sshape(), budget=-1) == B.PA_ERR_SHAPE
    for name in ("k", "v", "sc", "bt", "cl"):
        assert ccall(sshape(), **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    assert ccall(sshape(), ws=None) == B.PA_ERR_WORKSPACE
    assert ccall(sshape(), wsb=16) == B.PA_ERR_WORKSPACE
    assert ccall(sshape(), k=ctypes.c_void_p(0x100008)) == B.PA_ERR_ALIGNMENT
    assert ccall(sshape(), ws=ctypes.c_void_p(0x100004)) == B.PA_ERR_ALIGNMENT
    assert ccall(sshape(num_seqs=0), k=None, v=None, sc=None, bt=None, cl=None, ws=None) == B.PA_OK
    assert L.paged_kv_compress_prefill_int8(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 8,
                                            ctypes.byref(sshape()), FAKE, 1 << 20, None) == B.PA_ERR_NULL
    assert L.paged_kv_compress_prefill_fp8(FAKE, ctypes.c_void_p(0x100004), FAKE, FAKE, FAKE, 8,
                                           ctypes.byref(sshape()), FAKE, 1 << 20, None) == B.PA_ERR_ALIGNMENT


# ---- chunked prefill (include/paged_prefill.h) ----

def pshape(**kw):
    base = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                max_blocks_per_seq=8, num_blocks=16, max_q_len=64)
    base.update(kw)
    return B.PaPrefillShape(*[base[n] for n, _ in B.PaPrefillShape._fields_])


def pcall(sh, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, qo=FAKE, out=FAKE):
    return lib().paged_attn_prefill(q, k, v, bt, cl, qo, ctypes.c_float(0.1), out,
                                    ctypes.byref(sh), None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_seqs=-1), B.PA_ERR_SHAPE),
    (dict(num_q_heads=6, num_kv_heads=4), B.PA_ERR_SHAPE),
    (dict(max_q_len=0), B.PA_ERR_SHAPE),
    (dict(num_blocks=0), B.PA_ERR_SHAPE),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=8), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=48), B.PA_ERR_UNSUPPORTED),
])
def test_prefill_shape_errors(kw, code):
    assert pcall(pshape(**kw)) == code


def test_prefill_null_alignment_and_empty():
    for name in ("q", "k", "v", "bt", "cl", "qo", "out"):
        assert pcall(pshape(), **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    for name in ("q", "k", "v", "out"):
        assert pcall(pshape(), **{name: ctypes.c_void_p(0x100008)}) == B.PA_ERR_ALIGNMENT, name
    assert pcall(pshape(num_seqs=0), q=None, k=None) == B.PA_OK


def pcall_q(kind, sh, q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, cl=FAKE, qo=FAKE, out=FAKE):
    if kind == "int8":
        return lib().paged_attn_prefill_int8(q, k, v, ks, vs, bt, cl, qo, ctypes.c_float(0.1), out,
                                             ctypes.byref(sh), None)
    return lib().paged_attn_prefill_fp8(q, k, v, bt, cl, qo, ctypes.c_float(0.1), out,
                                        ctypes.byref(sh), None)


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantized_prefill_host_checks(kind):
    assert pcall_q(kind, pshape(head_dim=96)) == B.PA_ERR_UNSUPPORTED
    assert pcall_q(kind, pshape(num_q_heads=6, num_kv_heads=4)) == B.PA_ERR_SHAPE
    names = ("q", "k", "v", "bt", "cl", "qo", "out") + (("ks", "vs") if kind == "int8" else ())
    for name in names:
        assert pcall_q(kind, pshape(), **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    # the codes need 8-byte alignment only; q and out 16 bytes; int8 scales 4 bytes
    assert pcall_q(kind, pshape(), k=ctypes.c_void_p(0x100004)) == B.PA_ERR_ALIGNMENT
    assert pcall_q(kind, pshape(), q=ctypes.c_void_p(0x100008)) == B.PA_ERR_ALIGNMENT
    if kind == "int8":
        assert pcall_q(kind, pshape(), vs=ctypes.c_void_p(0x100002)) == B.PA_ERR_ALIGNMENT
    assert pcall_q(kind, pshape(num_seqs=0), q=None, k=None) == B.PA_OK


def test_prefill_workspace_size():
    # 2 sequences x 2 kv heads x ceil(64 * 4 / 256) = 1 row tile x K pieces x 256 rows x (D + 2) floats
    for k in (2, 3, 64):
        assert lib().paged_attn_prefill_workspace_bytes(ctypes.byref(pshape()), k) == 2 * 2 * 1 * k * 256 * 130 * 4
    # max_q_len 65 needs a second row tile; head_dim 64
    assert (lib().paged_attn_prefill_workspace_bytes(ctypes.byref(pshape(max_q_len=65, head_dim=64)), 4)
            == 2 * 2 * 2 * 4 * 256 * 66 * 4)
    assert lib().paged_attn_prefill_workspace_bytes(ctypes.byref(pshape()), 1) == 0
    for k in (0, -1, 65):
        assert lib().paged_attn_prefill_workspace_bytes(ctypes.byref(pshape()), k) == 0
    assert lib().paged_attn_prefill_workspace_bytes(ctypes.byref(pshape(head_dim=96)), 2) == 0
    assert lib().paged_attn_prefill_workspace_bytes(None, 2) == 0


def test_prefill_plan_host_checks():
    k = ctypes.c_int32(-5)
    assert lib().paged_attn_prefill_plan(ctypes.byref(pshape()), None) == B.PA_ERR_NULL
    assert lib().paged_attn_prefill_plan(None, ctypes.byref(k)) == B.PA_ERR_NULL
    assert lib().paged_attn_prefill_plan(ctypes.byref(pshape(head_dim=96)), ctypes.byref(k)) == B.PA_ERR_UNSUPPORTED
    assert lib().paged_attn_prefill_plan(ctypes.byref(pshape(max_q_len=0)), ctypes.byref(k)) == B.PA_ERR_SHAPE
    # no sequences: no device query, one piece
    assert lib().paged_attn_prefill_plan(ctypes.byref(pshape(num_seqs=0)), ctypes.byref(k)) == B.PA_OK
    assert k.value == 1


def pcall_split(kind, sh, key_splits, ws=FAKE, wsb=1 << 30, q=FAKE, k=FAKE, out=FAKE):
    L = lib()
    tail = (ctypes.c_float(0.1), out, ctypes.byref(sh), key_splits, ws, wsb, None)
    if kind == "int8":
        return L.paged_attn_prefill_split_int8(q, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, *tail)
    fn = L.paged_attn_prefill_split_fp8 if kind == "fp8" else L.paged_attn_prefill_split
    return fn(q, k, FAKE, FAKE, FAKE, FAKE, *tail)


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_split_prefill_host_checks(kind):
    need = lib().paged_attn_prefill_workspace_bytes(ctypes.byref(pshape()), 4)
    for k in (0, -3, 65):
        assert pcall_split(kind, pshape(), k) == B.PA_ERR_SHAPE, k
    assert pcall_split(kind, pshape(), 4, ws=None) == B.PA_ERR_WORKSPACE
    assert pcall_split(kind, pshape(), 4, wsb=need - 1) == B.PA_ERR_WORKSPACE
    assert pcall_split(kind, pshape(), 4, ws=ctypes.c_void_p(0x100008), wsb=need) == B.PA_ERR_ALIGNMENT
    assert pcall_split(kind, pshape(), 4, q=None) == B.PA_ERR_NULL
    assert pcall_split(kind, pshape(), 4, out=ctypes.c_void_p(0x100008)) == B.PA_ERR_ALIGNMENT
    assert pcall_split(kind, pshape(head_dim=96), 4) == B.PA_ERR_UNSUPPORTED
    # the shape is checked before key_splits; no sequences is a no-op either way
    assert pcall_split(kind, pshape(num_seqs=0), 4, ws=None, q=None, k=None) == B.PA_OK


def call_noalloc(sh, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, out=FAKE):
    return lib().paged_attn_decode_noalloc(q, k, v, bt, cl, ctypes.c_float(0.125), out,
                                           ctypes.byref(sh), None)


def test_noalloc_decode_host_checks():
    # Shape, NULL and alignment errors as for paged_attn_decode; zero sequences
    # is a no-op; a shape whose fixed items need more than the 32 MiB static
    # scratch is rejected before any device call.
    assert call_noalloc(shape(num_q_heads=6, num_kv_heads=4)) == B.PA_ERR_SHAPE
    assert call_noalloc(shape(head_dim=96)) == B.PA_ERR_UNSUPPORTED
    for name in ("q", "k", "v", "bt", "cl", "out"):
        assert call_noalloc(shape(), **{name: ctypes.c_void_p(0)}) == B.PA_ERR_NULL, name
    assert call_noalloc(shape(), q=ctypes.c_void_p(0x100008)) == B.PA_ERR_ALIGNMENT
    assert call_noalloc(shape(num_seqs=0)) == B.PA_OK
    # 4096 sequences of up to 1024 tokens in 16-token items: 262144 items of
    # 4 records of 2 heads x 66 floats, far beyond 32 MiB.
    big = shape(num_seqs=4096, max_blocks_per_seq=64, split_tokens=16)
    assert call_noalloc(big) == B.PA_ERR_SCRATCH
    assert "32 MiB" in B.strerror(B.PA_ERR_SCRATCH)
