"""GPU test of paged_attn_check_tables: the device-side check of the caller
contract (context lengths within the table row, used table entries within the
pool).  The check reads only tables and lengths, so contract-breaking inputs
are safe to give it.  Expected counts are known by construction, and the
oracle, which validates the same contract, rejects exactly the broken
inputs."""
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


def test_valid_workloads_pass():
    for name in ("tiny", "llama3_8b", "long_context"):
        wl = I.WORKLOADS[name]
        note(f"check tables {name}")
        v = I.layer_views(I.make_inputs(wl, DEV), 0)
        NB = v["k_cache"].shape[0]
        assert B.check_tables(v["block_tables"], v["context_lens"], NB, wl.block_size) == (0, -1)


def test_planted_violations_are_counted_and_the_first_is_named():
    ctx = (40, 17, 100, 64, 33, 80, 5, 48, 16, 90, 1, 0)
    bs = 16
    note(f"check tables planted violations ctx={ctx}")
    _, v = C.make_case(len(ctx), 8, 2, 64, bs, ctx=ctx, seed=90, device=DEV)
    NB, MB = v["k_cache"].shape[0], v["block_tables"].shape[1]
    bt = v["block_tables"].clone()
    cl = v["context_lens"].clone()
    # entries past a context's last block are not checked: garbage there is fine
    bt[0, 3:] = -7
    assert B.check_tables(bt, cl, NB, bs) == (0, -1)
    bt[3, 2] = -1            # used entry below zero
    bt[5, 4] = NB            # used entry past the pool
    cl[7] = MB * bs + 1      # context longer than the row can address
    cl[9] = -5               # negative context
    assert B.check_tables(bt, cl, NB, bs) == (4, 3)
    # the oracle rejects each broken sequence on its own, and accepts the rest
    q, k, vv = I.bf16_bits(v["q"]), I.bf16_bits(v["k_cache"]), I.bf16_bits(v["v_cache"])
    bt_h, cl_h = bt.cpu().numpy(), cl.cpu().numpy()
    for s in range(len(ctx)):
        one = lambda: oracle.paged_decode_bf16(q[s:s + 1], k, vv, bt_h[s:s + 1], cl_h[s:s + 1],
                                               v["scale"])
        if s in (3, 5, 7, 9):
            with pytest.raises(ValueError):
                one()
        else:
            one()


def test_no_sequences():
    bt = torch.zeros((1, 4), dtype=torch.int32, device=DEV)[:0]
    cl = torch.zeros(0, dtype=torch.int32, device=DEV)
    assert B.check_tables(bt, cl, 8, 16) == (0, -1)
