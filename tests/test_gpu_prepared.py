"""Prepared calls (sfa.prepare_*) give the same bits as the plain binding calls, call after call,
and keep following the bound tensors' contents."""

import numpy as np
import pytest

from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_prepared_decode_matches_plain_call(sfa_lib):
    import torch

    inp = W.generate(batch=3, s1=2, n_q=64, act_seqs=[700, 129, 2000], topk=256, seed=11)
    d = sfa_lib.to_device(inp)
    ref = sfa_lib.run(inp, d).clone()
    call = sfa_lib.prepare_run(inp, d)
    for _ in range(3):
        out = call()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # new contents in the same storage are picked up
    d["query_nope"].neg_()
    ref2 = sfa_lib.run(inp, d).clone()
    out = call()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref2.view(torch.int16))
    assert not torch.equal(ref2.view(torch.int16), ref.view(torch.int16))


def test_prepared_indexer_matches_plain_calls(sfa_lib):
    import torch

    inp = W.indexer_generate(batch=2, s1=2, act_seqs=[1000, 300], topk=128, seed=3)
    d = sfa_lib.indexer_to_device(inp)
    sc, idx = sfa_lib.run_indexer(inp, d)
    call = sfa_lib.prepare_indexer(d["q_index"], d["k_index"], d["weights"], d["block_table"], d["kv_act_seqs"],
                                   batch=inp.batch, s1=inp.s1, topk=inp.topk)
    got = call()
    torch.cuda.synchronize()
    assert torch.equal(got, idx)


def test_prepared_cache_write_matches_plain_call(sfa_lib):
    import torch

    inp = W.cache_write_generate(batch=2, s1=40, n_pool_blocks=8, max_blocks_per_batch=4, kv_dtype="int8", seed=2)
    a, b = sfa_lib.cache_to_device(inp), sfa_lib.cache_to_device(inp)
    sfa_lib.run_cache_write(inp, a)
    call = sfa_lib.prepare_cache_write(b["new_nope"], b["new_rope"], b["positions"], b["block_table"], b["key_nope"],
                                       b["key_rope"], b["k_nope_scales"], batch=inp.batch, s1=inp.s1)
    call()
    torch.cuda.synchronize()
    assert torch.equal(a["key_nope"], b["key_nope"])
    assert np.array_equal(a["key_rope"].view(torch.int16).cpu().numpy(), b["key_rope"].view(torch.int16).cpu().numpy())
    assert np.array_equal(a["k_nope_scales"].cpu().numpy().view(np.uint32), b["k_nope_scales"].cpu().numpy().view(np.uint32))
