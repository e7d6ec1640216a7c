"""sfa_decode_noalloc (the library's fixed per-GPU scratch as workspace) gives the same output as
sfa_decode with a caller workspace, on two calls in a row, the second with a smaller input."""

import pytest

from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _args(inp, d):
    return (d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"], d["topk_indices"],
            d["block_table"], d["kv_act_seqs"], inp.softmax_scale)


def test_noalloc_matches_decode_on_two_calls(sfa_lib):
    import torch

    big = W.generate(batch=8, s1=2, n_q=128, act_seqs=[8192, 5000, 3000, 8000, 2048, 7000, 6500, 4096], topk=2048,
                     seed=31)
    small = W.generate(batch=2, s1=1, n_q=64, act_seqs=[1900, 300], topk=1024, kv_dtype="int8", seed=32)
    for inp in (big, small):
        d = sfa_lib.to_device(inp)
        dims_need = sfa_lib.workspace_size(sfa_lib.make_dims(
            batch=inp.batch, s1=inp.s1, n_q=inp.n_q, topk=inp.topk, max_blocks_per_batch=d["block_table"].shape[1],
            num_cache_rows=d["key_rope"].shape[0], kv_dtype=sfa_lib.KV_INT8 if inp.kv_dtype == "int8" else 0))
        assert 0 < dims_need <= sfa_lib.NOALLOC_SCRATCH_BYTES
        ref = sfa_lib.decode(*_args(inp, d), batch=inp.batch, s1=inp.s1).clone()
        out = torch.full_like(ref, float("nan"))
        got = sfa_lib.decode_noalloc(*_args(inp, d), batch=inp.batch, s1=inp.s1, out=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), inp.kv_dtype
