"""One decode step composed from the three entry points, on small shapes: the cache write of
the new tokens' latent rows (INT8), the indexer's scores and top-k, and the sparse attention
over the selected rows of the written cache. It is checked against the composed oracles: the
written cache bit for bit, the selection as an exact top-k of the kernel's scores, and the
attention output at the accuracy standard."""

import numpy as np
import pytest

import oracle.cache_oracle as CO
import oracle.indexer_oracle as IO
import oracle.sfa_oracle as O
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_cache_write_indexer_attention_step(sfa_lib):
    import torch

    sfa = sfa_lib
    acts = [1500, 700, 2300]
    att = W.generate(batch=3, s1=2, n_q=64, act_seqs=acts, topk=256, kv_dtype="int8", seed=61,
                     max_blocks_per_batch=20)
    idx_inp = W.indexer_generate(batch=3, s1=2, act_seqs=acts, topk=256, seed=61, max_blocks_per_batch=20)
    pos = np.array([[a - 2, a - 1] for a in acts], dtype=np.int32).reshape(-1)
    new = W.cache_write_generate(batch=3, s1=2, n_pool_blocks=1, max_blocks_per_batch=20, kv_dtype="int8", seed=62,
                                 positions=pos, block_table=att.block_table)
    d = sfa.to_device(att)
    nw = sfa.cache_to_device(new)
    # 1. the new rows into the latent cache
    sfa.cache_write(nw["new_nope"], nw["new_rope"], nw["positions"], d["block_table"], d["key_nope"], d["key_rope"],
                    d["k_nope_scales"], batch=3, s1=2)
    # 2. the indexer's top-k
    xd = sfa.indexer_to_device(idx_inp)
    sc, sel = sfa.run_indexer(idx_inp, xd)
    # 3. the attention over the selected rows
    out = sfa.decode(d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"], sel,
                     d["block_table"], d["kv_act_seqs"], att.softmax_scale, batch=3, s1=2)
    torch.cuda.synchronize()

    kn, kr, ks = CO.cache_write(new.new_nope, new.new_rope, new.positions, new.block_table, 2, att.key_nope,
                                att.key_rope, att.k_nope_scales)
    assert np.array_equal(d["key_nope"].cpu().numpy(), kn)
    assert np.array_equal(d["k_nope_scales"].cpu().numpy().view(np.uint32), ks.view(np.uint32))
    sel_np = sel.cpu().numpy()
    assert IO.check_topk(sel_np, sc.cpu().numpy().astype(np.float64), 256)["bad"] == []
    chosen = W.SfaInputs(**{**att.__dict__, "topk_indices": sel_np, "key_nope": kn, "key_rope": kr,
                            "k_nope_scales": ks})
    ref = O.sparse_mla_attention(chosen).reshape(att.n_tokens, att.n_q, 512)
    got = out.float().cpu().numpy().astype(np.float64).reshape(att.n_tokens, att.n_q, 512)
    rep = O.allclose_report(got, ref)
    assert rep["fails"] == 0, rep
