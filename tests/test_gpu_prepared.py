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


def test_concurrent_decodes_on_two_streams(sfa_lib):
    """Decodes queued on two streams at once, each with the binding's cached workspace, give the
    same bits as the same calls run one after the other: the streams never share a workspace."""
    import torch

    inps = [W.generate(batch=4, s1=2, n_q=128, act_seqs=[6000, 4100, 3000, 5000], topk=2048, seed=s)
            for s in (21, 22)]
    devs = [sfa_lib.to_device(i) for i in inps]
    refs = [sfa_lib.run(i, d, num_splits=4).clone() for i, d in zip(inps, devs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in refs]
    for _ in range(4):
        for o in outs:
            o.fill_(0)
        # both streams wait for the fills, then run with no ordering between them
        ev = torch.cuda.Event()
        ev.record()
        for st, i, d, o in zip(streams, inps, devs, outs):
            st.wait_event(ev)
            for _rep in range(3):
                sfa_lib.decode(d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"],
                               d["topk_indices"], d["block_table"], d["kv_act_seqs"], i.softmax_scale,
                               batch=i.batch, s1=i.s1, num_splits=4, out=o, stream=st)
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16))
    keys = [k for k in sfa_lib._WORKSPACES if k[2] in (streams[0].cuda_stream, streams[1].cuda_stream)]
    assert len(keys) == 2


def test_workspace_contents_do_not_matter(sfa_lib):
    """The merge counters in the workspace carry each call's own generation: a workspace full of
    arbitrary bytes (or of an earlier call with other shapes) gives the same bits as a fresh one."""
    import torch

    inp = W.generate(batch=5, s1=2, n_q=128, act_seqs=[6000, 300, 4100, 2048, 8000], topk=2048, seed=41)
    d = sfa_lib.to_device(inp)
    args = (d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], d["k_nope_scales"], d["topk_indices"],
            d["block_table"], d["kv_act_seqs"], inp.softmax_scale)
    need = sfa_lib.workspace_size(sfa_lib.make_dims(batch=5, s1=2, n_q=128, topk=2048,
                                                    max_blocks_per_batch=d["block_table"].shape[1],
                                                    num_cache_rows=d["key_rope"].shape[0], num_splits=4))
    ref = sfa_lib.decode(*args, batch=5, s1=2, num_splits=4,
                         workspace=torch.zeros(need, dtype=torch.uint8, device="cuda")).clone()
    g = torch.Generator(device="cuda").manual_seed(5)
    for fill in ("ones", "random", "reuse"):
        ws = torch.empty(need + 4096, dtype=torch.uint8, device="cuda")
        if fill == "ones":
            ws.fill_(255)
        elif fill == "random":
            ws.random_(0, 256, generator=g)
        else:
            # an earlier call with other shapes and partition count leaves its partials here
            small = W.generate(batch=2, s1=1, n_q=64, act_seqs=[900, 4000], topk=1024, seed=42)
            ds = sfa_lib.to_device(small)
            sfa_lib.decode(ds["query_nope"], ds["query_rope"], ds["key_nope"], ds["key_rope"], None,
                           ds["topk_indices"], ds["block_table"], ds["kv_act_seqs"], small.softmax_scale, batch=2,
                           s1=1, num_splits=8, workspace=ws)
        for _ in range(2):
            out = sfa_lib.decode(*args, batch=5, s1=2, num_splits=4, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), fill
