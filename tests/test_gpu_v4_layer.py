"""One decode step of a DeepSeek-V4 attention layer on 512-wide rows, end to end on the GPU. SCFA
layer: the V4 MLA prolog, the cache write of the new latent rows, the compressor (512 channels)
and the index-key compressor (128 channels, Hadamard), the indexer prolog on the prolog's cq, the
Lightning Indexer over the compressed index keys with its top-k, and SCFA over the original and
compressed caches. CFA layer: the prolog, the cache write, the compressor at ratio 128, CFA over
every causal compressed entry. SWA layer: the prolog, the cache write, SWA
("NPU DeepSeek-V4 model PyPTO fused-operator optimisation": MlaProlog, Compressor, IndexerProlog,
FA-class operators; "CANN DeepSeek Indexer attention optimisation": Lightning Indexer).

Every step is checked against its oracle on the GPU's own inputs to that step (the outputs of
the steps before it), so each comparison tests one kernel: the bf16 outputs to the attention's
bar (|gpu - ref| <= 1e-4 + 5e-3 |ref|), copies and states bit for bit, the index scores to the
indexer's fp32 accumulation bound, the selection as an exact top-k of the GPU's scores."""

import numpy as np
import pytest

import oracle.compress_oracle as C
import oracle.indexer_oracle as IO
import oracle.prolog_oracle as P
import oracle.sfa_oracle as O
import oracle.window_oracle as WO
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch

    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _close(name, got, want):
    err = np.abs(got - want)
    bound = 1e-4 + 5e-3 * np.abs(want)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{name}: {len(bad)} off, first {bad[:3].tolist()}, worst {np.max(err / bound):.3f}"


def run_layer(sfa, L):
    """The step's launches on the current stream; returns the device tensors of every stage."""
    import torch

    B, S1 = L.window.batch, L.window.s1
    T, K = B * S1, L.topk_cmp
    r = {}
    pro_d = sfa.prolog_v4_to_device(L.prolog)
    win_d = sfa.window_to_device(L.window)
    pos = torch.from_numpy(L.positions).cuda()
    cq = torch.empty((T, L.prolog.q_lora_rank), dtype=torch.bfloat16, device="cuda")
    q, kv = sfa.run_prolog_v4(L.prolog, pro_d, cq_out=cq)
    sfa.cache_write(kv, None, pos, win_d["block_table_ori"], win_d["key_nope"], None, None, batch=B, s1=S1)
    if L.compress_att is not None:
        catt_d = sfa.compress_to_device(L.compress_att)
        catt_d["key_nope"] = win_d["key_nope"]          # the compressed entries share the window's pool
        sfa.run_compress(L.compress_att, catt_d)
        r["catt"] = catt_d
    if L.kind == "scfa":
        cidx_d = sfa.compress_to_device(L.compress_idx)  # the index-key pool
        sfa.run_compress(L.compress_idx, cidx_d)
        ip_d = sfa.indexer_prolog_to_device(L.indexer_prolog)
        ip_d["qr"] = cq
        q_index, _k, w = sfa.run_indexer_prolog(L.indexer_prolog, ip_d)
        scores = sfa.indexer_scores(q_index, cidx_d["key_nope"], w, win_d["block_table_cmp"], win_d["cmp_len"],
                                    batch=B, s1=S1, topk=K)
        sel = sfa.topk_select(scores, win_d["cmp_len"], batch=B, s1=S1, topk=K)
        win_d["cmp_indices"] = sel
        r.update(cidx=cidx_d, q_index=q_index, w=w, scores=scores, sel=sel)
    win_d["query_nope"] = q
    out = sfa.run_window(L.window, win_d)
    torch.cuda.synchronize()
    r.update(q=q, kv=kv, cq=cq, pool=win_d["key_nope"], out=out)
    return r


@pytest.mark.parametrize("kind,seed", [("scfa", 0), ("scfa", 1), ("cfa", 0), ("swa", 0)])
def test_v4_layer_step(sfa_lib, kind, seed):
    # lengths that are multiples of 128: every sequence's second token closes a window at ratio
    # 128 as well as at ratio 4
    L = W.v4_layer_generate(kind=kind, batch=3, s1=2, n_q=16, hidden=256, q_lora_rank=256,
                            ori_lens=[640, 384, 256], window=64, topk_cmp=24 if kind == "scfa" else 0, seed=seed)
    r = run_layer(sfa_lib, L)
    pro, win = L.prolog, L.window
    T = pro.tokens

    # 1. the V4 prolog
    q_ref, kv_ref = P.mla_prolog_v4(pro.x, pro.w_dq, pro.gamma_cq, pro.w_uq, pro.w_dkv, pro.gamma_ckv,
                                    pro.positions, pro.rope_cos, pro.rope_sin, pro.eps, pro.n_q)
    q_bits, kv_bits = _bits(r["q"]), _bits(r["kv"])
    _close("q", P.bf16_bits_to_f64(q_bits).reshape(q_ref.shape), q_ref)
    _close("kv", P.bf16_bits_to_f64(kv_bits), kv_ref)

    # 2. the cache write: the new rows at the tokens' positions, bit for bit
    pool = _bits(r["pool"])
    rows = [int(win.block_table_ori[t // 2, p // 128]) * 128 + p % 128 for t, p in enumerate(pro.positions)]
    assert np.array_equal(pool[rows], kv_bits)

    # 3-4. the compressors: states bit for bit, every written row to the bar (each sequence's
    # second token closes a window)
    comps = [] if kind == "swa" else [("compress_att", L.compress_att, r["catt"])]
    if kind == "scfa":
        comps.append(("compress_idx", L.compress_idx, r["cidx"]))
    for name, inp, d in comps:
        ks, ss, entries = C.compress(inp)
        np.testing.assert_array_equal(d["kv_state"].cpu().numpy().view(np.uint32), ks.view(np.uint32))
        np.testing.assert_array_equal(d["score_state"].cpu().numpy().view(np.uint32), ss.view(np.uint32))
        got = _bits(d["key_nope"])
        assert len(entries) == win.batch
        for b, c, row, y in entries:
            assert row >= 0 and c == int(win.cmp_len[b]) - 1, name
            _close(f"{name} row {row}", P.bf16_bits_to_f64(got[row]), y)

    if kind != "scfa":
        # 7. SWA / CFA over the GPU's pool and queries (CFA: every causal entry, the newest one
        # just written by the compressor)
        win.query_nope, win.key_nope = q_bits, pool
        out_ref = WO.window_attention(win)
        rep = O.allclose_report(r["out"].float().cpu().numpy().astype(np.float64).reshape(out_ref.shape), out_ref)
        assert rep["fails"] == 0, rep
        return

    # 5. the indexer prolog on the GPU's cq
    ip = L.indexer_prolog
    qi_ref, _, w_ref = P.indexer_prolog(ip.x, _bits(r["cq"]), ip.w_idx_qb, ip.w_idx_k, ip.ln_gamma_k, ip.ln_beta_k,
                                        ip.w_idx_proj, ip.positions, ip.rope_cos, ip.rope_sin, ip.eps, ip.n_heads,
                                        ip.rotate)
    qi_bits = _bits(r["q_index"])
    _close("q_index", P.bf16_bits_to_f64(qi_bits).reshape(qi_ref.shape), qi_ref)
    w_gpu = r["w"].cpu().numpy()
    _close("weights", w_gpu.astype(np.float64), w_ref)

    # 6. index scores over the compressed index keys (the GPU's pool), and an exact top-k of them
    kpool = _bits(r["cidx"]["key_nope"])
    n_pos = win.block_table_cmp.shape[1] * 128
    ref = IO.indexer_scores(qi_bits.reshape(T, 64, 128), w_gpu, kpool, win.block_table_cmp, win.cmp_len, 2, n_pos)
    got = r["scores"].cpu().numpy().astype(np.float64)
    live = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), live)
    qa = np.abs(IO.bf16_bits_to_f64(qi_bits.reshape(T, 64, 128)))
    ka = np.abs(IO.bf16_bits_to_f64(kpool))
    mag = np.zeros_like(ref)
    for t in range(T):
        act = int(win.cmp_len[t // 2])
        mag[t, :act] = np.abs(w_gpu[t].astype(np.float64)) @ (qa[t] @ ka[IO.live_rows(win.block_table_cmp, act,
                                                                                       t // 2)].T)
    assert np.all(np.abs(got[live] - ref[live]) <= 2.0 ** -15 * mag[live] + 1e-30)
    sel = r["sel"].cpu().numpy()
    assert IO.check_topk(sel, r["scores"].cpu().numpy(), L.topk_cmp)["bad"] == []

    # 7. SCFA over the GPU's pools, queries and compressed list
    win.query_nope, win.key_nope, win.cmp_indices = q_bits, pool, sel
    out_ref = WO.window_attention(win)
    rep = O.allclose_report(r["out"].float().cpu().numpy().astype(np.float64).reshape(out_ref.shape), out_ref)
    assert rep["fails"] == 0, rep
