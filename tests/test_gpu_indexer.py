"""GPU parity for the Lightning Indexer and the top-k selection (through the C ABI).

* Scores against the fp64 oracle. Bound per element: 2^-15 * sum_h |w_h| * sum_d |q_hd k_d|.
  That is four times a first-order bound on fp32 accumulation of 128 exact bf16 products and a
  64-term weighted sum.
* The selection is a decision taken on floating-point scores, so it is checked in the
  kernel's own precision: on the GPU's fp32 scores it must be an exact top-k (distinct live
  positions, min(k, live) of them, nothing unselected above the lowest selected, ties at the
  lowest positions). Against the fp64 scores, it may differ only within the score bound
  around the k-th value.
* End to end: indexer -> top-k -> sfa_decode equals the attention oracle run on the selected
  positions.
"""

import numpy as np
import pytest
import torch

import oracle.indexer_oracle as IO
import oracle.sfa_oracle as O
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")


def _lib():
    from mla_sparse_top_amd import sfa
    return sfa


def _oracle(inp):
    T, H, D = inp.n_tokens, inp.n_heads, inp.head_dim
    q = inp.q_index.reshape(T, H, D)
    ref = IO.indexer_scores(q, inp.weights, inp.k_index, inp.block_table, inp.kv_act_seqs, inp.s1, inp.n_positions)
    # sum_h |w_h| sum_d |q_hd k_jd| for the bound
    qa = np.abs(IO.bf16_bits_to_f64(q))
    ka = np.abs(IO.bf16_bits_to_f64(inp.k_index))
    wa = np.abs(inp.weights.astype(np.float64))
    mag = np.zeros_like(ref)
    for t in range(T):
        b = t // inp.s1
        act = int(inp.kv_act_seqs[b])
        if act > 0:
            rows = IO.live_rows(inp.block_table, act, b)
            mag[t, :act] = wa[t] @ (qa[t] @ ka[rows].T)
    return ref, mag


def _ties_take_lowest(sel, scores):
    """Among the scores equal to the lowest selected one, the selected positions are the lowest."""
    for t in range(sel.shape[0]):
        pos = sel[t][sel[t] >= 0]
        if len(pos) == 0:
            continue
        kth = scores[t][pos].min()
        eq = np.nonzero(scores[t] == kth)[0]
        taken = np.sort(np.intersect1d(pos, eq))
        assert np.array_equal(taken, eq[:len(taken)]), t


def _check(inp, label):
    sfa = _lib()
    sc, idx = sfa.run_indexer(inp)
    torch.cuda.synchronize()
    got = sc.cpu().numpy().astype(np.float64)
    sel = idx.cpu().numpy()
    ref, mag = _oracle(inp)
    live = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), live), label
    bound = 2.0 ** -15 * mag + 1e-30
    err = np.abs(got[live] - ref[live])
    ratio = float((err / bound[live]).max()) if live.any() else 0.0
    print(f"[indexer] {label}: live={int(live.sum())} worst_err/bound={ratio:.3g}", flush=True)
    assert ratio <= 1.0, label
    # the selection, in the kernel's precision
    rep = IO.check_topk(sel, got, inp.topk)
    assert rep["bad"] == [], (label, rep["bad"][:5])
    _ties_take_lowest(sel, got)
    # the selection against the fp64 scores: differences only inside the bound near the k-th value
    for t in range(inp.n_tokens):
        pos = sel[t][sel[t] >= 0]
        if len(pos) == 0 or len(pos) == int(live[t].sum()):
            continue
        rest = live[t].copy()
        rest[pos] = False
        lo = (ref[t, pos] + bound[t, pos]).min()      # a selected score can be at most this low
        hi = (ref[t, rest] - bound[t, rest]).max()    # an unselected score at least this high
        assert hi <= lo + 1e-30, (label, t)
    return sc, idx


def test_small_ragged_pages():
    inp = W.indexer_generate(batch=3, s1=2, act_seqs=[1000, 130, 77], topk=100, seed=1, max_blocks_per_batch=9,
                             extra_pool_blocks=3)
    _check(inp, "small_ragged")


@pytest.mark.parametrize("topk", [1, 64, 127, 128, 129, 1000])
def test_topk_edges(topk):
    inp = W.indexer_generate(batch=2, s1=1, act_seqs=[900, 129], topk=topk, seed=topk, max_blocks_per_batch=8)
    _check(inp, f"topk{topk}")


def test_many_tokens_per_batch():
    # more than one 8-token chunk per batch, and a batch with nothing live
    inp = W.indexer_generate(batch=3, s1=19, act_seqs=[700, 0, 2500], topk=300, seed=3, max_blocks_per_batch=20)
    _check(inp, "s1_19")


def test_tokens_beyond_one_chunk():
    # s1 = 5: one workgroup takes 4 tokens, another the fifth; s1 = 3 takes 3 at once
    _check(W.indexer_generate(batch=2, s1=5, act_seqs=[900, 300], topk=200, seed=7, max_blocks_per_batch=8),
           "s1_5")
    _check(W.indexer_generate(batch=2, s1=3, act_seqs=[640, 1000], topk=333, seed=8, max_blocks_per_batch=8),
           "s1_3")


def test_several_pages_per_workgroup_ragged():
    # 14 x 301 pages: each workgroup runs 4 pages, the last run of a batch is short, and the
    # lengths give dead runs, dead pages inside a run and partial pages
    rng = np.random.default_rng(11)
    act = [int(v) for v in rng.integers(1, 301 * 128, size=14)]
    act[0], act[1], act[2], act[3] = 0, 100, 128 * 4, 301 * 128
    inp = W.indexer_generate(batch=14, s1=3, act_seqs=act, topk=1500, seed=11, max_blocks_per_batch=301)
    _check(inp, "pages_per_wg_4")


def test_rows_longer_than_the_lds_key_cache():
    # 313 pages = 40064 positions per token: the selection reads its keys from global memory
    inp = W.indexer_generate(batch=2, s1=1, act_seqs=[40000, 33000], topk=3000, seed=12, max_blocks_per_batch=313)
    _check(inp, "uncached_select")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_shape_full(seed):
    _check(W.indexer_decode(seed=seed), f"decode_b64_s2_seed{seed}")


def test_select_ties_take_lowest_positions():
    sfa = _lib()
    n_pos = 512
    scores = torch.zeros((3, n_pos), dtype=torch.float32, device="cuda")
    scores[0, 100:110] = 5.0          # 10 above, then ties at 0
    scores[1, :] = -2.5               # everything tied
    scores[2, ::2] = 1.0              # 256 tied at the top
    act = torch.tensor([512, 300, 512], dtype=torch.int32, device="cuda")
    out = sfa.topk_select(scores, act, batch=3, s1=1, topk=40).cpu().numpy()
    assert set(out[0].tolist()) == set(range(100, 110)) | set(range(30))
    assert sorted(out[1].tolist()) == list(range(40))
    assert sorted(out[2].tolist()) == list(range(0, 80, 2))


@pytest.mark.parametrize("n_pos", [8192, 40960])
def test_select_large_ties_and_signs(n_pos):
    # every score equal, then scores that differ only in their lowest bits, then mixed signs,
    # then -0.0 beside +0.0; both the LDS-cached and the global-memory selection
    sfa = _lib()
    g = torch.Generator().manual_seed(5)
    sc = torch.zeros((4, n_pos), dtype=torch.float32)
    sc[0] = 0.75
    base = torch.full((n_pos,), 1.0).view(torch.int32)
    sc[1] = (base + torch.randint(0, 8, (n_pos,), generator=g, dtype=torch.int32)).view(torch.float32)
    sc[2] = torch.randn(n_pos, generator=g)
    sc[3, ::2] = -0.0
    sc[3, 1::2] = 0.0
    act = torch.full((4,), n_pos - 5, dtype=torch.int32)
    K = 1000
    out = sfa.topk_select(sc.cuda(), act.cuda(), batch=4, s1=1, topk=K).cpu().numpy()
    scn = sc.numpy().astype(np.float64)
    rep = IO.check_topk(out, np.where(np.arange(n_pos) < n_pos - 5, scn, -np.inf), K)
    assert rep["bad"] == []
    _ties_take_lowest(out, scn)
    assert sorted(out[0].tolist()) == list(range(K))          # ties: the lowest positions
    # row 3: -0.0 and +0.0 are equal scores, so again the lowest positions
    assert sorted(out[3].tolist()) == list(range(K))


def test_end_to_end_indexer_topk_attention():
    sfa = _lib()
    # one cache layout for both the latent and the index keys: the same block table and lengths
    att = W.generate(batch=4, s1=2, n_q=128, act_seqs=[3000, 700, 5000, 129], topk=512, seed=41,
                     max_blocks_per_batch=40)
    idx_inp = W.indexer_generate(batch=4, s1=2, act_seqs=[3000, 700, 5000, 129], topk=512, seed=41,
                                 max_blocks_per_batch=40)
    # give the indexer the attention workload's block table (its pool is laid out the same way)
    n_pool = att.num_cache_rows // 128
    k = np.zeros((n_pool * 128, 128), dtype=np.uint16)
    rng = np.random.default_rng(41)
    k[:] = W._bf16_bits(torch.from_numpy(rng.standard_normal(k.shape).astype(np.float32)))
    idx_inp = W.IndexerInputs(**{**idx_inp.__dict__, "k_index": k, "block_table": att.block_table.copy()})
    d = sfa.indexer_to_device(idx_inp)
    sc, sel = sfa.run_indexer(idx_inp, d)
    dev = sfa.to_device(att)
    dev["topk_indices"] = sel
    out = sfa.decode(dev["query_nope"], dev["query_rope"], dev["key_nope"], dev["key_rope"], None, sel,
                     dev["block_table"], dev["kv_act_seqs"], att.softmax_scale, batch=att.batch, s1=att.s1)
    torch.cuda.synchronize()
    chosen = W.SfaInputs(**{**att.__dict__, "topk_indices": sel.cpu().numpy()})
    ref = O.sparse_mla_attention(chosen).reshape(att.n_tokens, att.n_q, 512)
    got = out.float().cpu().numpy().astype(np.float64).reshape(att.n_tokens, att.n_q, 512)
    rep = O.allclose_report(got, ref, 5e-3, 1e-4)
    assert rep["fails"] == 0, rep
    # and the selection is a top-k of the index scores
    assert IO.check_topk(sel.cpu().numpy(), sc.cpu().numpy().astype(np.float64), 512)["bad"] == []
