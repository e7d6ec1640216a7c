"""GPU parity of the cache write (sfa_cache_write) against the CPU oracle (oracle/cache_oracle.py).

Every output is integer or byte work (codes, copied bit patterns) or an fp32 scale fixed by one
IEEE division, so the bar is bit-exact: the whole cache after the write, including the rows no
token targets, must equal the oracle's. The full-size case is the benchmark's workload (every
position of a 64 x 8192 cache, 524,288 rows) in the same launch configuration.
"""

import numpy as np
import pytest

import oracle.cache_oracle as C
import oracle.sfa_oracle as O
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run(sfa, inp):
    import torch

    d = sfa.cache_to_device(inp)
    sfa.run_cache_write(inp, d)
    torch.cuda.synchronize()
    kn = d["key_nope"].cpu()
    kn = kn.numpy() if inp.kv_dtype == "int8" else kn.view(torch.int16).numpy().view(np.uint16)
    kr = (np.zeros((kn.shape[0], 0), dtype=np.uint16) if d["key_rope"] is None
          else d["key_rope"].cpu().view(torch.int16).numpy().view(np.uint16))
    ks = None if d["k_nope_scales"] is None else d["k_nope_scales"].cpu().numpy()
    return kn, kr, ks


def _oracle(inp):
    return C.cache_write(inp.new_nope, inp.new_rope, inp.positions, inp.block_table, inp.s1, inp.key_nope,
                         inp.key_rope, inp.k_nope_scales)


def _assert_same(got, want, label):
    kn, kr, ks = got
    wn, wr, ws = want
    bad = np.nonzero(np.any(kn != wn, axis=1))[0]
    assert bad.size == 0, f"{label}: nope rows differ: {bad[:8]}"
    assert np.array_equal(kr, wr), f"{label}: rope differs"
    if ws is not None:
        # compare the scale bit patterns (so -0.0 / +0.0 or a NaN would count)
        assert np.array_equal(ks.view(np.uint32), ws.view(np.uint32)), f"{label}: scales differ"


@pytest.mark.parametrize("kv_dtype", ["int8", "bf16"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_small_ragged_with_masked_tokens(sfa_lib, kv_dtype, seed):
    # 3 batches x 5 tokens (15: not a multiple of the 16 tokens of a workgroup) over a 12-block
    # pool; then some tokens are made unwritable in every way the contract names
    bt = np.array([[4, 7, -1], [0, 11, 3], [9, 15, 2]], dtype=np.int32)  # block 15 is past the pool
    inp = W.cache_write_generate(batch=3, s1=5, n_pool_blocks=12, max_blocks_per_batch=3, kv_dtype=kv_dtype,
                                 seed=seed, block_table=bt)
    pos = np.array([
        0, -1, 3 * 128, 255, 2 * 128 + 5,      # batch 0: padding, past mb*128, a -1 block entry
        1, 127, 128, 300, 383,                 # batch 1: block edges
        127, 1 * 128 + 7, 256, 2, 300,         # batch 2: its second block is outside the pool
    ], dtype=np.int32)
    pos = np.roll(pos.reshape(3, 5), seed, axis=1).reshape(-1)  # the order inside a batch is free
    inp.positions = pos
    assert inp.n_written() == 15 - 4
    _assert_same(_run(sfa_lib, inp), _oracle(inp), f"{kv_dtype} seed {seed}")


@pytest.mark.parametrize("rope_dim", [64, 0])
@pytest.mark.parametrize("kv_dtype", ["int8", "bf16"])
def test_many_tokens_random_positions(sfa_lib, kv_dtype, rope_dim):
    inp = W.cache_write_generate(batch=7, s1=301, n_pool_blocks=64, max_blocks_per_batch=9, kv_dtype=kv_dtype,
                                 seed=5, value_scale=3.0, rope_dim=rope_dim)
    _assert_same(_run(sfa_lib, inp), _oracle(inp), kv_dtype)


def test_special_groups(sfa_lib):
    """Hand-made groups: all zero, one non-zero element, exact ties (absmax 127 gives scale 1),
    negative zeros, large and small magnitudes, and a group whose scale is a subnormal fp32."""
    inp = W.cache_write_generate(batch=1, s1=8, n_pool_blocks=1, max_blocks_per_batch=1, kv_dtype="int8", seed=9)
    x = np.zeros((8, 512), dtype=np.float32)
    x[1, 200] = -0.375                                        # group 1: one element
    x[2, :128] = np.tile(np.array([0.5, 1.5, 2.5, -2.5, 3.5, 126.5, -0.75, 0.25], np.float32), 16)
    x[2, 0] = 127.0                                           # scale exactly 1: ties to even
    x[3, 256:384] = -0.0                                      # negative zeros: an all-zero group
    x[3, 0] = 254.0
    x[3, 1:128] = np.tile(np.array([5.0, 7.0, -3.0, 1.0], np.float32), 32)[:127]
    x[4] = np.linspace(-3e4, 3e4, 512).astype(np.float32)
    x[5] = np.linspace(-1e-30, 1e-30, 512).astype(np.float32)
    x[6] = np.where(np.arange(512) % 2 == 0, 1e-3, -2e-3).astype(np.float32)
    x[7] = np.float32(65504.0)
    x[7, 128:256] = np.linspace(-1e-37, 1e-37, 128).astype(np.float32)  # subnormal scale
    inp.new_nope = O.f32_to_bf16_bits_rne(x)
    got = _run(sfa_lib, inp)
    want = _oracle(inp)
    _assert_same(got, want, "special groups")
    row2 = int(inp.block_table[0, 0]) * 128 + int(inp.positions[2])
    assert list(got[0][row2, :8]) == [127, 2, 2, -2, 4, 126, -1, 0]
    assert got[2][row2, 0] == 1.0


def test_full_size_cache_fill_matches_oracle(sfa_lib):
    """The benchmark's workload: all 524,288 rows of the 64 x 8192 cache, INT8, bit-exact."""
    inp = W.cache_fill(seed=0)
    _assert_same(_run(sfa_lib, inp), _oracle(inp), "cache fill")


def test_decode_step_write_matches_oracle(sfa_lib):
    inp = W.cache_decode_step(seed=1)
    _assert_same(_run(sfa_lib, inp), _oracle(inp), "decode step")


def test_write_then_attention_reads_it(sfa_lib):
    """End to end: an INT8 cache written by sfa_cache_write equals the oracle-written cache, and
    sfa_decode over it meets the attention's accuracy standard against the oracle attention."""
    base = W.generate(batch=2, s1=2, n_q=32, act_seqs=[300, 256], topk=128, kv_dtype="int8", seed=3)
    rows = base.num_cache_rows
    # rewrite every live position of both sequences through the cache write;
    # per-batch token lists padded to one s1: batch 0 has 300 tokens, batch 1 256 (+44 padding)
    s1 = 300
    pos = np.concatenate([np.arange(300), np.arange(256), np.full(44, -1)]).astype(np.int32)
    cw = W.cache_write_generate(batch=2, s1=s1, n_pool_blocks=rows // 128, max_blocks_per_batch=base.block_table.shape[1],
                                kv_dtype="int8", seed=4, positions=pos, block_table=base.block_table)
    cw.key_nope, cw.key_rope, cw.k_nope_scales = base.key_nope, base.key_rope, base.k_nope_scales
    kn, kr, ks = _run(sfa_lib, cw)
    wn, wr, ws = _oracle(cw)
    _assert_same((kn, kr, ks), (wn, wr, ws), "end to end cache")
    base.key_nope, base.key_rope, base.k_nope_scales = kn, kr, ks
    out = sfa_lib.run(base).float().cpu().numpy()
    ref = O.sparse_mla_attention(base)
    rep = O.allclose_report(out, ref)
    assert rep["fails"] == 0, rep


@pytest.mark.parametrize("kv_dtype", ["int8", "bf16"])
def test_512_wide_rows_small_ragged(sfa_lib, kv_dtype):
    """512-wide rows (rope_dim 0): masked tokens as in the 576-wide case, nothing but the 512
    channels written."""
    bt = np.array([[4, 7, -1], [0, 11, 3], [9, 15, 2]], dtype=np.int32)  # block 15 is past the pool
    inp = W.cache_write_generate(batch=3, s1=5, n_pool_blocks=12, max_blocks_per_batch=3, kv_dtype=kv_dtype,
                                 seed=21, block_table=bt, rope_dim=0)
    inp.positions = np.array([0, -1, 3 * 128, 255, 2 * 128 + 5, 1, 127, 128, 300, 383, 127, 1 * 128 + 7, 256, 2, 300],
                             dtype=np.int32)
    assert inp.n_written() == 15 - 4
    _assert_same(_run(sfa_lib, inp), _oracle(inp), f"512-wide {kv_dtype}")


def test_512_wide_write_then_window_attention_reads_it(sfa_lib):
    """The 512-wide chain: the decode step's two new rows per sequence are quantised into an INT8
    pool of 512-wide rows, and SWA on that pool (rope_dim 0) reads them: the cache equals the
    oracle-written one and the attention meets the accuracy standard against the window oracle."""
    import torch

    import oracle.window_oracle as WO

    win = W.window_generate(batch=3, s1=2, n_q=32, ori_lens=[700, 300, 130], window=64, cmp_mode="none",
                            kv_dtype="int8", seed=22, rope_dim=0)
    pos = np.array([[int(v) - 2, int(v) - 1] for v in win.ori_len], dtype=np.int32).reshape(-1)
    cw = W.cache_write_generate(batch=3, s1=2, n_pool_blocks=win.num_cache_rows // 128,
                                max_blocks_per_batch=win.block_table_ori.shape[1], kv_dtype="int8", seed=23,
                                positions=pos, block_table=win.block_table_ori, rope_dim=0)
    cw.key_nope, cw.k_nope_scales = win.key_nope, win.k_nope_scales
    cw.key_rope = np.zeros((win.num_cache_rows, 0), dtype=np.uint16)
    kn, kr, ks = _run(sfa_lib, cw)
    _assert_same((kn, kr, ks), _oracle(cw), "512-wide chain cache")
    win.key_nope, win.k_nope_scales = kn, ks
    out = sfa_lib.run_window(win).float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    ref = WO.window_attention(win)
    rep = O.allclose_report(out.reshape(ref.shape), ref)
    assert rep["fails"] == 0, rep
