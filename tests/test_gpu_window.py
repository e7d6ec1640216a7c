"""GPU parity of the sliding-window + compressed-cache attention variants (sfa_window_decode:
SWA, CFA, SCFA) against the CPU oracle (oracle/window_oracle.py), at the attention's accuracy
standard (|got - ref| <= 1e-4 + 5e-3 |ref| on every element), plus exact closed forms."""

import numpy as np
import pytest

import oracle.sfa_oracle as O
import oracle.window_oracle as WO
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _check(sfa, inp, tokens=None, splits=0):
    out = sfa.run_window(inp, num_splits=splits).float().cpu().numpy().astype(np.float64)
    ref = WO.window_attention(inp, tokens=tokens)
    got = out.reshape(inp.n_tokens, inp.n_q, 512)
    if tokens is not None:
        got = got[list(tokens)]
    else:
        ref = ref.reshape(inp.n_tokens, inp.n_q, 512)
    rep = O.allclose_report(got, ref)
    assert rep["fails"] == 0, rep
    return out


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
@pytest.mark.parametrize("mode", ["none", "all", "sparse"])
def test_small_variants(sfa_lib, kv_dtype, mode):
    # ragged lengths; windows that reach below position 0; compressed lists with -1 padding
    inp = W.window_generate(batch=3, s1=2, n_q=32, ori_lens=[700, 40, 2], window=64, ratio=4, cmp_mode=mode,
                            topk_cmp=24, kv_dtype=kv_dtype, seed=1)
    _check(sfa_lib, inp)


@pytest.mark.parametrize("splits", [1, 2, 4])
def test_partitions_agree(sfa_lib, splits):
    inp = W.window_generate(batch=2, s1=2, n_q=64, ori_lens=[3000, 1500], window=700, ratio=4, cmp_mode="sparse",
                            topk_cmp=300, seed=2)
    _check(sfa_lib, inp, splits=splits)


def test_one_position_window_is_the_value_row_bit_exact(sfa_lib):
    inp = W.window_generate(batch=2, s1=2, n_q=16, ori_lens=[300, 129], window=1, cmp_mode="none", seed=3)
    out = sfa_lib.run_window(inp).view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)
    for t in range(4):
        b, s = divmod(t, 2)
        p = int(inp.ori_len[b]) - 2 + s
        row = int(inp.block_table_ori[b, p // 128]) * 128 + p % 128
        assert np.array_equal(out[b, s], np.broadcast_to(inp.key_nope[row], (16, 512)))


def test_window_only_equals_sparse_decode_bit_exact(sfa_lib):
    """SWA gives the same bits as sfa_decode given the window positions as its top-k list: the
    window instantiation resolves the same rows in the same order."""
    import torch

    inp = W.window_generate(batch=2, s1=2, n_q=32, ori_lens=[500, 200], window=96, cmp_mode="none", seed=4)
    got = sfa_lib.run_window(inp)
    idx = np.full((4, 96), -1, dtype=np.int32)
    for t in range(4):
        p = int(inp.ori_len[t // 2]) - 2 + t % 2
        w = WO.window_positions(p, 96)
        idx[t, :len(w)] = w
    d = sfa_lib.window_to_device(inp)
    ref = sfa_lib.decode(d["query_nope"], d["query_rope"], d["key_nope"], d["key_rope"], None,
                         torch.from_numpy(idx).cuda(), d["block_table_ori"], d["ori_len"], inp.softmax_scale,
                         batch=2, s1=2)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_swa_decode_shape_full(sfa_lib):
    _check(sfa_lib, W.swa_decode(seed=0))


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_scfa_decode_shape_full(sfa_lib, kv_dtype):
    _check(sfa_lib, W.scfa_decode(seed=1, kv_dtype=kv_dtype))


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_cfa_decode_shape_full(sfa_lib, kv_dtype):
    _check(sfa_lib, W.cfa_decode(seed=2, kv_dtype=kv_dtype))


@pytest.mark.parametrize("rope_dim", [64, 0])
@pytest.mark.parametrize("mode", ["none", "sparse"])
def test_prefill_form(sfa_lib, mode, rope_dim):
    """Prefill is s1 = ori_len: query s sits at position s, so early queries have short windows
    (down to one position) and few causal compressed entries (none below position 3)."""
    inp = W.window_generate(batch=1, s1=300, n_q=16, ori_lens=[300], window=64, ratio=4, cmp_mode=mode, topk_cmp=16,
                            seed=7, rope_dim=rope_dim)
    _check(sfa_lib, inp)


@pytest.mark.parametrize("rope_dim", [64, 0])
@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_pool_beyond_4gib_matches_small_pool(sfa_lib, kv_dtype, rope_dim):
    """The window instantiation with 64-bit row addressing (a pool of more than 4 Mi rows): the
    same SCFA problem with its blocks moved there, some below and some above row 4 Mi, gives the
    bit-identical result."""
    import torch

    inp = W.window_generate(batch=2, s1=2, n_q=64, ori_lens=[3000, 1400], window=200, ratio=4, cmp_mode="sparse",
                            topk_cmp=150, kv_dtype=kv_dtype, seed=8, rope_dim=rope_dim)
    d = sfa_lib.window_to_device(inp)
    ref = sfa_lib.run_window(inp, d).clone()
    n_small = inp.num_cache_rows // 128
    n_big = (1 << 22) // 128 + 64
    rng = np.random.default_rng(9)
    below = rng.choice(np.arange(1000, (1 << 22) // 128), size=n_small // 2, replace=False)
    above = rng.choice(np.arange((1 << 22) // 128, n_big), size=n_small - n_small // 2, replace=False)
    place = torch.from_numpy(np.concatenate([below, above]).astype(np.int64)).cuda()
    big = dict(d)
    for key, width in (("key_nope", 512), ("key_rope", 64), ("k_nope_scales", 4)):
        small = d[key]
        if small is None:
            continue
        t = torch.empty((n_big * 128, width), dtype=small.dtype, device="cuda")
        t.view(n_big, 128, width)[place] = small.view(n_small, 128, width)
        big[key] = t
    p32 = place.to(torch.int32)
    big["block_table_ori"] = p32[d["block_table_ori"].long()].contiguous()
    big["block_table_cmp"] = p32[d["block_table_cmp"].long()].contiguous()
    got = sfa_lib.run_window(inp, big)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    del big
    torch.cuda.empty_cache()


# ---- 512-wide rows (the DeepSeek-V4 layout: rotary channels inside the row, rope_dim 0) -----

@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
@pytest.mark.parametrize("mode", ["none", "all", "sparse"])
def test_d512_small_variants(sfa_lib, kv_dtype, mode):
    inp = W.window_generate(batch=3, s1=2, n_q=32, ori_lens=[700, 40, 2], window=64, ratio=4, cmp_mode=mode,
                            topk_cmp=24, kv_dtype=kv_dtype, seed=21, rope_dim=0)
    assert inp.rope_dim == 0
    _check(sfa_lib, inp)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
@pytest.mark.parametrize("splits", [1, 2, 4])
def test_d512_partitions_agree(sfa_lib, splits, kv_dtype):
    inp = W.window_generate(batch=2, s1=2, n_q=64, ori_lens=[3000, 1500], window=700, ratio=4, cmp_mode="sparse",
                            topk_cmp=300, kv_dtype=kv_dtype, seed=22, rope_dim=0)
    _check(sfa_lib, inp, splits=splits)


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_d512_equals_the_rope_kernel_with_zero_rope_bit_exact(sfa_lib, kv_dtype):
    """The same rows run through the 576-channel instantiation with 64 zero rope channels added
    to every query and row: each score gains four MFMA steps of exact zeros, so both kernels give
    the same bits (the 512-wide one skips the rope DMA and those steps)."""
    import torch

    inp = W.window_generate(batch=4, s1=2, n_q=128, ori_lens=[2000, 900, 130, 3000], window=128, ratio=4,
                            cmp_mode="sparse", topk_cmp=200, kv_dtype=kv_dtype, seed=23, rope_dim=0)
    d = sfa_lib.window_to_device(inp)
    got = sfa_lib.run_window(inp, d).clone()
    z = dict(d)
    z["query_rope"] = torch.zeros((d["query_nope"].shape[0], 64), dtype=torch.bfloat16, device="cuda")
    z["key_rope"] = torch.zeros((d["key_nope"].shape[0], 64), dtype=torch.bfloat16, device="cuda")
    ref = sfa_lib.run_window(inp, z)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_d512_one_position_window_is_the_row_bit_exact(sfa_lib):
    inp = W.window_generate(batch=2, s1=2, n_q=16, ori_lens=[300, 129], window=1, cmp_mode="none", seed=24,
                            rope_dim=0)
    out = sfa_lib.run_window(inp).view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)
    for t in range(4):
        b, s = divmod(t, 2)
        p = int(inp.ori_len[b]) - 2 + s
        row = int(inp.block_table_ori[b, p // 128]) * 128 + p % 128
        assert np.array_equal(out[b, s], np.broadcast_to(inp.key_nope[row], (16, 512)))


def test_d512_swa_decode_shape_full(sfa_lib):
    _check(sfa_lib, W.swa_decode_d512(seed=0))


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_d512_cfa_decode_shape_full(sfa_lib, kv_dtype):
    _check(sfa_lib, W.cfa_decode_d512(seed=2, kv_dtype=kv_dtype))


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_d512_scfa_decode_shape_full(sfa_lib, kv_dtype):
    _check(sfa_lib, W.scfa_decode_d512(seed=1, kv_dtype=kv_dtype))
