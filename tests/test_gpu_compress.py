"""GPU parity of the compressor (sfa_compress) against the CPU oracle (oracle/compress_oracle.py).

The refreshed state is a copy plus one fp32 addition, so it must be bit-exact. Each compressed
row is fp32 arithmetic (softmax over the slots, sum, RMS, rotation) rounded once to bf16; the
oracle is float64. The bar is the attention's: |gpu - ref| <= 1e-4 + 5e-3 * |ref| for every
element (a bf16 rounding moves a value by at most 2^-8 of itself, under the 5e-3 bound, and the
fp32 arithmetic adds ~1e-6). Every pool row no entry targets must be unchanged, bit for bit. The
full-size case is the benchmark's workload in the same launch configuration.
"""

import numpy as np
import pytest

import oracle.compress_oracle as C
import oracle.sfa_oracle as O
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run(sfa_lib, inp, d=None):
    import torch

    d = sfa_lib.compress_to_device(inp) if d is None else d
    sfa_lib.run_compress(inp, d)
    torch.cuda.synchronize()
    return d


def _host(d):
    import torch

    bits = lambda t: None if t is None else t.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    return d["kv_state"].cpu().numpy(), d["score_state"].cpu().numpy(), bits(d["key_nope"]), bits(d["key_rope"])


def _assert_matches(inp, got, want=None, pool=None):
    ks, ss, kn, kr = got
    wks, wss, entries = C.compress(inp) if want is None else want
    np.testing.assert_array_equal(ks.view(np.uint32), wks.view(np.uint32))
    np.testing.assert_array_equal(ss.view(np.uint32), wss.view(np.uint32))
    base_n, base_r = (inp.key_nope, inp.key_rope) if pool is None else pool
    written = {}
    for b, c, row, y in entries:
        if row >= 0:
            written[row] = (b, c, y)
    untouched = np.ones(kn.shape[0], dtype=bool)
    untouched[list(written)] = False
    np.testing.assert_array_equal(kn[untouched], base_n[untouched])
    if kr is not None:
        np.testing.assert_array_equal(kr[untouched], base_r[untouched])
    for row, (b, c, y) in written.items():
        g = (np.concatenate([O.bf16_bits_to_f64(kn[row]), O.bf16_bits_to_f64(kr[row])]) if kr is not None
             else O.bf16_bits_to_f64(kn[row]))
        err = np.abs(g - y)
        bound = 1e-4 + 5e-3 * np.abs(y)
        bad = np.nonzero(err > bound)[0]
        assert bad.size == 0, (f"entry (b={b}, c={c}) row {row}: {bad.size} channels off, first {bad[:4]}, "
                               f"worst ratio {np.max(err / bound):.3f}")
    return len(written)


def test_decode_workload_full_size(sfa_lib):
    """64 sequences, two new tokens each, ratio 4: every sequence closes a window (entry 2047)."""
    inp = W.compress_decode(seed=0)
    n = _assert_matches(inp, _host(_run(sfa_lib, inp)))
    assert n == 64


@pytest.mark.parametrize("seed", [1, 2])
def test_decode_workload_seeds(sfa_lib, seed):
    inp = W.compress_decode(seed=seed)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 64


def test_ratio_128_peaky_scores(sfa_lib):
    """A long window (128 slots, the loop over slots with no unrolled tail) and scores spread
    wide enough that a few slots carry each channel."""
    inp = W.compress_generate(batch=8, s1=1, ratio=128, start_pos=[127 + 128 * k for k in range(8)],
                              rope_positions=2048, max_blocks=2, seed=3, score_scale=4.0)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 8


def test_tokens_span_two_windows(sfa_lib):
    """Seven tokens at ratio 4 (positions 5..11): two entries in one call, the second pooling
    slots refreshed earlier in the same call; every slot is refreshed and the last writer wins."""
    inp = W.compress_generate(batch=3, s1=7, ratio=4, start_pos=[5, 5, 5], rope_positions=64, max_blocks=2, seed=4)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 6


def test_ratio_one_every_token_emits(sfa_lib):
    inp = W.compress_generate(batch=4, s1=3, ratio=1, start_pos=[0, 10, 100, 250], rope_positions=256,
                              max_blocks=2, seed=5)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 12


def test_ragged_positions_and_unwritable_entries(sfa_lib):
    """Mixed start positions: before position 0, past the RoPE tables, an entry whose block is
    negative, an entry past the block table, and an entry whose row is past the pool."""
    starts = [-3, 60, 6, 6, 1021, 6]
    inp = W.compress_generate(batch=6, s1=4, ratio=2, start_pos=starts, rope_positions=64, max_blocks=2,
                              n_pool_blocks=12, seed=6)
    inp.block_table_cmp[2, 0] = -1                 # sequence 2: its entries (3, 4) sit in block 0
    inp.rope_cos = W.rope_tables(1024)[0]          # sequence 4 reaches entry 511, past the table
    inp.rope_sin = W.rope_tables(1024)[1]
    inp.block_table_cmp[5, 0] = 12                 # a row past the 12-block pool
    n = _assert_matches(inp, _host(_run(sfa_lib, inp)))
    assert n == 2 + 2         # sequences 1 (61 and 63 close) and 3; 0 closes none; 2, 4, 5 write none


def test_state_carries_across_calls(sfa_lib):
    """Two calls in a row, the second reading the state the first refreshed."""
    inp = W.compress_generate(batch=4, s1=3, ratio=4, start_pos=[4] * 4, rope_positions=64, max_blocks=2, seed=7)
    d = _run(sfa_lib, inp)
    ks1, ss1, e1 = C.compress(inp)
    got1 = _host(d)
    _assert_matches(inp, got1, (ks1, ss1, e1))
    nxt = W.compress_generate(batch=4, s1=3, ratio=4, start_pos=[7] * 4, rope_positions=64, max_blocks=2, seed=8)
    nxt.kv_state, nxt.score_state = ks1, ss1
    nxt.block_table_cmp, nxt.ape, nxt.gamma = inp.block_table_cmp, inp.ape, inp.gamma
    for k in ("kv", "score"):
        d[k].copy_(sfa_lib.compress_to_device(nxt)[k])
    d["start_pos"].fill_(7)
    got2 = _host(_run(sfa_lib, nxt, d))
    _assert_matches(nxt, got2, pool=(got1[2], got1[3]))


def test_no_tokens_is_a_no_op(sfa_lib):
    inp = W.compress_generate(batch=2, s1=0, ratio=4, start_pos=[3, 3], rope_positions=64, max_blocks=2, seed=9)
    got = _host(_run(sfa_lib, inp))
    np.testing.assert_array_equal(got[0], inp.kv_state)
    np.testing.assert_array_equal(got[2], inp.key_nope)


def test_compressed_entry_feeds_scfa(sfa_lib):
    """One SCFA decode step after the compressor, on one shared pool: each sequence's second new
    token closes a window, the compressor writes that newest compressed entry, and the token's
    compressed list names it. The rows match the compressor oracle (and every other pool row is
    unchanged); the attention over the pool the GPU wrote matches the window oracle."""
    import torch

    import oracle.window_oracle as WO

    ratio = 4
    win = W.window_generate(batch=2, s1=2, n_q=32, ori_lens=[512, 300], window=64, ratio=ratio, cmp_mode="sparse",
                            topk_cmp=24, seed=11)
    for b in range(win.batch):
        win.cmp_indices[b * win.s1 + 1, 0] = int(win.cmp_len[b]) - 1   # closed by position ori_len - 1
    cmp = W.compress_generate(batch=2, s1=2, ratio=ratio, start_pos=[int(v) - 2 for v in win.ori_len],
                              rope_positions=1024, max_blocks=win.block_table_cmp.shape[1], seed=12)
    cmp.block_table_cmp, cmp.key_nope, cmp.key_rope = win.block_table_cmp, win.key_nope, win.key_rope
    dw = sfa_lib.window_to_device(win)
    dc = sfa_lib.compress_to_device(cmp)
    dc["key_nope"], dc["key_rope"] = dw["key_nope"], dw["key_rope"]
    sfa_lib.run_compress(cmp, dc)
    out = sfa_lib.run_window(win, dw)
    torch.cuda.synchronize()
    got = _host(dc)
    assert _assert_matches(cmp, got) == 2
    win.key_nope, win.key_rope = got[2], got[3]
    ref = WO.window_attention(win)
    rep = O.allclose_report(out.float().cpu().numpy().astype(np.float64).reshape(ref.shape), ref)
    assert rep["fails"] == 0, rep


def test_compressed_entry_feeds_int8_scfa(sfa_lib):
    """An INT8 compressed pool: the compressor writes its newest entry into a bf16 staging pool
    (same block table), sfa_cache_write quantises that row into the INT8 pool at the entry's
    position, and INT8 SCFA reads it. The staged rows match the compressor oracle; the codes and
    scales equal the cache oracle's quantisation of the staged bf16 rows (bit for bit, the rule
    decided in the same fp32 on both sides); the attention over the pool the GPU wrote matches the
    window oracle."""
    import torch

    import oracle.cache_oracle as CO
    import oracle.window_oracle as WO

    ratio = 4
    win = W.window_generate(batch=2, s1=2, n_q=32, ori_lens=[512, 300], window=64, ratio=ratio, cmp_mode="sparse",
                            topk_cmp=24, kv_dtype="int8", seed=13)
    for b in range(win.batch):
        win.cmp_indices[b * win.s1 + 1, 0] = int(win.cmp_len[b]) - 1   # closed by position ori_len - 1
    cmp = W.compress_generate(batch=2, s1=2, ratio=ratio, start_pos=[int(v) - 2 for v in win.ori_len],
                              rope_positions=1024, max_blocks=win.block_table_cmp.shape[1], seed=14)
    rows = win.key_rope.shape[0]
    cmp.block_table_cmp = win.block_table_cmp
    cmp.key_nope = np.zeros((rows, 512), dtype=np.uint16)      # the bf16 staging pool
    cmp.key_rope = np.zeros((rows, 64), dtype=np.uint16)
    dw = sfa_lib.window_to_device(win)
    dc = sfa_lib.compress_to_device(cmp)
    sfa_lib.run_compress(cmp, dc)
    torch.cuda.synchronize()
    staged = _host(dc)
    assert _assert_matches(cmp, staged, pool=(cmp.key_nope, cmp.key_rope)) == 2
    # the two new entries (one per sequence) go into the INT8 pool at their positions
    entries = [int(win.cmp_len[b]) - 1 for b in range(win.batch)]
    srow = [int(win.block_table_cmp[b, c // 128]) * 128 + c % 128 for b, c in enumerate(entries)]
    new_nope = dc["key_nope"][srow].contiguous()
    new_rope = dc["key_rope"][srow].contiguous()
    pos = torch.tensor(entries, dtype=torch.int32, device="cuda")
    sfa_lib.cache_write(new_nope, new_rope, pos, dw["block_table_cmp"], dw["key_nope"], dw["key_rope"],
                        dw["k_nope_scales"], batch=win.batch, s1=1)
    out = sfa_lib.run_window(win, dw)
    torch.cuda.synchronize()
    codes = dw["key_nope"].cpu().numpy()
    scales = dw["k_nope_scales"].cpu().numpy()
    want_c, want_s = CO.quantize_groups(staged[2][srow])
    np.testing.assert_array_equal(codes[srow], want_c)
    np.testing.assert_array_equal(scales[srow].view(np.uint32), want_s.view(np.uint32))
    win.key_nope, win.k_nope_scales = codes, scales
    win.key_rope = dw["key_rope"].cpu().view(torch.int16).numpy().view(np.uint16)
    ref = WO.window_attention(win)
    rep = O.allclose_report(out.float().cpu().numpy().astype(np.float64).reshape(ref.shape), ref)
    assert rep["fails"] == 0, rep


# ---- 128-channel rows (index keys) and the rotate = true branch (Hadamard transform) ----

@pytest.mark.parametrize("seed", [0, 1])
def test_index_keys_rotated_full_size(sfa_lib, seed):
    """The page's D = 128 configuration with rotate = true on the decode step: 64 sequences,
    positions 8190 and 8191, ratio 4, every sequence closing a window."""
    inp = W.compress_index_decode(seed=seed)
    assert inp.channels == 128 and inp.rotate
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 64


@pytest.mark.parametrize("rotate", [False, True])
def test_index_keys_windows_and_ragged_positions(sfa_lib, rotate):
    """128 channels, with and without the transform: seven tokens spanning two windows, a
    sequence starting before position 0 and one running past the RoPE tables."""
    inp = W.compress_generate(batch=4, s1=7, ratio=4, start_pos=[5, -2, 58, 5], rope_positions=64, max_blocks=2,
                              seed=13, channels=128, rotate=rotate)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 2 + 1 + 2 + 2


def test_index_keys_ratio_one_peaky(sfa_lib):
    """Ratio 1 (every token emits, so the entry is the token's own normalised, rotated and
    transformed row) and ratio 128 with peaky scores, both rotated."""
    inp = W.compress_generate(batch=3, s1=2, ratio=1, start_pos=[0, 40, 90], rope_positions=128, max_blocks=2,
                              seed=14, channels=128, rotate=True)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 6
    inp = W.compress_generate(batch=4, s1=1, ratio=128, start_pos=[127 + 128 * k for k in range(4)],
                              rope_positions=1024, max_blocks=2, seed=15, score_scale=4.0, channels=128, rotate=True)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 4


# ---- 512-channel rows (the DeepSeek-V4 D = 512 layout: the rotary channels inside the row) ----

@pytest.mark.parametrize("seed", [0, 1])
def test_d512_c128a_full_size(sfa_lib, seed):
    """The page's c128a case at the decode step: ratio 128, every sequence closes a window."""
    inp = W.compress_c128a(seed=seed)
    assert inp.channels == 512 and inp.key_rope is None
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 64


def test_d512_windows_and_ragged_positions(sfa_lib):
    inp = W.compress_generate(batch=3, s1=7, ratio=4, start_pos=[5, -2, 60], rope_positions=64, max_blocks=2,
                              seed=25, channels=512)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 2 + 1 + 1


def test_d512_compressed_entry_feeds_scfa(sfa_lib):
    """The 512-wide chain: the compressor writes each sequence's newest entry into a 512-wide
    pool, and SCFA on 512-wide rows reads it through the token's compressed list."""
    import torch

    import oracle.window_oracle as WO

    ratio = 4
    win = W.window_generate(batch=2, s1=2, n_q=32, ori_lens=[512, 300], window=64, ratio=ratio, cmp_mode="sparse",
                            topk_cmp=24, seed=26, rope_dim=0)
    for b in range(win.batch):
        win.cmp_indices[b * win.s1 + 1, 0] = int(win.cmp_len[b]) - 1   # closed by position ori_len - 1
    cmp = W.compress_generate(batch=2, s1=2, ratio=ratio, start_pos=[int(v) - 2 for v in win.ori_len],
                              rope_positions=1024, max_blocks=win.block_table_cmp.shape[1], seed=27, channels=512)
    cmp.block_table_cmp, cmp.key_nope = win.block_table_cmp, win.key_nope
    dw = sfa_lib.window_to_device(win)
    dc = sfa_lib.compress_to_device(cmp)
    dc["key_nope"] = dw["key_nope"]
    sfa_lib.run_compress(cmp, dc)
    out = sfa_lib.run_window(win, dw)
    torch.cuda.synchronize()
    got = _host(dc)
    assert _assert_matches(cmp, got) == 2
    win.key_nope = got[2]
    ref = WO.window_attention(win)
    rep = O.allclose_report(out.float().cpu().numpy().astype(np.float64).reshape(ref.shape), ref)
    assert rep["fails"] == 0, rep


# ---- long windows (ratio >= 10): the slots split over channel groups, merged through LDS ----

@pytest.mark.parametrize("channels", [576, 512, 128])
def test_long_window_groups_without_slots(sfa_lib, channels):
    """Ratio 16: 15 other slots in batches of 4 leave some of the channel groups without a slot
    (their running max stays -inf and they must add nothing to the merge)."""
    inp = W.compress_generate(batch=5, s1=1, ratio=16, start_pos=[15 + 16 * k for k in range(5)],
                              rope_positions=256, max_blocks=2, seed=31, score_scale=3.0, channels=channels,
                              rotate=channels == 128)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 5


@pytest.mark.parametrize("channels", [576, 512])
def test_long_window_two_entries_in_one_call(sfa_lib, channels):
    """Ratio 12, twenty tokens (positions 5..24): entries 0 and 1 close in one call; the second
    pools slots that earlier tokens of the same call refreshed, taken from their inputs."""
    inp = W.compress_generate(batch=3, s1=20, ratio=12, start_pos=[5, 5, 5], rope_positions=64, max_blocks=2,
                              seed=32, channels=channels)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 6


def test_long_window_index_keys_rotated(sfa_lib):
    inp = W.compress_generate(batch=8, s1=1, ratio=128, start_pos=[127 + 128 * k for k in range(8)],
                              rope_positions=2048, max_blocks=2, seed=33, score_scale=4.0, channels=128, rotate=True)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 8


@pytest.mark.parametrize("channels", [576, 512, 128])
def test_long_window_several_entries_in_one_call(sfa_lib, channels):
    """300 tokens at ratio 128 from positions 0 and 100: two and three entries per sequence in one
    call, the later ones pooling slots that earlier tokens of the call refreshed."""
    inp = W.compress_generate(batch=2, s1=300, ratio=128, start_pos=[0, 100], rope_positions=512, max_blocks=2,
                              seed=34, score_scale=2.0, channels=channels, rotate=channels == 128)
    assert _assert_matches(inp, _host(_run(sfa_lib, inp))) == 5


def test_long_window_c128a_repeats_bit_identically(sfa_lib):
    """The c128a workload run three times from the same inputs writes the same bits."""
    inp = W.compress_c128a(seed=3)
    rows = None
    for _ in range(3):
        got = _host(_run(sfa_lib, inp))
        if rows is None:
            rows = got[2]
            assert _assert_matches(inp, got) == 64
        else:
            np.testing.assert_array_equal(got[2], rows)
