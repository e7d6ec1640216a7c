"""Pins of the window / compressed-cache attention oracle (oracle/window_oracle.py): hand-worked
windows and rows, a window covering the whole causal prefix against dense causal attention on
the unpaged cache (a separate plain routine), a one-position window returning its value row,
agreement with the pinned sparse-attention oracle when both sources are one sequence, and
planted mistakes. No GPU needed.

Source: "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section "FA-class operators:
SWA, CFA and SCFA" (a sliding window over the original cache, plus causal or index-selected
entries of the compressed cache).
"""

import math

import numpy as np
import pytest

import oracle.sfa_oracle as O
import oracle.window_oracle as WO
from mla_sparse_top_amd import workloads as W


def test_window_positions_hand_worked():
    assert WO.window_positions(5, 3) == [3, 4, 5]
    assert WO.window_positions(1, 4) == [0, 1]
    assert WO.window_positions(0, 1) == [0]
    assert WO.window_positions(-1, 8) == []
    assert list(WO.query_positions([10, 3], 2)) == [8, 9, 1, 2]


def test_token_rows_hand_worked():
    bt_o = np.array([[2, 0]], dtype=np.int32)   # positions 0..127 -> block 2, 128..255 -> block 0
    bt_c = np.array([[1]], dtype=np.int32)
    # one token (s1 = 1) of a 130-long sequence: p = 129, window 3 -> positions 127, 128, 129
    rows = WO.token_rows(0, 1, 3, np.array([[4, -1, 40, 7]]), bt_o, bt_c, [130], [32], 3 * 128)
    assert rows == [2 * 128 + 127, 0 * 128 + 0, 0 * 128 + 1, 1 * 128 + 4, 1 * 128 + 7]  # 40 >= cmp_len 32


def _dense_causal(q_n, q_r, k_n, k_r, scale):
    """Plain softmax attention of one query over contiguous rows, for the closed form."""
    s = scale * (q_n @ k_n.T + q_r @ k_r.T)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ k_n


def test_full_window_equals_dense_causal_attention():
    inp = W.window_generate(batch=2, s1=2, n_q=4, ori_lens=[200, 70], window=10_000, cmp_mode="none", seed=3)
    out = WO.window_attention(inp)
    for b in range(2):
        bt = inp.block_table_ori[b]
        L = int(inp.ori_len[b])
        rows = np.array([int(bt[j // 128]) * 128 + j % 128 for j in range(L)])
        kn = O.bf16_bits_to_f64(inp.key_nope[rows])
        kr = O.bf16_bits_to_f64(inp.key_rope[rows])
        for s in range(2):
            t = b * 2 + s
            p = L - 2 + s
            qn = O.bf16_bits_to_f64(inp.query_nope[t * 4:(t + 1) * 4])
            qr = O.bf16_bits_to_f64(inp.query_rope[t * 4:(t + 1) * 4])
            want = _dense_causal(qn, qr, kn[:p + 1], kr[:p + 1], inp.softmax_scale)
            assert np.allclose(out[b, s], want, rtol=0, atol=1e-12)


def test_one_position_window_returns_its_value_row():
    inp = W.window_generate(batch=1, s1=2, n_q=4, ori_lens=[300], window=1, cmp_mode="none", seed=4)
    out = WO.window_attention(inp)
    for s in range(2):
        p = 300 - 2 + s
        row = int(inp.block_table_ori[0, p // 128]) * 128 + p % 128
        assert np.array_equal(out[0, s], np.broadcast_to(O.bf16_bits_to_f64(inp.key_nope[row]), (4, 512)))


def test_single_sequence_sources_match_sparse_attention_oracle():
    """With the compressed source aliased to the original one (same block table, same length),
    the variant is sparse attention over the window positions followed by the listed indices."""
    inp = W.window_generate(batch=2, s1=2, n_q=8, ori_lens=[260, 140], window=16, ratio=1, cmp_mode="sparse",
                            topk_cmp=20, seed=5)
    inp.block_table_cmp = inp.block_table_ori
    inp.cmp_len = inp.ori_len
    out = WO.window_attention(inp)
    idx = np.full((4, 16 + 20), -1, dtype=np.int32)
    for t in range(4):
        p = int(inp.ori_len[t // 2]) - 2 + t % 2
        win = WO.window_positions(p, 16)
        idx[t, :len(win)] = win
        idx[t, 16:] = inp.cmp_indices[t]

    class S:
        pass

    s = S()
    s.n_q, s.batch, s.s1, s.softmax_scale = 8, 2, 2, inp.softmax_scale
    s.query_nope, s.query_rope = inp.query_nope, inp.query_rope
    s.key_nope, s.key_rope, s.k_nope_scales = inp.key_nope, inp.key_rope, inp.k_nope_scales
    s.topk_indices, s.block_table, s.kv_act_seqs = idx, inp.block_table_ori, inp.ori_len
    want = O.sparse_mla_attention(s)
    assert np.allclose(out, want, rtol=0, atol=1e-12)


def test_cfa_lists_every_causal_entry():
    inp = W.window_generate(batch=1, s1=2, n_q=4, ori_lens=[520], window=4, ratio=128, cmp_mode="all", seed=6)
    # p = 518 and 519: entries c with (c + 1) * 128 <= p + 1, i.e. 0..3 (4 * 128 = 512 <= 519)
    assert [list(r[r >= 0]) for r in inp.cmp_indices] == [[0, 1, 2, 3], [0, 1, 2, 3]]
    rows = WO.token_rows(1, 2, 4, inp.cmp_indices, inp.block_table_ori, inp.block_table_cmp, inp.ori_len,
                         inp.cmp_len, inp.num_cache_rows)
    assert len(rows) == 4 + 4


def _scalar_shared_kv_attention(q, rows_k, scale):
    """One head over rows that serve as both key and value, in scalar loops: softmax over the
    rows of scale * <q, k_j>, then the weighted sum of the rows."""
    s = [scale * sum(qd * kd for qd, kd in zip(q, k)) for k in rows_k]
    m = max(s)
    w = [math.exp(v - m) for v in s]
    tot = sum(w)
    return [sum(w[j] * rows_k[j][d] for j in range(len(rows_k))) / tot for d in range(len(q))]


@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_d512_rows_match_scalar_attention_with_shared_kv(kv_dtype):
    """The 512-wide row layout (zero-width rope): each head's output is the softmax-weighted sum
    of the attended 512-channel rows themselves, the score taken over all 512 channels."""
    inp = W.window_generate(batch=2, s1=2, n_q=2, ori_lens=[9, 140], window=3, ratio=2, cmp_mode="sparse",
                            topk_cmp=3, kv_dtype=kv_dtype, rope_dim=0, seed=7)
    assert inp.rope_dim == 0 and inp.query_rope.shape == (8, 0)
    assert inp.softmax_scale == float(np.float32(1 / math.sqrt(512)))
    out = WO.window_attention(inp)
    for t in range(4):
        rows = WO.token_rows(t, 2, 3, inp.cmp_indices, inp.block_table_ori, inp.block_table_cmp, inp.ori_len,
                             inp.cmp_len, inp.num_cache_rows)
        assert len(rows) == 6
        if kv_dtype == "int8":
            ks = O.dequant_int8_chain(inp.key_nope[rows], inp.k_nope_scales[rows])
        else:
            ks = O.bf16_bits_to_f64(inp.key_nope[rows])
        ks = [list(map(float, r)) for r in ks]
        for hh in range(2):
            q = list(map(float, O.bf16_bits_to_f64(inp.query_nope[2 * t + hh])))
            want = _scalar_shared_kv_attention(q, ks, inp.softmax_scale)
            np.testing.assert_allclose(out[t // 2, t % 2, hh], want, rtol=1e-12, atol=1e-13)


def test_d512_equals_the_576_layout_with_zero_rope():
    """Appending 64 zero rope channels to every query and row changes no score, so the 576-wide
    formula gives the same output, bit for bit."""
    inp = W.window_generate(batch=2, s1=2, n_q=4, ori_lens=[300, 77], window=20, ratio=4, cmp_mode="sparse",
                            topk_cmp=10, rope_dim=0, seed=8)
    out = WO.window_attention(inp)
    inp.key_rope = np.zeros((inp.key_nope.shape[0], 64), dtype=np.uint16)
    inp.query_rope = np.zeros((inp.query_nope.shape[0], 64), dtype=np.uint16)
    assert np.array_equal(WO.window_attention(inp), out)


# ---- planted mistakes (CPU only) ----------------------------------------------------------

_real_wp = WO.window_positions
_real_rows = WO.token_rows


def _window_excludes_query(p, w):
    return _real_wp(p - 1, w)


def _window_one_short(p, w):
    return _real_wp(p, w - 1)


def _cmp_through_ori_table(t, s1, window, cmp, bt_o, bt_c, ol, cl, n):
    return _real_rows(t, s1, window, cmp, bt_o, bt_o, ol, cl, n)


_PINS = [test_window_positions_hand_worked, test_token_rows_hand_worked,
         test_full_window_equals_dense_causal_attention, test_one_position_window_returns_its_value_row,
         test_single_sequence_sources_match_sparse_attention_oracle]


_real_token = O.sparse_mla_attention_token


def _d512_scores_skip_rotary_channels(qn, qr, kn, kr, scale):
    # a 512-wide row taken as 448 nope channels plus 64 rope channels that have no query part
    if qr.shape[1] == 0:
        qn = qn.copy()
        qn[:, 448:] = 0.0
    return _real_token(qn, qr, kn, kr, scale)


def test_d512_pin_catches_planted_mistake(monkeypatch):
    monkeypatch.setattr(O, "sparse_mla_attention_token", _d512_scores_skip_rotary_channels)
    with pytest.raises(AssertionError):
        test_d512_rows_match_scalar_attention_with_shared_kv("bf16")


@pytest.mark.parametrize("name", ["excludes_query", "one_short", "cmp_through_ori_table"])
def test_some_pin_catches_planted_mistake(name, monkeypatch):
    if name == "excludes_query":
        monkeypatch.setattr(WO, "window_positions", _window_excludes_query)
    elif name == "one_short":
        monkeypatch.setattr(WO, "window_positions", _window_one_short)
    else:
        monkeypatch.setattr(WO, "token_rows", _cmp_through_ori_table)
    caught = 0
    for pin in _PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught, f"no pin caught {name}"
