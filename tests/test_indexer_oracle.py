"""Pins for the Lightning Indexer oracle (oracle/indexer_oracle.py), all on the CPU.

The score is a plain definition ("CANN DeepSeek Indexer attention optimisation", section
"Lightning Indexer"): I[i, j] = sum_h w[i, h] * ReLU(q_index[i, h] . k_index[j]). It is pinned
against a scalar brute force, closed forms (a key scored against itself, against its negation,
one-hot weights), positive homogeneity and additivity in the weights, and block-permutation
invariance of the paged cache. The selection rule is pinned against numpy's sort and against
planted wrong selections. Planted mistakes in copies of the oracle must each fail a pin.
"""

import math
import struct

import numpy as np
import pytest

import oracle.indexer_oracle as IO
from mla_sparse_top_amd import workloads as W


def _small(seed=0, act=(300, 77), s1=2, heads=3, dim=8, topk=50, extra=2):
    return W.indexer_generate(batch=len(act), s1=s1, act_seqs=list(act), topk=topk, seed=seed, n_heads=heads,
                              head_dim=dim, max_blocks_per_batch=3, extra_pool_blocks=extra)


def _bf16_scalar(bits) -> float:
    """bf16 bits to a Python float through struct: an independent route from the oracle's
    numpy bit shift (the four bytes of the binary32 pattern hi:lo:0:0, big-endian)."""
    b = int(bits) & 0xFFFF
    return struct.unpack(">f", bytes([b >> 8, b & 0xFF, 0, 0]))[0]


def _bf16_array(bits) -> np.ndarray:
    flat = np.asarray(bits).reshape(-1)
    return np.array([_bf16_scalar(x) for x in flat], dtype=np.float64).reshape(np.shape(bits))


def _scores(inp, fn=None):
    fn = fn or IO.indexer_scores
    T = inp.n_tokens
    return fn(inp.q_index.reshape(T, inp.n_heads, inp.head_dim), inp.weights, inp.k_index, inp.block_table,
              inp.kv_act_seqs, inp.s1, inp.n_positions)


def test_scores_match_scalar_brute_force():
    inp = _small(seed=1)
    got = _scores(inp)
    T, H, D = inp.n_tokens, inp.n_heads, inp.head_dim
    q = _bf16_array(inp.q_index).reshape(T, H, D)
    k = _bf16_array(inp.k_index)
    for t in range(T):
        b = t // inp.s1
        for j in range(0, inp.n_positions, 7):
            if j >= inp.kv_act_seqs[b]:
                assert got[t, j] == -math.inf
                continue
            row = int(inp.block_table[b][j // 128]) * 128 + j % 128
            want = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += q[t, h, d] * k[row, d]
                want += float(inp.weights[t, h]) * max(dot, 0.0)
            assert abs(got[t, j] - want) <= 1e-12 * (1 + abs(want)), (t, j)


def test_closed_forms_self_and_negated_key():
    # one head, weight 1: a query equal to key j scores |k_j|^2; its negation scores 0 (ReLU)
    inp = _small(seed=2, heads=1)
    T = inp.n_tokens
    j = 5
    row = int(inp.block_table[0][0]) * 128 + j
    q = np.repeat(inp.k_index[row][None, :], T, axis=0)
    inp.q_index = q
    inp.weights = np.ones((T, 1), dtype=np.float32)
    kj = _bf16_array(inp.k_index[row])
    assert _scores(inp)[0, j] == pytest.approx(float(kj @ kj), rel=1e-15)
    inp.q_index = q ^ np.uint16(0x8000)  # flip every sign bit: q = -k_j
    assert _scores(inp)[0, j] == 0.0


# bf16 is the upper half of an IEEE binary32 (sign, 8 exponent bits with bias 127, 7 stored
# fraction bits); each value below is worked out by hand from that definition.
_BF16_CASES = [
    (0x0000, 0.0), (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3FC0, 1.5), (0x3F00, 0.5),
    (0x4049, 3.140625),                              # 2 * (1 + 73/128)
    (0xC2F7, -123.5),                                # -(2^6) * (1 + 119/128)
    (0x0080, math.ldexp(1.0, -126)),                 # smallest normal
    (0x0001, math.ldexp(1.0, -133)),                 # smallest subnormal: 2^-126 * 2^-7
    (0x007F, math.ldexp(127.0, -133)),               # largest subnormal
    (0x7F7F, math.ldexp(255.0, 120)),                # largest finite: 2^127 * (1 + 127/128)
    (0x7F80, math.inf), (0xFF80, -math.inf),
]


@pytest.mark.parametrize("bits,value", _BF16_CASES)
def test_bf16_bits_to_f64_hand_worked(bits, value):
    got = IO.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))
    assert got.dtype == np.float64 and got[0] == value


def test_bf16_bits_to_f64_sign_zero_and_nan():
    got = IO.bf16_bits_to_f64(np.array([0x8000, 0x7FC0, 0xFFC1], dtype=np.uint16))
    assert got[0] == 0.0 and math.copysign(1.0, got[0]) == -1.0
    assert np.isnan(got[1]) and np.isnan(got[2])


def test_bf16_bits_to_f64_every_pattern_matches_struct_route():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = IO.bf16_bits_to_f64(bits)
    want = np.array(struct.unpack(">65536f", b"".join(bytes([b >> 8, b & 0xFF, 0, 0]) for b in range(65536))))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_one_hot_weights_select_a_head():
    inp = _small(seed=3)
    T, H = inp.n_tokens, inp.n_heads
    base = inp.weights.copy()
    per_head = []
    for h in range(H):
        inp.weights = np.zeros((T, H), dtype=np.float32)
        inp.weights[:, h] = 1.0
        per_head.append(_scores(inp))
    inp.weights = base
    full = _scores(inp)
    live = np.isfinite(full)
    combo = sum(base[:, h][:, None].astype(np.float64) * np.where(live, per_head[h], 0.0) for h in range(H))
    assert np.allclose(full[live], combo[live], rtol=1e-12, atol=1e-12)
    assert all(np.all(p[live] >= 0) for p in per_head)


def test_homogeneous_and_additive_in_weights():
    # small integer weights, so that 2w and w1 + w2 are exact in fp32 and the checks are tight
    inp = _small(seed=4)
    rng = np.random.default_rng(0)
    w1 = rng.integers(-4, 5, size=inp.weights.shape).astype(np.float32)
    w2 = rng.integers(-4, 5, size=inp.weights.shape).astype(np.float32)
    inp.weights = w1
    s1 = _scores(inp)
    inp.weights = 2 * w1
    s2 = _scores(inp)
    inp.weights = w2
    s3 = _scores(inp)
    inp.weights = w1 + w2
    s4 = _scores(inp)
    live = np.isfinite(s1)
    assert np.array_equal(np.isfinite(s4), live)
    assert np.allclose(s2[live], 2 * s1[live], rtol=1e-14, atol=0)
    assert np.allclose(s4[live], s1[live] + s3[live], rtol=1e-12, atol=1e-12)


def test_block_permutation_and_dead_rows():
    inp = _small(seed=5, extra=3)
    ref = _scores(inp)
    # dead rows are NaN in the pool, yet every live score is finite and every dead one is -inf
    for t in range(inp.n_tokens):
        act = int(inp.kv_act_seqs[t // inp.s1])
        assert np.all(np.isfinite(ref[t, :act])) and np.all(ref[t, act:] == -np.inf)
    n_pool = inp.num_cache_rows // 128
    perm = np.random.default_rng(1).permutation(n_pool)
    k = np.empty_like(inp.k_index)
    for p in range(n_pool):
        k[perm[p] * 128:(perm[p] + 1) * 128] = inp.k_index[p * 128:(p + 1) * 128]
    inp.k_index = k
    inp.block_table = perm[inp.block_table].astype(np.int32)
    assert np.array_equal(_scores(inp), ref)


def test_topk_positions_against_sort():
    rng = np.random.default_rng(6)
    scores = rng.standard_normal((5, 400))
    scores[2, 123:] = -np.inf      # 123 live positions
    scores[4, :] = -np.inf         # nothing live
    sel = IO.topk_positions(scores, 150)
    for t in range(5):
        live = np.nonzero(np.isfinite(scores[t]))[0]
        want = set(live[np.argsort(-scores[t][live])][:150].tolist())
        got = sel[t][sel[t] >= 0]
        assert set(got.tolist()) == want and len(got) == min(150, len(live))
        assert np.all(sel[t][len(got):] == -1)
    assert IO.check_topk(sel, scores, 150)["bad"] == []


def test_check_topk_catches_planted_mistakes():
    rng = np.random.default_rng(7)
    scores = rng.standard_normal((4, 300))
    scores[3, 40:] = -np.inf
    sel = IO.topk_positions(scores, 64)
    assert IO.check_topk(sel, scores, 64)["bad"] == []
    wrong = sel.copy()
    out_pos = np.setdiff1d(np.arange(300), sel[0])[0]
    wrong[0, 0] = out_pos                     # replace the best with an unselected position
    wrong[1, 5] = wrong[1, 6]                 # duplicate
    wrong[2, 10] = -1                         # too few
    wrong[3, 0] = 200                         # a dead position (row 3 has 40 live)
    bad = dict(IO.check_topk(wrong, scores, 64)["bad"])
    assert bad == {0: "order", 1: "invalid", 2: "count", 3: "invalid"}
    # ties at the boundary may go either way
    tie = np.zeros((1, 10))
    tie[0, :3] = 1.0
    assert IO.check_topk(np.array([[0, 1, 2, 7]]), tie, 4)["bad"] == []
    assert IO.check_topk(np.array([[0, 1, 2, 9]]), tie, 4)["bad"] == []
    assert IO.check_topk(np.array([[0, 1, 7, 9]]), tie, 4)["bad"] == [(0, "order")]


# ---- planted mistakes in copies of the oracle: each must fail a pin above ----

_real = IO.indexer_scores


def _relu_after_weight(q_bits, w, k_bits, bt, act, s1, n):
    out = _real(q_bits, np.abs(w), k_bits, bt, act, s1, n)
    return np.where(np.isfinite(out), out * np.sign(w.sum(axis=1))[:, None], out)


def _no_relu(q_bits, w, k_bits, bt, act, s1, n):
    return _real(q_bits, w, k_bits, bt, act, s1, n) - _real(q_bits ^ np.uint16(0x8000), w, k_bits, bt, act, s1, n)


def _swapped_block_math(q_bits, w, k_bits, bt, act, s1, n):
    bt = np.asarray(bt)
    return _real(q_bits, w, k_bits, bt[:, ::-1].copy(), act, s1, n)


def _inclusive_bound(q_bits, w, k_bits, bt, act, s1, n):
    out = _real(q_bits, w, k_bits, bt, act, s1, n)
    for t in range(out.shape[0]):
        a = int(act[t // s1])
        if a < n:
            out[t, a] = 0.0
    return out


_real_decode = IO.bf16_bits_to_f64


def _decode_shift_15(bits):
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return u32.view(np.float32).astype(np.float64)


def _decode_drops_sign(bits):
    return np.abs(_real_decode(bits))


def _decode_byte_swapped(bits):
    return _real_decode(np.asarray(bits, dtype=np.uint16).byteswap())


@pytest.mark.parametrize("mutant", [_decode_shift_15, _decode_drops_sign, _decode_byte_swapped])
def test_pins_catch_planted_decode_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(IO, "bf16_bits_to_f64", mutant)
    pins = [test_scores_match_scalar_brute_force, test_closed_forms_self_and_negated_key,
            test_bf16_bits_to_f64_every_pattern_matches_struct_route,
            lambda: [test_bf16_bits_to_f64_hand_worked(b, v) for b, v in _BF16_CASES]]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    # the score pins see the mutant through the oracle's own use of the decode
    assert caught >= 2, mutant.__name__


@pytest.mark.parametrize("mutant", [_relu_after_weight, _no_relu, _swapped_block_math, _inclusive_bound])
def test_pins_catch_planted_oracle_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(IO, "indexer_scores", mutant)
    pins = [test_scores_match_scalar_brute_force, test_closed_forms_self_and_negated_key,
            test_one_hot_weights_select_a_head, test_block_permutation_and_dead_rows]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, mutant.__name__
