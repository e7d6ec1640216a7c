"""Pins of the compressor oracle ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation",
section "Compressor"): closed forms, an invariant, a scalar brute force, the refresh / emission
rules, and planted mistakes that each pin set must catch. CPU only."""

from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.linalg

from mla_sparse_top_amd import workloads as W
from oracle import compress_oracle as C

C_ = C.CHANNELS


def _small(seed=0, *, ratio=4, s1=2, start=6, batch=2, n_pos=64, score_scale=1.0, channels=576, rotate=False):
    return W.compress_generate(batch=batch, s1=s1, ratio=ratio, start_pos=[start] * batch, rope_positions=n_pos,
                               max_blocks=2, seed=seed, score_scale=score_scale, channels=channels, rotate=rotate)


def _rope_complex(x, cos, sin):
    """RoPE as complex multiplication: pair (a, b) is a + ib, times cos + i sin."""
    z = (x[0::2] + 1j * x[1::2]) * (cos.astype(np.float64) + 1j * sin.astype(np.float64))
    out = np.empty_like(x)
    out[0::2], out[1::2] = z.real, z.imag
    return out


# ---- pins, written as checks so that the planted mistakes below can run them ----

def _pin_one_slot():
    """ratio 1: the softmax over one slot is 1, so the entry is RoPE(RMSNorm(kv)) of the token."""
    x = _small(ratio=1, s1=1, start=9)
    x.eps = 0.0
    _, _, e = C.compress(x)
    assert len(e) == 2
    for b, c, _, y in e:
        assert c == 9
        kv = x.kv[b].astype(np.float64)
        want = kv * math.sqrt(C_) / np.linalg.norm(kv) * x.gamma.astype(np.float64)
        want[512:] = _rope_complex(want[512:], x.rope_cos[9], x.rope_sin[9])
        np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def _pin_equal_scores_mean():
    """Equal scores in every slot: the pool is the plain mean of the slots."""
    x = _small(ratio=4, s1=1, start=7)
    x.score[:] = 0.0
    x.score_state[:] = 0.0
    x.ape[:] = 0.0
    ks, _, e = C.compress(x)
    for b, _, _, _ in e:
        np.testing.assert_allclose(C.pool(ks[b], np.zeros_like(ks[b])), ks[b].astype(np.float64).mean(axis=0),
                                   rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(C.pool(ks[0], x.score_state[0]), ks[0].astype(np.float64).mean(axis=0), atol=1e-13)


def _pin_per_channel_dominant_slot():
    """A slot far above the others wins its channel alone; which slot wins varies by channel, so
    the softmax must run over the slots for each channel separately."""
    ratio = 4
    kv = np.random.default_rng(1).standard_normal((ratio, C_)).astype(np.float32)
    sc = np.zeros((ratio, C_), dtype=np.float32)
    win = np.arange(C_) % ratio
    sc[win, np.arange(C_)] = 200.0
    np.testing.assert_allclose(C.pool(kv, sc), kv[win, np.arange(C_)].astype(np.float64), rtol=1e-12, atol=1e-12)


def _pin_unit_rms():
    """gamma = 1, eps = 0: the entry has mean square exactly 1, since RoPE rotations keep norms."""
    x = _small(ratio=4, s1=2, start=6, score_scale=3.0)
    x.gamma[:] = 1.0
    x.eps = 0.0
    # tables of exact quarter turns, so that cos^2 + sin^2 = 1 holds exactly in fp32
    k = np.random.default_rng(2).integers(0, 4, size=x.rope_cos.shape)
    x.rope_cos[:] = np.array([1, 0, -1, 0], dtype=np.float32)[k]
    x.rope_sin[:] = np.array([0, 1, 0, -1], dtype=np.float32)[k]
    _, _, e = C.compress(x)
    assert e
    for *_, y in e:
        assert abs(np.mean(y * y) - 1.0) < 1e-12


def _pin_quarter_turn():
    """cos 0, sin 1 maps the pair (a, b) to (-b, a)."""
    v = np.arange(1.0, 65.0)
    y = C.rope_pairs(v, np.zeros(32), np.ones(32))
    np.testing.assert_array_equal(y[0::2], -v[1::2])
    np.testing.assert_array_equal(y[1::2], v[0::2])
    np.testing.assert_array_equal(C.rope_pairs(v, np.ones(32), np.zeros(32)), v)


def _fwht(v):
    """Hadamard transform by the butterfly: for strides h = 1, 2, 4, ..., each pair (i, i + h) with
    bit h of i clear becomes (a + b, a - b); then the 1/sqrt(n) scale."""
    v = list(v)
    n = len(v)
    h = 1
    while h < n:
        for i in range(n):
            if i & h == 0:
                a, b = v[i], v[i + h]
                v[i], v[i + h] = a + b, a - b
        h *= 2
    return [u / math.sqrt(n) for u in v]


def _brute(x):
    """Pure-Python scalar loops over the same steps."""
    C_ = x.channels
    R0 = C_ - 64
    ratio, n_pos = x.ratio, x.rope_cos.shape[0]
    kvs = [[[float(v) for v in x.kv_state[b, r]] for r in range(ratio)] for b in range(x.batch)]
    scs = [[[float(v) for v in x.score_state[b, r]] for r in range(ratio)] for b in range(x.batch)]
    out = []
    for b in range(x.batch):
        for s in range(x.s1):
            t, p = b * x.s1 + s, int(x.start_pos[b]) + s
            if not 0 <= p < n_pos:
                continue
            r0 = p - (p // ratio) * ratio
            kvs[b][r0] = [float(v) for v in x.kv[t]]
            scs[b][r0] = [float(np.float32(x.score[t, ch]) + np.float32(x.ape[r0, ch])) for ch in range(C_)]
            if (p + 1) - ((p + 1) // ratio) * ratio != 0:
                continue
            y = []
            for ch in range(C_):
                m = max(scs[b][r][ch] for r in range(ratio))
                ws = [math.exp(scs[b][r][ch] - m) for r in range(ratio)]
                y.append(sum(ws[r] * kvs[b][r][ch] for r in range(ratio)) / sum(ws))
            ms = sum(v * v for v in y) / C_
            y = [y[ch] / math.sqrt(ms + x.eps) * float(x.gamma[ch]) for ch in range(C_)]
            for i in range(32):
                a, bb = y[R0 + 2 * i], y[R0 + 1 + 2 * i]
                co, si = float(x.rope_cos[p, i]), float(x.rope_sin[p, i])
                y[R0 + 2 * i], y[R0 + 1 + 2 * i] = a * co - bb * si, a * si + bb * co
            if x.rotate:
                y = _fwht(y)
            out.append((b, (p + 1) // ratio - 1, y))
    return kvs, scs, out


def _pin_brute_force():
    for ch, rot in ((576, False), (512, False), (128, False), (128, True)):
        x = _small(seed=3, ratio=3, s1=5, start=1, n_pos=5, channels=ch, rotate=rot)  # positions 1..5; 5 past the tables
        ks, ss, e = C.compress(x)
        bk, bs, be = _brute(x)
        np.testing.assert_array_equal(ks, np.array(bk, dtype=np.float32))
        np.testing.assert_array_equal(ss, np.array(bs, dtype=np.float32))
        assert [(b, c) for b, c, _, _ in e] == [(b, c) for b, c, _ in be] == [(0, 0), (1, 0)]
        for (_, _, _, y), (_, _, yb) in zip(e, be):
            np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)


def _pin_hadamard_rows():
    """The transform's first rows in natural (Sylvester) order: e_0 -> all 1/sqrt(n), e_1 ->
    alternating +-1/sqrt(n), e_2 -> (+, +, -, -, ...); it is its own inverse and keeps norms."""
    n = 128
    e = np.eye(n)
    np.testing.assert_allclose(C.hadamard_rotate(e[0]), np.full(n, n ** -0.5), rtol=1e-15)
    np.testing.assert_allclose(C.hadamard_rotate(e[1]), np.tile([1.0, -1.0], n // 2) * n ** -0.5, rtol=1e-15)
    np.testing.assert_allclose(C.hadamard_rotate(e[2]), np.tile([1.0, 1.0, -1.0, -1.0], n // 4) * n ** -0.5,
                               rtol=1e-15)
    v = np.random.default_rng(7).standard_normal(n)
    np.testing.assert_allclose(C.hadamard_rotate(C.hadamard_rotate(v)), v, rtol=1e-12, atol=1e-13)
    assert abs(np.linalg.norm(C.hadamard_rotate(v)) - np.linalg.norm(v)) < 1e-12
    for m in (2, 8, 64):
        w = np.random.default_rng(m).standard_normal(m)
        np.testing.assert_allclose(C.hadamard_rotate(w), _fwht(w), rtol=1e-12, atol=1e-13)


def _pin_rotated_one_slot():
    """ratio 1, 128 channels, rotate: the entry is H(RoPE(RMSNorm(kv)))/sqrt(128) of the token,
    rebuilt here with the butterfly on a quarter-turn rotation."""
    x = _small(ratio=1, s1=1, start=9, channels=128, rotate=True)
    x.eps = 0.0
    x.gamma[:] = 1.0
    x.rope_cos[9], x.rope_sin[9] = 0.0, 1.0
    _, _, e = C.compress(x)
    assert len(e) == 2
    for b, c, _, y in e:
        kv = x.kv[b].astype(np.float64)
        want = kv * math.sqrt(128) / np.linalg.norm(kv)
        a, bb = want[64::2].copy(), want[65::2].copy()
        want[64::2], want[65::2] = -bb, a
        np.testing.assert_allclose(y, _fwht(want), rtol=1e-12, atol=1e-12)


def _pin_refresh_and_emission():
    """Positions 5..11 at ratio 4: windows close at 7 and 11 (entries 1 and 2); each slot ends
    holding its last writer; the stored score is the fp32 sum with the slot's ape."""
    x = _small(seed=4, ratio=4, s1=7, start=5, batch=1)
    ks, ss, e = C.compress(x)
    assert [c for _, c, _, _ in e] == [1, 2]
    last = {p % 4: s for s, p in enumerate(range(5, 12))}
    for slot, s in last.items():
        np.testing.assert_array_equal(ks[0, slot], x.kv[s])
        np.testing.assert_array_equal(ss[0, slot], (x.score[s] + x.ape[slot]).astype(np.float32))


def _pin_skips_and_rows():
    """Tokens before position 0 or past the tables refresh nothing; entry rows follow the block
    table, and negative blocks, entries past the table and rows past the pool are not written."""
    x = _small(seed=5, ratio=2, s1=4, start=-2, batch=1)
    ks, ss, e = C.compress(x)
    assert [c for _, c, _, _ in e] == [0]                  # positions -2, -1, 0, 1: only 1 closes
    np.testing.assert_array_equal(ks[0, 0], x.kv[2])
    np.testing.assert_array_equal(ks[0, 1], x.kv[3])
    bt = np.array([3, -1], dtype=np.int32)
    assert C.entry_row(bt, 5, 1 << 20) == 3 * 128 + 5
    assert C.entry_row(bt, 130, 1 << 20) == -1
    assert C.entry_row(bt, 256, 1 << 20) == -1
    assert C.entry_row(bt, 5, 3 * 128 + 5) == -1
    assert C.entry_row(bt, -1, 1 << 20) == -1


PINS = [_pin_one_slot, _pin_equal_scores_mean, _pin_per_channel_dominant_slot, _pin_unit_rms, _pin_quarter_turn,
        _pin_brute_force, _pin_refresh_and_emission, _pin_skips_and_rows, _pin_hadamard_rows, _pin_rotated_one_slot]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[5:] for p in PINS])
def test_pin(pin):
    pin()


def test_decode_workload_shape():
    x = W.compress_decode()
    ks, ss, e = C.compress(x)
    assert len(e) == 64 and all(c == 2047 and r >= 0 for _, c, r, _ in e)
    assert len({r for _, _, r, _ in e}) == 64


# ---- planted mistakes: each must make at least one pin fail ----

def _axis_channels(kv_slots, score_slots):
    s = np.asarray(score_slots, dtype=np.float64)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return (w * np.asarray(kv_slots, dtype=np.float64)).sum(axis=0)


_ORIG = {n: getattr(C, n) for n in ("pool", "rope_pairs", "rms_norm", "hadamard_rotate", "compressed_row")}


def _walsh_sequency(y):
    """rows ordered by sign changes (Walsh order) instead of the natural order"""
    y = np.asarray(y, np.float64)
    n = len(y)
    h = scipy.linalg.hadamard(n)
    order = np.argsort([np.count_nonzero(np.diff(r) != 0) for r in h], kind="stable")
    return h[order] @ y / np.sqrt(n)


def _rotate_before_rope(kv_slots, score_slots, gamma, eps, cos, sin, rotate=False):
    y = C.rms_norm(C.pool(kv_slots, score_slots), gamma, eps)
    if rotate:
        y = C.hadamard_rotate(y)
    y[-64:] = C.rope_pairs(y[-64:], cos, sin)
    return y

MUTANTS = {
    "softmax over channels": ("pool", _axis_channels),
    "rope sign flipped": ("rope_pairs", lambda x, c, s: _ORIG["rope_pairs"](x, c, -np.asarray(s))),
    "rmsnorm without gamma": ("rms_norm", lambda x, g, e: _ORIG["rms_norm"](x, np.ones_like(g), e)),
    "rmsnorm over sum, not mean": ("rms_norm", lambda x, g, e: np.asarray(x, np.float64) / np.sqrt(
        np.sum(np.asarray(x, np.float64) ** 2) + e) * np.asarray(g, np.float64)),
    "slot off by one": ("slot_of", lambda p, r: (p + 1) % r),
    "emits on p % ratio == 0": ("closes_window", lambda p, r: p % r == 0),
    "entry index off by one": ("entry_index", lambda p, r: (p + 1) // r),
    "pool is the plain mean": ("pool", lambda kv, sc: np.asarray(kv, np.float64).mean(axis=0)),
    "hadamard without 1/sqrt(n)": ("hadamard_rotate", lambda y: _ORIG["hadamard_rotate"](y) * np.sqrt(len(y))),
    "hadamard in sequency order": ("hadamard_rotate", _walsh_sequency),
    "hadamard before RoPE": ("compressed_row", _rotate_before_rope),
    "rotate flag ignored": ("compressed_row", lambda *a, rotate=False: _ORIG["compressed_row"](*a[:6], False)),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(C, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin catches: {name}"
