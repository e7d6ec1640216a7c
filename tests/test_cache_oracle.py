"""Pins of the cache-write oracle (oracle/cache_oracle.py) against what the page and the
mathematics fix: hand-derived rounding cases (tests/golden/int8_quant_cases.txt), exact rational
arithmetic for the scale and the nearest-integer property, a scalar brute force, the page
mapping of positions to rows, and invariants of the write. No GPU needed.

Source: "DeepSeek V3/V2 Sparse Flash Attention with Quantization", sections "INT8 quantisation
rule" (groups of 128, absmax scale, codes in [-128, 127]) and "Algorithm overview"
(PagedAttention: 128-row blocks through block_table).
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.cache_oracle as C
import oracle.sfa_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "int8_quant_cases.txt")


def _bits(x) -> np.ndarray:
    """fp32 values that are exactly bf16 -> their bf16 bit patterns (asserts exactness)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & np.uint32(0xFFFF)), "value is not a bf16 number"
    return (u >> np.uint32(16)).astype(np.uint16)


def _random_rows(rng, rows, scale=1.0):
    x = (rng.standard_normal((rows, 512)) * scale).astype(np.float32)
    return O.f32_to_bf16_bits_rne(x)


def _f32_of_bits(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        a, x, q = line.split()[:3]
        cases.append((float(a), float(x), int(q)))
    assert len(cases) >= 15
    return cases


def test_golden_rounding_cases():
    for absmax, x, code in _golden_cases():
        g = np.zeros(512, dtype=np.float32)
        g[0] = absmax
        g[5] = x if x != absmax else 0.0
        if x == absmax or x == -absmax:
            g[0] = x
        codes, scales = C.quantize_groups(_bits(g)[None, :])
        assert scales[0, 0] == np.float32(abs(absmax) / 127.0 if absmax in (127.0, 254.0) else scales[0, 0])
        got = codes[0, 0] if abs(x) == absmax else codes[0, 5]
        assert got == code, (absmax, x, got, code)
        assert np.all(scales[0, 1:] == 0) and np.all(codes[0, 128:] == 0)


def _nearest_f32(fr: Fraction) -> np.float32:
    """The binary32 value nearest to a positive rational, ties to even (by checking neighbours)."""
    c = np.float32(float(fr))  # within one ulp; fix up exactly
    best = c
    for cand in (np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))):
        d_c, d_b = abs(Fraction(float(cand)) - fr), abs(Fraction(float(best)) - fr)
        if d_c < d_b or (d_c == d_b and (cand.view(np.uint32) & 1) == 0 and cand != best):
            best = cand
    return np.float32(best)


def test_scale_is_nearest_fp32_to_absmax_over_127():
    rng = np.random.default_rng(1)
    bits = _random_rows(rng, 16, scale=3.0)
    _, scales = C.quantize_groups(bits)
    x = _f32_of_bits(bits).reshape(16, 4, 128)
    for r in range(16):
        for g in range(4):
            am = Fraction(float(np.abs(x[r, g]).max()))
            assert scales[r, g] == _nearest_f32(am / 127), (r, g)


def test_codes_are_nearest_integers_and_extremes_are_127():
    rng = np.random.default_rng(2)
    bits = _random_rows(rng, 24)
    codes, scales = C.quantize_groups(bits)
    x = _f32_of_bits(bits).reshape(24, 4, 128)
    q = codes.reshape(24, 4, 128).astype(np.int64)
    ties = 0
    for r in range(24):
        for g in range(4):
            s = Fraction(float(scales[r, g]))
            am = np.abs(x[r, g]).max()
            for i in range(128):
                exact = Fraction(float(x[r, g, i])) / s
                dist = abs(exact - q[r, g, i])
                # the quotient is rounded to fp32 before the integer rounding: 2^-16 of slack
                assert dist <= Fraction(1, 2) + Fraction(1, 1 << 16), (r, g, i, float(exact), q[r, g, i])
                if dist == Fraction(1, 2):
                    ties += 1
                    assert q[r, g, i] % 2 == 0
                if abs(x[r, g, i]) == am:
                    assert q[r, g, i] == (127 if x[r, g, i] > 0 else -127)
    assert q.min() >= -127 and q.max() <= 127


def _scalar_quantize(vals):
    """Brute force for one group: pure Python, exact rationals for the quotient, with the fp32
    roundings the reading fixes done by numpy on single scalars."""
    am = max(abs(v) for v in vals)
    if am == 0:
        return [0] * len(vals), 0.0
    s = float(np.float32(np.float32(am) / np.float32(127)))
    out = []
    for v in vals:
        qf = float(np.float32(np.float32(v) / np.float32(s)))
        lo = int(np.floor(qf))
        frac = Fraction(qf) - lo
        if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
            lo += 1
        out.append(max(-128, min(127, lo)))
    return out, s


def test_matches_scalar_brute_force():
    rng = np.random.default_rng(3)
    bits = _random_rows(rng, 3, scale=0.01)
    codes, scales = C.quantize_groups(bits)
    x = _f32_of_bits(bits).reshape(3, 4, 128)
    for r in range(3):
        for g in range(4):
            want, s = _scalar_quantize([float(v) for v in x[r, g]])
            assert float(scales[r, g]) == s
            assert list(codes[r, 128 * g:128 * (g + 1)].astype(int)) == want


def test_zero_group_and_single_element_group():
    g = np.zeros((1, 512), dtype=np.float32)
    g[0, 130] = -0.375  # group 1: one non-zero element
    codes, scales = C.quantize_groups(_bits(g))
    assert scales[0, 0] == 0 and scales[0, 2] == 0 and scales[0, 3] == 0
    assert np.all(codes[0, :128] == 0) and np.all(codes[0, 256:] == 0)
    assert codes[0, 130] == -127 and np.count_nonzero(codes[0, 128:256]) == 1
    # an all-zero group dequantises to exact zeros through the attention oracle's chain
    deq = O.dequant_int8_chain(codes, scales)
    assert np.all(deq[0, :128] == 0)


def test_round_trip_error_bound():
    """The dequantised value (the attention's chain) is within half a scale step of the input,
    plus the bf16 rounding of the chain."""
    rng = np.random.default_rng(4)
    bits = _random_rows(rng, 32)
    codes, scales = C.quantize_groups(bits)
    x = _f32_of_bits(bits).astype(np.float64)
    deq = O.dequant_int8_chain(codes, scales)
    step = np.repeat(scales.astype(np.float64), 128, axis=1)
    bound = 0.5 * step * (1 + 2.0 ** -16) + np.abs(deq) * 2.0 ** -8
    assert np.all(np.abs(deq - x) <= bound)


def test_target_rows_hand_worked():
    bt = np.array([[3, 0, -1], [1, 2, 4]], dtype=np.int32)  # pool of 5 blocks = 640 rows
    pos = np.array([0, 130, 300, -1, 127, 383, 384, 200], dtype=np.int32)
    # s1 = 4: tokens 0..3 belong to batch 0, tokens 4..7 to batch 1
    rows = C.target_rows(pos, bt, 4, 640)
    assert list(rows) == [3 * 128 + 0, 0 * 128 + 2, -1, -1, 1 * 128 + 127, 4 * 128 + 127, -1, 2 * 128 + 72]
    # a block past the pool is not written
    assert list(C.target_rows(np.array([1]), np.array([[5]]), 1, 640)) == [-1]


def test_target_rows_agree_with_attention_resolve():
    """The write and the attention's read resolve a position to the same row (two independent
    codings of the page mapping)."""
    rng = np.random.default_rng(5)
    bt = rng.permutation(16).reshape(4, 4).astype(np.int32)
    pos = rng.integers(0, 512, size=8).astype(np.int32)
    rows = C.target_rows(pos, bt, 2, 16 * 128)
    act = np.full(4, 512, dtype=np.int32)
    rr = O.resolve_rows(pos.reshape(8, 1), bt, act, 2)
    assert np.array_equal(rows, rr[:, 0])


def _pool(rng, n_blocks, int8):
    rows = n_blocks * 128
    rope = rng.integers(0, 1 << 16, size=(rows, 64), dtype=np.uint16)
    if int8:
        return rng.integers(-128, 128, size=(rows, 512), dtype=np.int8), rope, rng.random((rows, 4), dtype=np.float32)
    return rng.integers(0, 1 << 16, size=(rows, 512), dtype=np.uint16), rope, None


@pytest.mark.parametrize("int8", [False, True])
def test_write_touches_only_target_rows(int8):
    rng = np.random.default_rng(6)
    kn, kr, ks = _pool(rng, 6, int8)
    bt = np.array([[2, 5], [0, 4]], dtype=np.int32)
    pos = np.array([0, 255, -1, 17], dtype=np.int32)  # s1 = 2
    new_n, new_r = _random_rows(rng, 4), rng.integers(0, 1 << 16, size=(4, 64), dtype=np.uint16)
    kn2, kr2, ks2 = C.cache_write(new_n, new_r, pos, bt, 2, kn, kr, ks)
    rows = [2 * 128 + 0, 5 * 128 + 127, 0 * 128 + 17]
    toks = [0, 1, 3]
    mask = np.ones(kr.shape[0], dtype=bool)
    mask[rows] = False
    assert np.array_equal(kn2[mask], kn[mask]) and np.array_equal(kr2[mask], kr[mask])
    assert np.array_equal(kr2[rows], new_r[toks])
    if int8:
        codes, scales = C.quantize_groups(new_n[toks])
        assert np.array_equal(kn2[rows], codes) and np.array_equal(ks2[rows], scales)
        assert np.array_equal(ks2[mask], ks[mask])
    else:
        assert np.array_equal(kn2[rows], new_n[toks])


def test_write_is_invariant_under_block_permutation():
    rng = np.random.default_rng(7)
    kn, kr, ks = _pool(rng, 8, True)
    bt = rng.permutation(8).reshape(2, 4).astype(np.int32)
    pos = rng.permutation(512)[:6].astype(np.int32)
    new_n, new_r = _random_rows(rng, 6), rng.integers(0, 1 << 16, size=(6, 64), dtype=np.uint16)
    a = C.cache_write(new_n, new_r, pos, bt, 3, kn, kr, ks)
    perm = rng.permutation(8)
    def move(t):
        m = np.empty_like(t.reshape(8, 128, -1))
        m[perm] = t.reshape(8, 128, -1)
        return m.reshape(t.shape)
    b = C.cache_write(new_n, new_r, pos, perm[bt].astype(np.int32), 3, move(kn), move(kr), move(ks))
    for x, y in zip(a, b):
        assert np.array_equal(move(x), y)


def test_write_then_attention_reads_back_the_dequantised_row():
    """A single key written through the cache write and read by the attention oracle returns the
    chain-dequantised row (the attention's single-key closed form)."""
    rng = np.random.default_rng(8)
    kn, kr, ks = _pool(rng, 2, True)
    bt = np.array([[1, 0]], dtype=np.int32)
    new_n, new_r = _random_rows(rng, 1), O.f32_to_bf16_bits_rne(rng.standard_normal((1, 64)).astype(np.float32))
    kn2, kr2, ks2 = C.cache_write(new_n, new_r, np.array([200], dtype=np.int32), bt, 1, kn, kr, ks)
    rows = O.resolve_rows(np.array([[200, -1]]), bt, np.array([256]), 1)
    r = rows[0][rows[0] >= 0]
    kn_g, kr_g = O.gather_latents(r, kn2, kr2, ks2)
    q = O.bf16_bits_to_f64(O.f32_to_bf16_bits_rne(rng.standard_normal((4, 512)).astype(np.float32)))
    qr = O.bf16_bits_to_f64(O.f32_to_bf16_bits_rne(rng.standard_normal((4, 64)).astype(np.float32)))
    out = O.sparse_mla_attention_token(q, qr, kn_g, kr_g, 0.05)
    assert np.array_equal(kr_g[0], O.bf16_bits_to_f64(new_r[0]))
    codes, scales = C.quantize_groups(new_n)
    want = O.dequant_int8_chain(codes, scales)[0]
    assert np.allclose(out.reshape(4, 512), want[None, :], rtol=0, atol=1e-12)


def test_512_wide_rows_match_the_nope_part_of_576_rows():
    """Zero-width rope arrays (the 512-wide layout): the write of the 512 channels is the nope
    part of the same write with rope rows beside it, bit for bit, for both cache types."""
    from mla_sparse_top_amd import workloads as W

    for kv in ("int8", "bf16"):
        inp = W.cache_write_generate(batch=3, s1=7, n_pool_blocks=9, max_blocks_per_batch=3, kv_dtype=kv, seed=12,
                                     rope_dim=0)
        assert inp.new_rope.shape == (21, 0) and inp.key_rope.shape == (9 * 128, 0)
        n0, r0, s0 = C.cache_write(inp.new_nope, inp.new_rope, inp.positions, inp.block_table, 7, inp.key_nope,
                                   inp.key_rope, inp.k_nope_scales)
        rng = np.random.default_rng(13)
        nr = rng.integers(0, 1 << 16, (21, 64)).astype(np.uint16)
        kr = rng.integers(0, 1 << 16, (9 * 128, 64)).astype(np.uint16)
        n1, r1, s1 = C.cache_write(inp.new_nope, nr, inp.positions, inp.block_table, 7, inp.key_nope, kr,
                                   inp.k_nope_scales)
        assert r0.shape == (9 * 128, 0) and np.array_equal(n0, n1)
        if kv == "int8":
            assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
        assert inp.n_written() == 21 and np.sum(np.any(n0 != inp.key_nope, axis=1)) > 0


def test_duplicate_targets_rejected():
    rng = np.random.default_rng(9)
    kn, kr, ks = _pool(rng, 1, False)
    with pytest.raises(ValueError):
        C.cache_write(_random_rows(rng, 2), kr[:2], np.array([3, 3]), np.array([[0]]), 2, kn, kr, ks)


# ---- planted mistakes (CPU only): each must make at least one pin above fail ----------------

_real_quant = C.quantize_groups
_real_rows = C.target_rows


def _q_generic(bits, scale_div=127.0, rounder=np.rint):
    x = C._bf16_bits_to_f32(bits).reshape(-1, 4, 128)
    am = np.abs(x).max(axis=2)
    s = (am / np.float32(scale_div)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s).astype(np.float32)
    q = np.clip(rounder((x / safe[:, :, None]).astype(np.float32)), -128, 127)
    q = np.where((s == 0)[:, :, None], 0, q)
    return q.astype(np.int8).reshape(-1, 512), s


_MUTANTS = {
    "floor": lambda b: _q_generic(b, rounder=np.floor),
    "ties_away": lambda b: _q_generic(b, rounder=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)),
    "scale_128": lambda b: _q_generic(b, scale_div=128.0),
    "trunc": lambda b: _q_generic(b, rounder=np.trunc),
    "group_roll": lambda b: tuple((lambda q, s: (q, np.roll(s, 1, axis=1)))(*_real_quant(b))),
}


def _rows_swapped(positions, bt, s1, n):
    p = np.asarray(positions, dtype=np.int64)
    swapped = np.where(p >= 0, (p % 128) * 128 + p // 128, p)
    return _real_rows(swapped, bt, s1, n)


_PINS = [test_golden_rounding_cases, test_scale_is_nearest_fp32_to_absmax_over_127,
         test_codes_are_nearest_integers_and_extremes_are_127, test_matches_scalar_brute_force,
         test_round_trip_error_bound, test_target_rows_hand_worked, test_target_rows_agree_with_attention_resolve,
         test_write_then_attention_reads_back_the_dequantised_row]


@pytest.mark.parametrize("name", sorted(_MUTANTS) + ["rows_swapped"])
def test_some_pin_catches_planted_mistake(name, monkeypatch):
    if name == "rows_swapped":
        monkeypatch.setattr(C, "target_rows", _rows_swapped)
    else:
        monkeypatch.setattr(C, "quantize_groups", _MUTANTS[name])
    caught = 0
    for pin in _PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught, f"no pin caught {name}"
