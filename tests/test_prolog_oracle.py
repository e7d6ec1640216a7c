"""Pins of the MLA prolog oracle ("CANN DeepSeek Indexer attention optimisation", section "MLA
Prolog"; "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section "MlaProlog",
computation steps): a pure-Python scalar brute force, closed forms, invariants, and planted
mistakes that the pins must catch. CPU only."""

from __future__ import annotations

import math
import struct

import numpy as np
import pytest

from mla_sparse_top_amd import workloads as W
from oracle import prolog_oracle as P


def _bits(a) -> np.ndarray:
    """float values that are exact in bf16 -> their bf16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _tiny(seed=0, *, tokens=3, hidden=16, q=8, n_q=2, dn=4, n_pos=16, positions=(3, 0, 15)):
    return W.prolog_generate(tokens=tokens, n_q=n_q, hidden=hidden, q_lora_rank=q, nope_dim=dn,
                             positions=list(positions), rope_positions=n_pos, seed=seed)


def _run(p, **over):
    a = dict(x=p.x, w_dq=p.w_dq, gamma_cq=p.gamma_cq, w_uq_qr=p.w_uq_qr, w_uk=p.w_uk, w_dkv_kr=p.w_dkv_kr,
             gamma_ckv=p.gamma_ckv, positions=p.positions, rope_cos=p.rope_cos, rope_sin=p.rope_sin, eps=p.eps,
             n_q=p.n_q)
    a.update(over)
    return P.mla_prolog(**a)


# ---- a scalar route: struct decode, nested loops, math.sqrt, explicit rotation ----

def _dec(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute(p):
    t_n, h_n = p.x.shape
    qn_rows = p.w_dq.shape[0]
    n_q, dn = p.n_q, p.nope_dim
    x = [[_dec(p.x[t, k]) for k in range(h_n)] for t in range(t_n)]
    out = []
    for t in range(t_n):
        pos = int(p.positions[t])
        live = 0 <= pos < p.rope_cos.shape[0]
        c = [sum(x[t][k] * _dec(p.w_dq[i, k]) for k in range(h_n)) for i in range(qn_rows)]
        inv = 1.0 / math.sqrt(sum(v * v for v in c) / qn_rows + p.eps)
        cq = [c[i] * inv * _dec(p.gamma_cq[i]) for i in range(qn_rows)]
        qn = [[0.0] * 512 for _ in range(n_q)]
        qr = [[0.0] * 64 for _ in range(n_q)]
        for h in range(n_q):
            base = h * (dn + 64)
            u = [sum(cq[i] * _dec(p.w_uq_qr[base + j, i]) for i in range(qn_rows)) for j in range(dn + 64)]
            for cc in range(512):
                qn[h][cc] = sum(u[d] * _dec(p.w_uk[h, cc, d]) for d in range(dn))
            for i in range(32):
                if live:
                    co, si = float(p.rope_cos[pos, i]), float(p.rope_sin[pos, i])
                    a, b = u[dn + 2 * i], u[dn + 2 * i + 1]
                    qr[h][2 * i], qr[h][2 * i + 1] = a * co - b * si, a * si + b * co
        kv = [sum(x[t][k] * _dec(p.w_dkv_kr[r, k]) for k in range(h_n)) for r in range(576)]
        inv = 1.0 / math.sqrt(sum(v * v for v in kv[:512]) / 512 + p.eps)
        kn = [kv[r] * inv * _dec(p.gamma_ckv[r]) for r in range(512)]
        kr = [0.0] * 64
        for i in range(32):
            if live:
                co, si = float(p.rope_cos[pos, i]), float(p.rope_sin[pos, i])
                a, b = kv[512 + 2 * i], kv[512 + 2 * i + 1]
                kr[2 * i], kr[2 * i + 1] = a * co - b * si, a * si + b * co
        out.append((qn, qr, kn, kr))
    return out


# ---- pins, written as checks so that the planted mistakes below can run them ----

def _pin_brute_force():
    """The vectorised oracle equals the scalar route on tiny shapes (one token past the tables)."""
    for seed, pos in ((0, (3, 0, 15)), (1, (7, 16, -1))):
        p = _tiny(seed, positions=pos)
        qn, qr, kn, kr = _run(p)
        for t, (bqn, bqr, bkn, bkr) in enumerate(_brute(p)):
            np.testing.assert_allclose(qn[t], np.array(bqn), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(qr[t], np.array(bqr), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(kn[t], np.array(bkn), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(kr[t], np.array(bkr), rtol=1e-11, atol=1e-12)


def _pin_selector_weights_closed_form():
    """x = 2 e_t and down-projections that copy channels: with gamma 1 and eps 0 the normalised
    vectors are sqrt(width) e_t, so u is sqrt(Q) times column t of w_uq_qr; with w_uk the identity
    on its first dn channels, q_nope is that column's nope part (then zeros), q_rope its rope
    part turned by a quarter turn (cos 0, sin 1: (a, b) -> (-b, a)); kv_nope is sqrt(512) e_t and
    kv_rope is x's channels 512.. turned the same way."""
    t_n, h_n, q, n_q, dn = 3, 640, 8, 2, 4
    p = _tiny(2, tokens=t_n, hidden=h_n, q=q, n_q=n_q, dn=dn, positions=(5, 5, 5))
    x = np.zeros((t_n, h_n), np.float32)
    for t in range(t_n):
        x[t, t] = 2.0
        x[t, 512 + 2 * t] = 0.5      # a rope channel of the key
    w_dq = np.eye(q, h_n, dtype=np.float32)
    w_dkv = np.eye(576, h_n, dtype=np.float32)
    w_uk = np.zeros((n_q, 512, dn), np.float32)
    for h in range(n_q):
        w_uk[h, :dn, :dn] = np.eye(dn)
    cos = p.rope_cos.copy()
    sin = p.rope_sin.copy()
    cos[5], sin[5] = 0.0, 1.0
    qn, qr, kn, kr = _run(p, x=_bits(x), w_dq=_bits(w_dq), w_dkv_kr=_bits(w_dkv), w_uk=_bits(w_uk),
                          gamma_cq=_bits(np.ones(q)), gamma_ckv=_bits(np.ones(512)), eps=0.0, rope_cos=cos,
                          rope_sin=sin)
    wq = P.bf16_bits_to_f64(p.w_uq_qr)
    for t in range(t_n):
        col = math.sqrt(q) * wq[:, t].reshape(n_q, dn + 64)
        for h in range(n_q):
            np.testing.assert_allclose(qn[t, h, :dn], col[h, :dn], rtol=1e-14, atol=1e-15)
            assert np.all(qn[t, h, dn:] == 0.0)
            a, b = col[h, dn::2], col[h, dn + 1::2]
            np.testing.assert_allclose(qr[t, h, 0::2], -b, rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(qr[t, h, 1::2], a, rtol=1e-14, atol=1e-15)
        want = np.zeros(512)
        want[t] = math.sqrt(512)
        np.testing.assert_allclose(kn[t], want, rtol=1e-14, atol=1e-15)
        want_r = np.zeros(64)
        want_r[2 * t + 1] = 0.5         # (0.5, 0) turned by a quarter turn is (0, 0.5)
        np.testing.assert_allclose(kr[t], want_r, rtol=0, atol=1e-15)


def _pin_scale_invariance():
    """eps 0: doubling x leaves the normalised outputs (everything that passes through an RMSNorm)
    exactly unchanged and doubles the rotary key, which is not normalised."""
    p = _tiny(3)
    x2 = _bits(P.bf16_bits_to_f64(p.x) * 2.0)
    a = _run(p, eps=0.0)
    b = _run(p, eps=0.0, x=x2)
    for i in range(3):
        assert np.array_equal(a[i], b[i])
    assert np.array_equal(b[3], 2.0 * a[3])


def _pin_unit_mean_square():
    """gamma 1, eps 0: the latent row has mean square 1."""
    p = _tiny(4)
    kn = _run(p, eps=0.0, gamma_ckv=_bits(np.ones(512)))[2]
    np.testing.assert_allclose(np.mean(kn * kn, axis=1), 1.0, rtol=1e-13)


def _pin_zero_angle_and_rotation_norm():
    """Position 0 of the tables is angle 0 (cos 1, sin 0): q_rope is the rope part of u as is,
    and at any position each rotated pair keeps its length (to the fp32 tables' cos^2 + sin^2 = 1,
    about 1e-7)."""
    p = _tiny(5, positions=(0, 9, 0))
    base = _run(p, rope_cos=np.ones_like(p.rope_cos), rope_sin=np.zeros_like(p.rope_sin))
    got = _run(p)
    for t in (0, 2):
        np.testing.assert_allclose(got[1][t], base[1][t], rtol=1e-15, atol=0)
        np.testing.assert_allclose(got[3][t], base[3][t], rtol=1e-15, atol=0)
    for o, b0 in ((got[1][1], base[1][1]), (got[3][1], base[3][1])):
        ln = np.hypot(o[..., 0::2], o[..., 1::2])
        lb = np.hypot(b0[..., 0::2], b0[..., 1::2])
        np.testing.assert_allclose(ln, lb, rtol=1e-6)
        assert not np.allclose(o, b0)


def _pin_head_permutation():
    """Permuting the heads' rows of w_uq_qr and of w_uk permutes the heads of the query outputs
    exactly, and leaves the key outputs unchanged."""
    p = _tiny(6, n_q=3)
    perm = np.array([2, 0, 1])
    dn = p.nope_dim
    wq = p.w_uq_qr.reshape(3, dn + 64, -1)[perm].reshape(p.w_uq_qr.shape)
    a = _run(p)
    b = _run(p, w_uq_qr=wq, w_uk=p.w_uk[perm])
    assert np.array_equal(b[0], a[0][:, perm])
    assert np.array_equal(b[1], a[1][:, perm])
    assert np.array_equal(b[2], a[2]) and np.array_equal(b[3], a[3])


def _pin_positions_outside_tables():
    """A token whose position lies outside the tables gets zero rotary outputs and its other
    outputs unchanged."""
    p = _tiny(7, positions=(2, 2, 2))
    a = _run(p)
    b = _run(p, positions=np.array([2, -1, 16], np.int32))
    for t in (1, 2):
        assert np.all(b[1][t] == 0) and np.all(b[3][t] == 0)
        assert np.array_equal(b[0][t], a[0][t]) and np.array_equal(b[2][t], a[2][t])
    assert np.array_equal(b[1][0], a[1][0])


PINS = [_pin_brute_force, _pin_selector_weights_closed_form, _pin_scale_invariance, _pin_unit_mean_square,
        _pin_zero_angle_and_rotation_norm, _pin_head_permutation, _pin_positions_outside_tables]


@pytest.mark.parametrize("pin", PINS, ids=[f.__name__[5:] for f in PINS])
def test_pin(pin):
    pin()


def test_decode_workload_shapes():
    p = W.prolog_decode()
    assert p.x.shape == (128, 7168) and p.w_dq.shape == (1536, 7168) and p.w_uq_qr.shape == (128 * 192, 1536)
    assert p.w_uk.shape == (128, 512, 128) and p.w_dkv_kr.shape == (576, 7168)
    assert set(p.positions.tolist()) == {8190, 8191} and p.rope_positions == 8192


# ---- planted mistakes: each must make at least one pin fail ----

_ORIG = {n: getattr(P, n) for n in ("rms_norm", "rope_interleaved", "split_heads", "absorb", "rope_rows")}


def _rope_halves(v, c, s):
    """rotate-half pairing (v[i], v[i+32]) instead of adjacent pairs"""
    v = np.asarray(v, np.float64)
    h = v.shape[-1] // 2
    a, b = v[..., :h], v[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _split_rope_first(u, n_q, dn):
    u = u.reshape(u.shape[0], n_q, dn + 64)
    return u[:, :, 64:], u[:, :, :64]


def _split_planar(u, n_q, dn):
    """all heads' nope parts first, then all rope parts"""
    qn = u[:, : n_q * dn].reshape(u.shape[0], n_q, dn)
    qp = u[:, n_q * dn:].reshape(u.shape[0], n_q, 64)
    return qn, qp


def _absorb_reshaped(qn, wuk):
    """w_uk taken as (N, dn, 512) row-major"""
    w = wuk.reshape(wuk.shape[0], wuk.shape[2], wuk.shape[1]).transpose(0, 2, 1)
    return np.einsum("thd,hcd->thc", qn, w)


def _rows_next(positions, c, s):
    return _ORIG["rope_rows"](np.asarray(positions) + 1, c, s)


MUTANTS = {
    "rope sign flipped": ("rope_interleaved", lambda v, c, s: _ORIG["rope_interleaved"](v, c, -np.asarray(s))),
    "rope on halves, not adjacent pairs": ("rope_interleaved", _rope_halves),
    "rmsnorm without gamma": ("rms_norm", lambda v, g, e: _ORIG["rms_norm"](v, np.ones_like(g), e)),
    "rmsnorm over the sum, not the mean": ("rms_norm", lambda v, g, e: np.asarray(v, np.float64) / np.sqrt(
        np.sum(np.asarray(v, np.float64) ** 2, axis=-1, keepdims=True) + e) * np.asarray(g, np.float64)),
    "rmsnorm eps outside the root": ("rms_norm", lambda v, g, e: np.asarray(v, np.float64) / (np.sqrt(
        np.mean(np.asarray(v, np.float64) ** 2, axis=-1, keepdims=True)) + e + 1e-3) * np.asarray(g, np.float64)),
    "head rows rope first": ("split_heads", _split_rope_first),
    "heads split planar": ("split_heads", _split_planar),
    "w_uk read transposed": ("absorb", _absorb_reshaped),
    "position off by one": ("rope_rows", _rows_next),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(P, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin catches: {name}"


def test_key_norm_covering_the_rotary_part_is_caught(monkeypatch):
    """A latent RMSNorm taken over all 576 key channels (rotary part included) is caught."""
    orig = P.mla_prolog

    def mutant(x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin, eps, n_q):
        qn, qr, _, _ = orig(x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin,
                            eps, n_q)
        kv = P.bf16_bits_to_f64(x) @ P.bf16_bits_to_f64(w_dkv_kr).T
        inv = 1.0 / np.sqrt(np.mean(kv * kv, axis=1, keepdims=True) + eps)
        cos, sin, live = P.rope_rows(positions, rope_cos, rope_sin)
        kn = kv[:, :512] * inv * P.bf16_bits_to_f64(gamma_ckv)
        kr = P.rope_interleaved(kv[:, 512:] * inv, cos, sin)
        kr[~live] = 0.0
        return qn, qr, kn, kr

    monkeypatch.setattr(P, "mla_prolog", mutant)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


# ---- the V4 form (mla_prolog_v4): 512-wide query heads and latent row, rotary part inside ----

def _tiny_v4(seed=0, *, tokens=3, hidden=16, q=8, n_q=2, n_pos=16, positions=(3, 0, 17)):
    return W.prolog_v4_generate(tokens=tokens, n_q=n_q, hidden=hidden, q_lora_rank=q, positions=list(positions),
                                rope_positions=n_pos, seed=seed)


def _run_v4(p, **over):
    a = dict(x=p.x, w_dq=p.w_dq, gamma_cq=p.gamma_cq, w_uq=p.w_uq, w_dkv=p.w_dkv, gamma_ckv=p.gamma_ckv,
             positions=p.positions, rope_cos=p.rope_cos, rope_sin=p.rope_sin, eps=p.eps, n_q=p.n_q)
    a.update(over)
    return P.mla_prolog_v4(**a)


def _brute_v4(p):
    """Scalar route: struct decode, loops, math.sqrt, each pair turned by hand."""
    t_n, h_n = p.x.shape
    qr_n = p.w_dq.shape[0]
    x = [[_dec(p.x[t, k]) for k in range(h_n)] for t in range(t_n)]
    out = []
    for t in range(t_n):
        pos = int(p.positions[t])
        live = 0 <= pos < p.rope_cos.shape[0]

        def turn(v):
            for i in range(32):
                a, b = v[448 + 2 * i], v[449 + 2 * i]
                if live:
                    c, s = float(p.rope_cos[pos, i]), float(p.rope_sin[pos, i])
                    v[448 + 2 * i], v[449 + 2 * i] = a * c - b * s, a * s + b * c
                else:
                    v[448 + 2 * i], v[449 + 2 * i] = 0.0, 0.0
            return v

        c = [sum(x[t][k] * _dec(p.w_dq[i, k]) for k in range(h_n)) for i in range(qr_n)]
        inv = 1.0 / math.sqrt(sum(v * v for v in c) / qr_n + p.eps)
        cq = [c[i] * inv * _dec(p.gamma_cq[i]) for i in range(qr_n)]
        heads = []
        for h in range(p.n_q):
            u = [sum(cq[i] * _dec(p.w_uq[h * 512 + j, i]) for i in range(qr_n)) for j in range(512)]
            iu = 1.0 / math.sqrt(sum(v * v for v in u) / 512 + p.eps)
            heads.append(turn([v * iu for v in u]))
        k = [sum(x[t][m] * _dec(p.w_dkv[j, m]) for m in range(h_n)) for j in range(512)]
        ik = 1.0 / math.sqrt(sum(v * v for v in k) / 512 + p.eps)
        out.append((heads, turn([k[j] * ik * _dec(p.gamma_ckv[j]) for j in range(512)])))
    return out


def _pin_v4_brute_force():
    """The vectorised V4 form equals the scalar route (one token past the tables)."""
    for seed, pos in ((0, (3, 0, 17)), (1, (15, -1, 8))):
        p = _tiny_v4(seed, positions=pos)
        q, kv = _run_v4(p)
        for t, (bq, bkv) in enumerate(_brute_v4(p)):
            np.testing.assert_allclose(q[t], np.array(bq), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(kv[t], np.array(bkv), rtol=1e-11, atol=1e-12)


def _pin_v4_unit_mean_square():
    """At angle zero (table row 0) each query head has mean square ms / (ms + eps) of its raw
    projection (unit weight), and kv / gamma the same for the latent row."""
    p = _tiny_v4(2, positions=(0, 0, 0))
    q, kv = _run_v4(p)
    X = P.bf16_bits_to_f64(p.x)
    cq = P.rms_norm(X @ P.bf16_bits_to_f64(p.w_dq).T, P.bf16_bits_to_f64(p.gamma_cq), p.eps)
    raw = (cq @ P.bf16_bits_to_f64(p.w_uq).T).reshape(3, p.n_q, 512)
    ms = np.mean(raw * raw, axis=-1)
    np.testing.assert_allclose(np.mean(q * q, axis=-1), ms / (ms + p.eps), rtol=1e-12)
    rk = X @ P.bf16_bits_to_f64(p.w_dkv).T
    mk = np.mean(rk * rk, axis=-1)
    kn = kv / P.bf16_bits_to_f64(p.gamma_ckv)
    np.testing.assert_allclose(np.mean(kn * kn, axis=-1), mk / (mk + p.eps), rtol=1e-12)


def _pin_v4_scale_invariance_and_quarter_turn():
    """With eps 0, scaling x by 2 (exact in bf16) changes nothing; a quarter turn (cos 0, sin 1)
    maps each rotary pair (a, b) of the zero-angle result to (-b, a) and leaves the rest alone."""
    p = _tiny_v4(3, positions=(0, 1, 2))
    q0, k0 = _run_v4(p, eps=0.0)
    x2 = (p.x.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # bf16 exponent + 1: times 2
    q1, k1 = _run_v4(p, x=x2, eps=0.0)
    np.testing.assert_allclose(q1, q0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(k1, k0, rtol=1e-12, atol=1e-13)
    cos = np.zeros((3, 32), np.float32)
    sin = np.ones((3, 32), np.float32)
    one = np.ones((3, 32), np.float32)
    qz, kz = _run_v4(p, rope_cos=one, rope_sin=np.zeros((3, 32), np.float32))
    qt, kt = _run_v4(p, rope_cos=cos, rope_sin=sin)
    for a, b in ((qz, qt), (kz, kt)):
        np.testing.assert_array_equal(b[..., :448], a[..., :448])
        np.testing.assert_array_equal(b[..., 448::2], -a[..., 449::2])
        np.testing.assert_array_equal(b[..., 449::2], a[..., 448::2])


V4_PINS = [_pin_v4_brute_force, _pin_v4_unit_mean_square, _pin_v4_scale_invariance_and_quarter_turn]


@pytest.mark.parametrize("pin", V4_PINS, ids=[f.__name__[5:] for f in V4_PINS])
def test_v4_pin(pin):
    pin()


def test_v4_decode_workload_shapes():
    p = W.prolog_v4_decode()
    assert p.x.shape == (128, 4096) and p.w_uq.shape == (128 * 512, 1536) and p.w_dkv.shape == (512, 4096)
    assert set(p.positions.tolist()) == {8190, 8191}


_ORIG_V4 = {n: getattr(P, n) for n in ("head_rms_norm", "rope_last")}


def _norm_whole_row(q, eps):
    t = q.shape[0]
    return _ORIG_V4["head_rms_norm"](q.reshape(t, -1), eps).reshape(q.shape)


def _rope_first(v, c, s, live):
    out = np.array(v, dtype=np.float64, copy=True)
    out[..., :64] = P.rope_interleaved(out[..., :64], c, s)
    out[~live, ..., :64] = 0.0
    return out


def _rope_no_zeroing(v, c, s, live):
    return _ORIG_V4["rope_last"](v, c, s, np.ones_like(live))


V4_MUTANTS = {
    "query norm over all heads at once": ("head_rms_norm", _norm_whole_row),
    "query norm with the key's gamma": ("head_rms_norm", lambda q, e: P.rms_norm(q, 1.0 + 0.1 * np.arange(
        q.shape[-1]) / q.shape[-1], e)),
    "rope on the first 64 channels": ("rope_last", _rope_first),
    "out-of-table positions rotated by row 0": ("rope_last", _rope_no_zeroing),
}


@pytest.mark.parametrize("name", list(V4_MUTANTS))
def test_v4_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = V4_MUTANTS[name]
    monkeypatch.setattr(P, attr, fn)
    failed = 0
    for pin in V4_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin catches: {name}"
