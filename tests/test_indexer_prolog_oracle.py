"""Pins of the indexer prolog oracle (oracle/prolog_oracle.py, indexer_prolog): "CANN DeepSeek
Indexer attention optimisation", section "Indexer Prolog"; "NPU DeepSeek-V4 model PyPTO
fused-operator optimisation", section "IndexerProlog". A scalar brute force, closed forms,
invariants and planted mistakes. CPU only."""

from __future__ import annotations

import math
import struct

import numpy as np
import pytest

from mla_sparse_top_amd import workloads as W
from oracle import prolog_oracle as P


def _tiny(seed=0, *, tokens=3, hidden=16, q=8, n_heads=2, positions=(3, 0, 15), rotate=True, n_pos=16):
    return W.indexer_prolog_generate(tokens=tokens, hidden=hidden, q_lora_rank=q, n_heads=n_heads,
                                     positions=list(positions), rope_positions=n_pos, rotate=rotate, seed=seed)


def _run(p, **over):
    a = dict(x=p.x, qr=p.qr, w_idx_qb=p.w_idx_qb, w_idx_k=p.w_idx_k, ln_gamma_k=p.ln_gamma_k, ln_beta_k=p.ln_beta_k,
             w_idx_proj=p.w_idx_proj, positions=p.positions, rope_cos=p.rope_cos, rope_sin=p.rope_sin, eps=p.eps,
             n_heads=p.n_heads, rotate=p.rotate)
    a.update(over)
    return P.indexer_prolog(**a)


def _bits(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _dec(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def _fwht(v):
    v = list(v)
    n, h = len(v), 1
    while h < n:
        for i in range(n):
            if i & h == 0:
                v[i], v[i + h] = v[i] + v[i + h], v[i] - v[i + h]
        h *= 2
    return [u / math.sqrt(n) for u in v]


def _brute(p):
    t_n, hid = p.x.shape
    qn, d, nh = p.qr.shape[1], p.head_dim, p.n_heads
    out = []
    for t in range(t_n):
        pos = int(p.positions[t])
        live = 0 <= pos < p.rope_cos.shape[0]
        x = [_dec(p.x[t, k]) for k in range(hid)]
        qr = [_dec(p.qr[t, k]) for k in range(qn)]

        def rope(v):
            for i in range(32):
                a, b = v[64 + 2 * i], v[65 + 2 * i]
                if live:
                    c, s = float(p.rope_cos[pos, i]), float(p.rope_sin[pos, i])
                    v[64 + 2 * i], v[65 + 2 * i] = a * c - b * s, a * s + b * c
                else:
                    v[64 + 2 * i], v[65 + 2 * i] = 0.0, 0.0
            return _fwht(v) if p.rotate else v

        qs = []
        for h in range(nh):
            qs.append(rope([sum(qr[k] * _dec(p.w_idx_qb[h * d + j, k]) for k in range(qn)) for j in range(d)]))
        kv = [sum(x[k] * _dec(p.w_idx_k[j, k]) for k in range(hid)) for j in range(d)]
        mu = sum(kv) / d
        var = sum((v - mu) ** 2 for v in kv) / d
        kv = [(kv[j] - mu) / math.sqrt(var + p.eps) * _dec(p.ln_gamma_k[j]) + _dec(p.ln_beta_k[j]) for j in range(d)]
        w = [sum(x[k] * _dec(p.w_idx_proj[h, k]) for k in range(hid)) / math.sqrt(nh * d) for h in range(nh)]
        out.append((qs, rope(kv), w))
    return out


# ---- pins ----

def _pin_brute_force():
    for rot, pos in ((True, (3, 0, 15)), (False, (7, 16, -1))):
        p = _tiny(1, rotate=rot, positions=pos)
        q, k, w = _run(p)
        for t, (bq, bk, bw) in enumerate(_brute(p)):
            np.testing.assert_allclose(q[t], np.array(bq), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(k[t], np.array(bk), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(w[t], np.array(bw), rtol=1e-11, atol=1e-12)


def _pin_layer_norm_moments():
    """gamma 1, beta 0, eps 0, angle 0, no transform: the key has mean 0 and variance 1."""
    p = _tiny(2, rotate=False, positions=(0, 0, 0))
    _, k, _ = _run(p, ln_gamma_k=_bits(np.ones(128)), ln_beta_k=_bits(np.zeros(128)), eps=0.0,
                   rope_cos=np.ones_like(p.rope_cos), rope_sin=np.zeros_like(p.rope_sin))
    np.testing.assert_allclose(k.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((k * k).mean(axis=1), 1.0, rtol=1e-13)


def _pin_scores_unchanged_by_the_transform():
    """The Hadamard transform is orthogonal and applied to query and key alike: every q . k is
    the same with and without it, while the vectors themselves change."""
    p = _tiny(3, tokens=4, n_heads=3, positions=(1, 5, 9, 2))
    q1, k1, _ = _run(p, rotate=True)
    q0, k0, _ = _run(p, rotate=False)
    s1 = np.einsum("thd,ud->thu", q1, k1)
    s0 = np.einsum("thd,ud->thu", q0, k0)
    np.testing.assert_allclose(s1, s0, rtol=1e-11, atol=1e-12)
    assert not np.allclose(q1, q0)


def _pin_weights_selector():
    """Projection rows that each pick one hidden channel (times 2): w = 2 x[ch_h] / sqrt(H * D)."""
    p = _tiny(4, n_heads=4, hidden=16)
    sel = np.array([3, 0, 15, 7])
    wp = np.zeros((4, 16), np.float32)
    wp[np.arange(4), sel] = 2.0
    _, _, w = _run(p, w_idx_proj=_bits(wp))
    x = P.bf16_bits_to_f64(p.x)
    np.testing.assert_allclose(w, 2.0 * x[:, sel] / math.sqrt(4 * 128), rtol=1e-15)


def _pin_first_half_not_rotated():
    """Without the transform only the second half of the head dimension turns: the first 64
    channels of q and k do not depend on the position."""
    a = _run(_tiny(5, rotate=False, positions=(2, 3, 4)))
    b = _run(_tiny(5, rotate=False, positions=(9, 10, 11)))
    np.testing.assert_array_equal(a[0][:, :, :64], b[0][:, :, :64])
    np.testing.assert_array_equal(a[1][:, :64], b[1][:, :64])
    assert not np.allclose(a[0][:, :, 64:], b[0][:, :, 64:])


def _pin_hadamard_last():
    v = np.random.default_rng(6).standard_normal((3, 128))
    for row in v:
        np.testing.assert_allclose(P.hadamard_last(row), _fwht(row), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(P.hadamard_last(np.eye(128)[1]), np.tile([1.0, -1.0], 64) / math.sqrt(128),
                               rtol=1e-15)


PINS = [_pin_brute_force, _pin_layer_norm_moments, _pin_scores_unchanged_by_the_transform, _pin_weights_selector,
        _pin_first_half_not_rotated, _pin_hadamard_last]


@pytest.mark.parametrize("pin", PINS, ids=[f.__name__[5:] for f in PINS])
def test_pin(pin):
    pin()


def test_decode_workload_shapes():
    p = W.indexer_prolog_decode()
    assert p.x.shape == (128, 7168) and p.qr.shape == (128, 1536) and p.w_idx_qb.shape == (64 * 128, 1536)
    assert p.w_idx_k.shape == (128, 7168) and p.w_idx_proj.shape == (64, 7168) and p.rotate


# ---- planted mistakes ----

_ORIG = {n: getattr(P, n) for n in ("layer_norm", "hadamard_last", "rope_interleaved", "indexer_prolog")}


def _ln_rms(v, g, b, eps):
    v = np.asarray(v, np.float64)
    return v / np.sqrt((v * v).mean(axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64) + np.asarray(b, np.float64)


def _ln_sample_var(v, g, b, eps):
    v = np.asarray(v, np.float64)
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).sum(axis=-1, keepdims=True) / (v.shape[-1] - 1)
    return (v - mu) / np.sqrt(var + eps) * np.asarray(g, np.float64) + np.asarray(b, np.float64)


def _q_only(*a, **kw):
    rot = kw.get("rotate", a[12] if len(a) > 12 else False)
    kw2 = dict(kw)
    if len(a) > 12:
        a = a[:12]
    kw2["rotate"] = False
    q, k, w = _ORIG["indexer_prolog"](*a, **kw2)
    return (P.hadamard_last(q) if rot else q), k, w


def _no_weight_scale(*a, **kw):
    q, k, w = _ORIG["indexer_prolog"](*a, **kw)
    return q, k, w * np.sqrt(kw.get("n_heads", 2) * 128)


MUTANTS = {
    "layer norm without the mean (an RMSNorm)": ("layer_norm", _ln_rms),
    "layer norm with the sample variance": ("layer_norm", _ln_sample_var),
    "hadamard unnormalised": ("hadamard_last", lambda v: _ORIG["hadamard_last"](v) * np.sqrt(np.shape(v)[-1])),
    "rope sign flipped": ("rope_interleaved", lambda v, c, s: _ORIG["rope_interleaved"](v, c, -np.asarray(s))),
    "transform on the query only": ("indexer_prolog", _q_only),
    "weights without 1/sqrt(heads * dim)": ("indexer_prolog", _no_weight_scale),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(P, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin catches: {name}"
