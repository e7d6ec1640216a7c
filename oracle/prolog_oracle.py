"""CPU oracle for the MLA prolog (hidden state -> absorbed query and latent cache row) -- TEST
INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU-baseline leg import this module. The GPU path shares no
code with it, and it imports nothing from the GPU path or from the input generators.

What it computes. "CANN DeepSeek Indexer attention optimisation", section "MLA Prolog": the
prolog turns the hidden state X into the query and the latent key/value with DeepSeek V3's
structure, and in decode it uses weight absorption; its parameter list names a query
down-projection w_dq with the RMSNorm scale gamma_cq, a query up-projection that also yields
the rotary part (w_uq_qr), the absorption weight w_uk, a down-projection that yields the latent
row and the rotary key (w_dkv_kr) with the RMSNorm scale gamma_ckv, and sin/cos tables.
"NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section "MlaProlog", computation
steps: the query is a down-projection, RMSNorm, up-projection, with interleaved RoPE on the
last rope_dim channels; the key is a projection, RMSNorm, and the same RoPE on its last
rope_dim channels. For one token t (hidden row x):

  cq        = RMSNorm(x . w_dq^T) * gamma_cq                            (Q channels)
  u         = cq . w_uq_qr^T ;  per head h: qn_h = u[h, :Dn],  qp_h = u[h, Dn:Dn+64]
  q_nope[h] = qn_h . w_uk[h]^T                                          (absorbed: 512 channels)
  q_rope[h] = RoPE(qp_h, p)
  kv        = x . w_dkv_kr^T ;  kv_nope = RMSNorm(kv[:512]) * gamma_ckv ;  kv_rope = RoPE(kv[512:], p)

Readings (each is listed with its reason in the design notes):
  * the layout is the one the sparse attention consumes (512 latent + 64 rotary channels per
    row, absorbed query per head); the V4 page's second query RMSNorm (unit weight) and its
    512-wide key with the rotary part inside belong to the V4 layout and are not applied;
  * weights are (out_features, in_features) row-major; head h owns rows h*(Dn+64) + [0, Dn)
    (nope) and + [Dn, Dn+64) (rope) of w_uq_qr; w_uk is (N, 512, Dn); w_dkv_kr rows [0, 512)
    are the latent row and [512, 576) the rotary key;
  * the pages fix the inputs and weights as bf16 and the products' outputs as fp32, but not
    the precision of the values handed from one step to the next (cq, qn_h); they are taken
    unrounded, so the prolog is the exact composition of its steps. (Rounding them to bf16
    on both sides does not give a checkable definition: a one-ulp difference in cq or qn_h,
    which fp32 and fp64 arithmetic reach in different places, moves q_nope by more than the
    output tolerance in about 0.4 % of elements);
  * RMSNorm(v) = v / sqrt(mean(v^2) + eps), then times gamma, per token over that vector;
  * RoPE rotates adjacent pairs (2i, 2i+1) by the angle whose cosine and sine are row p,
    column i of the caller's tables, p = positions[t]; a token whose p lies outside the tables
    gets zero rotary outputs;
  * the four outputs are stored as bf16 (round to nearest even); this oracle returns them
    before that last rounding, in float64.

Pinned by tests/test_prolog_oracle.py: a pure-Python scalar brute force on tiny shapes, closed
forms (identity absorption, quarter-turn and zero-angle rotation, scale invariance of the
normalised outputs, unit mean square), head permutation, and planted mistakes. The indexer
prolog at the end of this module is pinned in tests/test_indexer_prolog_oracle.py.

The V4 form (mla_prolog_v4 below) follows "NPU DeepSeek-V4 model PyPTO fused-operator
optimisation", section "MlaProlog", computation steps, in its own layout: the query of head h is
RMSNorm(cq . w_uq^T) over that head's 512 channels with unit weight (the page's second RMSNorm,
whose weight is fixed at 1), then RoPE in place on its last 64 channels; the latent row is
RMSNorm(x . w_dkv^T) * gamma_ckv over 512 channels, then RoPE in place on its last 64. No
weight absorption and no separate rotary outputs: query rows and the latent row are 512 wide
with the rotary part inside, the rows the 512-wide window attention reads. Its readings:
per-head normalisation (the rotation is applied to the last axis, so the query's last axis is
the head's 512 channels); the same RoPE, table and out-of-table rule as above; cq unrounded
between the steps. Pinned in tests/test_prolog_oracle.py (scalar brute force, unit mean square,
scale invariance, quarter turn, planted mistakes).
"""

from __future__ import annotations

import numpy as np

LATENT = 512
ROPE = 64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: the pattern is the upper half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def rms_norm(v: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * gamma over the last axis."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)


def rope_interleaved(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotates the pairs (v[..., 2i], v[..., 2i+1]) by the angle with cosine cos[..., i] and sine
    sin[..., i] (cos and sin broadcast against the pair axis)."""
    v = np.asarray(v, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def rope_rows(positions, rope_cos, rope_sin):
    """Per token, the table row of its position: (cos (T, 32), sin (T, 32), live (T,)); a token
    whose position lies outside the tables gets row 0 and live = False."""
    pos = np.asarray(positions, dtype=np.int64)
    n_pos = np.asarray(rope_cos).shape[0]
    live = (pos >= 0) & (pos < n_pos)
    safe = np.where(live, pos, 0)
    return (np.asarray(rope_cos, dtype=np.float64)[safe], np.asarray(rope_sin, dtype=np.float64)[safe], live)


def split_heads(u: np.ndarray, n_q: int, dn: int):
    """The up-projection's output (T, n_q*(dn+64)) as per-head nope (T, n_q, dn) and rope
    (T, n_q, 64) parts: head h owns channels h*(dn+64) + [0, dn) and + [dn, dn+64)."""
    u = u.reshape(u.shape[0], n_q, dn + ROPE)
    return u[:, :, :dn], u[:, :, dn:]


def absorb(qn: np.ndarray, wuk: np.ndarray) -> np.ndarray:
    """Weight absorption: q_nope[t, h, c] = sum over d of qn[t, h, d] * w_uk[h, c, d]."""
    return np.einsum("thd,hcd->thc", qn, wuk)


def mla_prolog(x, w_dq, gamma_cq, w_uq_qr, w_uk, w_dkv_kr, gamma_ckv, positions, rope_cos, rope_sin, eps,
               n_q: int):
    """The prolog over T tokens. bf16 arrays arrive as uint16 bit patterns: x (T, H), w_dq (Q, H),
    gamma_cq (Q), w_uq_qr (n_q*(Dn+64), Q), w_uk (n_q, 512, Dn), w_dkv_kr (576, H),
    gamma_ckv (512). positions int32 (T); rope_cos / rope_sin float32 (P, 32).

    Returns float64 arrays before the final bf16 rounding: q_nope (T, n_q, 512),
    q_rope (T, n_q, 64), kv_nope (T, 512), kv_rope (T, 64)."""
    X = bf16_bits_to_f64(x)
    wuk = bf16_bits_to_f64(w_uk)
    cos, sin, live = rope_rows(positions, rope_cos, rope_sin)

    # query: down-projection, RMSNorm with gamma_cq, up-projection split per head into the nope
    # part (which feeds the absorption) and the rope part
    cq = rms_norm(X @ bf16_bits_to_f64(w_dq).T, bf16_bits_to_f64(gamma_cq), eps)
    qn, qp = split_heads(cq @ bf16_bits_to_f64(w_uq_qr).T, n_q, wuk.shape[2])
    q_nope = absorb(qn, wuk)
    q_rope = rope_interleaved(qp, cos[:, None, :], sin[:, None, :])
    q_rope[~live] = 0.0

    # key: down-projection into the latent row (RMSNorm with gamma_ckv) and the rotary key
    kv = X @ bf16_bits_to_f64(w_dkv_kr).T
    kv_nope = rms_norm(kv[:, :LATENT], bf16_bits_to_f64(gamma_ckv), eps)
    kv_rope = rope_interleaved(kv[:, LATENT:LATENT + ROPE], cos, sin)
    kv_rope[~live] = 0.0
    return q_nope, q_rope, kv_nope, kv_rope


def head_rms_norm(q: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with unit weight over the last axis (each head's channels)."""
    return rms_norm(q, np.ones(q.shape[-1]), eps)


def rope_last(v: np.ndarray, cos: np.ndarray, sin: np.ndarray, live: np.ndarray) -> np.ndarray:
    """v with its last ROPE channels rotated in place (pairs as rope_interleaved; cos / sin
    broadcast against them), zero where the token's position is outside the tables."""
    out = np.array(v, dtype=np.float64, copy=True)
    out[..., -ROPE:] = rope_interleaved(out[..., -ROPE:], cos, sin)
    out[~live, ..., -ROPE:] = 0.0
    return out


def mla_prolog_v4(x, w_dq, gamma_cq, w_uq, w_dkv, gamma_ckv, positions, rope_cos, rope_sin, eps, n_q: int):
    """The V4 prolog over T tokens. bf16 arrays arrive as uint16 bit patterns: x (T, H),
    w_dq (Q, H), gamma_cq (Q), w_uq (n_q*512, Q) (head h owns rows h*512 .. +512), w_dkv (512, H),
    gamma_ckv (512). Returns float64 before the final bf16 rounding: q (T, n_q, 512) and
    kv (T, 512), each with its rotary part in its last 64 channels."""
    X = bf16_bits_to_f64(x)
    cos, sin, live = rope_rows(positions, rope_cos, rope_sin)
    cq = rms_norm(X @ bf16_bits_to_f64(w_dq).T, bf16_bits_to_f64(gamma_cq), eps)
    q = (cq @ bf16_bits_to_f64(w_uq).T).reshape(X.shape[0], n_q, LATENT)
    q = rope_last(head_rms_norm(q, eps), cos[:, None, :], sin[:, None, :], live)
    kv = rms_norm(X @ bf16_bits_to_f64(w_dkv).T, bf16_bits_to_f64(gamma_ckv), eps)
    kv = rope_last(kv, cos, sin, live)
    return q, kv


# ---- Indexer prolog ---------------------------------------------------------------------
# "CANN DeepSeek Indexer attention optimisation", section "Indexer Prolog": the index query of
# head h is RoPE(RMSNorm(X W_qa) W_qb), the index key RoPE(LayerNorm(X W_k)); RoPE only on the
# second half of the head dimension; the per-head weights w_h of the Lightning Indexer come from
# a projection of x. "NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
# "IndexerProlog": the query's rotary part is the part after nope_dim, the result goes through
# a Hadamard transform, and the weights are x . weights_proj times 1 / sqrt(heads * head_dim).
# Readings: qr (RMSNorm(X W_qa) times its scale) is the MLA prolog's normalised query, taken
# as a bf16 input; LayerNorm(v) = (v - mean) / sqrt(var + eps) * gamma + beta, with the
# population variance; rotate applies the same Sylvester Hadamard transform (scaled by
# 1/sqrt(head_dim)) to the query of every head and to the key, after RoPE; the V4 page's INT8
# quantisation of the query is not applied (the Lightning Indexer here scores bf16 queries).

def hadamard_last(v: np.ndarray) -> np.ndarray:
    """H v / sqrt(n) over the last axis, H the Sylvester Hadamard matrix of order n (symmetric,
    natural order), n a power of two."""
    import scipy.linalg

    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    return v @ scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)


def layer_norm(v: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """(v - mean) / sqrt(var + eps) * gamma + beta over the last axis (population variance)."""
    v = np.asarray(v, dtype=np.float64)
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    return (v - mu) / np.sqrt(var + float(eps)) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def indexer_prolog(x, qr, w_idx_qb, w_idx_k, ln_gamma_k, ln_beta_k, w_idx_proj, positions, rope_cos, rope_sin,
                   eps, n_heads: int, rotate: bool):
    """bf16 inputs as uint16 bits: x (T, H), qr (T, Q), w_idx_qb (n_heads*D, Q), w_idx_k (D, H),
    ln_gamma_k / ln_beta_k (D), w_idx_proj (n_heads, H). Returns float64 before the outputs'
    rounding: q_index (T, n_heads, D), k_index (T, D), weights (T, n_heads)."""
    X = bf16_bits_to_f64(x)
    t = X.shape[0]
    wk = bf16_bits_to_f64(w_idx_k)
    d = wk.shape[0]
    cos, sin, live = rope_rows(positions, rope_cos, rope_sin)
    half = d - ROPE

    q = (bf16_bits_to_f64(qr) @ bf16_bits_to_f64(w_idx_qb).T).reshape(t, n_heads, d)
    q[:, :, half:] = rope_interleaved(q[:, :, half:], cos[:, None, :], sin[:, None, :])
    q[~live, :, half:] = 0.0
    k = layer_norm(X @ wk.T, bf16_bits_to_f64(ln_gamma_k), bf16_bits_to_f64(ln_beta_k), eps)
    k[:, half:] = rope_interleaved(k[:, half:], cos, sin)
    k[~live, half:] = 0.0
    if rotate:
        q = hadamard_last(q)
        k = hadamard_last(k)
    w = (X @ bf16_bits_to_f64(w_idx_proj).T) / np.sqrt(n_heads * d)
    return q, k, w
