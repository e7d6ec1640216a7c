"""fp64 CPU oracle for DeepSeek-style sparse flash attention (SFA) over a paged MLA latent cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU baseline import
this module. The GPU path shares no code with it, and it shares none with the GPU path.

What it computes (sources, by page title and section):
  * "CANN DeepSeek Indexer attention optimisation" (custom_pypto.npu_sparse_attention_pto),
    section "Sparse Flash Attention": for each query token, attention restricted to the cache
    entries (MLA latents) that the indexer ranked in its top-k.
  * "DeepSeek V3/V2 Sparse Flash Attention with Quantization", sections "Algorithm overview",
    "Operator specification" and "Implementation notes":
      - the query and key are each split into a 512-d nope part and a 64-d rope part, and the
        two parts are concatenated for the score;
      - the cache is paged in blocks of 128 rows, and block_table maps each batch's logical
        block to a physical block;
      - kv_act_seqs gives each batch's live length;
      - the value is the nope part of the key, and the output has 512 columns;
      - optionally the nope part is INT8 with one FP32 scale per 128-element group. The
        dequant path casts INT8 -> FP16 -> FP32, multiplies by the group scale, and casts
        the product to BF16 before use;
      - the score is scaled before the softmax: Softmax(S * scale).

Written out, for token t of batch b, head h and valid slot set V_t:
    score[k] = scale * (q_nope[t,h] . Kn[k] + q_rope[t,h] . Kr[k])
    w        = softmax over k in V_t of score
    out[t,h] = sum over k in V_t of w[k] * Kn[k]
The method (decode softmax, or the prefill online max/sum/output update) reaches exactly this
value up to rounding order. So the oracle is this dense definition, in float64, with no tiling.

Readings of points the pages leave open (each is listed with its reason in the design notes):
  * A slot is valid iff 0 <= index < kv_act_seqs[b]. Other slots (-1 padding, past the live
    length) are masked wherever they sit in the row. Both query tokens of a batch share the
    bound.
  * A token with no valid slot outputs zeros.
  * Duplicate indices count once per occurrence, like a gather list.
  * The INT8 chain rounds twice: first to FP32 (RNE), then to BF16 (RNE).

Inputs are raw bit patterns (bf16 as uint16), exactly the bytes the GPU path receives.

Every function here is pinned by a test in tests/test_oracle_pins.py against closed forms,
library routines, hand-derived goldens (tests/golden/) or a scalar brute force.
"""

from __future__ import annotations

import numpy as np

KV_LORA_RANK = 512
ROPE_DIM = 64
BLOCK_SIZE = 128
QUANT_GROUP = 128


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE binary32. Widening (to fp32, then fp64) is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_rne(x) -> np.ndarray:
    """Round binary32 values to bfloat16 bit patterns, to nearest with ties to even.

    In the bit pattern, add 0x7FFF plus the lowest kept bit, then drop the low 16 bits. A carry
    into the exponent is correct rounding, up to and including overflow to infinity. A NaN stays
    a NaN, made quiet.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = (u >> np.uint64(16)) | np.uint64(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def dequant_int8_chain(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """INT8 k_nope -> the bf16 values the attention uses, returned as float64.

    This follows the cast chain of "DeepSeek V3/V2 Sparse Flash Attention with Quantization"
    (sections "INT8 quantisation path" and the PyPTO API table's cast entry):
      1. INT8 -> FP16 -> FP32. Both steps are exact, since |code| <= 128.
      2. Multiply by the FP32 scale of the element's 128-group. numpy's float32 multiply rounds
         the product to nearest even.
      3. Cast to BF16, round to nearest even (f32_to_bf16_bits_rne above).
    codes: int8 (R, 512); scales: float32 (R, 4). Group g covers columns [128g, 128g+128).
    """
    c = np.asarray(codes, dtype=np.int8)
    s = np.asarray(scales, dtype=np.float32)
    assert c.shape[-1] == KV_LORA_RANK and s.shape[-1] == KV_LORA_RANK // QUANT_GROUP
    c32 = c.astype(np.float16).astype(np.float32)
    s_per_col = np.repeat(s, QUANT_GROUP, axis=-1)
    prod = (c32 * s_per_col).astype(np.float32)
    return bf16_bits_to_f64(f32_to_bf16_bits_rne(prod))


def resolve_rows(topk_indices: np.ndarray, block_table: np.ndarray, kv_act_seqs: np.ndarray,
                 s1: int) -> np.ndarray:
    """Logical top-k slot -> physical cache row, or -1 for a masked slot.

    Token t belongs to batch b = t // s1. For slot index j, the slot is valid iff
    0 <= j < kv_act_seqs[b]. A valid slot's row is block_table[b, j // 128] * 128 + j % 128
    (PagedAttention, blocks of 128 rows).
    """
    idx = np.asarray(topk_indices, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    act = np.asarray(kv_act_seqs, dtype=np.int64)
    n_tok = idx.shape[0]
    b_of_t = np.arange(n_tok) // s1
    live = act[b_of_t][:, None]
    valid = (idx >= 0) & (idx < live)
    if valid.any():
        assert int((idx[valid] // BLOCK_SIZE).max()) < bt.shape[1], \
            "a valid index names a block past max_blocks_per_batch"
    safe = np.where(valid, idx, 0)
    blocks = bt[b_of_t[:, None], safe // BLOCK_SIZE]
    rows = blocks * BLOCK_SIZE + safe % BLOCK_SIZE
    return np.where(valid, rows, -1)


def gather_latents(rows: np.ndarray, key_nope: np.ndarray, key_rope: np.ndarray,
                   k_nope_scales) -> tuple:
    """Gather the cache rows named by `rows` (all valid) and decode them to float64.
    Returns (Kn (n, 512), Kr (n, 64)). For an int8 cache, Kn follows the INT8 -> bf16 chain."""
    rows = np.asarray(rows, dtype=np.int64)
    if key_nope.dtype == np.int8:
        kn = dequant_int8_chain(key_nope[rows], k_nope_scales[rows])
    else:
        kn = bf16_bits_to_f64(key_nope[rows])
    kr = bf16_bits_to_f64(key_rope[rows])
    return kn, kr


def sparse_mla_attention_token(qn: np.ndarray, qr: np.ndarray, kn: np.ndarray, kr: np.ndarray,
                               scale: float) -> np.ndarray:
    """One token, all heads: dense softmax attention over the gathered latents, in float64.
    qn (H, 512), qr (H, 64), kn (n, 512), kr (n, 64) -> out (H, 512). An empty set gives zeros.
    """
    h = qn.shape[0]
    if kn.shape[0] == 0:
        return np.zeros((h, KV_LORA_RANK), dtype=np.float64)
    scores = float(scale) * (qn @ kn.T + qr @ kr.T)
    scores = scores - scores.max(axis=1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ kn


def sparse_mla_attention(inp, tokens=None) -> np.ndarray:
    """Full operation over an input instance (fields as in mla_sparse_top_amd.workloads.SfaInputs,
    or any object with the same attributes). Returns float64 (B, S1, N_Q, 512).

    tokens: optional iterable of token ids (b*s1 + s). When given, the result has only those
    tokens (shape (len(tokens), N_Q, 512)), which keeps large instances within CPU budgets.
    """
    h = inp.n_q
    rows_all = resolve_rows(inp.topk_indices, inp.block_table, inp.kv_act_seqs, inp.s1)
    toks = range(inp.batch * inp.s1) if tokens is None else list(tokens)
    out = np.zeros((len(toks), h, KV_LORA_RANK), dtype=np.float64)
    for i, t in enumerate(toks):
        r = rows_all[t]
        r = r[r >= 0]
        kn, kr = gather_latents(r, inp.key_nope, inp.key_rope, inp.k_nope_scales)
        qn = bf16_bits_to_f64(inp.query_nope[t * h:(t + 1) * h])
        qr = bf16_bits_to_f64(inp.query_rope[t * h:(t + 1) * h])
        out[i] = sparse_mla_attention_token(qn, qr, kn, kr, inp.softmax_scale)
    if tokens is None:
        return out.reshape(inp.batch, inp.s1, h, KV_LORA_RANK)
    return out


def allclose_report(got: np.ndarray, ref: np.ndarray, rtol: float = 5e-3, atol: float = 1e-4) -> dict:
    """Element-wise |got - ref| <= atol + rtol * |ref| on every element (the operation's stated
    accuracy standard, read as a strict all-element check). Returns the fail count, the worst
    ratio err / bound and where it sits."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = atol + rtol * np.abs(ref)
    err = np.abs(got - ref)
    bad = ~(err <= bound)  # NaN counts as a failure
    ratio = np.where(np.isfinite(err), err / bound, np.inf)
    worst = int(np.argmax(ratio)) if ratio.size else 0
    return {
        "n": int(ref.size),
        "fails": int(bad.sum()),
        "worst_ratio": float(ratio.flat[worst]) if ratio.size else 0.0,
        "worst_index": np.unravel_index(worst, ref.shape) if ratio.size else None,
        "max_abs_err": float(np.nanmax(err)) if err.size else 0.0,
    }
