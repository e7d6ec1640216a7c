"""CPU oracle for the sliding-window + compressed-cache attention variants (SWA, CFA, SCFA) --
TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU-baseline leg import this module. The GPU path shares no
code with it.

What it computes ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section "FA-class
operators: SWA, CFA and SCFA"): the attention of a query token runs over cache rows from two
sources. The original cache (ori_kv) contributes a sliding window of the most recent positions;
the compressed cache (cmp_kv) contributes either every causal entry (CFA) or the entries a
sparse index list selects (SCFA); SWA has the window alone. The attention itself is the one of
"DeepSeek V3/V2 Sparse Flash Attention with Quantization" (scores over [nope|rope], softmax of
scale * S, V = nope), applied to the union of the two row sets, so this module builds the row
sets and hands them to the pinned attention core of oracle.sfa_oracle.

Readings (the page gives the names and the two sources, not these details; each is listed with
its reason in the design notes):
  * query token t = b * s1 + s sits at position p = ori_len[b] - s1 + s (the s1 newest
    positions of its sequence, as in decode with MTP; prefill is s1 = ori_len);
  * the window is the positions max(0, p - window + 1) .. p of ori_kv;
  * compressed entries come as an index list per token (-1 padding), valid iff
    0 <= j < cmp_len[b]; for CFA the caller lists every causal entry;
  * both caches are rows of one paged pool with block_size 128; each has its own block table;
  * duplicates across the two sources count once per occurrence (a gather list);
  * rows of the page's D = 512 configuration (the head size its timing table gives these
    operators): query and cache rows are 512 channels whose last 64 already carry the rotary
    embedding (the page's MlaProlog and Compressor rotate them in place), the score runs over
    all 512 and V is the same row. Such inputs carry zero-width rope arrays, so the formula
    below applies unchanged (the rope term of the score is an empty sum).
"""

from __future__ import annotations

import numpy as np

from . import sfa_oracle as O

BLOCK_SIZE = 128


def query_positions(ori_len, s1: int) -> np.ndarray:
    """Position of each query token in its sequence: ori_len[b] - s1 + s."""
    ori_len = np.asarray(ori_len, dtype=np.int64)
    b = np.arange(len(ori_len) * s1) // s1
    s = np.arange(len(ori_len) * s1) % s1
    return ori_len[b] - s1 + s


def window_positions(p: int, window: int) -> list:
    """The window of a query at position p: max(0, p - window + 1) .. p (empty when p < 0)."""
    if p < 0 or window <= 0:
        return []
    return list(range(max(0, p - window + 1), p + 1))


def _row(bt_row, j: int, num_rows: int) -> int:
    blk = int(bt_row[j // BLOCK_SIZE])
    if blk < 0:
        return -1
    r = blk * BLOCK_SIZE + j % BLOCK_SIZE
    return r if r < num_rows else -1


def token_rows(t: int, s1: int, window: int, cmp_indices, bt_ori, bt_cmp, ori_len, cmp_len, num_rows: int) -> list:
    """Physical rows token t attends to: its window over ori_kv, then its valid compressed
    entries over cmp_kv, in that order."""
    b = t // s1
    p = int(ori_len[b]) - s1 + t % s1
    rows = []
    for j in window_positions(p, window):
        if j < bt_ori.shape[1] * BLOCK_SIZE:
            r = _row(bt_ori[b], j, num_rows)
            if r >= 0:
                rows.append(r)
    if cmp_indices is not None:
        for j in np.asarray(cmp_indices[t], dtype=np.int64):
            if 0 <= j < int(cmp_len[b]) and j < bt_cmp.shape[1] * BLOCK_SIZE:
                r = _row(bt_cmp[b], int(j), num_rows)
                if r >= 0:
                    rows.append(r)
    return rows


def window_attention(inp, tokens=None) -> np.ndarray:
    """The variant over an input instance (fields as in workloads.WindowInputs): float64
    (B, S1, N_Q, 512), or (len(tokens), N_Q, 512) for a token subset."""
    h = inp.n_q
    toks = range(inp.batch * inp.s1) if tokens is None else list(tokens)
    out = np.zeros((len(toks), h, O.KV_LORA_RANK), dtype=np.float64)
    for i, t in enumerate(toks):
        rows = token_rows(t, inp.s1, inp.window, inp.cmp_indices, inp.block_table_ori, inp.block_table_cmp,
                          inp.ori_len, inp.cmp_len, inp.num_cache_rows)
        kn, kr = O.gather_latents(np.asarray(rows, dtype=np.int64), inp.key_nope, inp.key_rope, inp.k_nope_scales)
        qn = O.bf16_bits_to_f64(inp.query_nope[t * h:(t + 1) * h])
        qr = O.bf16_bits_to_f64(inp.query_rope[t * h:(t + 1) * h])
        out[i] = O.sparse_mla_attention_token(qn, qr, kn, kr, inp.softmax_scale)
    if tokens is None:
        return out.reshape(inp.batch, inp.s1, h, O.KV_LORA_RANK)
    return out
