"""fp64 CPU oracle for the Lightning Indexer scores and the top-k selection that feeds sparse
flash attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU baseline import
this module. The GPU path shares no code with it.

What it computes (source: "CANN DeepSeek Indexer attention optimisation"
(custom_pypto.npu_sparse_attention_pto), sections "Lightning Indexer" and "Sparse Flash
Attention"):
  * for query token i and cache position j, the index score is a multi-query, MLP-like sum over
    the index heads h: I[i, j] = sum_h w[i, h] * ReLU(q_index[i, h] . k_index[j]), where the
    head weights w[i, :] are per query token (the Indexer Prolog computes them);
  * the attention of token i then runs over the k positions with the largest I[i, :].

Readings of points the pages leave open (listed with reasons in the design notes):
  * k_index lives in a paged cache with the same block table and live lengths as the latent
    cache (the function prototype passes index_k_cache beside block_table and act_seqs).
    Position j of batch b is live iff 0 <= j < kv_act_seqs[b]; its row is
    block_table[b][j // 128] * 128 + j % 128. Both query tokens of a batch share the bound.
  * Only live positions are candidates. With fewer live positions than k, all of them are
    selected and the rest of the row is -1.
  * Equal scores at the selection boundary may be broken either way; a selection is correct
    iff it holds min(k, live) distinct live positions and no unselected live position scores
    above a selected one.

Inputs are raw bit patterns (bf16 as uint16), exactly the bytes the GPU path receives.
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 128


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE binary32; widening is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def live_rows(block_table: np.ndarray, act: int, b: int) -> np.ndarray:
    """Physical row of each live position j < act of batch b (PagedAttention, blocks of 128)."""
    j = np.arange(int(act), dtype=np.int64)
    return np.asarray(block_table, dtype=np.int64)[b, j // BLOCK_SIZE] * BLOCK_SIZE + j % BLOCK_SIZE


def indexer_scores(q_bits: np.ndarray, weights: np.ndarray, k_bits: np.ndarray, block_table: np.ndarray,
                   kv_act_seqs: np.ndarray, s1: int, n_positions: int) -> np.ndarray:
    """I[t, j] for every token t and position j < n_positions, in float64; -inf where j is not
    live. q_bits (T, H, D) bf16 bits, weights (T, H) float32, k_bits (rows, D) bf16 bits."""
    q = bf16_bits_to_f64(q_bits)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    k = bf16_bits_to_f64(k_bits)
    n_tok = q.shape[0]
    out = np.full((n_tok, n_positions), -np.inf)
    for t in range(n_tok):
        b = t // s1
        act = int(kv_act_seqs[b])
        if act <= 0:
            continue
        rows = live_rows(block_table, act, b)
        dots = q[t] @ k[rows].T                      # (H, act)
        out[t, :act] = w[t] @ np.maximum(dots, 0.0)  # sum over heads of w_h * ReLU(.)
    return out


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """One correct selection: for each row, the k largest finite scores (ties to the lower
    position), as positions in descending score order, padded with -1."""
    scores = np.asarray(scores)
    out = np.full((scores.shape[0], k), -1, dtype=np.int32)
    for t in range(scores.shape[0]):
        live = np.nonzero(np.isfinite(scores[t]))[0]
        order = live[np.lexsort((live, -scores[t][live]))]
        sel = order[:k]
        out[t, :len(sel)] = sel
    return out


def check_topk(selected: np.ndarray, scores: np.ndarray, k: int) -> dict:
    """Whether `selected` (T, k) is a correct top-k of `scores` (T, N), where -inf marks a
    position that is not live. Per row: the non-negative entries come first and are distinct
    live positions, there are min(k, live) of them, the rest are -1, and no unselected live
    position scores above the lowest selected score."""
    selected = np.asarray(selected)
    scores = np.asarray(scores)
    bad = []
    for t in range(scores.shape[0]):
        row = selected[t]
        live = np.isfinite(scores[t])
        n_live = int(live.sum())
        want = min(k, n_live)
        pos = row[row >= 0]
        if len(pos) != want or not np.all(row[:want] >= 0) or not np.all(row[want:] == -1):
            bad.append((t, "count"))
            continue
        if len(np.unique(pos)) != want or np.any(pos >= scores.shape[1]) or not np.all(live[pos]):
            bad.append((t, "invalid"))
            continue
        if want == 0:
            continue
        lowest = scores[t][pos].min()
        rest = live.copy()
        rest[pos] = False
        if np.any(scores[t][rest] > lowest):
            bad.append((t, "order"))
    return {"rows": scores.shape[0], "bad": bad}
