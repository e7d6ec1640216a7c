"""CPU oracle for the compressor that produces compressed-cache rows -- TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU-baseline leg import this module. The GPU path shares no
code with it, and it imports nothing from the GPU path or from the input generators.

What it computes ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
"Compressor", its computation steps): two projections of the hidden state, kv = X W_kv and
score = X W_gate + ape, refresh a per-sequence state (kv_state, score_state). When position p
closes a window (p + 1 is a multiple of the compression ratio), the state is pooled into one
compressed entry: for every channel, the softmax of score_state over the state's slots weights
kv_state, and the weighted sum over the slots is RMS-normalised and then rotated (RoPE). With
rotate = true the row then goes through a Hadamard transform.

Readings (the page gives the formula, not these details; each is listed with its reason in the
design notes):
  * the projections are plain GEMMs outside this step: kv and score arrive as fp32 (T, C), the
    precision the page gives the matmul outputs;
  * C = 576 channels, the row of the compressed cache the window attention reads (512 nope
    channels, then 64 rope channels), C = 512, the same row in the page's D = 512 layout (the
    rotary channels inside the row), or C = 128, the row of a compressed index-key cache (the
    page's D = 128 configuration, whose keys the Lightning Indexer scores); the last 64 channels
    are the rotary ones in all three;
  * the state of sequence b holds `ratio` slots of C channels; the token at position p writes
    slot p mod ratio; ape is (ratio, C), indexed by that slot; the stored score is the fp32 sum
    score + ape[slot];
  * token t = b * s1 + s sits at position p = start_pos[b] + s, and the tokens of a sequence
    refresh the state in order of s; a token is skipped (no refresh, no entry) unless
    0 <= p < rope_positions;
  * the window closed at p is compressed entry c = (p + 1) / ratio - 1; it lands at row
    block_table_cmp[b][c // 128] * 128 + c % 128 of the compressed pool, and is not written if
    c >= max_blocks * 128, the block entry is negative, or the row is outside the pool;
  * the softmax runs over the slots, separately for every channel (dim 1 of the (b, ratio, C)
    state);
  * RMSNorm over all C channels: y = x / sqrt(mean(x^2) + eps) * gamma;
  * RoPE on the 64 rope channels, as 32 adjacent pairs (2i, 2i+1) rotated by the angle whose
    cosine and sine are row p, column i of the caller's tables (p = the closing token's
    position);
  * rotate = true (C = 128 only, a power of two): after RoPE the row is multiplied by the
    Sylvester Hadamard matrix of order C (rows in natural order, H_2n = [[H_n, H_n],
    [H_n, -H_n]]) scaled by 1/sqrt(C), an orthogonal and self-inverse map;
  * the row is stored as bf16, rounded to nearest even.

The arithmetic is float64 except the stored score (an fp32 addition, as stored). Pinned by
tests/test_compress_oracle.py against closed forms (one slot, equal scores, a dominant slot, a
quarter-turn rotation), an invariant (unit RMS under rotation), a pure-Python scalar brute
force, and planted mistakes; the Hadamard step by an explicit butterfly transform, its first
rows, self-inversion and norm preservation.
"""

from __future__ import annotations

import numpy as np
import scipy.linalg

CHANNELS = 576
NOPE = 512
ROPE = 64
BLOCK_SIZE = 128


def slot_of(p: int, ratio: int) -> int:
    """State slot the token at position p refreshes."""
    return p % ratio


def closes_window(p: int, ratio: int) -> bool:
    """The step at position p emits a compressed entry when p + 1 is a multiple of the ratio."""
    return (p + 1) % ratio == 0


def entry_index(p: int, ratio: int) -> int:
    """Index of the compressed entry the window closed at p produces."""
    return (p + 1) // ratio - 1


def entry_row(bt_row, c: int, num_rows: int) -> int:
    """Physical row of compressed entry c through the sequence's block table; -1 = not written."""
    if c < 0 or c >= len(bt_row) * BLOCK_SIZE:
        return -1
    blk = int(bt_row[c // BLOCK_SIZE])
    if blk < 0:
        return -1
    r = blk * BLOCK_SIZE + c % BLOCK_SIZE
    return r if r < num_rows else -1


def pool(kv_slots: np.ndarray, score_slots: np.ndarray) -> np.ndarray:
    """Per channel, the softmax over the slots of the scores weights the kv values; returns the
    weighted sum over the slots. kv_slots, score_slots: (ratio, C)."""
    s = np.asarray(score_slots, dtype=np.float64)
    w = np.exp(s - s.max(axis=0, keepdims=True))
    w = w / w.sum(axis=0, keepdims=True)
    return (w * np.asarray(kv_slots, dtype=np.float64)).sum(axis=0)


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the channel axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x) + float(eps)) * np.asarray(gamma, dtype=np.float64)


def rope_pairs(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotates adjacent pairs (x[2i], x[2i+1]) by the angle with cosine cos[i] and sine sin[i]."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    even, odd = x[0::2], x[1::2]
    out = np.empty_like(x)
    out[0::2] = even * c - odd * s
    out[1::2] = even * s + odd * c
    return out


def hadamard_rotate(y: np.ndarray) -> np.ndarray:
    """H y / sqrt(n), H the Sylvester Hadamard matrix of order n = len(y) (a power of two)."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[0]
    return scipy.linalg.hadamard(n).astype(np.float64) @ y / np.sqrt(n)


def compressed_row(kv_slots, score_slots, gamma, eps, cos, sin, rotate: bool = False) -> np.ndarray:
    """RoPE(RMSNorm(pool)) for one closed window, then the Hadamard transform when rotate is set:
    float64 (C,). The last ROPE channels are the rotary ones."""
    y = rms_norm(pool(kv_slots, score_slots), gamma, eps)
    y[-ROPE:] = rope_pairs(y[-ROPE:], cos, sin)
    if rotate:
        y = hadamard_rotate(y)
    return y


def compress(inp):
    """Runs the step over an input instance (fields as in workloads.CompressInputs).

    Returns (kv_state, score_state, entries): the refreshed fp32 states, and a list of
    (b, c, row, y) for every closed window in token order, with y the float64 row and row its
    physical row (-1 when it is not written).
    """
    kv_state = np.array(inp.kv_state, dtype=np.float32, copy=True)
    score_state = np.array(inp.score_state, dtype=np.float32, copy=True)
    ratio = int(inp.ratio)
    n_pos = inp.rope_cos.shape[0]
    entries = []
    for b in range(inp.batch):
        for s in range(inp.s1):
            t = b * inp.s1 + s
            p = int(inp.start_pos[b]) + s
            if p < 0 or p >= n_pos:
                continue
            slot = slot_of(p, ratio)
            kv_state[b, slot] = inp.kv[t]
            score_state[b, slot] = (inp.score[t].astype(np.float32) + inp.ape[slot].astype(np.float32)).astype(np.float32)
            if closes_window(p, ratio):
                c = entry_index(p, ratio)
                y = compressed_row(kv_state[b], score_state[b], inp.gamma, inp.eps, inp.rope_cos[p], inp.rope_sin[p],
                                   bool(getattr(inp, "rotate", False)))
                entries.append((b, c, entry_row(inp.block_table_cmp[b], c, inp.num_cache_rows), y))
    return kv_state, score_state, entries
