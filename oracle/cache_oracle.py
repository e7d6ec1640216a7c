"""CPU oracle for the cache write of the paged MLA latent cache -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module. The GPU
path shares no code with it, and it imports nothing from the GPU path or from the input
generators.

What it computes (sources, by page title and section):
  * "DeepSeek V3/V2 Sparse Flash Attention with Quantization", section "Algorithm overview"
    (PagedAttention): the cache is paged in blocks of 128 rows; block_table maps a batch's
    logical block to a physical block, so logical position p of batch b is physical row
        block_table[b][p // 128] * 128 + p % 128.
  * The same page, section "INT8 quantisation rule": the nope part of a key is quantised in
    groups of 128 elements, the group's absolute maximum sets the scale, and the codes lie in
    [-128, 127]. Its dequant chain (int8 -> fp32, times the group scale, -> bf16) is what the
    attention reads back, so the scale is the fp32 value that maps the absolute maximum to 127.

Written out, for one 128-element group x (bf16 values, widened exactly to fp32):
    scale = fp32(absmax(x) / 127)                      (IEEE division, round to nearest even)
    code  = clamp(round_half_even(fp32(x / scale)), -128, 127)
    an all-zero group has scale 0 and codes 0.
Readings (the pages leave them open; each is listed with its reason in the design notes):
  * the division x / scale is one IEEE fp32 division, rounded to nearest even, and the quotient
    is then rounded to an integer with ties to even;
  * an all-zero group stores scale 0 and codes 0, so that it dequantises to exact zeros;
  * a token whose position is negative, at or past max_blocks_per_batch * 128, whose block entry
    is negative, or whose row falls outside the pool is not written (the masking rule of the
    attention's slots, applied to the write);
  * the rope part and a bf16 cache's nope part are copied bit for bit;
  * rows of the 512-wide layout ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation",
    D = 512, the rotary channels inside the row) come with zero-width rope arrays: the 512
    channels are the nope part, quantised or copied as above, and there is nothing else.

Inputs are raw bit patterns (bf16 as uint16), the bytes the GPU path receives. The arithmetic is
numpy float32, whose division and rounding are IEEE binary32 round-to-nearest-even.

Every function here is pinned by tests/test_cache_oracle.py against hand-derived cases, the
mathematics of rounding (exact rational arithmetic), and brute force.
"""

from __future__ import annotations

import numpy as np

KV_LORA_RANK = 512
ROPE_DIM = 64
BLOCK_SIZE = 128
QUANT_GROUP = 128
N_GROUPS = KV_LORA_RANK // QUANT_GROUP


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of a binary32 pattern: widening is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32)


def quantize_groups(nope_bits: np.ndarray):
    """The INT8 quantisation rule on rows of 512 bf16 values ("INT8 quantisation rule").

    nope_bits: uint16 (rows, 512). Returns (codes int8 (rows, 512), scales float32 (rows, 4)).
    """
    x = _bf16_bits_to_f32(nope_bits).reshape(-1, N_GROUPS, QUANT_GROUP)
    absmax = np.abs(x).max(axis=2)                          # exact: a maximum of fp32 values
    scale = (absmax / np.float32(127.0)).astype(np.float32)  # one fp32 division, RNE
    zero = scale == np.float32(0.0)
    safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    quot = (x / safe[:, :, None]).astype(np.float32)       # one fp32 division per element, RNE
    q = np.rint(quot)                                       # ties to even
    q = np.clip(q, -128.0, 127.0)
    q = np.where(zero[:, :, None], np.float32(0.0), q)
    return q.astype(np.int8).reshape(-1, KV_LORA_RANK), scale.astype(np.float32)


def target_rows(positions: np.ndarray, block_table: np.ndarray, s1: int, num_cache_rows: int) -> np.ndarray:
    """Physical row of each new token, -1 where the token is not written ("Algorithm overview",
    PagedAttention). Token t belongs to batch t // s1."""
    positions = np.asarray(positions, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    mb = bt.shape[1]
    out = np.full(positions.shape[0], -1, dtype=np.int64)
    for t, p in enumerate(positions):
        b = t // s1
        if p < 0 or p >= mb * BLOCK_SIZE:
            continue
        blk = bt[b, p // BLOCK_SIZE]
        if blk < 0:
            continue
        row = blk * BLOCK_SIZE + p % BLOCK_SIZE
        if row >= num_cache_rows:
            continue
        out[t] = row
    return out


def cache_write(new_nope_bits, new_rope_bits, positions, block_table, s1, key_nope, key_rope, k_nope_scales=None):
    """Write new latent rows into copies of the cache and return the copies.

    new_nope_bits uint16 (T, 512), new_rope_bits uint16 (T, 64); key_nope is uint16 (rows, 512)
    for a bf16 cache or int8 (rows, 512) for an INT8 cache (then k_nope_scales float32 (rows, 4)
    is required); key_rope uint16 (rows, 64). Rows no token targets keep their contents.
    """
    key_nope = np.array(key_nope, copy=True)
    key_rope = np.array(key_rope, copy=True)
    int8 = key_nope.dtype == np.int8
    if int8:
        if k_nope_scales is None:
            raise ValueError("an INT8 cache needs its scales")
        k_nope_scales = np.array(k_nope_scales, dtype=np.float32, copy=True)
    rows = target_rows(positions, block_table, s1, key_rope.shape[0])
    sel = np.nonzero(rows >= 0)[0]
    dst = rows[sel]
    if len(np.unique(dst)) != len(dst):
        raise ValueError("two tokens target the same cache row")
    key_rope[dst] = np.asarray(new_rope_bits, dtype=np.uint16)[sel]
    if int8:
        codes, scales = quantize_groups(np.asarray(new_nope_bits, dtype=np.uint16)[sel])
        key_nope[dst] = codes
        k_nope_scales[dst] = scales
    else:
        key_nope[dst] = np.asarray(new_nope_bits, dtype=np.uint16)[sel]
    return key_nope, key_rope, k_nope_scales
