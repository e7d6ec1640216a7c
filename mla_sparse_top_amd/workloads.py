"""Seeded synthetic inputs for sparse MLA attention over a paged latent KV cache.

This module only draws random inputs and lays them out the way the operation consumes them
("DeepSeek V3/V2 Sparse Flash Attention with Quantization", input/output table: query_nope,
query_rope, key_nope_2d, key_rope_2d, k_nope_scales, topk_indices, block_table, kv_act_seqs).
It contains no attention arithmetic. Its one transformation is the INT8 quantisation of the
cache's nope part, one FP32 scale per 128-element group, which gives the INT8 attention
workloads their inputs (the same page's "INT8 quantisation rule": the scale comes from the
group's absolute maximum and the codes span [-128, 127]). The cache-write kernel is checked
against its own oracle (oracle/cache_oracle.py), never against this module.

All floating data are returned as raw bit patterns (bf16 as uint16), so the GPU path and the
CPU oracle consume identical bytes.

Draws use ``torch.Generator`` on the CPU. Normals are drawn as float32 and rounded to bfloat16
by torch (round to nearest even). Distinct top-k indices come from ``torch.randperm``.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

KV_LORA_RANK = 512
ROPE_DIM = 64
BLOCK_SIZE = 128
QUANT_GROUP = 128
N_GROUPS = KV_LORA_RANK // QUANT_GROUP
BF16_QNAN = 0x7FC0

# Rows are drawn in chunks so that a pool of a million rows never holds more than one chunk
# of float32 normals at once.
_ROW_CHUNK = 1 << 16


@dataclasses.dataclass
class SfaInputs:
    """One problem instance in the layouts of the operation's input table.

    Shapes (T = batch * s1 query tokens, H = n_q heads, R = num_cache_rows):
      query_nope     uint16 (T*H, 512)  bf16 bits, row = (b*s1 + s)*H + h
      query_rope     uint16 (T*H, 64)   bf16 bits
      key_nope       uint16 (R, 512) bf16 bits, or int8 (R, 512) when kv_dtype == "int8"
      key_rope       uint16 (R, 64)     bf16 bits
      k_nope_scales  float32 (R, 4) for int8, else None
      topk_indices   int32 (T, topk), -1 = padding
      block_table    int32 (batch, max_blocks_per_batch)
      kv_act_seqs    int32 (batch,)
    """

    batch: int
    s1: int
    n_q: int
    topk: int
    kv_dtype: str
    query_nope: np.ndarray
    query_rope: np.ndarray
    key_nope: np.ndarray
    key_rope: np.ndarray
    k_nope_scales: Optional[np.ndarray]
    topk_indices: np.ndarray
    block_table: np.ndarray
    kv_act_seqs: np.ndarray
    softmax_scale: float
    poison_blocks: tuple
    name: str = ""

    @property
    def n_tokens(self) -> int:
        return self.batch * self.s1

    @property
    def num_cache_rows(self) -> int:
        return int(self.key_rope.shape[0])

    @property
    def max_blocks_per_batch(self) -> int:
        return int(self.block_table.shape[1])

    def valid_counts(self) -> np.ndarray:
        """Number of slots per token that name a position inside its batch's live range."""
        b = np.arange(self.n_tokens) // self.s1
        act = self.kv_act_seqs[b][:, None]
        idx = self.topk_indices
        return ((idx >= 0) & (idx < act)).sum(axis=1)


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(g: torch.Generator, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, _ROW_CHUNK):
        r1 = min(rows, r0 + _ROW_CHUNK)
        out[r0:r1] = _bf16_bits(torch.randn(r1 - r0, cols, generator=g, dtype=torch.float32))
    return out


def _quantize_rows(x_bf16: torch.Tensor):
    """Cache-write quantisation of bf16 latents (rows, 512): per 128-element group,
    scale = absmax / 127 (float32) and code = clamp(round_half_even(x / scale), -128, 127).
    All-zero groups get scale 0 and code 0."""
    x = x_bf16.to(torch.float32).reshape(-1, N_GROUPS, QUANT_GROUP)
    scale = x.abs().amax(dim=2) / 127.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = torch.round(x / safe[:, :, None]).clamp_(-128, 127)  # torch.round: ties to even
    q = torch.where((scale > 0)[:, :, None], q, torch.zeros_like(q))
    return q.to(torch.int8).reshape(-1, KV_LORA_RANK), scale


def quantize_int8_groups(nope_bf16_bits: np.ndarray):
    """Quantise bf16 bit patterns (rows, 512) -> (int8 codes (rows, 512), float32 scales (rows, 4))."""
    x = torch.from_numpy(np.ascontiguousarray(nope_bf16_bits).view(np.int16)).view(torch.bfloat16)
    q, s = _quantize_rows(x)
    return q.numpy(), s.numpy()


def _normal_nope(g: torch.Generator, rows: int, int8: bool):
    """Draw the cache's nope rows as bf16 N(0,1); for int8 also quantise them, chunk by chunk."""
    if not int8:
        return _normal_bf16(g, rows, KV_LORA_RANK), None
    codes = np.empty((rows, KV_LORA_RANK), dtype=np.int8)
    scales = np.empty((rows, N_GROUPS), dtype=np.float32)
    for r0 in range(0, rows, _ROW_CHUNK):
        r1 = min(rows, r0 + _ROW_CHUNK)
        xb = torch.randn(r1 - r0, KV_LORA_RANK, generator=g, dtype=torch.float32).to(torch.bfloat16)
        q, s = _quantize_rows(xb)
        codes[r0:r1] = q.numpy()
        scales[r0:r1] = s.numpy()
    return codes, scales


def generate(
    *,
    batch: int,
    s1: int,
    n_q: int,
    act_seqs: Sequence[int],
    topk: int,
    kv_dtype: str = "bf16",
    seed: int = 0,
    max_blocks_per_batch: Optional[int] = None,
    index_mode: str = "uniform",
    softmax_scale: Optional[float] = None,
    extra_pool_blocks: int = 0,
    fixed_block_table: Optional[Sequence[Sequence[int]]] = None,
    pool_blocks: Optional[int] = None,
    name: str = "",
) -> SfaInputs:
    """Draw one instance.

    index_mode:
      "uniform" -- every token of batch b takes min(topk, act[b]) distinct positions drawn
                   uniformly from [0, act[b]), in random order, then -1 padding up to topk.
      "causal"  -- token s of batch b sits at position p = act[b] - s1 + s and draws
                   min(topk, p+1) distinct positions from [0, p], then -1 padding.

    The physical pool holds the blocks the batches use (in random order), any extra unused
    blocks, and one trailing poison block. block_table entries past a batch's last live block
    point at the poison block. The poison block, and every row of a live block at or past
    act[b], is filled with NaN (bf16) or NaN scales (int8), so reading one shows up as NaN.
    """
    assert kv_dtype in ("bf16", "int8")
    assert index_mode in ("uniform", "causal")
    act = [int(a) for a in act_seqs]
    assert len(act) == batch
    g = torch.Generator().manual_seed(int(seed))
    nblk = [math.ceil(a / BLOCK_SIZE) for a in act]
    mb = max_blocks_per_batch if max_blocks_per_batch is not None else max(1, max(nblk) if nblk else 1)
    assert all(n <= mb for n in nblk), "kv_act_seqs exceeds max_blocks_per_batch * block_size"

    if fixed_block_table is not None:
        bt = np.array(fixed_block_table, dtype=np.int32).reshape(batch, mb)
        n_pool = int(pool_blocks) if pool_blocks is not None else int(bt.max()) + 2
        used = set(int(v) for b in range(batch) for v in bt[b, : nblk[b]])
        poison = tuple(sorted(set(range(n_pool)) - used))
        assert poison, "a fixed block table needs at least one spare block for poison"
        for b in range(batch):
            bt[b, nblk[b]:] = poison[-1]
    else:
        n_used = sum(nblk)
        n_pool = n_used + int(extra_pool_blocks) + 1
        poison = (n_pool - 1,)
        perm = torch.randperm(n_used + int(extra_pool_blocks), generator=g).numpy().astype(np.int32)
        bt = np.full((batch, mb), poison[0], dtype=np.int32)
        off = 0
        for b in range(batch):
            bt[b, : nblk[b]] = perm[off: off + nblk[b]]
            off += nblk[b]

    rows = n_pool * BLOCK_SIZE
    nope, scales = _normal_nope(g, rows, kv_dtype == "int8")
    rope = _normal_bf16(g, rows, ROPE_DIM)

    # Rows nobody may read: the poison blocks, and rows of live blocks past the live length.
    dead = np.zeros(rows, dtype=bool)
    for p in poison:
        dead[p * BLOCK_SIZE:(p + 1) * BLOCK_SIZE] = True
    for b in range(batch):
        tail = nblk[b] * BLOCK_SIZE - act[b]
        if tail > 0:
            last = int(bt[b, nblk[b] - 1])
            dead[last * BLOCK_SIZE + (BLOCK_SIZE - tail):(last + 1) * BLOCK_SIZE] = True

    dead_rows = np.nonzero(dead)[0]
    if kv_dtype == "int8":
        scales[dead_rows] = np.float32(np.nan)
        nope[dead_rows] = 0
    else:
        nope[dead_rows] = BF16_QNAN
    key_nope = nope
    rope[dead_rows] = BF16_QNAN

    t_count = batch * s1
    qn = _normal_bf16(g, t_count * n_q, KV_LORA_RANK)
    qr = _normal_bf16(g, t_count * n_q, ROPE_DIM)

    idx = np.full((t_count, topk), -1, dtype=np.int32)
    for t in range(t_count):
        b, s = divmod(t, s1)
        if index_mode == "uniform":
            span = act[b]
        else:
            span = max(0, min(act[b], act[b] - s1 + s + 1))
        k = min(topk, span)
        if k > 0:
            idx[t, :k] = torch.randperm(span, generator=g)[:k].numpy().astype(np.int32)

    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(KV_LORA_RANK + ROPE_DIM)))
    else:
        softmax_scale = float(np.float32(softmax_scale))

    return SfaInputs(
        batch=batch, s1=s1, n_q=n_q, topk=topk, kv_dtype=kv_dtype,
        query_nope=qn, query_rope=qr, key_nope=key_nope, key_rope=rope, k_nope_scales=scales,
        topk_indices=idx, block_table=bt, kv_act_seqs=np.array(act, dtype=np.int32),
        softmax_scale=softmax_scale, poison_blocks=tuple(int(p) for p in poison), name=name,
    )


# ----------------------------------------------------------------------------------------
# The named workloads. Shapes follow the decode case the pages time their attention ops on
# (64 sequences, two query tokens per step, 8K of cache) and the page-2 test table.
# ----------------------------------------------------------------------------------------

def tiny(seed: int = 0) -> SfaInputs:
    """B=1, S1=1, 16 heads, 256 live positions in 2 blocks mapped [1, 0] over a 4-block pool,
    64 distinct indices."""
    return generate(batch=1, s1=1, n_q=16, act_seqs=[256], topk=64, seed=seed,
                    fixed_block_table=[[1, 0]], pool_blocks=4, name="tiny_b1_s1_h16_topk64")


def decode_mtp1(seed: int = 0, kv_dtype: str = "bf16") -> SfaInputs:
    """B=64, S1=2, 128 heads, 8192 live positions each, 4096-block pool in random order,
    2048 distinct indices per token."""
    return generate(batch=64, s1=2, n_q=128, act_seqs=[8192] * 64, topk=2048, kv_dtype=kv_dtype,
                    seed=seed, name=f"decode_b64_s2_h128_kv8192_topk2048_{kv_dtype}")


def decode_mtp1_int8(seed: int = 0) -> SfaInputs:
    return decode_mtp1(seed=seed, kv_dtype="int8")


def varlen_decode(seed: int = 0) -> SfaInputs:
    """B=32, S1=1, 128 heads, live lengths uniform in [512, 65536], 512 block slots per batch,
    min(2048, len) distinct indices padded with -1."""
    g = torch.Generator().manual_seed(10_000 + int(seed))
    act = torch.randint(512, 65536 + 1, (32,), generator=g).tolist()
    return generate(batch=32, s1=1, n_q=128, act_seqs=act, topk=2048, seed=seed,
                    max_blocks_per_batch=512, name="varlen_b32_s1_h128_topk2048")


def prefill(seed: int = 0, s1: int = 4096, kv_dtype: str = "bf16") -> SfaInputs:
    """B=1, S1=4096 query tokens over 4096 live positions in 32 randomly placed blocks; query i
    takes min(i+1, 2048) distinct positions from [0, i], padded with -1."""
    return generate(batch=1, s1=s1, n_q=128, act_seqs=[s1], topk=2048, kv_dtype=kv_dtype,
                    seed=seed, index_mode="causal", name=f"prefill_b1_s{s1}_h128_topk2048_{kv_dtype}")


def page_case(name: str, seed: int = 0) -> SfaInputs:
    """The page-2 test table's shapes (B, S1, N_Q=128, N_KV=1, per-batch lengths, key mode)."""
    if name == "total_int8_d":
        return generate(batch=4, s1=2, n_q=128, act_seqs=[65536, 16381, 666, 15], topk=2048,
                        kv_dtype="int8", seed=seed, max_blocks_per_batch=512, name=name)
    if name == "per_int8_d":
        return generate(batch=4, s1=2, n_q=128, act_seqs=[65536] * 4, topk=2048, kv_dtype="int8",
                        seed=seed, name=name)
    if name == "per_bf16_d":
        return generate(batch=4, s1=2, n_q=128, act_seqs=[65536] * 4, topk=2048, kv_dtype="bf16",
                        seed=seed, name=name)
    if name == "int8_p":
        return generate(batch=1, s1=256, n_q=128, act_seqs=[65536], topk=2048, kv_dtype="int8",
                        seed=seed, index_mode="causal", name=name)
    raise KeyError(name)


PAGE_CASES = ("total_int8_d", "per_int8_d", "per_bf16_d", "int8_p")


# ----------------------------------------------------------------------------------------
# Lightning Indexer inputs ("CANN DeepSeek Indexer attention optimisation", sections "Indexer
# Prolog" and "Lightning Indexer"): per query token, index queries for each index head and the
# head weights; per cache position, one index key, in a paged cache with the same block table
# and live lengths as the latent cache.
# ----------------------------------------------------------------------------------------

INDEX_HEADS = 64
INDEX_DIM = 128


@dataclasses.dataclass
class IndexerInputs:
    """Shapes (T = batch * s1, H = index heads, D = index head dim, R = cache rows):
      q_index      uint16 (T*H, D)   bf16 bits, row t*H + h
      weights      float32 (T, H)
      k_index      uint16 (R, D)     bf16 bits
      block_table  int32 (batch, max_blocks_per_batch)
      kv_act_seqs  int32 (batch,)
    """

    batch: int
    s1: int
    n_heads: int
    head_dim: int
    topk: int
    q_index: np.ndarray
    weights: np.ndarray
    k_index: np.ndarray
    block_table: np.ndarray
    kv_act_seqs: np.ndarray
    name: str = ""

    @property
    def n_tokens(self) -> int:
        return self.batch * self.s1

    @property
    def num_cache_rows(self) -> int:
        return int(self.k_index.shape[0])

    @property
    def max_blocks_per_batch(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def n_positions(self) -> int:
        return self.max_blocks_per_batch * BLOCK_SIZE


def indexer_generate(*, batch: int, s1: int, act_seqs: Sequence[int], topk: int, seed: int = 0,
                     n_heads: int = INDEX_HEADS, head_dim: int = INDEX_DIM,
                     max_blocks_per_batch: Optional[int] = None, extra_pool_blocks: int = 0,
                     name: str = "") -> IndexerInputs:
    """q_index and k_index are N(0,1) rounded to bf16. The head weights are N(0,1) times
    1/sqrt(n_heads * head_dim), the normalisation the Indexer Prolog applies to its weights.
    The pool holds the batches' blocks in a random order, any extra blocks and one trailing
    poison block; block_table entries past a batch's live blocks point at the poison block,
    and the poison block and every row of a live block at or past the live length are NaN."""
    act = [int(a) for a in act_seqs]
    assert len(act) == batch
    g = torch.Generator().manual_seed(50_000 + int(seed))
    nblk = [math.ceil(a / BLOCK_SIZE) for a in act]
    mb = max_blocks_per_batch if max_blocks_per_batch is not None else max(1, max(nblk) if nblk else 1)
    assert all(n <= mb for n in nblk), "kv_act_seqs exceeds max_blocks_per_batch * block_size"
    n_used = sum(nblk)
    n_pool = n_used + int(extra_pool_blocks) + 1
    poison = n_pool - 1
    perm = torch.randperm(n_used + int(extra_pool_blocks), generator=g).numpy().astype(np.int32)
    bt = np.full((batch, mb), poison, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    rows = n_pool * BLOCK_SIZE
    k = _normal_bf16(g, rows, head_dim)
    k[poison * BLOCK_SIZE:] = BF16_QNAN
    for b in range(batch):
        tail = nblk[b] * BLOCK_SIZE - act[b]
        if tail > 0:
            last = int(bt[b, nblk[b] - 1])
            k[last * BLOCK_SIZE + (BLOCK_SIZE - tail):(last + 1) * BLOCK_SIZE] = BF16_QNAN
    t_count = batch * s1
    q = _normal_bf16(g, t_count * n_heads, head_dim)
    w = (torch.randn(t_count, n_heads, generator=g, dtype=torch.float32)
         * float(1.0 / math.sqrt(n_heads * head_dim))).numpy()
    return IndexerInputs(batch=batch, s1=s1, n_heads=n_heads, head_dim=head_dim, topk=topk, q_index=q,
                         weights=w, k_index=k, block_table=bt, kv_act_seqs=np.array(act, dtype=np.int32),
                         name=name)


def indexer_decode(seed: int = 0) -> IndexerInputs:
    """The decode shape of the attention workload: B=64, S1=2, 8192 live positions each in a
    4096-block pool, 64 index heads of 128 dims, top-k 2048."""
    return indexer_generate(batch=64, s1=2, act_seqs=[8192] * 64, topk=2048, seed=seed,
                            name="indexer_b64_s2_h64_d128_kv8192_topk2048")


# ----------------------------------------------------------------------------------------
# Cache-write inputs ("DeepSeek V3/V2 Sparse Flash Attention with Quantization", sections
# "Algorithm overview" and "INT8 quantisation rule"): new latent rows for each new token, the
# logical position each one takes, a block table, and the existing cache they are written into.
# Only random draws and layout here; the existing INT8 cache holds random codes and scales.
# ----------------------------------------------------------------------------------------


@dataclasses.dataclass
class CacheWriteInputs:
    """Shapes (T = batch * s1, R = cache rows):
      new_nope     uint16 (T, 512)  bf16 bits
      new_rope     uint16 (T, 64)   bf16 bits
      positions    int32 (T,)       logical position of token t in batch t // s1 (-1: not written)
      block_table  int32 (batch, max_blocks_per_batch)
      key_nope     uint16 (R, 512) bf16 bits, or int8 (R, 512)
      key_rope     uint16 (R, 64)
      k_nope_scales float32 (R, 4) or None
    """

    batch: int
    s1: int
    kv_dtype: str
    new_nope: np.ndarray
    new_rope: np.ndarray
    positions: np.ndarray
    block_table: np.ndarray
    key_nope: np.ndarray
    key_rope: np.ndarray
    k_nope_scales: Optional[np.ndarray]
    name: str = ""

    @property
    def n_tokens(self) -> int:
        return self.batch * self.s1

    @property
    def num_cache_rows(self) -> int:
        return int(self.key_rope.shape[0])

    def n_written(self) -> int:
        p = self.positions.astype(np.int64)
        mb = self.block_table.shape[1]
        b = np.arange(self.n_tokens) // self.s1
        ok = (p >= 0) & (p < mb * BLOCK_SIZE)
        blk = np.where(ok, self.block_table[b, np.where(ok, p, 0) // BLOCK_SIZE], -1).astype(np.int64)
        ok &= (blk >= 0) & (blk * BLOCK_SIZE + np.where(ok, p, 0) % BLOCK_SIZE < self.num_cache_rows)
        return int(ok.sum())


def cache_write_generate(*, batch: int, s1: int, n_pool_blocks: int, max_blocks_per_batch: int,
                         kv_dtype: str = "int8", seed: int = 0, positions: Optional[np.ndarray] = None,
                         block_table: Optional[np.ndarray] = None, value_scale: float = 1.0,
                         name: str = "", rope_dim: int = ROPE_DIM) -> CacheWriteInputs:
    """New rows are N(0,1) * value_scale rounded to bf16. Unless given, the block table is a
    random permutation of the pool's blocks (it needs n_pool_blocks >= batch * mb) and each
    batch's s1 tokens take distinct random positions in [0, mb * 128). The existing cache is
    random bytes (bf16: random bit patterns; INT8: random codes, scales uniform in [0, 1)).
    rope_dim 0: 512-wide rows with the rotary channels inside; the rope arrays are zero-width."""
    assert rope_dim in (0, ROPE_DIM)
    g = torch.Generator().manual_seed(70_000 + int(seed))
    mb = int(max_blocks_per_batch)
    if block_table is None:
        assert n_pool_blocks >= batch * mb
        block_table = torch.randperm(n_pool_blocks, generator=g)[: batch * mb].view(batch, mb).numpy()
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    if positions is None:
        positions = np.concatenate([torch.randperm(mb * BLOCK_SIZE, generator=g)[:s1].numpy()
                                    for _ in range(batch)]) if batch * s1 else np.zeros(0)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    t = batch * s1
    nn = np.empty((t, KV_LORA_RANK), dtype=np.uint16)
    for r0 in range(0, t, _ROW_CHUNK):
        r1 = min(t, r0 + _ROW_CHUNK)
        nn[r0:r1] = _bf16_bits(torch.randn(r1 - r0, KV_LORA_RANK, generator=g) * float(value_scale))
    nr = _normal_bf16(g, t, ROPE_DIM) if rope_dim else np.zeros((t, 0), dtype=np.uint16)
    rows = n_pool_blocks * BLOCK_SIZE
    kr = (torch.randint(0, 1 << 16, (rows, ROPE_DIM), generator=g, dtype=torch.int32).numpy().astype(np.uint16)
          if rope_dim else np.zeros((rows, 0), dtype=np.uint16))
    if kv_dtype == "int8":
        kn = torch.randint(-128, 128, (rows, KV_LORA_RANK), generator=g, dtype=torch.int8).numpy()
        ks = torch.rand(rows, N_GROUPS, generator=g).numpy()
    else:
        kn = torch.randint(0, 1 << 16, (rows, KV_LORA_RANK), generator=g, dtype=torch.int32).numpy().astype(np.uint16)
        ks = None
    return CacheWriteInputs(batch=batch, s1=s1, kv_dtype=kv_dtype, new_nope=nn, new_rope=nr, positions=positions,
                            block_table=block_table, key_nope=kn, key_rope=kr, k_nope_scales=ks, name=name)


def cache_fill(seed: int = 0, kv_dtype: str = "int8") -> CacheWriteInputs:
    """Every position of the decode workload's cache written at once (a prefill of 64 sequences
    of 8192 tokens): B=64, S1=8192, positions 0..8191 in order, the block table a random
    permutation of a 4096-block pool (524,288 rows)."""
    pos = np.tile(np.arange(8192, dtype=np.int32), 64)
    return cache_write_generate(batch=64, s1=8192, n_pool_blocks=4096, max_blocks_per_batch=64, kv_dtype=kv_dtype,
                                seed=seed, positions=pos, name=f"cache_write_b64_s8192_{kv_dtype}")


def cache_decode_step(seed: int = 0, kv_dtype: str = "int8") -> CacheWriteInputs:
    """The decode step's write: B=64 sequences, S1=2 new tokens at positions 8190 and 8191, into
    the decode workload's 4096-block pool."""
    pos = np.tile(np.array([8190, 8191], dtype=np.int32), 64)
    return cache_write_generate(batch=64, s1=2, n_pool_blocks=4096, max_blocks_per_batch=64, kv_dtype=kv_dtype,
                                seed=seed, positions=pos, name=f"cache_write_b64_s2_{kv_dtype}")


# ----------------------------------------------------------------------------------------
# Sliding-window + compressed-cache attention inputs ("NPU DeepSeek-V4 model PyPTO fused-operator
# optimisation", section "FA-class operators: SWA, CFA and SCFA"): per sequence an original
# cache (ori_kv, a window of it is read) and a compressed cache (cmp_kv, compress_ratio times
# shorter), both as rows of one paged pool with their own block tables.
# ----------------------------------------------------------------------------------------


@dataclasses.dataclass
class WindowInputs:
    """Shapes (T = batch * s1):
      query_nope/query_rope  uint16 (T*n_q, 512/64)     bf16 bits (rope (T*n_q, 0) for 512-wide rows)
      key_nope/key_rope      the shared pool, as in SfaInputs (k_nope_scales for int8; key_rope
                             (rows, 0) for 512-wide rows)
      cmp_indices            int32 (T, topk_cmp) or None  compressed-entry indices, -1 padded
      block_table_ori/_cmp   int32 (batch, mb_ori/mb_cmp)
      ori_len, cmp_len       int32 (batch,)
    """

    batch: int
    s1: int
    n_q: int
    window: int
    topk_cmp: int
    kv_dtype: str
    query_nope: np.ndarray
    query_rope: np.ndarray
    key_nope: np.ndarray
    key_rope: np.ndarray
    k_nope_scales: Optional[np.ndarray]
    cmp_indices: Optional[np.ndarray]
    block_table_ori: np.ndarray
    block_table_cmp: np.ndarray
    ori_len: np.ndarray
    cmp_len: np.ndarray
    softmax_scale: float
    name: str = ""

    @property
    def n_tokens(self) -> int:
        return self.batch * self.s1

    @property
    def num_cache_rows(self) -> int:
        return int(self.key_rope.shape[0])

    @property
    def rope_dim(self) -> int:
        return int(self.key_rope.shape[1])


def window_generate(*, batch: int, s1: int, n_q: int, ori_lens: Sequence[int], window: int, ratio: int = 4,
                    cmp_mode: str = "sparse", topk_cmp: int = 0, kv_dtype: str = "bf16", seed: int = 0,
                    name: str = "", rope_dim: int = ROPE_DIM) -> WindowInputs:
    """cmp_mode: "none" (SWA: window only), "all" (CFA: every causal compressed entry, in order)
    or "sparse" (SCFA: min(topk_cmp, causal) distinct causal entries in random order). A query at
    position p sees the compressed entries c with (c + 1) * ratio <= p + 1 (entry c summarises
    positions c*ratio .. c*ratio + ratio - 1). cmp_len[b] = ori_len[b] // ratio. Both caches' blocks
    are drawn in one random order from a shared pool with one trailing NaN poison block, which
    every unused block-table entry names; rows past a cache's length are NaN too.
    rope_dim 64: 512 nope + 64 rope channels per row, scale 1/sqrt(576). rope_dim 0: the 512-wide
    rows of the DeepSeek-V4 layout, whose rotary channels sit inside the row; the rope arrays are
    then zero-width and the scale is 1/sqrt(512)."""
    assert kv_dtype in ("bf16", "int8") and cmp_mode in ("none", "all", "sparse") and rope_dim in (0, ROPE_DIM)
    g = torch.Generator().manual_seed(90_000 + int(seed))
    ori = [int(v) for v in ori_lens]
    cmp_len = [v // ratio for v in ori]
    nb_o = [math.ceil(v / BLOCK_SIZE) for v in ori]
    nb_c = [math.ceil(v / BLOCK_SIZE) for v in cmp_len]
    mb_o, mb_c = max(1, max(nb_o)), max(1, max(nb_c))
    n_used = sum(nb_o) + sum(nb_c)
    poison = n_used
    perm = torch.randperm(n_used, generator=g).numpy().astype(np.int32)
    bt_o = np.full((batch, mb_o), poison, dtype=np.int32)
    bt_c = np.full((batch, mb_c), poison, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt_o[b, :nb_o[b]] = perm[off:off + nb_o[b]]
        off += nb_o[b]
        bt_c[b, :nb_c[b]] = perm[off:off + nb_c[b]]
        off += nb_c[b]
    rows = (n_used + 1) * BLOCK_SIZE
    nope, scales = _normal_nope(g, rows, kv_dtype == "int8")
    rope = _normal_bf16(g, rows, ROPE_DIM) if rope_dim else np.zeros((rows, 0), dtype=np.uint16)
    dead = np.zeros(rows, dtype=bool)
    dead[poison * BLOCK_SIZE:] = True
    for b in range(batch):
        for bt, nb, ln in ((bt_o, nb_o[b], ori[b]), (bt_c, nb_c[b], cmp_len[b])):
            tail = nb * BLOCK_SIZE - ln
            if nb and tail > 0:
                last = int(bt[b, nb - 1])
                dead[last * BLOCK_SIZE + (BLOCK_SIZE - tail):(last + 1) * BLOCK_SIZE] = True
    dead_rows = np.nonzero(dead)[0]
    if kv_dtype == "int8":
        scales[dead_rows] = np.float32(np.nan)
        nope[dead_rows] = 0
    else:
        nope[dead_rows] = BF16_QNAN
    rope[dead_rows] = BF16_QNAN
    t_count = batch * s1
    qn = _normal_bf16(g, t_count * n_q, KV_LORA_RANK)
    qr = _normal_bf16(g, t_count * n_q, ROPE_DIM) if rope_dim else np.zeros((t_count * n_q, 0), dtype=np.uint16)
    cmp_idx = None
    if cmp_mode != "none":
        causal = [max(0, (ori[t // s1] - s1 + t % s1 + 1) // ratio) for t in range(t_count)]
        k = max(causal) if cmp_mode == "all" else int(topk_cmp)
        cmp_idx = np.full((t_count, max(1, k)), -1, dtype=np.int32)
        for t in range(t_count):
            n = causal[t]
            if cmp_mode == "all":
                cmp_idx[t, :n] = np.arange(n, dtype=np.int32)
            elif n > 0:
                m = min(k, n)
                cmp_idx[t, :m] = torch.randperm(n, generator=g)[:m].numpy().astype(np.int32)
    scale = float(np.float32(1.0 / math.sqrt(KV_LORA_RANK + rope_dim)))
    return WindowInputs(batch=batch, s1=s1, n_q=n_q, window=int(window),
                        topk_cmp=0 if cmp_idx is None else int(cmp_idx.shape[1]), kv_dtype=kv_dtype,
                        query_nope=qn, query_rope=qr, key_nope=nope, key_rope=rope, k_nope_scales=scales,
                        cmp_indices=cmp_idx, block_table_ori=bt_o, block_table_cmp=bt_c,
                        ori_len=np.array(ori, dtype=np.int32), cmp_len=np.array(cmp_len, dtype=np.int32),
                        softmax_scale=scale, name=name)


def swa_decode(seed: int = 0, kv_dtype: str = "bf16") -> WindowInputs:
    """SWA at the pages' timed shape (64 sequences, 2 query tokens, 8K of cache): a 128-position
    window, no compressed cache (the window size is a reading; the page gives none)."""
    return window_generate(batch=64, s1=2, n_q=128, ori_lens=[8192] * 64, window=128, cmp_mode="none",
                           kv_dtype=kv_dtype, seed=seed, name=f"swa_b64_s2_w128_{kv_dtype}")


def cfa_decode(seed: int = 0, kv_dtype: str = "bf16") -> WindowInputs:
    """CFA at the pages' timed shape with compress_ratio 128: a 128-position window plus every
    causal compressed entry (63 or 64 of the 64 entries that 8K positions give at ratio 128; the
    window size is a reading, the same as SWA's and SCFA's)."""
    return window_generate(batch=64, s1=2, n_q=128, ori_lens=[8192] * 64, window=128, ratio=128, cmp_mode="all",
                           kv_dtype=kv_dtype, seed=seed, name=f"cfa_b64_s2_w128_r128_{kv_dtype}")


def scfa_decode(seed: int = 0, kv_dtype: str = "bf16") -> WindowInputs:
    """SCFA at the pages' timed shape with compress_ratio 4: a 128-position window plus 512
    compressed entries per token picked from the 2048 causal ones (window size and top-k are
    readings; 512 entries of ratio 4 cover 2048 original positions, the top-k of the SFA page)."""
    return window_generate(batch=64, s1=2, n_q=128, ori_lens=[8192] * 64, window=128, ratio=4, cmp_mode="sparse",
                           topk_cmp=512, kv_dtype=kv_dtype, seed=seed, name=f"scfa_b64_s2_w128_k512_{kv_dtype}")


def swa_decode_d512(seed: int = 0, kv_dtype: str = "bf16") -> WindowInputs:
    """SWA as swa_decode, on the 512-wide rows of the DeepSeek-V4 layout (D = 512, the head size
    the page's timing table gives the FA-class operators)."""
    return window_generate(batch=64, s1=2, n_q=128, ori_lens=[8192] * 64, window=128, cmp_mode="none",
                           kv_dtype=kv_dtype, seed=seed, rope_dim=0, name=f"swa_b64_s2_w128_d512_{kv_dtype}")


def cfa_decode_d512(seed: int = 0, kv_dtype: str = "bf16") -> WindowInputs:
    """CFA as cfa_decode (ratio 128), on 512-wide rows."""
    return window_generate(batch=64, s1=2, n_q=128, ori_lens=[8192] * 64, window=128, ratio=128, cmp_mode="all",
                           kv_dtype=kv_dtype, seed=seed, rope_dim=0, name=f"cfa_b64_s2_w128_r128_d512_{kv_dtype}")


def scfa_decode_d512(seed: int = 0, kv_dtype: str = "bf16") -> WindowInputs:
    """SCFA as scfa_decode (ratio 4, 512 listed entries), on 512-wide rows."""
    return window_generate(batch=64, s1=2, n_q=128, ori_lens=[8192] * 64, window=128, ratio=4, cmp_mode="sparse",
                           topk_cmp=512, kv_dtype=kv_dtype, seed=seed, rope_dim=0,
                           name=f"scfa_b64_s2_w128_k512_d512_{kv_dtype}")


# ----------------------------------------------------------------------------------------
# Compressor inputs ("NPU DeepSeek-V4 model PyPTO fused-operator optimisation", section
# "Compressor"): the fp32 outputs of the two projections for the new tokens, the per-sequence
# state, the gate's position embedding, the RMSNorm weight, RoPE tables, and the compressed
# pool that receives the entries.
# ----------------------------------------------------------------------------------------

COMPRESS_CHANNELS = KV_LORA_RANK + ROPE_DIM


@dataclasses.dataclass
class CompressInputs:
    batch: int
    s1: int
    ratio: int
    kv: np.ndarray              # float32 (T, 576)
    score: np.ndarray           # float32 (T, 576)
    ape: np.ndarray             # float32 (ratio, 576)
    gamma: np.ndarray           # float32 (576)
    eps: float
    rope_cos: np.ndarray        # float32 (rope_positions, 32)
    rope_sin: np.ndarray        # float32 (rope_positions, 32)
    start_pos: np.ndarray       # int32 (B)
    kv_state: np.ndarray        # float32 (B, ratio, 576)
    score_state: np.ndarray     # float32 (B, ratio, 576)
    block_table_cmp: np.ndarray  # int32 (B, max_blocks)
    key_nope: np.ndarray        # uint16 (rows, 512), or (rows, 128) for 128 channels: the pool's bf16 bits
    key_rope: Optional[np.ndarray]  # uint16 (rows, 64); None for 128 channels
    name: str = ""
    rotate: bool = False        # the Hadamard transform after RoPE (128 channels)

    @property
    def num_cache_rows(self) -> int:
        return int(self.key_nope.shape[0])

    @property
    def rope_positions(self) -> int:
        return int(self.rope_cos.shape[0])

    @property
    def channels(self) -> int:
        return int(self.kv.shape[1])


def rope_tables(n_pos: int, base: float = 10000.0):
    """cos and sin of p * base^(-2i/64) for p < n_pos, i < 32, computed in float64 and rounded
    to float32 (the usual rotary frequencies; the tables are inputs of the step)."""
    inv = base ** (-np.arange(0, ROPE_DIM, 2, dtype=np.float64) / ROPE_DIM)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def compress_generate(*, batch: int, s1: int, ratio: int, start_pos: Sequence[int], rope_positions: int,
                      max_blocks: int, n_pool_blocks: Optional[int] = None, seed: int = 0,
                      score_scale: float = 1.0, block_table: Optional[np.ndarray] = None,
                      name: str = "", channels: int = COMPRESS_CHANNELS, rotate: bool = False) -> CompressInputs:
    """kv, score, kv_state and score_state are N(0,1) float32 (scores times score_scale); ape is
    N(0, 0.1^2); gamma is 1 + N(0, 0.1^2); eps 1e-6. Unless given, the block table is a random
    permutation of the pool's blocks, and the pool holds random bf16 bit patterns, so a row the
    step should not touch shows up if it changes."""
    g = torch.Generator().manual_seed(90_000 + int(seed))
    c = int(channels)
    t = batch * s1
    n_pool_blocks = batch * max_blocks if n_pool_blocks is None else int(n_pool_blocks)
    if block_table is None:
        assert n_pool_blocks >= batch * max_blocks
        block_table = torch.randperm(n_pool_blocks, generator=g)[: batch * max_blocks].view(batch, max_blocks).numpy()
    kv = torch.randn(t, c, generator=g).numpy()
    score = (torch.randn(t, c, generator=g) * float(score_scale)).numpy()
    ape = (torch.randn(ratio, c, generator=g) * 0.1).numpy()
    gamma = (1.0 + torch.randn(c, generator=g) * 0.1).numpy()
    kv_state = torch.randn(batch, ratio, c, generator=g).numpy()
    score_state = (torch.randn(batch, ratio, c, generator=g) * float(score_scale)).numpy()
    cos, sin = rope_tables(rope_positions)
    rows = n_pool_blocks * BLOCK_SIZE
    wide = c - ROPE_DIM if c == COMPRESS_CHANNELS else c
    kn = torch.randint(0, 1 << 16, (rows, wide), generator=g, dtype=torch.int32).numpy().astype(np.uint16)
    kr = (torch.randint(0, 1 << 16, (rows, ROPE_DIM), generator=g, dtype=torch.int32).numpy().astype(np.uint16)
          if c == COMPRESS_CHANNELS else None)
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)  # noqa: E731
    return CompressInputs(batch=batch, s1=s1, ratio=int(ratio), kv=f32(kv), score=f32(score), ape=f32(ape),
                          gamma=f32(gamma), eps=1e-6, rope_cos=cos, rope_sin=sin,
                          start_pos=np.ascontiguousarray(start_pos, dtype=np.int32), kv_state=f32(kv_state),
                          score_state=f32(score_state),
                          block_table_cmp=np.ascontiguousarray(block_table, dtype=np.int32),
                          key_nope=kn, key_rope=kr, name=name, rotate=bool(rotate))


def compress_c128a(seed: int = 0) -> CompressInputs:
    """The page's c128a compressor case (ratio 128, one state window, D = 512) at the decode
    step: 64 sequences, two new tokens at positions 8190 and 8191, so 8191 closes a window and
    writes entry 63 into 512-wide rows (the rotary channels are the last 64 of the row)."""
    return compress_generate(batch=64, s1=2, ratio=128, start_pos=[8190] * 64, rope_positions=8192,
                             max_blocks=1, seed=seed, channels=KV_LORA_RANK, name="compress_c128a_b64_s2_d512")


def compress_decode(seed: int = 0, ratio: int = 4) -> CompressInputs:
    """The decode step of the page's compressor case (64 sequences, MTP 1 so two new tokens,
    every sequence compressing): positions 8190 and 8191, so 8191 closes a window of ratio 4
    and writes compressed entry 2047, the last of the 2048 entries the SCFA workload reads.
    The compressed pool has 16 blocks of 128 entries per sequence."""
    return compress_generate(batch=64, s1=2, ratio=ratio, start_pos=[8190] * 64, rope_positions=8192,
                             max_blocks=2048 // BLOCK_SIZE, seed=seed, name=f"compress_b64_s2_r{ratio}")


# ---- MLA prolog ------------------------------------------------------------------------
# The hidden state of the new tokens, the projection weights (random, scaled so that every
# product has unit variance), the RMSNorm scales, positions and RoPE tables.
# ----------------------------------------------------------------------------------------

PROLOG_ROPE = ROPE_DIM


@dataclasses.dataclass
class PrologInputs:
    tokens: int
    n_q: int
    x: np.ndarray               # uint16 bf16 bits (T, hidden)
    w_dq: np.ndarray            # uint16 (q_lora_rank, hidden)
    gamma_cq: np.ndarray        # uint16 (q_lora_rank)
    w_uq_qr: np.ndarray         # uint16 (n_q * (nope_dim + 64), q_lora_rank)
    w_uk: np.ndarray            # uint16 (n_q, 512, nope_dim)
    w_dkv_kr: np.ndarray        # uint16 (576, hidden)
    gamma_ckv: np.ndarray       # uint16 (512)
    positions: np.ndarray       # int32 (T)
    rope_cos: np.ndarray        # float32 (rope_positions, 32)
    rope_sin: np.ndarray        # float32 (rope_positions, 32)
    eps: float
    name: str = ""

    @property
    def hidden(self) -> int:
        return int(self.x.shape[1])

    @property
    def q_lora_rank(self) -> int:
        return int(self.w_dq.shape[0])

    @property
    def nope_dim(self) -> int:
        return int(self.w_uk.shape[2])

    @property
    def rope_positions(self) -> int:
        return int(self.rope_cos.shape[0])


def _scaled_bf16(g: torch.Generator, shape, std: float) -> np.ndarray:
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = np.empty((rows, shape[-1]), dtype=np.uint16)
    for r0 in range(0, rows, _ROW_CHUNK):
        r1 = min(rows, r0 + _ROW_CHUNK)
        out[r0:r1] = _bf16_bits(torch.randn(r1 - r0, shape[-1], generator=g, dtype=torch.float32) * std)
    return out.reshape(shape)


def prolog_generate(*, tokens: int, n_q: int, hidden: int = 7168, q_lora_rank: int = 1536, nope_dim: int = 128,
                    positions: Optional[Sequence[int]] = None, rope_positions: int = 8192, seed: int = 0,
                    name: str = "") -> PrologInputs:
    """x is N(0,1); each weight is N(0, 1/fan_in) so that every product has unit variance; the
    RMSNorm scales are 1 + N(0, 0.1^2); all rounded to bf16. Positions default to the decode
    step's 8190, 8191 alternating (two new tokens per sequence); eps is 1e-6."""
    g = torch.Generator().manual_seed(110_000 + int(seed))
    x = _scaled_bf16(g, (tokens, hidden), 1.0)
    w_dq = _scaled_bf16(g, (q_lora_rank, hidden), hidden ** -0.5)
    gamma_cq = _bf16_bits(1.0 + torch.randn(q_lora_rank, generator=g) * 0.1)
    w_uq_qr = _scaled_bf16(g, (n_q * (nope_dim + PROLOG_ROPE), q_lora_rank), q_lora_rank ** -0.5)
    w_uk = _scaled_bf16(g, (n_q, KV_LORA_RANK, nope_dim), nope_dim ** -0.5)
    w_dkv_kr = _scaled_bf16(g, (KV_LORA_RANK + PROLOG_ROPE, hidden), hidden ** -0.5)
    gamma_ckv = _bf16_bits(1.0 + torch.randn(KV_LORA_RANK, generator=g) * 0.1)
    if positions is None:
        positions = [8190 + (t % 2) for t in range(tokens)]
    cos, sin = rope_tables(rope_positions)
    return PrologInputs(tokens=int(tokens), n_q=int(n_q), x=x, w_dq=w_dq, gamma_cq=gamma_cq, w_uq_qr=w_uq_qr,
                        w_uk=w_uk, w_dkv_kr=w_dkv_kr, gamma_ckv=gamma_ckv,
                        positions=np.ascontiguousarray(positions, dtype=np.int32), rope_cos=cos, rope_sin=sin,
                        eps=1e-6, name=name)


def prolog_decode(seed: int = 0) -> PrologInputs:
    """The decode step's prolog: 64 sequences x 2 new tokens (MTP 1), 128 heads, hidden 7168,
    query rank 1536, nope head dim 128, positions 8190 and 8191."""
    return prolog_generate(tokens=128, n_q=128, seed=seed, name="mla_prolog_b64_s2")


@dataclasses.dataclass
class PrologV4Inputs:
    tokens: int
    n_q: int
    x: np.ndarray               # uint16 bf16 bits (T, hidden)
    w_dq: np.ndarray            # uint16 (q_lora_rank, hidden)
    gamma_cq: np.ndarray        # uint16 (q_lora_rank)
    w_uq: np.ndarray            # uint16 (n_q * 512, q_lora_rank)
    w_dkv: np.ndarray           # uint16 (512, hidden)
    gamma_ckv: np.ndarray       # uint16 (512)
    positions: np.ndarray       # int32 (T)
    rope_cos: np.ndarray        # float32 (rope_positions, 32)
    rope_sin: np.ndarray        # float32 (rope_positions, 32)
    eps: float
    name: str = ""

    @property
    def hidden(self) -> int:
        return int(self.x.shape[1])

    @property
    def q_lora_rank(self) -> int:
        return int(self.w_dq.shape[0])

    @property
    def rope_positions(self) -> int:
        return int(self.rope_cos.shape[0])


def prolog_v4_generate(*, tokens: int, n_q: int, hidden: int = 4096, q_lora_rank: int = 1536,
                       positions: Optional[Sequence[int]] = None, rope_positions: int = 8192, seed: int = 0,
                       name: str = "") -> PrologV4Inputs:
    """The V4 prolog's inputs, drawn as prolog_generate's: x N(0,1), weights N(0, 1/fan_in), RMSNorm
    scales 1 + N(0, 0.1^2), all rounded to bf16; positions 8190, 8191 alternating; eps 1e-6."""
    g = torch.Generator().manual_seed(120_000 + int(seed))
    x = _scaled_bf16(g, (tokens, hidden), 1.0)
    w_dq = _scaled_bf16(g, (q_lora_rank, hidden), hidden ** -0.5)
    gamma_cq = _bf16_bits(1.0 + torch.randn(q_lora_rank, generator=g) * 0.1)
    w_uq = _scaled_bf16(g, (n_q * KV_LORA_RANK, q_lora_rank), q_lora_rank ** -0.5)
    w_dkv = _scaled_bf16(g, (KV_LORA_RANK, hidden), hidden ** -0.5)
    gamma_ckv = _bf16_bits(1.0 + torch.randn(KV_LORA_RANK, generator=g) * 0.1)
    if positions is None:
        positions = [8190 + (t % 2) for t in range(tokens)]
    cos, sin = rope_tables(rope_positions)
    return PrologV4Inputs(tokens=int(tokens), n_q=int(n_q), x=x, w_dq=w_dq, gamma_cq=gamma_cq, w_uq=w_uq,
                          w_dkv=w_dkv, gamma_ckv=gamma_ckv, positions=np.ascontiguousarray(positions, dtype=np.int32),
                          rope_cos=cos, rope_sin=sin, eps=1e-6, name=name)


def prolog_v4_decode(seed: int = 0) -> PrologV4Inputs:
    """The V4 prolog at the decode step: 64 sequences x 2 new tokens, 128 heads of 512 channels,
    hidden 4096 (the page's MlaProlog shapes), query rank 1536 (not given by the page: the V3
    value), positions 8190 and 8191."""
    return prolog_v4_generate(tokens=128, n_q=128, seed=seed, name="mla_prolog_v4_b64_s2")


@dataclasses.dataclass
class V4LayerInputs:
    """The inputs of one decode step of a DeepSeek-V4 attention layer on 512-wide rows, consistent
    across its steps. kind "swa" (compression ratio 1): the V4 MLA prolog, the cache write of the
    new latent rows into the original cache, SWA. kind "cfa" (ratio 128): also the compressor
    (512 channels) into the compressed cache, and CFA over every causal compressed entry. kind
    "scfa" (ratio 4): also the index-key compressor (128 channels, Hadamard), the indexer prolog
    (whose qr is the prolog's cq, filled in on the device), the Lightning Indexer over the
    compressed index keys, and SCFA over its top-k."""
    kind: str
    prolog: PrologV4Inputs
    window: WindowInputs        # pools, block tables and lengths (SCFA: its cmp_indices are replaced)
    compress_att: Optional[CompressInputs]  # 512-channel rows into the window's pool (block_table_cmp)
    compress_idx: Optional[CompressInputs]  # 128-channel rows into the index-key pool (same block table)
    indexer_prolog: Optional[IndexerPrologInputs]
    topk_cmp: int

    @property
    def positions(self) -> np.ndarray:
        return self.prolog.positions


def v4_layer_generate(*, kind: str, batch: int, s1: int, n_q: int, hidden: int, q_lora_rank: int,
                      ori_lens: Sequence[int], window: int, topk_cmp: int = 0, seed: int = 0,
                      name: str = "") -> V4LayerInputs:
    """Token t = b * s1 + s sits at position ori_len[b] - s1 + s (the window inputs' rule); the
    RoPE tables cover max(ori_lens) positions. The compressors' kv and score are random fp32 (the
    outputs of projection GEMMs outside the step). SCFA's ratio is 4, CFA's 128."""
    assert kind in ("swa", "cfa", "scfa")
    ratio = {"swa": 1, "cfa": 128, "scfa": 4}[kind]
    ori = [int(v) for v in ori_lens]
    pos = [ori[t // s1] - s1 + t % s1 for t in range(batch * s1)]
    n_pos = max(ori)
    mode = {"swa": "none", "cfa": "all", "scfa": "sparse"}[kind]
    win = window_generate(batch=batch, s1=s1, n_q=n_q, ori_lens=ori, window=window, ratio=max(ratio, 4),
                          cmp_mode=mode, topk_cmp=topk_cmp, seed=seed, rope_dim=0, name=name)
    pro = prolog_v4_generate(tokens=batch * s1, n_q=n_q, hidden=hidden, q_lora_rank=q_lora_rank, positions=pos,
                             rope_positions=n_pos, seed=seed + 7)
    catt = cidx = ip = None
    if kind != "swa":
        starts = [v - s1 for v in ori]
        mb_cmp = win.block_table_cmp.shape[1]
        rows = win.num_cache_rows
        catt = compress_generate(batch=batch, s1=s1, ratio=ratio, start_pos=starts, rope_positions=n_pos,
                                 max_blocks=mb_cmp, n_pool_blocks=rows // BLOCK_SIZE, seed=seed + 11,
                                 block_table=win.block_table_cmp, channels=KV_LORA_RANK)
        catt.key_nope = win.key_nope
    if kind == "scfa":
        cidx = compress_generate(batch=batch, s1=s1, ratio=ratio, start_pos=starts, rope_positions=n_pos,
                                 max_blocks=mb_cmp, n_pool_blocks=rows // BLOCK_SIZE, seed=seed + 13,
                                 block_table=win.block_table_cmp, channels=128, rotate=True)
        # the index keys already in the compressed index-key cache: N(0,1) bf16 (the generator's
        # random bit patterns, which catch stray writes in the compressor's own tests, hold NaNs)
        cidx.key_nope = _normal_bf16(torch.Generator().manual_seed(130_000 + int(seed)), rows, 128)
        ip = indexer_prolog_generate(tokens=batch * s1, hidden=hidden, q_lora_rank=q_lora_rank, positions=pos,
                                     rope_positions=n_pos, rotate=True, seed=seed + 17)
        ip.x = pro.x  # one hidden state per token feeds both prologs
    return V4LayerInputs(kind=kind, prolog=pro, window=win, compress_att=catt, compress_idx=cidx, indexer_prolog=ip,
                         topk_cmp=int(topk_cmp))


def v4_scfa_layer_generate(**kw) -> V4LayerInputs:
    return v4_layer_generate(kind="scfa", **kw)


def v4_layer_decode(kind: str, seed: int = 0) -> V4LayerInputs:
    """One decode step of a V4 layer at the pages' shape: 64 sequences x 2 new tokens, 8K of
    original cache, window 128; SCFA with ratio 4 (2,048 compressed entries) and 512 entries
    selected per token, CFA with ratio 128 (every causal entry of 64); 128 heads of 512 channels,
    hidden 4096, query rank 1536."""
    return v4_layer_generate(kind=kind, batch=64, s1=2, n_q=128, hidden=4096, q_lora_rank=1536, ori_lens=[8192] * 64,
                             window=128, topk_cmp=512 if kind == "scfa" else 0, seed=seed,
                             name=f"v4_{kind}_layer_b64_s2")


def v4_scfa_layer_decode(seed: int = 0) -> V4LayerInputs:
    return v4_layer_decode("scfa", seed)


def v4_swa_layer_decode(seed: int = 0) -> V4LayerInputs:
    return v4_layer_decode("swa", seed)


def v4_cfa_layer_decode(seed: int = 0) -> V4LayerInputs:
    return v4_layer_decode("cfa", seed)


def compress_index_decode(seed: int = 0, ratio: int = 4) -> CompressInputs:
    """The page's D = 128 compressor configuration (the index keys the Lightning Indexer scores
    over the compressed cache) on the same decode step: 64 sequences, positions 8190 and 8191,
    ratio 4, rotate = true."""
    return compress_generate(batch=64, s1=2, ratio=ratio, start_pos=[8190] * 64, rope_positions=8192,
                             max_blocks=2048 // BLOCK_SIZE, seed=seed, channels=128, rotate=True,
                             name=f"compress_b64_s2_r{ratio}_c128_rot")


# ---- Indexer prolog ----------------------------------------------------------------------

@dataclasses.dataclass
class IndexerPrologInputs:
    tokens: int
    n_heads: int
    x: np.ndarray               # uint16 bf16 bits (T, hidden)
    qr: np.ndarray              # uint16 (T, q_lora_rank): the normalised query of the MLA prolog
    w_idx_qb: np.ndarray        # uint16 (n_heads * head_dim, q_lora_rank)
    w_idx_k: np.ndarray         # uint16 (head_dim, hidden)
    ln_gamma_k: np.ndarray      # uint16 (head_dim)
    ln_beta_k: np.ndarray       # uint16 (head_dim)
    w_idx_proj: np.ndarray      # uint16 (n_heads, hidden)
    positions: np.ndarray       # int32 (T)
    rope_cos: np.ndarray        # float32 (rope_positions, 32)
    rope_sin: np.ndarray
    eps: float
    rotate: bool
    name: str = ""

    @property
    def hidden(self) -> int:
        return int(self.x.shape[1])

    @property
    def q_lora_rank(self) -> int:
        return int(self.qr.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.w_idx_k.shape[0])

    @property
    def rope_positions(self) -> int:
        return int(self.rope_cos.shape[0])


def indexer_prolog_generate(*, tokens: int, hidden: int = 7168, q_lora_rank: int = 1536, n_heads: int = 64,
                            head_dim: int = 128, positions: Optional[Sequence[int]] = None,
                            rope_positions: int = 8192, rotate: bool = True, seed: int = 0,
                            name: str = "") -> IndexerPrologInputs:
    """x and qr are N(0,1) (qr stands for the MLA prolog's RMS-normalised query); each weight is
    N(0, 1/fan_in); the LayerNorm scale is 1 + N(0, 0.1^2) and its shift N(0, 0.1^2); all bf16.
    Positions default to 8190, 8191 alternating; eps is 1e-6."""
    g = torch.Generator().manual_seed(120_000 + int(seed))
    x = _scaled_bf16(g, (tokens, hidden), 1.0)
    qr = _scaled_bf16(g, (tokens, q_lora_rank), 1.0)
    w_qb = _scaled_bf16(g, (n_heads * head_dim, q_lora_rank), q_lora_rank ** -0.5)
    w_k = _scaled_bf16(g, (head_dim, hidden), hidden ** -0.5)
    gamma = _bf16_bits(1.0 + torch.randn(head_dim, generator=g) * 0.1)
    beta = _bf16_bits(torch.randn(head_dim, generator=g) * 0.1)
    w_proj = _scaled_bf16(g, (n_heads, hidden), hidden ** -0.5)
    if positions is None:
        positions = [8190 + (t % 2) for t in range(tokens)]
    cos, sin = rope_tables(rope_positions)
    return IndexerPrologInputs(tokens=int(tokens), n_heads=int(n_heads), x=x, qr=qr, w_idx_qb=w_qb, w_idx_k=w_k,
                               ln_gamma_k=gamma, ln_beta_k=beta, w_idx_proj=w_proj,
                               positions=np.ascontiguousarray(positions, dtype=np.int32), rope_cos=cos, rope_sin=sin,
                               eps=1e-6, rotate=bool(rotate), name=name)


def indexer_prolog_decode(seed: int = 0) -> IndexerPrologInputs:
    """The decode step's indexer prolog: 64 sequences x 2 new tokens, hidden 7168, query rank
    1536, 64 index heads of 128, with the Hadamard transform."""
    return indexer_prolog_generate(tokens=128, seed=seed, name="indexer_prolog_b64_s2")
