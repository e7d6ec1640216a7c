"""Pins for the fp64 oracle: each check ties the oracle to something other than itself.

What pins what:
  bf16 decode        -- IEEE bit patterns with known values
  bf16 RNE           -- hand-derived ties / overflow / NaN cases; torch's own bf16 cast on many values
  INT8 chain         -- hand-derived double-rounding cases; per-group scale placement; torch's
                        float32 multiply + bf16 cast as a second route
  resolve            -- a hand-worked block table; a scalar loop
  attention          -- scalar brute force (pure Python, math.exp, struct decoding) on tiny inputs;
                        closed forms CF1 (dense equivalence vs torch SDPA on the unpaged sequence),
                        CF2 (single key), CF3 (equal scores -> mean), CF4 (block permutation),
                        CF5 (slot order / padding position), CF6 (hardmax limit); duplicates;
                        empty set
Run on the CPU (no GPU marker).
"""

import math
import struct

import numpy as np
import pytest
import torch

import oracle.sfa_oracle as O
from mla_sparse_top_amd import workloads as W


# ----------------------------------------------------------------------------------------
# scalar helpers (an independent route: Python floats, struct packing, integer rounding)
# ----------------------------------------------------------------------------------------

def _bf16_scalar(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _round_f32_to_bf16_scalar(x32: float) -> int:
    u = _f32_bits(x32)
    hi, lo = u >> 16, u & 0xFFFF
    if lo > 0x8000 or (lo == 0x8000 and (hi & 1)):
        hi += 1
    return hi & 0xFFFF


def _dequant_scalar(code: int, scale_f32: float) -> float:
    # code * scale is exact in a Python float (8-bit times 24-bit significands);
    # struct.pack('<f') rounds it to binary32, to nearest even.
    p32 = struct.unpack("<f", struct.pack("<f", float(code) * scale_f32))[0]
    return _bf16_scalar(_round_f32_to_bf16_scalar(p32))


def _brute_force(inp, token: int):
    """Plain loops over heads, slots and dimensions for one token."""
    h_n = inp.n_q
    b = token // inp.s1
    act = int(inp.kv_act_seqs[b])
    rows = []
    for j in inp.topk_indices[token].tolist():
        if 0 <= j < act:
            blk = int(inp.block_table[b][j // 128])
            rows.append(blk * 128 + (j % 128))
    out = [[0.0] * 512 for _ in range(h_n)]
    if not rows:
        return out

    def kn(r, d):
        if inp.kv_dtype == "int8":
            return _dequant_scalar(int(inp.key_nope[r][d]), float(inp.k_nope_scales[r][d // 128]))
        return _bf16_scalar(int(inp.key_nope[r][d]))

    kcache = {r: ([kn(r, d) for d in range(512)], [_bf16_scalar(int(inp.key_rope[r][d])) for d in range(64)])
              for r in set(rows)}
    for h in range(h_n):
        qrow = token * h_n + h
        qn = [_bf16_scalar(int(v)) for v in inp.query_nope[qrow]]
        qr = [_bf16_scalar(int(v)) for v in inp.query_rope[qrow]]
        scores = []
        for r in rows:
            kn_r, kr_r = kcache[r]
            s = 0.0
            for d in range(512):
                s += qn[d] * kn_r[d]
            for d in range(64):
                s += qr[d] * kr_r[d]
            scores.append(inp.softmax_scale * s)
        mx = max(scores)
        e = [math.exp(s - mx) for s in scores]
        tot = sum(e)
        for k, r in enumerate(rows):
            w = e[k] / tot
            kn_r = kcache[r][0]
            for d in range(512):
                out[h][d] += w * kn_r[d]
    return out


# ----------------------------------------------------------------------------------------
# bf16 decode / round
# ----------------------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x3E80], dtype=np.uint16)
    want = [1.0, -2.0, 3.140625, math.inf, -math.inf, 2.0 ** -133, -0.0, 0.25]
    got = O.bf16_bits_to_f64(bits)
    for g, w in zip(got.tolist(), want):
        assert g == w
    assert math.copysign(1.0, got[6]) == -1.0
    assert np.isnan(O.bf16_bits_to_f64(np.array([0x7FC1], dtype=np.uint16)))[0]


@pytest.mark.parametrize("f32_bits,bf16_bits", [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: exact tie between 0x3F80 and 0x3F81, keep the even 0x3F80
    (0x3F818000, 0x3F82),  # 1 + 3*2^-8: tie between 0x3F81 and 0x3F82, go to the even 0x3F82
    (0x3F808001, 0x3F81),  # just above the tie: up
    (0x3F807FFF, 0x3F80),  # just below the tie: down
    (0xBF808000, 0xBF80),  # negative tie, magnitude rounds to even
    (0x7F7FFFFF, 0x7F80),  # FLT_MAX: the discarded half is above the tie, carries into +inf
    (0x7F7F7FFF, 0x7F7F),  # below the tie: stays finite
    (0x7F800000, 0x7F80),  # +inf
    (0x7FC00000, 0x7FC0),  # quiet NaN
    (0x7F800001, 0x7FC0),  # signalling NaN becomes quiet, never inf
    (0x00008000, 0x0000),  # subnormal tie toward the even zero
    (0x00018000, 0x0002),  # subnormal tie toward the even 0x0002
])
def test_bf16_rne_hand_cases(f32_bits, bf16_bits):
    x = np.array([f32_bits], dtype=np.uint32).view(np.float32)
    assert int(O.f32_to_bf16_bits_rne(x)[0]) == bf16_bits


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # force a quarter of them onto exact ties
    u[::4] = (u[::4] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = O.f32_to_bf16_bits_rne(f)
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


# ----------------------------------------------------------------------------------------
# INT8 dequant chain
# ----------------------------------------------------------------------------------------

def _chain_one(code, scale_bits):
    s = np.array([[scale_bits] * 4], dtype=np.uint32).view(np.float32)
    c = np.full((1, 512), code, dtype=np.int8)
    return O.dequant_int8_chain(c, s)[0, 0]


def test_int8_chain_double_rounding_down():
    # scale 0x3EAB5556 = 11228502 * 2^-25. Times 3: 33685506 * 2^-25 = 8421376.5 * 2^-23,
    # an exact fp32 tie that rounds to the even 8421376 * 2^-23 = 1 + 2^-8.
    # That is a bf16 tie, which rounds to the even 0x3F80 = 1.0.
    # Rounding the exact product (just above 1 + 2^-8) straight to bf16 would give 0x3F81.
    assert _chain_one(3, 0x3EAB5556) == 1.0


def test_int8_chain_double_rounding_up():
    # scale 0x3EACAAAA = 11315882 * 2^-25. Times 3: 33947646 * 2^-25 = 8486911.5 * 2^-23,
    # an fp32 tie that goes to the even 8486912 * 2^-23 = 1 + 3 * 2^-8.
    # That is a bf16 tie between 0x3F81 and 0x3F82, which goes to the even 0x3F82 = 1 + 2^-6.
    # Rounding the exact product (just below the tie) straight to bf16 would give 0x3F81.
    assert _chain_one(3, 0x3EACAAAA) == 1.0 + 2.0 ** -6


def test_int8_chain_extreme_codes_and_group_placement():
    # Scales that are powers of two make every product exact in bf16. So each output column
    # equals code * scale of ITS group. This catches a wrong group index (d // 128).
    codes = np.zeros((3, 512), dtype=np.int8)
    codes[0, :] = 1
    codes[1, :] = -128
    codes[2, :] = 127
    scales = np.array([[1.0, 2.0, 4.0, 0.5]] * 3, dtype=np.float32)
    got = O.dequant_int8_chain(codes, scales)
    want_scale = np.repeat(np.array([1.0, 2.0, 4.0, 0.5]), 128)
    assert np.array_equal(got[0], want_scale)
    assert np.array_equal(got[1], -128.0 * want_scale)
    # 127 * 2 = 254 is bf16-exact (8 significant bits: 0b11111110)
    assert np.array_equal(got[2], 127.0 * want_scale)


def test_int8_chain_matches_torch_route_and_scalar_route():
    rng = np.random.default_rng(3)
    codes = rng.integers(-128, 128, size=(64, 512), dtype=np.int64).astype(np.int8)
    scales = (rng.random((64, 4)) * 0.05 + 1e-3).astype(np.float32)
    ours = O.dequant_int8_chain(codes, scales)
    t = (torch.from_numpy(codes).to(torch.float16).to(torch.float32)
         * torch.from_numpy(np.repeat(scales, 128, axis=1))).to(torch.bfloat16).to(torch.float64)
    assert np.array_equal(ours, t.numpy())
    for r in range(0, 64, 9):
        for d in range(0, 512, 37):
            assert ours[r, d] == _dequant_scalar(int(codes[r, d]), float(scales[r, d // 128]))


# ----------------------------------------------------------------------------------------
# resolve
# ----------------------------------------------------------------------------------------

def test_resolve_hand_worked():
    # batch 0: live 200 positions in logical blocks [3, 1]; batch 1: live 129 in blocks [0, 2]
    bt = np.array([[3, 1], [0, 2]], dtype=np.int32)
    act = np.array([200, 129], dtype=np.int32)
    idx = np.array([
        [0, 127, 128, 199, 200, -1, 5],
        [0, 128, 129, 255, -7, 64, 127],
    ], dtype=np.int32)
    want = np.array([
        [3 * 128 + 0, 3 * 128 + 127, 1 * 128 + 0, 1 * 128 + 71, -1, -1, 3 * 128 + 5],
        [0 * 128 + 0, 2 * 128 + 0, -1, -1, -1, 64, 127],
    ])
    assert np.array_equal(O.resolve_rows(idx, bt, act, s1=1), want)


def test_resolve_two_tokens_per_batch_share_bound():
    bt = np.array([[2, 0]], dtype=np.int32)
    act = np.array([130], dtype=np.int32)
    idx = np.array([[129, 130], [0, 131]], dtype=np.int32)
    assert np.array_equal(O.resolve_rows(idx, bt, act, s1=2), [[1, -1], [256, -1]])


def test_resolve_matches_scalar_loop():
    inp = W.generate(batch=3, s1=2, n_q=16, act_seqs=[700, 129, 5], topk=300, seed=4,
                     max_blocks_per_batch=8)
    rows = O.resolve_rows(inp.topk_indices, inp.block_table, inp.kv_act_seqs, inp.s1)
    for t in range(inp.n_tokens):
        b = t // inp.s1
        for k, j in enumerate(inp.topk_indices[t].tolist()):
            if 0 <= j < int(inp.kv_act_seqs[b]):
                assert rows[t, k] == int(inp.block_table[b][j // 128]) * 128 + j % 128
            else:
                assert rows[t, k] == -1


# ----------------------------------------------------------------------------------------
# attention: brute force and closed forms
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype", ["bf16", "int8"])
def test_oracle_matches_scalar_brute_force(kv_dtype):
    inp = W.generate(batch=2, s1=2, n_q=2, act_seqs=[150, 9], topk=6, kv_dtype=kv_dtype, seed=11,
                     max_blocks_per_batch=3)
    # plant slots the oracle must mask: an index at the live length, and padding in the middle
    inp.topk_indices[0, 1] = 150
    inp.topk_indices[1, 2] = -1
    ref = O.sparse_mla_attention(inp).reshape(inp.n_tokens, inp.n_q, 512)
    for t in range(inp.n_tokens):
        bf = np.array(_brute_force(inp, t))
        assert np.max(np.abs(bf - ref[t])) <= 1e-12


def _contiguous_instance(seq_len, n_q, seed, scale=None, n_tokens=2):
    """A paged instance built FROM an unpaged sequence: the test scatters logical blocks into a
    random physical order itself, so the dense reference below never sees the block table."""
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    nblk = -(-seq_len // 128)
    seq_nope = torch.randn(nblk * 128, 512, generator=g).to(torch.bfloat16)
    seq_rope = torch.randn(nblk * 128, 64, generator=g).to(torch.bfloat16)
    q_nope = torch.randn(n_tokens * n_q, 512, generator=g).to(torch.bfloat16)
    q_rope = torch.randn(n_tokens * n_q, 64, generator=g).to(torch.bfloat16)
    phys = rng.permutation(nblk + 2)[:nblk]  # two spare physical blocks stay NaN
    pool_n = np.full(((nblk + 2) * 128, 512), W.BF16_QNAN, dtype=np.uint16)
    pool_r = np.full(((nblk + 2) * 128, 64), W.BF16_QNAN, dtype=np.uint16)
    sn = seq_nope.view(torch.int16).numpy().view(np.uint16)
    sr = seq_rope.view(torch.int16).numpy().view(np.uint16)
    for lb, pb in enumerate(phys):
        pool_n[pb * 128:(pb + 1) * 128] = sn[lb * 128:(lb + 1) * 128]
        pool_r[pb * 128:(pb + 1) * 128] = sr[lb * 128:(lb + 1) * 128]
    idx = np.stack([rng.permutation(seq_len) for _ in range(n_tokens)]).astype(np.int32)
    inp = W.SfaInputs(
        batch=1, s1=n_tokens, n_q=n_q, topk=seq_len, kv_dtype="bf16",
        query_nope=q_nope.view(torch.int16).numpy().view(np.uint16),
        query_rope=q_rope.view(torch.int16).numpy().view(np.uint16),
        key_nope=pool_n, key_rope=pool_r, k_nope_scales=None, topk_indices=idx,
        block_table=phys.astype(np.int32)[None, :], kv_act_seqs=np.array([seq_len], dtype=np.int32),
        softmax_scale=float(np.float32(scale if scale is not None else 1 / math.sqrt(576))),
        poison_blocks=())
    return inp, seq_nope[:seq_len], seq_rope[:seq_len], q_nope, q_rope


def test_cf1_topk_covering_all_positions_equals_dense_attention():
    inp, kn, kr, qn, qr = _contiguous_instance(seq_len=300, n_q=8, seed=5)
    ref = O.sparse_mla_attention(inp).reshape(inp.n_tokens, inp.n_q, 512)
    k = torch.cat([kn, kr], dim=1).to(torch.float64)          # (S, 576)
    v = kn.to(torch.float64)                                  # (S, 512)
    for t in range(inp.n_tokens):
        q = torch.cat([qn[t * 8:(t + 1) * 8], qr[t * 8:(t + 1) * 8]], dim=1).to(torch.float64)
        dense = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], scale=inp.softmax_scale)[0]
        assert np.max(np.abs(dense.numpy() - ref[t])) <= 1e-12


def test_cf2_single_selected_key_returns_its_value_row():
    inp = W.generate(batch=1, s1=1, n_q=4, act_seqs=[256], topk=8, seed=2)
    inp.topk_indices[0, :] = -1
    inp.topk_indices[0, 5] = 200
    out = O.sparse_mla_attention(inp)[0, 0]
    row = int(inp.block_table[0, 1]) * 128 + 72
    want = O.bf16_bits_to_f64(inp.key_nope[row])
    for h in range(4):
        assert np.array_equal(out[h], want)


def test_cf3_equal_scores_give_mean_of_selected_rows():
    inp = W.generate(batch=1, s1=1, n_q=2, act_seqs=[256], topk=40, seed=3)
    inp.query_nope[:] = 0
    inp.query_rope[:] = 0
    out = O.sparse_mla_attention(inp)[0, 0]
    rows = [int(inp.block_table[0, j // 128]) * 128 + j % 128 for j in inp.topk_indices[0]]
    vals = np.array([[_bf16_scalar(int(x)) for x in inp.key_nope[r]] for r in rows])
    mean = vals.mean(axis=0)
    assert np.max(np.abs(out - mean)) <= 1e-13


def test_cf4_block_permutation_invariance_is_exact():
    inp = W.generate(batch=2, s1=2, n_q=8, act_seqs=[600, 300], topk=64, seed=8, extra_pool_blocks=3)
    ref = O.sparse_mla_attention(inp)
    rng = np.random.default_rng(0)
    n_pool = inp.num_cache_rows // 128
    perm = rng.permutation(n_pool)                 # physical block p moves to perm[p]
    kn = np.empty_like(inp.key_nope)
    kr = np.empty_like(inp.key_rope)
    for p in range(n_pool):
        kn[perm[p] * 128:(perm[p] + 1) * 128] = inp.key_nope[p * 128:(p + 1) * 128]
        kr[perm[p] * 128:(perm[p] + 1) * 128] = inp.key_rope[p * 128:(p + 1) * 128]
    moved = W.SfaInputs(**{**inp.__dict__, "key_nope": kn, "key_rope": kr,
                           "block_table": perm[inp.block_table].astype(np.int32)})
    assert np.array_equal(O.sparse_mla_attention(moved), ref)


def test_cf5_slot_order_and_padding_position_do_not_matter():
    inp = W.generate(batch=1, s1=2, n_q=4, act_seqs=[500], topk=48, seed=9)
    inp.topk_indices[:, 40:] = -1
    ref = O.sparse_mla_attention(inp)
    rng = np.random.default_rng(1)
    shuffled = inp.topk_indices[:, rng.permutation(48)].copy()
    moved = W.SfaInputs(**{**inp.__dict__, "topk_indices": shuffled})
    assert np.max(np.abs(O.sparse_mla_attention(moved) - ref)) <= 1e-12


def test_cf6_large_scale_selects_the_argmax_row():
    inp = W.generate(batch=1, s1=1, n_q=3, act_seqs=[128], topk=16, seed=12, softmax_scale=4096.0)
    out = O.sparse_mla_attention(inp)[0, 0]
    rows = [int(inp.block_table[0, 0]) * 128 + j for j in inp.topk_indices[0]]
    for h in range(3):
        qn = np.array([_bf16_scalar(int(x)) for x in inp.query_nope[h]])
        qr = np.array([_bf16_scalar(int(x)) for x in inp.query_rope[h]])
        sc = [qn @ np.array([_bf16_scalar(int(x)) for x in inp.key_nope[r]])
              + qr @ np.array([_bf16_scalar(int(x)) for x in inp.key_rope[r]]) for r in rows]
        order = np.argsort(sc)
        assert sc[order[-1]] - sc[order[-2]] > 0.01  # a clear winner at this scale
        best = rows[order[-1]]
        want = np.array([_bf16_scalar(int(x)) for x in inp.key_nope[best]])
        assert np.max(np.abs(out[h] - want)) <= 1e-9


def test_duplicates_count_per_occurrence():
    inp = W.generate(batch=1, s1=1, n_q=2, act_seqs=[128], topk=3, seed=13)
    inp.topk_indices[0] = [5, 5, 9]
    out = O.sparse_mla_attention(inp)[0, 0]
    r5, r9 = int(inp.block_table[0, 0]) * 128 + 5, int(inp.block_table[0, 0]) * 128 + 9
    for h in range(2):
        q = np.concatenate([O.bf16_bits_to_f64(inp.query_nope[h]), O.bf16_bits_to_f64(inp.query_rope[h])])
        k5 = np.concatenate([O.bf16_bits_to_f64(inp.key_nope[r5]), O.bf16_bits_to_f64(inp.key_rope[r5])])
        k9 = np.concatenate([O.bf16_bits_to_f64(inp.key_nope[r9]), O.bf16_bits_to_f64(inp.key_rope[r9])])
        s5, s9 = inp.softmax_scale * (q @ k5), inp.softmax_scale * (q @ k9)
        m = max(s5, s9)
        w5 = 2 * math.exp(s5 - m) / (2 * math.exp(s5 - m) + math.exp(s9 - m))
        want = w5 * k5[:512] + (1 - w5) * k9[:512]
        assert np.max(np.abs(out[h] - want)) <= 1e-12


def test_empty_valid_set_gives_zeros():
    inp = W.generate(batch=1, s1=2, n_q=4, act_seqs=[64], topk=8, seed=14)
    inp.topk_indices[0, :] = -1
    inp.topk_indices[1, :] = 64  # at the live length: masked
    assert np.array_equal(O.sparse_mla_attention(inp), np.zeros((1, 2, 4, 512)))


def test_allclose_report_semantics():
    ref = np.array([0.0, 1.0, -2.0, 10.0])
    assert O.allclose_report(ref + np.array([0.9e-4, 5.0e-3, -1.0e-2, 0.0]), ref)["fails"] == 0
    assert O.allclose_report(ref + np.array([1.01e-4, 0, 0, 0]), ref)["fails"] == 1
    got = ref.copy()
    got[3] = np.nan
    assert O.allclose_report(got, ref)["fails"] == 1
