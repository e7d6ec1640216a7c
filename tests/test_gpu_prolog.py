"""GPU parity of the MLA prolog (sfa_mla_prolog) against the CPU oracle (oracle/prolog_oracle.py).

The oracle is float64 and returns the outputs before their bf16 rounding; the GPU accumulates in
fp32 and carries cq and the per-head nope parts as bf16 hi + lo pairs. The bar is the
attention's, for every element of all four outputs: |gpu - ref| <= 1e-4 + 5e-3 * |ref| (one bf16
rounding moves a value by at most 2^-9 of itself; the fp32 sums add ~1e-6 relative). The
full-size case is the benchmark's workload in the same launch configuration.
"""

import numpy as np
import pytest

import oracle.prolog_oracle as P
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu

NAMES = ("q_nope", "q_rope", "kv_nope", "kv_rope")


def _bits(t):
    import torch

    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _oracle(inp):
    return P.mla_prolog(inp.x, inp.w_dq, inp.gamma_cq, inp.w_uq_qr, inp.w_uk, inp.w_dkv_kr, inp.gamma_ckv,
                        inp.positions, inp.rope_cos, inp.rope_sin, inp.eps, inp.n_q)


def _assert_close(inp, got, want=None):
    want = _oracle(inp) if want is None else want
    t, n = inp.tokens, inp.n_q
    shapes = ((t, n, 512), (t, n, 64), (t, 512), (t, 64))
    for name, g, w, sh in zip(NAMES, got, want, shapes):
        gv = P.bf16_bits_to_f64(_bits(g)).reshape(sh)
        err = np.abs(gv - w)
        bound = 1e-4 + 5e-3 * np.abs(w)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (f"{name}: {len(bad)} elements off, first {bad[:3].tolist()}, worst ratio "
                               f"{np.max(err / bound):.3f}")


def _run(sfa_lib, inp):
    import torch

    d = sfa_lib.prolog_to_device(inp)
    out = sfa_lib.run_prolog(inp, d)
    torch.cuda.synchronize()
    return d, out


@pytest.mark.parametrize("tokens,hidden,q,n_q,dn,seed", [
    (37, 512, 256, 4, 64, 0),        # one partial token block
    (200, 1024, 512, 3, 128, 1),     # a full and a ragged token block, odd head count
    (1, 256, 256, 1, 64, 2),         # the smallest shapes
    (130, 4096, 1024, 16, 128, 3),   # V4's hidden width
    (70, 512, 192, 128, 64, 4),      # three k chunks in one range: an odd chunk count
])
def test_small_shapes(sfa_lib, tokens, hidden, q, n_q, dn, seed):
    pos = [(7 * t) % 300 for t in range(tokens)]
    inp = W.prolog_generate(tokens=tokens, n_q=n_q, hidden=hidden, q_lora_rank=q, nope_dim=dn, positions=pos,
                            rope_positions=256, seed=seed)
    _, out = _run(sfa_lib, inp)
    _assert_close(inp, out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_full_size(sfa_lib, seed):
    """64 sequences x 2 new tokens, 128 heads, hidden 7168, query rank 1536: every element."""
    inp = W.prolog_decode(seed=seed)
    _, out = _run(sfa_lib, inp)
    _assert_close(inp, out)


def test_positions_outside_tables_give_zero_rotary_parts(sfa_lib):
    inp = W.prolog_generate(tokens=6, n_q=2, hidden=256, q_lora_rank=256, nope_dim=64,
                            positions=[-1, 0, 63, 64, 1000, -7], rope_positions=64, seed=5)
    _, out = _run(sfa_lib, inp)
    for t in (0, 3, 4, 5):
        assert not _bits(out[1]).reshape(6, 2, 64)[t].any()
        assert not _bits(out[3])[t].any()
    _assert_close(inp, out)


def test_repeat_calls_are_bit_identical(sfa_lib):
    import torch

    inp = W.prolog_generate(tokens=128, n_q=8, hidden=1024, q_lora_rank=512, nope_dim=128, seed=6)
    d, a = _run(sfa_lib, inp)
    a = [x.clone() for x in a]
    b = sfa_lib.run_prolog(inp, d)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_empty_call_is_a_no_op(sfa_lib):
    import torch

    inp = W.prolog_generate(tokens=0, n_q=2, hidden=256, q_lora_rank=256, nope_dim=64, seed=7)
    d = sfa_lib.prolog_to_device(inp)
    out = sfa_lib.run_prolog(inp, d)
    torch.cuda.synchronize()
    assert all(o.numel() == 0 for o in out)


def test_prolog_feeds_cache_write_and_decode(sfa_lib):
    """The prolog's latent rows, written by sfa_cache_write, are the rows sfa_decode reads, and
    its absorbed query is sfa_decode's query: decode over a cache holding only the new token's row
    returns that row (a single valid key gives weight 1)."""
    import torch

    b, s1 = 2, 1
    inp = W.prolog_generate(tokens=b * s1, n_q=16, hidden=512, q_lora_rank=256, nope_dim=64, positions=[0, 0],
                            rope_positions=16, seed=8)
    d, (qn, qr, kn, kr) = _run(sfa_lib, inp)
    blocks = torch.tensor([[0], [1]], dtype=torch.int32, device="cuda")
    key_nope = torch.zeros((256, 512), dtype=torch.bfloat16, device="cuda")
    key_rope = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    sfa_lib.cache_write(kn, kr, d["positions"], blocks, key_nope, key_rope, batch=b, s1=s1)
    torch.cuda.synchronize()
    assert torch.equal(key_nope[0].view(torch.int16), kn[0].view(torch.int16))
    assert torch.equal(key_nope[128].view(torch.int16), kn[1].view(torch.int16))
    assert torch.equal(key_rope[128].view(torch.int16), kr[1].view(torch.int16))
    idx = torch.zeros((b * s1, 1), dtype=torch.int32, device="cuda")
    act = torch.ones((b,), dtype=torch.int32, device="cuda")
    out = sfa_lib.decode(qn, qr, key_nope, key_rope, None, idx, blocks, act, 0.0417, batch=b, s1=s1)
    torch.cuda.synchronize()
    for t in range(b):
        for h in range(16):
            assert torch.equal(out[t, 0, h].view(torch.int16), kn[t].view(torch.int16))


# ---- the V4 form (sfa_mla_prolog_v4): 512-wide query heads and latent row, rotary part inside ----

def _oracle_v4(inp):
    return P.mla_prolog_v4(inp.x, inp.w_dq, inp.gamma_cq, inp.w_uq, inp.w_dkv, inp.gamma_ckv, inp.positions,
                           inp.rope_cos, inp.rope_sin, inp.eps, inp.n_q)


def _assert_close_v4(inp, got):
    want = _oracle_v4(inp)
    for name, g, w, sh in zip(("q", "kv"), got, want, ((inp.tokens, inp.n_q, 512), (inp.tokens, 512))):
        gv = P.bf16_bits_to_f64(_bits(g)).reshape(sh)
        err = np.abs(gv - w)
        bound = 1e-4 + 5e-3 * np.abs(w)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (f"{name}: {len(bad)} elements off, first {bad[:3].tolist()}, worst ratio "
                               f"{np.max(err / bound):.3f}")


@pytest.mark.parametrize("tokens,hidden,q,n_q,seed", [
    (37, 512, 256, 4, 0),        # one partial token block
    (200, 1024, 512, 3, 1),      # a full and a ragged token block, odd head count
    (1, 256, 64, 1, 2),          # the smallest shapes
    (130, 4096, 1024, 16, 3),    # the page's hidden width
    (100, 512, 192, 64, 4),      # three k chunks in one range: an odd chunk count
])
def test_v4_small_shapes(sfa_lib, tokens, hidden, q, n_q, seed):
    """Positions (7t) mod 300 against 256 table rows: some tokens get zero rotary channels."""
    import torch

    pos = [(7 * t) % 300 for t in range(tokens)]
    inp = W.prolog_v4_generate(tokens=tokens, n_q=n_q, hidden=hidden, q_lora_rank=q, positions=pos,
                               rope_positions=256, seed=seed)
    out = sfa_lib.run_prolog_v4(inp)
    torch.cuda.synchronize()
    _assert_close_v4(inp, out)


@pytest.mark.parametrize("seed", [0, 1])
def test_v4_decode_full_size(sfa_lib, seed):
    """64 sequences x 2 new tokens, 128 heads of 512 channels, hidden 4096: every element."""
    import torch

    inp = W.prolog_v4_decode(seed=seed)
    d = sfa_lib.prolog_v4_to_device(inp)
    cq = torch.empty((inp.tokens, inp.q_lora_rank), dtype=torch.bfloat16, device="cuda")
    out = sfa_lib.run_prolog_v4(inp, d, cq_out=cq)
    again = sfa_lib.run_prolog_v4(inp, d)
    torch.cuda.synchronize()
    _assert_close_v4(inp, out)
    assert all(torch.equal(a, b) for a, b in zip(out, again))  # repeat calls are bit-identical
    X = P.bf16_bits_to_f64(inp.x)
    want_cq = P.rms_norm(X @ P.bf16_bits_to_f64(inp.w_dq).T, P.bf16_bits_to_f64(inp.gamma_cq), inp.eps)
    got_cq = P.bf16_bits_to_f64(_bits(cq))
    assert np.all(np.abs(got_cq - want_cq) <= 1e-4 + 5e-3 * np.abs(want_cq))


def test_v4_feeds_cache_write_and_512_wide_swa(sfa_lib):
    """The V4 chain on the GPU: the prolog's latent rows go through sfa_cache_write (rope_dim 0)
    into a 512-wide pool at the new tokens' positions, and SWA on that pool reads the prolog's
    query heads. The written rows equal the prolog's bits; the attention meets the accuracy
    standard against the window oracle on the GPU-written pool and queries."""
    import torch

    import oracle.sfa_oracle as O
    import oracle.window_oracle as WO

    win = W.window_generate(batch=2, s1=2, n_q=16, ori_lens=[300, 200], window=64, cmp_mode="none", seed=31,
                            rope_dim=0)
    pos = [298, 299, 198, 199]
    pro = W.prolog_v4_generate(tokens=4, n_q=16, hidden=256, q_lora_rank=128, positions=pos, rope_positions=512,
                               seed=32)
    dw = sfa_lib.window_to_device(win)
    q, kv = sfa_lib.run_prolog_v4(pro)
    sfa_lib.cache_write(kv, None, torch.tensor(pos, dtype=torch.int32, device="cuda"), dw["block_table_ori"],
                        dw["key_nope"], None, None, batch=2, s1=2)
    dw["query_nope"] = q
    out = sfa_lib.run_window(win, dw)
    torch.cuda.synchronize()
    pool = _bits(dw["key_nope"])
    rows = [int(win.block_table_ori[t // 2, p // 128]) * 128 + p % 128 for t, p in enumerate(pos)]
    assert np.array_equal(pool[rows], _bits(kv))
    win.key_nope, win.query_nope = pool, _bits(q)
    ref = WO.window_attention(win)
    rep = O.allclose_report(out.float().cpu().numpy().astype(np.float64).reshape(ref.shape), ref)
    assert rep["fails"] == 0, rep


def test_v4_kv_ready_event(sfa_lib):
    """The optional event is recorded once kv and cq are final: a second stream that waits for it
    copies them while the call's up-projection may still run, and the copies equal the finished
    outputs; q is unaffected (every element checked against the oracle)."""
    import torch

    inp = W.prolog_v4_generate(tokens=150, n_q=8, hidden=512, q_lora_rank=256,
                               positions=[(5 * t) % 300 for t in range(150)], rope_positions=256, seed=9)
    d = sfa_lib.prolog_v4_to_device(inp)
    cq = torch.empty((inp.tokens, inp.q_lora_rank), dtype=torch.bfloat16, device="cuda")
    ev = torch.cuda.Event()
    side = torch.cuda.Stream()
    call = sfa_lib.prepare_prolog_v4_run(inp, d, cq_out=cq, kv_ready=ev)
    q, kv = call.out
    for _ in range(2):
        call()
        side.wait_event(ev)
        with torch.cuda.stream(side):
            kv_early, cq_early = kv.clone(), cq.clone()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(kv_early.view(torch.int16), kv.view(torch.int16))
        assert torch.equal(cq_early.view(torch.int16), cq.view(torch.int16))
    _assert_close_v4(inp, (q, kv))
