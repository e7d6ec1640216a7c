"""GPU parity of the indexer prolog (sfa_indexer_prolog) against the CPU oracle
(oracle/prolog_oracle.py, indexer_prolog), and of the MLA prolog's cq output.

The oracle is float64 before the outputs' rounding; the GPU accumulates in fp32, rounds q_index
and k_index once to bf16 and keeps the weights in fp32. The bar, for every element:
|gpu - ref| <= 1e-4 + 5e-3 * |ref|.
"""

import numpy as np
import pytest

import oracle.prolog_oracle as P
from mla_sparse_top_amd import workloads as W

pytestmark = pytest.mark.gpu


def _f64(t):
    import torch

    if t.dtype == torch.bfloat16:
        return P.bf16_bits_to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def _assert_close(inp, got):
    want = P.indexer_prolog(inp.x, inp.qr, inp.w_idx_qb, inp.w_idx_k, inp.ln_gamma_k, inp.ln_beta_k, inp.w_idx_proj,
                            inp.positions, inp.rope_cos, inp.rope_sin, inp.eps, inp.n_heads, inp.rotate)
    for name, g, w in zip(("q_index", "k_index", "weights"), got, want):
        gv = _f64(g).reshape(w.shape)
        err = np.abs(gv - w)
        bound = 1e-4 + 5e-3 * np.abs(w)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, f"{name}: {len(bad)} off, first {bad[:3].tolist()}, worst {np.max(err / bound):.3f}"


def _run(sfa_lib, inp):
    import torch

    d = sfa_lib.indexer_prolog_to_device(inp)
    out = sfa_lib.run_indexer_prolog(inp, d)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_full_size(sfa_lib, seed):
    """64 sequences x 2 new tokens, hidden 7168, query rank 1536, 64 heads, rotate: every element."""
    inp = W.indexer_prolog_decode(seed=seed)
    _assert_close(inp, _run(sfa_lib, inp))


@pytest.mark.parametrize("tokens,hidden,q,rotate,seed", [
    (37, 512, 256, False, 2),     # one partial token block, no transform
    (200, 1024, 512, True, 3),    # a full and a ragged token block
    (1, 256, 256, True, 4),       # the smallest shapes
])
def test_small_shapes(sfa_lib, tokens, hidden, q, rotate, seed):
    pos = [(11 * t) % 300 for t in range(tokens)]
    inp = W.indexer_prolog_generate(tokens=tokens, hidden=hidden, q_lora_rank=q, positions=pos, rope_positions=256,
                                    rotate=rotate, seed=seed)
    _assert_close(inp, _run(sfa_lib, inp))


def test_rotation_keeps_the_scores(sfa_lib):
    """With and without the transform the GPU's q . k agree (to the bf16 rounding of q and k)."""
    a = W.indexer_prolog_generate(tokens=8, hidden=512, q_lora_rank=256, rope_positions=16, positions=list(range(8)),
                                  rotate=True, seed=5)
    b = W.indexer_prolog_generate(tokens=8, hidden=512, q_lora_rank=256, rope_positions=16, positions=list(range(8)),
                                  rotate=False, seed=5)
    qa, ka, _ = (_f64(x) for x in _run(sfa_lib, a))
    qb, kb, _ = (_f64(x) for x in _run(sfa_lib, b))
    sa = qa.reshape(8, 64, 128) @ ka.T
    sb = qb.reshape(8, 64, 128) @ kb.T
    scale = np.abs(sb).max()
    assert np.max(np.abs(sa - sb)) < 2e-2 * scale
    assert not np.allclose(qa, qb)


def test_mla_prolog_cq_output(sfa_lib):
    """sfa_mla_prolog's cq output is RMSNorm(x . w_dq^T) * gamma_cq rounded to bf16."""
    import torch

    inp = W.prolog_generate(tokens=40, n_q=4, hidden=1024, q_lora_rank=512, nope_dim=128, seed=6)
    d = sfa_lib.prolog_to_device(inp)
    cq = torch.empty((40, 512), dtype=torch.bfloat16, device="cuda")
    sfa_lib.run_prolog(inp, d, cq_out=cq)
    torch.cuda.synchronize()
    want = P.rms_norm(P.bf16_bits_to_f64(inp.x) @ P.bf16_bits_to_f64(inp.w_dq).T, P.bf16_bits_to_f64(inp.gamma_cq),
                      inp.eps)
    got = _f64(cq)
    assert np.all(np.abs(got - want) <= 1e-4 + 5e-3 * np.abs(want))
