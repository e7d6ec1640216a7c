"""Plant plausible mistakes in the oracle (on the CPU only) and check that the pins catch each.

Each mutant swaps one oracle function for a subtly wrong version and then re-runs a pin from
test_oracle_pins. The pins must fail with the mutant installed; otherwise they are too weak to
guard the oracle.
"""

import numpy as np
import pytest

import oracle.sfa_oracle as O
import tests.test_oracle_pins as P

_real_token = O.sparse_mla_attention_token
_real_resolve = O.resolve_rows
_real_chain = O.dequant_int8_chain
_real_gather = O.gather_latents


def _drop_rope(qn, qr, kn, kr, scale):
    return _real_token(qn, qr * 0.0, kn, kr, scale)


def _scale_after_softmax(qn, qr, kn, kr, scale):
    return _real_token(qn, qr, kn, kr, 1.0)


def _value_is_rope_padded(qn, qr, kn, kr, scale):
    out = _real_token(qn, qr, kn, kr, scale)
    out[:, :64] = _real_token(qn, qr, np.concatenate([kr, kn[:, 64:]], axis=1), kr, scale)[:, :64]
    return out


def _no_max_subtract_sign_flip(qn, qr, kn, kr, scale):
    return _real_token(-qn, -qr, kn, kr, scale)


def _resolve_inclusive_bound(idx, bt, act, s1):
    return _real_resolve(idx, bt, np.asarray(act) + 1, s1)


def _resolve_swapped_block_math(idx, bt, act, s1):
    idx = np.asarray(idx, dtype=np.int64)
    b_of_t = np.arange(idx.shape[0]) // s1
    valid = (idx >= 0) & (idx < np.asarray(act)[b_of_t][:, None])
    safe = np.where(valid, idx, 0)
    blocks = np.asarray(bt)[b_of_t[:, None], safe % np.asarray(bt).shape[1]]
    return np.where(valid, blocks * 128 + safe // 128, -1)


def _chain_exact(codes, scales):
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 128, axis=-1)


def _chain_wrong_group(codes, scales):
    return _real_chain(codes, np.roll(scales, 1, axis=-1))


def _gather_rope_from_nope(rows, key_nope, key_rope, scales):
    kn, kr = _real_gather(rows, key_nope, key_rope, scales)
    return kn, kn[:, :64].copy()


MUTANTS = {
    "drop_rope": ("sparse_mla_attention_token", _drop_rope),
    "scale_ignored": ("sparse_mla_attention_token", _scale_after_softmax),
    "value_mixes_rope": ("sparse_mla_attention_token", _value_is_rope_padded),
    "sign_flip": ("sparse_mla_attention_token", _no_max_subtract_sign_flip),
    "resolve_inclusive_bound": ("resolve_rows", _resolve_inclusive_bound),
    "resolve_swapped_block_math": ("resolve_rows", _resolve_swapped_block_math),
    "chain_exact_dequant": ("dequant_int8_chain", _chain_exact),
    "chain_wrong_group": ("dequant_int8_chain", _chain_wrong_group),
    "gather_rope_from_nope": ("gather_latents", _gather_rope_from_nope),
}

PINS = [
    P.test_resolve_hand_worked,
    lambda: P.test_oracle_matches_scalar_brute_force("bf16"),
    lambda: P.test_oracle_matches_scalar_brute_force("int8"),
    P.test_cf1_topk_covering_all_positions_equals_dense_attention,
    P.test_cf2_single_selected_key_returns_its_value_row,
    P.test_int8_chain_double_rounding_down,
    P.test_int8_chain_extreme_codes_and_group_placement,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin)
    assert caught, f"no pin caught mutant {name}"
