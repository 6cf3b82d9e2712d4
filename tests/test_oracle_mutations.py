"""Plant plausible mistakes in the oracle (CPU only) and check that at least
one pin in test_oracle_pins.py catches each one. This guards the pins
themselves: a pin that still passes on a broken oracle pins nothing."""
import numpy as np
import pytest

import oracle
import oracle.gmla_oracle as G
from tests import test_oracle_pins as P


def _rope_wrong_sign(u, pos, base):
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    theta = np.power(float(base), -2.0 * np.arange(d // 2) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    out = np.empty_like(u)
    out[..., 0::2] = u[..., 0::2] * np.cos(ang) + u[..., 1::2] * np.sin(ang)
    out[..., 1::2] = -u[..., 0::2] * np.sin(ang) + u[..., 1::2] * np.cos(ang)
    return out


def _rope_half_split(u, pos, base):
    # pairs (i, i + d/2) instead of (2i, 2i+1)
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    theta = np.power(float(base), -2.0 * np.arange(d // 2) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    a, b = u[..., : d // 2], u[..., d // 2:]
    return np.concatenate([a * np.cos(ang) - b * np.sin(ang), a * np.sin(ang) + b * np.cos(ang)], -1)


def _attend_strict(q_rows, k, v, t_rows, scale):
    # causal boundary s < t instead of s <= t (position 0 keeps itself)
    return _orig_attend(q_rows, k, v, [max(int(t) - 1, 0) for t in t_rows], scale)


def _attend_no_max(q_rows, k, v, t_rows, scale):
    o, lse = _orig_attend(q_rows, k, v, t_rows, scale)
    return o, lse - 1.0  # lse off by a constant


def _decode_drops_current_token(q_abs, cache, seq_start, seq_len, *a, **kw):
    # the current token's row left out of the softmax (exclusive boundary)
    return _orig_decode(q_abs, cache, seq_start, [max(int(n) - 1, 1) for n in seq_len], *a, **kw)


def _decode_lse_off(*a, **kw):
    o, lse = _orig_decode(*a, **kw)
    return o, lse + 0.5


def _decode_query_rotated_one_further(q_abs, cache, seq_start, seq_len, d_c, d_r, rope_base, sm_scale, **kw):
    # the RoPE query turned to position L_b instead of L_b - 1
    q = np.array(q_abs, dtype=np.float64)
    if d_r and rope_base:
        q[..., d_c:] = _orig_rope(q[..., d_c:], 1.0, rope_base)
    return _orig_decode(q, cache, seq_start, seq_len, d_c, d_r, rope_base, sm_scale, **kw)


def _sigmoid_wrong(z):
    return 1.0 / (1.0 + np.exp(np.asarray(z, dtype=np.float64)))


def _value_up_transposed_heads(o_lat, W_uv):
    o = np.einsum("thc,hdc->thd", np.asarray(o_lat, float), np.asarray(W_uv, float)[::-1])
    return o.reshape(o.shape[0], -1)


def _reconstruct_swapped(c, W_uk, W_uv):
    k, v = _orig_reconstruct(c, W_uk, W_uv)
    return k, np.einsum("...c,hdc->...hd", np.asarray(c, float), np.asarray(W_uv, float)[:, :, ::-1])


def _prepare_heads_swapped(x, W_c, W_kr, W_q, W_qr, W_uk, pos, base, **kw):
    # each head's query absorbed with another head's W_UK
    return _orig_prepare(x, W_c, W_kr, W_q, W_qr, np.asarray(W_uk, float)[::-1], pos, base, **kw)


def _prepare_pos_off_by_one(x, W_c, W_kr, W_q, W_qr, W_uk, pos, base, **kw):
    # the new RoPE key rotated to the previous position
    return _orig_prepare(x, W_c, W_kr, W_q, W_qr, W_uk, np.asarray(pos) - 1, base, **kw)


def _prepare_rotates_query(x, W_c, W_kr, W_q, W_qr, W_uk, pos, base, **kw):
    # the RoPE query rotated here as well as in the decode step
    row, q = _orig_prepare(x, W_c, W_kr, W_q, W_qr, W_uk, pos, base, **kw)
    d_c = row.shape[1] - (0 if W_kr is None else np.asarray(W_kr).shape[0])
    q = q.copy()
    q[..., d_c:] = G.rope_rotate(q[..., d_c:], np.asarray(pos, float)[:, None], base)
    return row, q


def _query_compression_permuted(x, W_dq):
    # the latent query's components in the wrong order
    return np.asarray(x, float) @ np.asarray(W_dq, float)[::-1].T


def _head_gate_tiled(x, o_tilde, W_g, b_g, W_o, return_gated=False):
    # channel n gated by head n % H instead of head n // d_v
    z = np.asarray(x, float) @ np.asarray(W_g, float).T + (0.0 if b_g is None else np.asarray(b_g, float))
    g = 1.0 / (1.0 + np.exp(-z))
    o = np.asarray(o_tilde, float)
    gated = o * np.tile(g, (1, o.shape[1] // g.shape[1]))
    y = gated @ np.asarray(W_o, float).T
    return (y, gated) if return_gated else y


def _prefill_no_rope_term(x, W_c, W_q, W_uk, W_uv, sm_scale, rows=None, **kw):
    # the RoPE query dropped from the score (the key part then adds nothing)
    if kw.get("W_qr") is not None:
        kw["W_qr"] = 0.0 * np.asarray(kw["W_qr"], float)
    return _orig_prefill(x, W_c, W_q, W_uk, W_uv, sm_scale, rows, **kw)


def _prefill_unrotated(x, W_c, W_q, W_uk, W_uv, sm_scale, rows=None, **kw):
    # decoupled RoPE parts used without rotating them
    kw["rope_base"] = 0.0
    return _orig_prefill(x, W_c, W_q, W_uk, W_uv, sm_scale, rows, **kw)


_orig_attend = G.attend_rows
_orig_decode = G.decode_reference
_orig_rope = G.rope_rotate
_orig_reconstruct = G.reconstruct_kv
_orig_prepare = G.decode_prepare_reference
_orig_prefill = G.prefill_reference

MUTATIONS = [
    ("rope_rotate", _rope_wrong_sign, [P.test_rope_matches_complex_rotation_and_is_relative,
                                       lambda: P.test_decode_matches_mqa_sdpa(8)]),
    ("rope_rotate", _rope_half_split, [P.test_rope_matches_complex_rotation_and_is_relative,
                                       lambda: P.test_decode_matches_mqa_sdpa(8)]),
    ("attend_rows", _attend_strict, [lambda: P.test_causal_attention_matches_torch_sdpa(7, 3, 5, 6),
                                     P.test_whole_layer_matches_scalar_brute_force]),
    ("attend_rows", _attend_no_max, [P.test_zero_query_gives_uniform_mean_and_log_count,
                                     P.test_first_position_returns_its_own_value_and_lse]),
    ("decode_reference", _decode_drops_current_token, [lambda: P.test_decode_matches_mqa_sdpa(0),
                                                       P.test_decode_equals_last_prefill_row]),
    ("decode_reference", _decode_lse_off, [P.test_decode_single_token_and_lse_closed_form,
                                           P.test_decode_equals_last_prefill_row]),
    ("decode_reference", _decode_query_rotated_one_further, [lambda: P.test_decode_matches_mqa_sdpa(8)]),
    ("sigmoid", _sigmoid_wrong, [P.test_sigmoid_matches_scipy_and_range, P.test_gate_special_cases,
                                 P.test_whole_layer_matches_scalar_brute_force]),
    ("value_up_projection", _value_up_transposed_heads,
     [P.test_decode_equals_last_prefill_row, P.test_value_up_projection_moves_wuv_past_the_weighted_sum]),
    ("reconstruct_kv", _reconstruct_swapped, [P.test_prefill_explicit_equals_absorbed_route,
                                              P.test_whole_layer_matches_scalar_brute_force]),
    ("decode_prepare_reference", _prepare_heads_swapped,
     [lambda: P.test_decode_prepare_then_decode_equals_explicit_attention(0),
      lambda: P.test_decode_prepare_then_decode_equals_explicit_attention(4),
      P.test_decode_prepare_absorbed_query_matches_scalar_loops]),
    ("decode_prepare_reference", _prepare_pos_off_by_one,
     [lambda: P.test_decode_prepare_then_decode_equals_explicit_attention(4)]),
    ("decode_prepare_reference", _prepare_rotates_query,
     [lambda: P.test_decode_prepare_then_decode_equals_explicit_attention(4)]),
    ("query_compression", _query_compression_permuted,
     [P.test_low_rank_query_equals_composed_projection, P.test_low_rank_query_decode_prepare_scalar_loops]),
    ("head_gate_out_reference", _head_gate_tiled,
     [P.test_head_gate_matches_scalar_loops, P.test_head_gate_equals_channel_gate_with_repeated_rows,
      P.test_head_gate_allows_folding_wo_wuv_in_decode]),
    ("prefill_reference", _prefill_no_rope_term,
     [P.test_rope_prefill_matches_scalar_brute_force, P.test_rope_prefill_rows_equal_absorbed_decode_steps]),
    ("prefill_reference", _prefill_unrotated,
     [P.test_rope_prefill_matches_scalar_brute_force, P.test_rope_prefill_rows_equal_absorbed_decode_steps]),
    ("rope_rotate", _rope_wrong_sign, [P.test_rope_prefill_matches_scalar_brute_force]),
]


@pytest.mark.parametrize("name,bad,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_every_planted_mistake_is_caught(monkeypatch, name, bad, pins):
    monkeypatch.setattr(G, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
