"""Pins for the fp64 oracle: each test checks it against something other than
itself -- a library routine, a closed form, an invariant, a special case, a
scalar brute force, or the numbers the pages print. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from gated_mla_latent_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _sdpa(q, k, v, scale, causal):
    """torch's own scaled_dot_product_attention in fp64 on the CPU.
    q,k,v: [L, H, d] numpy -> [L, H, dv]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o.numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("L,H,dk,dv", [(1, 1, 4, 4), (7, 3, 5, 6), (33, 2, 16, 8)])
def test_causal_attention_matches_torch_sdpa(L, H, dk, dv):
    q = rng.standard_normal((L, H, dk))
    k = rng.standard_normal((L, H, dk))
    v = rng.standard_normal((L, H, dv))
    scale = 0.37
    o, _ = O.causal_attention(q, k, v, scale)
    ref = _sdpa(q, k, v, scale, causal=True)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one_and_are_nonnegative():
    L, H = 9, 3
    q = rng.standard_normal((L, H, 4)) * 3
    k = rng.standard_normal((L, H, 4))
    # v = 1 everywhere: o_t = sum_s a_ts, which must be exactly one.
    o, _ = O.causal_attention(q, k, np.ones((L, H, 1)), 1.0)
    np.testing.assert_allclose(o, 1.0, atol=1e-12)
    # v_s = e_s (one-hot on the key index): o_t is the weight row itself.
    eye = np.broadcast_to(np.eye(L)[:, None, :], (L, H, L))
    a, _ = O.causal_attention(q, k, eye, 1.0)
    assert (a >= 0).all()
    # weights beyond t are exactly zero (causal, inclusive boundary)
    for t in range(L):
        assert np.all(a[t, :, t + 1:] == 0)
        assert np.all(a[t, :, t] > 0)


def test_first_position_returns_its_own_value_and_lse():
    L, H = 5, 2
    q = rng.standard_normal((L, H, 3))
    k = rng.standard_normal((L, H, 3))
    v = rng.standard_normal((L, H, 4))
    o, lse = O.causal_attention(q, k, v, 0.5)
    np.testing.assert_array_equal(o[0], v[0])
    np.testing.assert_allclose(lse[0], 0.5 * np.einsum("hd,hd->h", q[0], k[0]), atol=1e-12)


def test_zero_query_gives_uniform_mean_and_log_count():
    L, H = 6, 2
    q = np.zeros((L, H, 3))
    k = rng.standard_normal((L, H, 3))
    v = rng.standard_normal((L, H, 2))
    o, lse = O.causal_attention(q, k, v, 1.0)
    for t in range(L):
        np.testing.assert_allclose(o[t], v[: t + 1].mean(axis=0), atol=1e-12)
        np.testing.assert_allclose(lse[t], math.log(t + 1), atol=1e-12)


def test_dominant_key_selects_its_value():
    L, H, d = 4, 1, 2
    k = np.zeros((L, H, d))
    k[2, 0] = [50.0, 0.0]
    q = np.tile(np.array([50.0, 0.0]), (L, H, 1))
    v = rng.standard_normal((L, H, 3))
    o, _ = O.causal_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[3, 0], v[2, 0], atol=1e-12)


# ---------------------------------------------------------------- RoPE
def _rope_complex(u, pos, base):
    """RoPE as complex multiplication of interleaved pairs by e^{i pos theta}."""
    d = u.shape[-1]
    z = u[..., 0::2] + 1j * u[..., 1::2]
    theta = base ** (-np.arange(0, d, 2) / d)
    z = z * np.exp(1j * np.asarray(pos)[..., None] * theta)
    out = np.empty_like(u)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def test_rope_matches_complex_rotation_and_is_relative():
    d = 64
    q = rng.standard_normal((3, d))
    k = rng.standard_normal((3, d))
    for pos in [0, 1, 17, 1000, 131071]:
        np.testing.assert_allclose(O.rope_rotate(q, pos, 10000.0), _rope_complex(q, pos, 10000.0),
                                   rtol=0, atol=1e-10)
    np.testing.assert_array_equal(O.rope_rotate(q, 0, 10000.0), q)
    r = O.rope_rotate(q, 77, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # <R_t q, R_s k> depends only on t - s
    a = np.einsum("nd,nd->n", O.rope_rotate(q, 50, 10000.0), O.rope_rotate(k, 20, 10000.0))
    b = np.einsum("nd,nd->n", O.rope_rotate(q, 30, 10000.0), k)
    np.testing.assert_allclose(a, b, atol=1e-10)
    # d_r = 2 closed form: theta_0 = 1
    u = np.array([[1.0, 0.0]])
    np.testing.assert_allclose(O.rope_rotate(u, 0.5, 10000.0), [[math.cos(0.5), math.sin(0.5)]], atol=1e-15)


# ---------------------------------------------------------------- gate
def test_sigmoid_matches_scipy_and_range():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.sigmoid(z), scipy.special.expit(z), rtol=1e-14, atol=0)
    z = rng.standard_normal(1000) * 5
    s = O.sigmoid(z)
    assert ((s > 0) & (s < 1)).all()


def test_gate_special_cases():
    T, D, Hdv = 5, 8, 6
    x = rng.standard_normal((T, D))
    ot = rng.standard_normal((T, Hdv))
    W_o = rng.standard_normal((D, Hdv))
    # W_g = 0 -> every gate is exactly 1/2
    y = O.gate_out_reference(x, ot, np.zeros((Hdv, D)), W_o)
    np.testing.assert_allclose(y, 0.5 * ot @ W_o.T, atol=1e-12)
    # a gate driven to +inf lets o~ through unchanged (ungated MLA)
    W_g = np.zeros((Hdv, D)); W_g[:, 0] = 1.0
    x2 = x.copy(); x2[:, 0] = 80.0
    y = O.gate_out_reference(x2, ot, W_g, W_o)
    np.testing.assert_allclose(y, ot @ W_o.T, atol=1e-12)
    # driven to -inf, the layer output vanishes
    x2[:, 0] = -800.0
    y = O.gate_out_reference(x2, ot, W_g, W_o)
    np.testing.assert_allclose(y, 0.0, atol=1e-300)
    # the gate is per channel: channel j is scaled by sigmoid((W_g x)_j) alone
    W_g = rng.standard_normal((Hdv, D))
    _, gated = O.gate_out_reference(x, ot, W_g, W_o, return_gated=True)
    np.testing.assert_allclose(gated, scipy.special.expit(x @ W_g.T) * ot, atol=1e-14)


# ---------------------------------------------------------------- absorption
def test_prefill_explicit_equals_absorbed_route():
    """q.(W_UK c) = (W_UK^T q).c and sum_s a_s W_UV c_s = W_UV sum_s a_s c_s
    ([GF] §一, [N03] §5.1 / exercise 4): compute the layer through the
    absorbed route here and compare with the oracle's explicit route."""
    B, L, D, H, dc, dk, dv = 2, 11, 16, 3, 8, 5, 7
    x = rng.standard_normal((B, L, D))
    W_c = rng.standard_normal((dc, D))
    W_q = rng.standard_normal((H * dk, D))
    W_uk = rng.standard_normal((H, dk, dc))
    W_uv = rng.standard_normal((H, dv, dc))
    scale = 0.21
    c, ot, lse = O.prefill_reference(x, W_c, W_q, W_uk, W_uv, scale)
    for b in range(B):
        cb = x[b] @ W_c.T
        q = (x[b] @ W_q.T).reshape(L, H, dk)
        for h in range(H):
            qa = q[:, h] @ W_uk[h]  # [L, dc] absorbed query
            z = (qa @ cb.T) * scale
            z[np.triu_indices(L, 1)] = -np.inf
            a = scipy.special.softmax(z, axis=1)
            o_lat = a @ cb
            np.testing.assert_allclose(ot[b, :, h * dv:(h + 1) * dv], o_lat @ W_uv[h].T, atol=1e-11)
            np.testing.assert_allclose(lse[b, :, h], scipy.special.logsumexp(z, axis=1), atol=1e-11)


def test_prefill_matches_torch_sdpa_per_head():
    B, L, D, H, dc, dk, dv = 1, 20, 12, 2, 6, 4, 4
    x = rng.standard_normal((B, L, D))
    W_c = rng.standard_normal((dc, D)); W_q = rng.standard_normal((H * dk, D))
    W_uk = rng.standard_normal((H, dk, dc)); W_uv = rng.standard_normal((H, dv, dc))
    _, ot, _ = O.prefill_reference(x, W_c, W_q, W_uk, W_uv, 0.3)
    c = torch.nn.functional.linear(torch.from_numpy(x[0]), torch.from_numpy(W_c)).numpy()
    q = torch.nn.functional.linear(torch.from_numpy(x[0]), torch.from_numpy(W_q)).numpy().reshape(L, H, dk)
    k = np.stack([c @ W_uk[h].T for h in range(H)], axis=1)
    v = np.stack([c @ W_uv[h].T for h in range(H)], axis=1)
    ref = _sdpa(q, k, v, 0.3, causal=True).reshape(L, H * dv)
    np.testing.assert_allclose(ot[0], ref, atol=1e-12)


def test_prefill_rows_subset_equals_full():
    B, L, D, H, dc, dk, dv = 1, 13, 8, 2, 4, 3, 3
    x = rng.standard_normal((B, L, D))
    ws = [rng.standard_normal(s) for s in [(dc, D), (H * dk, D), (H, dk, dc), (H, dv, dc)]]
    _, full, lf = O.prefill_reference(x, *ws, 0.5)
    rows = [0, 4, 12]
    _, part, lp = O.prefill_reference(x, *ws, 0.5, rows=rows)
    np.testing.assert_allclose(part, full[:, rows], atol=1e-13)
    np.testing.assert_allclose(lp, lf[:, rows], atol=1e-13)


# ---------------------------------------------------------------- decode
def _decode_via_mqa_sdpa(inp):
    """Absorbed decode is MQA with one shared key [c; R k^R] and value c
    ([N03] §3.1): one torch SDPA call per sequence, RoPE via complex numbers."""
    q_abs = inp.q_abs.double().numpy()
    cache = inp.cache.double().numpy()
    outs = []
    for b in range(inp.B):
        L = int(inp.seq_len[b]); s0 = int(inp.seq_start[b])
        rows = cache[s0:s0 + L]
        q = q_abs[b].copy()
        if inp.d_r:
            q[:, inp.d_c:] = _rope_complex(q[:, inp.d_c:], L - 1, inp.rope_base)
        qt = torch.from_numpy(q)[:, None, :]  # [H, 1, W]
        kt = torch.from_numpy(rows)[None].expand(inp.H, L, rows.shape[1])
        vt = torch.from_numpy(rows[:, :inp.d_c])[None].expand(inp.H, L, inp.d_c)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=inp.sm_scale)
        outs.append(o[:, 0].numpy())
    return np.stack(outs)


@pytest.mark.parametrize("d_r", [0, 8])
def test_decode_matches_mqa_sdpa(d_r):
    inp = W.make_decode(4, 5, 16, d_r, 1, 40, dtype=torch.float32, seed=3)
    o, lse = O.decode_reference(inp.q_abs.numpy(), inp.cache.numpy(), inp.seq_start.numpy(),
                                inp.seq_len.numpy(), inp.d_c, inp.d_r, inp.rope_base, inp.sm_scale)
    np.testing.assert_allclose(o, _decode_via_mqa_sdpa(inp), atol=1e-12)
    assert np.isfinite(lse).all()


def test_decode_ignores_rows_outside_its_sequence():
    a = W.make_decode(3, 4, 16, 8, 5, 30, dtype=torch.float32, seed=5, gap_rows=0)
    b = W.make_decode(3, 4, 16, 8, 5, 30, dtype=torch.float32, seed=5, gap_rows=7)
    args = lambda i: (i.q_abs.numpy(), i.cache.numpy(), i.seq_start.numpy(), i.seq_len.numpy(),
                      i.d_c, i.d_r, i.rope_base, i.sm_scale)
    oa, la = O.decode_reference(*args(a))
    ob, lb = O.decode_reference(*args(b))
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_decode_single_token_and_lse_closed_form():
    inp = W.make_decode(2, 3, 8, 4, 1, 1, dtype=torch.float32, seed=9)
    q = inp.q_abs.double().numpy(); cache = inp.cache.double().numpy()
    o, lse = O.decode_reference(q, cache, inp.seq_start.numpy(), inp.seq_len.numpy(),
                                8, 4, inp.rope_base, inp.sm_scale)
    for b in range(2):
        row = cache[int(inp.seq_start[b])]
        np.testing.assert_array_equal(o[b], np.broadcast_to(row[:8], (3, 8)))
        # position 0: the rotation is the identity
        np.testing.assert_allclose(lse[b], inp.sm_scale * q[b] @ row, atol=1e-12)


def test_decode_equals_last_prefill_row():
    """Prefill's last row and a decode step over prefill's own latent agree
    once the query is absorbed (q~_h = W_UK^(h)T q_h) and W_UV is applied on
    the output side."""
    B, L, D, H, dc, dk, dv = 2, 9, 10, 3, 8, 4, 5
    x = rng.standard_normal((B, L, D))
    W_c = rng.standard_normal((dc, D)); W_q = rng.standard_normal((H * dk, D))
    W_uk = rng.standard_normal((H, dk, dc)); W_uv = rng.standard_normal((H, dv, dc))
    scale = 0.4
    c, ot, lse = O.prefill_reference(x, W_c, W_q, W_uk, W_uv, scale)
    q = (x[:, -1] @ W_q.T).reshape(B, H, dk)
    q_abs = np.einsum("bhk,hkc->bhc", q, W_uk)
    cache = c.reshape(B * L, dc)
    o_lat, lse_d = O.decode_reference(q_abs, cache, np.arange(B) * L, np.full(B, L), dc, 0, 0.0, scale)
    np.testing.assert_allclose(O.value_up_projection(o_lat, W_uv), ot[:, -1], atol=1e-11)
    np.testing.assert_allclose(lse_d, lse[:, -1], atol=1e-11)


def test_lse_merge_of_disjoint_key_sets_equals_whole():
    L, H, d = 37, 4, 6
    q = rng.standard_normal((1, H, d)); k = rng.standard_normal((L, H, d)); v = rng.standard_normal((L, H, 5))
    full_o, full_l = O.attend_rows(q, k, v, [L - 1], 0.7)
    parts = []
    for lo, hi in [(0, 10), (10, 11), (11, 37)]:
        # keys lo..hi-1 only: treat them as a sequence and attend from its end
        o, l = O.attend_rows(q, k[lo:hi], v[lo:hi], [hi - lo - 1], 0.7)
        parts.append((o, l))
    parts.append((np.zeros_like(full_o), np.full_like(full_l, -np.inf)))  # an empty split
    o, l = O.lse_merge(parts)
    np.testing.assert_allclose(o, full_o, atol=1e-12)
    np.testing.assert_allclose(l, full_l, atol=1e-12)


def test_value_up_projection_moves_wuv_past_the_weighted_sum():
    T, H, dc, dv, S = 3, 2, 5, 4, 7
    a = scipy.special.softmax(rng.standard_normal((T, H, S)), axis=-1)
    c = rng.standard_normal((S, dc))
    W_uv = rng.standard_normal((H, dv, dc))
    o_lat = np.einsum("ths,sc->thc", a, c)
    explicit = np.einsum("ths,shd->thd", a, np.einsum("sc,hdc->shd", c, W_uv)).reshape(T, H * dv)
    np.testing.assert_allclose(O.value_up_projection(o_lat, W_uv), explicit, atol=1e-12)


# ---------------------------------------------------------------- decode-step projections
def _explicit_rope_decode(x_all, W_c, W_kr, W_q, W_qr, W_uk, W_uv, scale, base):
    """The newest token of one sequence attending over all of it, with every
    head's keys [W_UK^(h) c_j ; RoPE(W^KR x_j, j)] and values W_UV^(h) c_j
    built explicitly (no absorption), the query [W_q^(h) x ; RoPE(W^QR(h) x, t)]
    at the last position t. Written with plain numpy, not the oracle."""
    T = x_all.shape[0]
    H, dk, dc = W_uk.shape
    dr = W_kr.shape[0]
    c = x_all @ W_c.T
    kr = _rope_complex(x_all @ W_kr.T, np.arange(T), base)
    x = x_all[-1]
    out = []
    for h in range(H):
        q = np.concatenate([W_q[h * dk:(h + 1) * dk] @ x, _rope_complex(W_qr[h * dr:(h + 1) * dr] @ x, T - 1, base)])
        k = np.concatenate([c @ W_uk[h].T, kr], axis=1)  # [T, dk + dr]
        z = scale * (k @ q)
        a = np.exp(z - z.max())
        a /= a.sum()
        out.append(a @ (c @ W_uv[h].T))
    return np.concatenate(out)


@pytest.mark.parametrize("dr", [0, 4])
def test_decode_prepare_then_decode_equals_explicit_attention(dr):
    """Appending the new token's latent (and rotated RoPE key) and absorbing
    W_UK into its query, then the latent-cache decode and the value
    up-projection, give what explicit per-head K/V attention gives."""
    D, H, dc, dk, dv, Lp, base, scale = 12, 3, 8, 5, 6, 7, 100.0, 0.4
    x_all = rng.standard_normal((Lp + 1, D))
    W_c, W_q = rng.standard_normal((dc, D)), rng.standard_normal((H * dk, D))
    W_uk, W_uv = rng.standard_normal((H, dk, dc)), rng.standard_normal((H, dv, dc))
    W_kr = rng.standard_normal((dr, D)) if dr else None
    W_qr = rng.standard_normal((H * dr, D)) if dr else None
    # earlier tokens' cache rows, written directly from the definition
    prev = x_all[:Lp] @ W_c.T
    if dr:
        prev = np.concatenate([prev, _rope_complex(x_all[:Lp] @ W_kr.T, np.arange(Lp), base)], axis=1)
    row, q_abs = O.decode_prepare_reference(x_all[Lp:], W_c, W_kr, W_q, W_qr, W_uk, [Lp], base)
    assert row.shape == (1, dc + dr) and q_abs.shape == (1, H, dc + dr)
    cache = np.concatenate([prev, row])
    o_lat, _ = O.decode_reference(q_abs, cache, [0], [Lp + 1], dc, dr, base, scale)
    o = O.value_up_projection(o_lat, W_uv).reshape(-1)
    if dr:
        ref = _explicit_rope_decode(x_all, W_c, W_kr, W_q, W_qr, W_uk, W_uv, scale, base)
    else:
        c = x_all @ W_c.T
        x = x_all[-1]
        ref = []
        for h in range(H):
            z = scale * ((c @ W_uk[h].T) @ (W_q[h * dk:(h + 1) * dk] @ x))
            a = np.exp(z - z.max())
            ref.append((a / a.sum()) @ (c @ W_uv[h].T))
        ref = np.concatenate(ref)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-11)


def test_decode_prepare_absorbed_query_matches_scalar_loops():
    D, H, dc, dk, dr = 4, 2, 3, 2, 2
    x = rng.standard_normal((2, D))
    W_c, W_q = rng.standard_normal((dc, D)), rng.standard_normal((H * dk, D))
    W_uk, W_kr, W_qr = rng.standard_normal((H, dk, dc)), rng.standard_normal((dr, D)), rng.standard_normal((H * dr, D))
    row, q_abs = O.decode_prepare_reference(x, W_c, W_kr, W_q, W_qr, W_uk, [3, 9], 0.0)  # base 0: no rotation
    for b in range(2):
        for c in range(dc):
            assert abs(row[b][c] - sum(W_c[c][j] * x[b][j] for j in range(D))) < 1e-12
        for i in range(dr):
            assert abs(row[b][dc + i] - sum(W_kr[i][j] * x[b][j] for j in range(D))) < 1e-12
        for h in range(H):
            q = [sum(W_q[h * dk + k][j] * x[b][j] for j in range(D)) for k in range(dk)]
            for c in range(dc):
                assert abs(q_abs[b][h][c] - sum(W_uk[h][k][c] * q[k] for k in range(dk))) < 1e-12
            for i in range(dr):
                assert abs(q_abs[b][h][dc + i] - sum(W_qr[h * dr + i][j] * x[b][j] for j in range(D))) < 1e-12


# ---------------------------------------------------------------- low-rank query
def test_low_rank_query_equals_composed_projection():
    """q = W^UQ (W^DQ x) and q^R = W^QR (W^DQ x) are the full-rank
    projections W^UQ W^DQ and W^QR W^DQ applied to x (matrix product
    associativity), in prefill and in the decode-step projections."""
    B, L, D, H, dc, dk, dv, dr, dcq = 2, 5, 9, 3, 6, 4, 5, 4, 7
    x = rng.standard_normal((B, L, D))
    W_c, W_uk, W_uv = rng.standard_normal((dc, D)), rng.standard_normal((H, dk, dc)), rng.standard_normal((H, dv, dc))
    W_dq, W_uq, W_qr = rng.standard_normal((dcq, D)), rng.standard_normal((H * dk, dcq)), rng.standard_normal((H * dr, dcq))
    W_kr = rng.standard_normal((dr, D))
    a = O.prefill_reference(x, W_c, W_uq, W_uk, W_uv, 0.3, W_dq=W_dq, W_kr=W_kr, W_qr=W_qr, rope_base=50.0)
    b = O.prefill_reference(x, W_c, W_uq @ W_dq, W_uk, W_uv, 0.3, W_kr=W_kr, W_qr=W_qr @ W_dq, rope_base=50.0)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=0, atol=1e-11)
    xs = x[:, -1]
    r1, q1 = O.decode_prepare_reference(xs, W_c, W_kr, W_uq, W_qr, W_uk, [3, 8], 50.0, W_dq=W_dq)
    r2, q2 = O.decode_prepare_reference(xs, W_c, W_kr, W_uq @ W_dq, W_qr @ W_dq, W_uk, [3, 8], 50.0)
    np.testing.assert_allclose(r1, r2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(q1, q2, rtol=0, atol=1e-11)


def test_low_rank_query_decode_prepare_scalar_loops():
    D, H, dc, dk, dr, dcq = 4, 2, 3, 2, 2, 3
    x = rng.standard_normal((2, D))
    W_c, W_dq = rng.standard_normal((dc, D)), rng.standard_normal((dcq, D))
    W_uq, W_uk = rng.standard_normal((H * dk, dcq)), rng.standard_normal((H, dk, dc))
    W_kr, W_qr = rng.standard_normal((dr, D)), rng.standard_normal((H * dr, dcq))
    _, q_abs = O.decode_prepare_reference(x, W_c, W_kr, W_uq, W_qr, W_uk, [1, 2], 0.0, W_dq=W_dq)
    for b in range(2):
        cq = [sum(W_dq[i][j] * x[b][j] for j in range(D)) for i in range(dcq)]
        for h in range(H):
            q = [sum(W_uq[h * dk + k][i] * cq[i] for i in range(dcq)) for k in range(dk)]
            for c in range(dc):
                assert abs(q_abs[b][h][c] - sum(W_uk[h][k][c] * q[k] for k in range(dk))) < 1e-12
            for i in range(dr):
                assert abs(q_abs[b][h][dc + i] - sum(W_qr[h * dr + i][j] * cq[j] for j in range(dcq))) < 1e-12


# ---------------------------------------------------------------- RoPE prefill
def _brute_rope_prefill(x, W_c, W_q, W_uk, W_uv, W_kr, W_qr, scale, base):
    """One sequence, scalar loops; the rotation is the complex-number form."""
    L, D = x.shape
    H, dk, dc = W_uk.shape
    dv, dr = W_uv.shape[1], W_kr.shape[0]
    c = [[sum(W_c[i][j] * x[s][j] for j in range(D)) for i in range(dc)] for s in range(L)]
    kr = _rope_complex(np.array([[sum(W_kr[i][j] * x[s][j] for j in range(D)) for i in range(dr)] for s in range(L)]),
                       np.arange(L), base)
    out = np.zeros((L, H * dv))
    for t in range(L):
        for h in range(H):
            q = [sum(W_q[h * dk + i][j] * x[t][j] for j in range(D)) for i in range(dk)]
            qr = _rope_complex(np.array([sum(W_qr[h * dr + i][j] * x[t][j] for j in range(D)) for i in range(dr)]),
                               t, base)
            z = []
            for s in range(t + 1):
                k = [sum(W_uk[h][i][m] * c[s][m] for m in range(dc)) for i in range(dk)]
                z.append(scale * (sum(q[i] * k[i] for i in range(dk)) + sum(qr[i] * kr[s][i] for i in range(dr))))
            mx = max(z)
            e = [math.exp(u - mx) for u in z]
            den = sum(e)
            for i in range(dv):
                out[t][h * dv + i] = sum(e[s] / den * sum(W_uv[h][i][m] * c[s][m] for m in range(dc))
                                         for s in range(t + 1))
    return out


def test_rope_prefill_matches_scalar_brute_force():
    L, D, H, dc, dk, dv, dr = 6, 5, 2, 4, 3, 3, 4
    x = rng.standard_normal((1, L, D))
    W_c, W_q = rng.standard_normal((dc, D)), rng.standard_normal((H * dk, D))
    W_uk, W_uv = rng.standard_normal((H, dk, dc)), rng.standard_normal((H, dv, dc))
    W_kr, W_qr = rng.standard_normal((dr, D)), rng.standard_normal((H * dr, D))
    _, o, _ = O.prefill_reference(x, W_c, W_q, W_uk, W_uv, 0.4, W_kr=W_kr, W_qr=W_qr, rope_base=7.0)
    ref = _brute_rope_prefill(x[0], W_c, W_q, W_uk, W_uv, W_kr, W_qr, 0.4, 7.0)
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-11)


def test_rope_prefill_rows_equal_absorbed_decode_steps():
    """Row t of the explicit RoPE prefill equals the absorbed route: the
    cache rows of tokens 0..t from the decode-step projections, the latent
    decode over them, then W_UV."""
    L, D, H, dc, dk, dv, dr, base, scale = 7, 6, 3, 5, 4, 3, 4, 100.0, 0.35
    x = rng.standard_normal((1, L, D))
    W_c, W_q = rng.standard_normal((dc, D)), rng.standard_normal((H * dk, D))
    W_uk, W_uv = rng.standard_normal((H, dk, dc)), rng.standard_normal((H, dv, dc))
    W_kr, W_qr = rng.standard_normal((dr, D)), rng.standard_normal((H * dr, D))
    _, o, lse = O.prefill_reference(x, W_c, W_q, W_uk, W_uv, scale, W_kr=W_kr, W_qr=W_qr, rope_base=base)
    rows, q_abs = O.decode_prepare_reference(x[0], W_c, W_kr, W_q, W_qr, W_uk, np.arange(L), base)
    for t in range(L):
        o_lat, l = O.decode_reference(q_abs[t:t + 1], rows, [0], [t + 1], dc, dr, base, scale)
        np.testing.assert_allclose(O.value_up_projection(o_lat, W_uv)[0], o[0, t], rtol=0, atol=1e-11)
        np.testing.assert_allclose(l[0], lse[0, t], rtol=0, atol=1e-11)


# ---------------------------------------------------------------- per-head gate
def test_head_gate_matches_scalar_loops():
    T, D, H, dv = 3, 4, 2, 3
    x, o = rng.standard_normal((T, D)), rng.standard_normal((T, H * dv))
    W_g, b_g, W_o = rng.standard_normal((H, D)), rng.standard_normal(H), rng.standard_normal((D, H * dv))
    y = O.head_gate_out_reference(x, o, W_g, b_g, W_o)
    for t in range(T):
        g = [1.0 / (1.0 + math.exp(-(sum(W_g[h][j] * x[t][j] for j in range(D)) + b_g[h]))) for h in range(H)]
        for i in range(D):
            want = sum(W_o[i][h * dv + j] * g[h] * o[t][h * dv + j] for h in range(H) for j in range(dv))
            assert abs(y[t][i] - want) < 1e-12


def test_head_gate_equals_channel_gate_with_repeated_rows():
    """A per-head gate is the per-channel gate whose rows repeat each head's
    gate row over its d_v channels."""
    T, D, H, dv = 4, 6, 3, 5
    x, o = rng.standard_normal((T, D)), rng.standard_normal((T, H * dv))
    W_g, W_o = rng.standard_normal((H, D)), rng.standard_normal((D, H * dv))
    y = O.head_gate_out_reference(x, o, W_g, None, W_o)
    y_ch = O.gate_out_reference(x, o, np.repeat(W_g, dv, axis=0), W_o)
    np.testing.assert_allclose(y, y_ch, rtol=0, atol=1e-12)
    # zero weights and bias: every gate is 1/2
    np.testing.assert_allclose(O.head_gate_out_reference(x, o, 0 * W_g, np.zeros(H), W_o), 0.5 * (o @ W_o.T),
                               rtol=0, atol=1e-12)


def test_head_gate_allows_folding_wo_wuv_in_decode():
    """With a scalar per head, W_o^(h) W_UV^(h) can be folded into one
    [d_model, d_c] matrix per head: y = sum_h g_h (W_o^(h) W_UV^(h)) o_lat_h."""
    T, D, H, dc, dv = 3, 7, 2, 5, 4
    x, o_lat = rng.standard_normal((T, D)), rng.standard_normal((T, H, dc))
    W_g, b_g = rng.standard_normal((H, D)), rng.standard_normal(H)
    W_uv, W_o = rng.standard_normal((H, dv, dc)), rng.standard_normal((D, H * dv))
    y = O.head_gate_out_reference(x, O.value_up_projection(o_lat, W_uv), W_g, b_g, W_o)
    g = 1.0 / (1.0 + np.exp(-(x @ W_g.T + b_g)))
    y_fold = sum(g[:, h:h + 1] * (o_lat[:, h] @ (W_o[:, h * dv:(h + 1) * dv] @ W_uv[h]).T) for h in range(H))
    np.testing.assert_allclose(y, y_fold, rtol=0, atol=1e-11)


# ---------------------------------------------------------------- brute force
def _brute_layer(x, W_c, W_q, W_uk, W_uv, W_g, W_o, scale):
    """Scalar loops over every index, math.exp only: one sequence."""
    L, D = len(x), len(x[0])
    H, dk, dc = len(W_uk), len(W_uk[0]), len(W_uk[0][0])
    dv = len(W_uv[0])
    c = [[sum(W_c[i][j] * x[s][j] for j in range(D)) for i in range(dc)] for s in range(L)]
    y = []
    for t in range(L):
        ot = []
        for h in range(H):
            q = [sum(W_q[h * dk + i][j] * x[t][j] for j in range(D)) for i in range(dk)]
            z = []
            for s in range(t + 1):
                k = [sum(W_uk[h][i][m] * c[s][m] for m in range(dc)) for i in range(dk)]
                z.append(scale * sum(q[i] * k[i] for i in range(dk)))
            mx = max(z)
            e = [math.exp(v - mx) for v in z]
            den = sum(e)
            for i in range(dv):
                acc = 0.0
                for s in range(t + 1):
                    v = sum(W_uv[h][i][m] * c[s][m] for m in range(dc))
                    acc += e[s] / den * v
                ot.append(acc)
        g = [1.0 / (1.0 + math.exp(-sum(W_g[n][j] * x[t][j] for j in range(D)))) for n in range(H * dv)]
        y.append([sum(W_o[i][n] * g[n] * ot[n] for n in range(H * dv)) for i in range(len(W_o))])
    return c, y


def test_whole_layer_matches_scalar_brute_force():
    L, D, H, dc, dk, dv = 6, 5, 2, 4, 3, 3
    x = rng.standard_normal((1, L, D))
    ws = dict(W_c=rng.standard_normal((dc, D)), W_q=rng.standard_normal((H * dk, D)),
              W_uk=rng.standard_normal((H, dk, dc)), W_uv=rng.standard_normal((H, dv, dc)),
              W_g=rng.standard_normal((H * dv, D)), W_o=rng.standard_normal((D, H * dv)))
    c, _, y = O.gated_mla_layer(x, *ws.values(), 0.45)
    cb, yb = _brute_layer(x[0].tolist(), *[w.tolist() for w in ws.values()], 0.45)
    np.testing.assert_allclose(c[0], cb, atol=1e-12)
    np.testing.assert_allclose(y[0], yb, atol=1e-11)


# ---------------------------------------------------------------- bytes
def _bytes(case):
    kw = {k: case[k] for k in ("h", "g", "d_h", "d_c", "d_r") if k in case}
    n = O.kv_bytes_per_token(case["mechanism"], layers=case["layers"],
                             bytes_per_elem=case["bytes_per_elem"], **kw)
    return n * case.get("context", 1)


def test_kv_bytes_reproduce_printed_worked_examples():
    with open(os.path.join(GOLDEN, "kv_bytes_worked_examples.json")) as f:
        g = json.load(f)
    unit = {"elements": 1, "B": 1, "KiB": 1024, "MiB": 2 ** 20, "GiB": 2 ** 30}
    for case in g["cases"]:
        val = _bytes(case) / unit[case["unit"]]
        tol = case.get("rounded_to", 0) / 2 + 1e-12
        assert abs(val - case["printed"]) <= tol, (case["cite"], val)
    mha = O.kv_bytes_per_token("MHA", h=128, d_h=128, layers=60)
    mla = O.kv_bytes_per_token("MLA", d_c=512, d_r=64, layers=60)
    assert abs(mha / mla - g["ratios"][0]["printed"]) <= g["ratios"][0]["tolerance"]
    gqa = O.kv_bytes_per_token("GQA", h=64, g=8, d_h=128)
    assert gqa / O.kv_bytes_per_token("MHA", h=64, d_h=128) == g["ratios"][1]["printed"]
    # GQA end points: g = 1 is MQA, g = h is MHA
    assert O.kv_bytes_per_token("GQA", h=8, g=1, d_h=64) == O.kv_bytes_per_token("MQA", d_h=64)
    assert O.kv_bytes_per_token("GQA", h=8, g=8, d_h=64) == O.kv_bytes_per_token("MHA", h=8, d_h=64)
    assert O.decode_step_cache_bytes([3, 4], 512, 64) == 7 * 1152
