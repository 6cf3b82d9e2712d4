"""Plain fp64 CPU oracle for Gated Multi-head Latent Attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code, tables or helpers with the HIP
library, and it never imports that library.

Everything here is the definition written out in float64 numpy, in the
un-absorbed form: every head's keys and values are reconstructed explicitly
from the cached latent, and nothing is fused, blocked or reordered beyond what
the definition states. Inputs may be any float dtype; they are upcast to
float64 (bf16 and fp32 values are exact in fp64, so the oracle sees the very
values the GPU receives).

Sources (page title, section):
  [GF]  "Gated MLA 计算公式：输出门与 FFN 的区别" (hackcha.cn)
        §一 latent and per-head reconstruction; §二 causal softmax, head
        concat and the boxed gated output equation; §四 data flow; NoPE note.
  [N03] "LLM 注意力与计算内核精读笔记 · 03 注意力头变体：MQA / GQA / MLA"
        §5.1 low-rank KV compression and absorption, and the low-rank query
        c^Q = W^DQ h, q = W^UQ c^Q; §5.2 decoupled RoPE (q^R from c^Q, k^R
        from h); 题4 answer (absorbed query (W^UK)^T q).
  [CD]  "Gated Multi-head Latent Attention (Gated MLA)" (concept page)
        Gating Mechanism / Mathematical Formulation: the per-head scalar
        gate g_h = sigmoid(W_g x + b_g) scaling head h's output.

Readings where the pages leave a step open (each one is listed with its
reason in the design notes of the repository):
  * softmax scale is an explicit argument (the pages write 1/sqrt(d_h));
  * RoPE pairs are interleaved (2i, 2i+1) with theta_i = base^(-2i/d_r); the
    query is rotated at position L_b - 1 and cached k^R rows are stored
    already rotated ([N03] §5.2 applies RoPE to k^R before it is cached);
  * V in absorbed decode is the latent part c[:d_c] only;
  * the gate is per channel (H*d_v wide), without bias, fed by x_t ([GF] §二);
  * head concat is head-major: channel h*d_v + j;
  * in prefill the RoPE parts sit after each head's content part: score
    q^C.k^C + RoPE(q^R, t).RoPE(k^R, s), with k^R shared by all heads;
  * without query compression c^Q is x itself (W^DQ = identity).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "latent_projection",
    "query_projection",
    "query_compression",
    "reconstruct_kv",
    "attend_rows",
    "causal_attention",
    "rope_rotate",
    "decode_reference",
    "decode_prepare_reference",
    "lse_merge",
    "value_up_projection",
    "sigmoid",
    "gate_out_reference",
    "head_gate_out_reference",
    "prefill_reference",
    "gated_mla_layer",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Projections  ([GF] §一, [N03] §5.1)
# --------------------------------------------------------------------------
def latent_projection(x, W_c) -> np.ndarray:
    """c_s = W_c x_s for every token ([GF] §一 first equation).

    x: [..., d_model]; W_c: [d_c, d_model] (row = output channel).
    Returns c: [..., d_c].
    """
    return _f64(x) @ _f64(W_c).T


def query_projection(x, W_q, H: int) -> np.ndarray:
    """q_t^(h) = W_q^(h) x_t, all heads stacked head-major in W_q.

    W_q: [H*d_k, d_model]; returns q: [..., H, d_k].
    """
    q = _f64(x) @ _f64(W_q).T
    return q.reshape(q.shape[:-1] + (H, q.shape[-1] // H))


def query_compression(x, W_dq) -> np.ndarray:
    """c_t^Q = W^DQ h_t, the low-rank query latent ([N03] §5.1, last
    paragraph); the per-head queries are then q_t = W^UQ c_t^Q and the RoPE
    queries W^QR c_t^Q ([N03] §5.2).

    x: [..., d_model]; W_dq: [d_cq, d_model]. Returns [..., d_cq].
    """
    return _f64(x) @ _f64(W_dq).T


def reconstruct_kv(c, W_uk, W_uv):
    """k_s^(h) = W_k^(h) c_s and v_s^(h) = W_v^(h) c_s for every head
    ([GF] §一 second and third equations; [N03] §5.1).

    c: [..., d_c]; W_uk: [H, d_k, d_c]; W_uv: [H, d_v, d_c].
    Returns k: [..., H, d_k], v: [..., H, d_v].
    """
    c = _f64(c)
    # optimize=True lets numpy hand the contraction over c to the BLAS matrix
    # product; the sums are the same
    k = np.einsum("...c,hdc->...hd", c, _f64(W_uk), optimize=True)
    v = np.einsum("...c,hdc->...hd", c, _f64(W_uv), optimize=True)
    return k, v


# --------------------------------------------------------------------------
# Softmax attention  ([GF] §二 first equation)
# --------------------------------------------------------------------------
def attend_rows(q_rows, k, v, t_rows, scale: float):
    """Causal softmax attention for selected query positions of one sequence.

    q_rows: [R, H, d_k] queries at positions t_rows (length R);
    k: [L, H, d_k]; v: [L, H, d_v] keys/values of the whole sequence.
    For query position t the keys s <= t take part (inclusive boundary):
        z_s = scale * q . k_s,  a = softmax_{s<=t}(z),  o = sum_s a_s v_s.
    Returns o: [R, H, d_v] and lse: [R, H] with lse = log sum_{s<=t} exp(z_s)
    (natural log).
    """
    q_rows = _f64(q_rows)
    k = _f64(k)
    v = _f64(v)
    R, H, _ = q_rows.shape
    t_rows = np.asarray([int(t) for t in t_rows], dtype=np.int64)
    S = int(t_rows.max()) + 1 if R else 0  # keys any requested row can see
    kh = np.ascontiguousarray(k[:S].transpose(1, 2, 0))  # [H, d_k, S]
    vh = np.ascontiguousarray(v[:S].transpose(1, 0, 2))  # [H, S, d_v]
    o = np.empty((R, H, v.shape[-1]))
    lse = np.empty((R, H))
    # Rows are independent; they are taken a few at a time so that each
    # head's scores of those rows are one matrix product (a library step).
    # Keys past a row's position get z = -inf, i.e. weight exp(-inf) = 0:
    # exactly the sums over s <= t.
    step = max(1, (1 << 24) // max(1, H * S))
    for r0 in range(0, R, step):
        rs = slice(r0, min(R, r0 + step))
        qh = q_rows[rs].transpose(1, 0, 2)  # [H, r, d_k]
        z = (qh @ kh) * scale  # [H, r, S]: z[h, i, s] = scale * q_(t_i)^(h) . k_s^(h)
        visible = np.arange(S)[None, :] <= t_rows[rs][:, None]  # [r, S]: s <= t
        z = np.where(visible[None], z, -np.inf)
        m = z.max(axis=2, keepdims=True)
        e = np.exp(z - m)
        den = e.sum(axis=2, keepdims=True)
        a = e / den
        o[rs] = (a @ vh).transpose(1, 0, 2)  # sum_s a_s v_s^(h)
        lse[rs] = (m + np.log(den))[:, :, 0].T
    return o, lse


def causal_attention(q, k, v, scale: float):
    """Causal attention for every query position of one sequence.

    q: [L, H, d_k], k: [L, H, d_k], v: [L, H, d_v] -> o [L, H, d_v], lse [L, H].
    """
    L = q.shape[0]
    return attend_rows(q, k, v, np.arange(L), scale)


# --------------------------------------------------------------------------
# Decoupled RoPE  ([N03] §5.2)
# --------------------------------------------------------------------------
def rope_rotate(u, pos, base: float) -> np.ndarray:
    """Rotate the last axis of u (width d_r, even) to position pos.

    Pairs are interleaved: (u[2i], u[2i+1]) is turned by the angle
    pos * theta_i with theta_i = base ** (-2i / d_r):
        u'[2i]   = u[2i] cos - u[2i+1] sin
        u'[2i+1] = u[2i] sin + u[2i+1] cos
    pos may be a scalar or broadcast against u[..., 0].
    """
    u = _f64(u)
    d_r = u.shape[-1]
    if d_r == 0:
        return u.copy()
    assert d_r % 2 == 0
    i = np.arange(d_r // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d_r)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    ev, od = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = ev * cos - od * sin
    out[..., 1::2] = ev * sin + od * cos
    return out


# --------------------------------------------------------------------------
# Decode over the latent cache  ([N03] §5.1, §5.2, 题4; [GF] §一, §二)
# --------------------------------------------------------------------------
def decode_reference(q_abs, cache, seq_start, seq_len, d_c: int, d_r: int,
                     rope_base: float, sm_scale: float, batches=None):
    """One decode step for every sequence b, written in the un-absorbed form.

    q_abs: [B, H, d_c + d_r]: the query with W_UK already applied to its
      content part (q~ = (W^UK)^T q, [N03] 题4) and its RoPE part not yet
      rotated.
    cache: [rows, d_c + d_r]: row j holds the latent c_j and (if d_r > 0)
      the shared RoPE key k^R_j, already rotated to its own position.
      Sequence b owns rows seq_start[b] .. seq_start[b] + seq_len[b] - 1.
    Because q~ is given, the per-head up-projection of the key is the identity
    on the latent: every head's key is k_j^h = [c_j ; k^R_j] and its value is
    v_j^h = c_j (the shared row itself). The query's RoPE part is rotated
    at position seq_len[b] - 1 (the current token); rope_base == 0 or
    d_r == 0 means NoPE.

    Returns o_lat [B, H, d_c] and lse [B, H] (natural log of the softmax
    denominator, scores already scaled). `batches` limits the work to some b
    (the other rows are left NaN).
    """
    q_abs = np.asarray(q_abs)
    B, H, W = q_abs.shape
    assert W == d_c + d_r
    o_lat = np.full((B, H, d_c), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seq_len[b])
        if L < 1:
            raise ValueError("a decode step needs at least one cached token")
        s0 = int(seq_start[b])
        rows = _f64(cache[s0: s0 + L])  # [L, d_c + d_r]
        q = _f64(q_abs[b])  # [H, d_c + d_r]
        q_c = q[:, :d_c]
        q_r = q[:, d_c:]
        if d_r > 0 and rope_base != 0.0:
            q_r = rope_rotate(q_r, L - 1, rope_base)
        qh = np.concatenate([q_c, q_r], axis=1)  # [H, d_c + d_r]
        # The up-projection of every head is the identity on the cached row,
        # so head h's key for row j is k_j^h = rows[j] and its value
        # v_j^h = rows[j, :d_c]. The H per-head dot products with the rows
        # are then one matrix product (a library step; nothing is blocked or
        # reordered beyond the sums the definition states).
        z = (qh @ rows.T) * sm_scale  # [H, L]: z[h, j] = scale * q~_h . k_j^h
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        den = e.sum(axis=1, keepdims=True)
        a = e / den  # softmax over the L_b cached rows (all j <= L_b - 1)
        o_lat[b] = a @ rows[:, :d_c]  # sum_j a_{h,j} v_j^h
        lse[b] = (m + np.log(den))[:, 0]
    return o_lat, lse


def decode_prepare_reference(x, W_c, W_kr, W_q, W_qr, W_uk, pos, rope_base: float, W_dq=None):
    """The projections of one decode step around the cached-latent attention
    ([N03] §5.1 low-rank KV compression, absorption and 题4; §5.2 decoupled
    RoPE), for the new token x_b of every sequence b at position pos[b]:

        c     = W_c x                       the latent, appended to the cache
        k^R   = RoPE(W^KR x, pos)           the shared RoPE key, stored rotated
        q^(h) = W_q^(h) x                   per-head query (d_k wide)
        q~^(h) = (W_UK^(h))^T q^(h)         absorbed query (d_c wide)
        q^R(h) = W^QR(h) x                  per-head RoPE query, not rotated here
                                            (the decode step rotates it)

    x: [B, d_model]; W_c: [d_c, d_model]; W_kr: [d_r, d_model] or None;
    W_q: [H*d_k, d_in]; W_qr: [H*d_r, d_in] or None; W_uk: [H, d_k, d_c];
    pos: [B]. With W_dq ([d_cq, d_model]) the query side starts from the
    low-rank query c^Q = W^DQ x (d_in = d_cq: W_q is W^UQ, and the RoPE
    query is W^QR c^Q); without it d_in = d_model and the query side reads x.
    Returns (cache_row [B, d_c + d_r], q_abs [B, H, d_c + d_r]).
    """
    x = _f64(x)
    B = x.shape[0]
    W_uk = _f64(W_uk)
    H = W_uk.shape[0]
    c = latent_projection(x, W_c)  # [B, d_c]
    xq = x if W_dq is None else query_compression(x, W_dq)
    q = query_projection(xq, W_q, H)  # [B, H, d_k]
    q_t = np.einsum("bhk,hkc->bhc", q, W_uk)  # (W_UK^(h))^T q^(h)
    if W_kr is None or np.asarray(W_kr).shape[0] == 0:
        return c, q_t
    k_r = x @ _f64(W_kr).T  # [B, d_r]
    if rope_base != 0.0:
        k_r = rope_rotate(k_r, np.asarray(pos, dtype=np.float64), rope_base)
    d_r = k_r.shape[-1]
    q_r = (xq @ _f64(W_qr).T).reshape(B, H, d_r)
    return np.concatenate([c, k_r], axis=1), np.concatenate([q_t, q_r], axis=2)


def lse_merge(parts):
    """Merge softmax-attention results computed over disjoint key sets.

    parts: list of (o_i [..., d], lse_i [...]) where o_i is the normalised
    attention output over key subset i and lse_i the natural log of its
    softmax denominator. Subsets with lse_i = -inf (no keys) contribute
    nothing. Returns (o, lse) over the union of the subsets:
        m = max_i lse_i;  w_i = exp(lse_i - m)
        o = sum_i w_i o_i / sum_i w_i;  lse = m + log sum_i w_i
    """
    lses = np.stack([_f64(p[1]) for p in parts])
    os_ = np.stack([_f64(p[0]) for p in parts])
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    w = np.where(np.isfinite(lses), w, 0.0)
    den = w.sum(axis=0)
    o = (w[..., None] * os_).sum(axis=0) / den[..., None]
    return o, m + np.log(den)


# --------------------------------------------------------------------------
# Output side: value up-projection, gate, W_o  ([GF] §一, §二 boxed equation)
# --------------------------------------------------------------------------
def value_up_projection(o_lat, W_uv) -> np.ndarray:
    """o~_t = Concat_h W_v^(h) o_lat_t^(h) (head-major).

    With v_s^(h) = W_v^(h) c_s, sum_s a_s v_s = W_v^(h) sum_s a_s c_s, so the
    up-projection is applied once per query to the latent-space output.
    o_lat: [T, H, d_c]; W_uv: [H, d_v, d_c] -> [T, H*d_v].
    """
    o = np.einsum("thc,hdc->thd", _f64(o_lat), _f64(W_uv))
    return o.reshape(o.shape[0], -1)


def sigmoid(z) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-_f64(z)))


def gate_out_reference(x, o_tilde, W_g, W_o, return_gated: bool = False):
    """y_t = W_o [ Sigmoid(W_g x_t) (.) o~_t ]  ([GF] §二 boxed equation).

    x: [T, d_model]; o_tilde: [T, H*d_v]; W_g: [H*d_v, d_model];
    W_o: [d_model, H*d_v]. The gate is per channel, input-dependent, and is
    applied after attention and before the output projection.
    """
    g = sigmoid(_f64(x) @ _f64(W_g).T)
    gated = g * _f64(o_tilde)
    y = gated @ _f64(W_o).T
    return (y, gated) if return_gated else y


def head_gate_out_reference(x, o_tilde, W_g, b_g, W_o, return_gated: bool = False):
    """Per-head scalar gate ([CD] Gating Mechanism and Mathematical
    Formulation): g_t = Sigmoid(W_g x_t + b_g) in R^H, head h's output block
    o~_t^(h) (channels h*d_v .. h*d_v + d_v - 1) scaled by g_t[h], then the
    heads merged and projected: y_t = W_o [ g_t[h] o~_t^(h) ]_h.

    x: [T, d_model]; o_tilde: [T, H*d_v]; W_g: [H, d_model]; b_g: [H] or
    None (zero); W_o: [d_model, H*d_v].
    """
    z = _f64(x) @ _f64(W_g).T
    if b_g is not None:
        z = z + _f64(b_g)
    g = sigmoid(z)  # [T, H]
    o = _f64(o_tilde)
    T, HV = o.shape
    H = g.shape[1]
    gated = (o.reshape(T, H, HV // H) * g[:, :, None]).reshape(T, HV)
    y = gated @ _f64(W_o).T
    return (y, gated) if return_gated else y


# --------------------------------------------------------------------------
# Prefill and the whole layer
# --------------------------------------------------------------------------
def prefill_reference(x, W_c, W_q, W_uk, W_uv, sm_scale: float, rows=None, *, W_dq=None, W_kr=None, W_qr=None,
                      rope_base: float = 0.0):
    """Causal prefill of a batch of sequences, explicit K/V per head.

    x: [B, L, d_model]. Returns (c [B, L, d_c], o_tilde, lse) where o_tilde is
    [B, L, H*d_v] (head-major concat, [GF] §二 second equation) and lse is
    [B, L, H]. With `rows` (a list of query positions) only those positions
    are attended (o_tilde/lse are then [B, R, ...]); c is always complete.

    Optional parts:
      * W_dq [d_cq, d_model]: low-rank query ([N03] §5.1): the queries come
        from c^Q = W^DQ x, and W_q ([H*d_k, d_cq]) is W^UQ;
      * W_kr [d_r, d_model], W_qr [H*d_r, d_in]: decoupled RoPE ([N03] §5.2):
        every head's key is [W_UK^(h) c_s ; RoPE(W^KR x_s, s)] (the RoPE part
        shared by the heads) and its query [q^C ; RoPE(W^QR(h) c^Q_t, t)]
        (c^Q = x without W_dq); rope_base 0 leaves both unrotated.
    """
    x = _f64(x)
    B, L, _ = x.shape
    H = np.asarray(W_uk).shape[0]
    c = latent_projection(x, W_c)
    t_rows = np.arange(L) if rows is None else np.asarray(rows)
    d_r = 0 if W_kr is None else np.asarray(W_kr).shape[0]
    outs, lses = [], []
    for b in range(B):
        k, v = reconstruct_kv(c[b], W_uk, W_uv)  # [L, H, d]
        xq = x[b, t_rows] if W_dq is None else query_compression(x[b, t_rows], W_dq)
        q = query_projection(xq, W_q, H)  # [R, H, d_k]
        if d_r > 0:
            k_r = x[b] @ _f64(W_kr).T  # [L, d_r], position s = row index
            q_r = (xq @ _f64(W_qr).T).reshape(len(t_rows), H, d_r)
            if rope_base != 0.0:
                k_r = rope_rotate(k_r, np.arange(L, dtype=np.float64), rope_base)
                q_r = rope_rotate(q_r, t_rows.astype(np.float64)[:, None], rope_base)
            k = np.concatenate([k, np.broadcast_to(k_r[:, None, :], (L, H, d_r))], axis=2)
            q = np.concatenate([q, q_r], axis=2)
        o, l = attend_rows(q, k, v, t_rows, sm_scale)
        outs.append(o.reshape(len(t_rows), -1))
        lses.append(l)
    return c, np.stack(outs), np.stack(lses)


def gated_mla_layer(x, W_c, W_q, W_uk, W_uv, W_g, W_o, sm_scale: float):
    """The whole attention sub-layer: x -> MLA -> o~ -> gate -> W_o -> y
    ([GF] §四 data flow, attention part only). x: [B, L, d_model]."""
    x = _f64(x)
    B, L, D = x.shape
    c, o_tilde, _ = prefill_reference(x, W_c, W_q, W_uk, W_uv, sm_scale)
    y = gate_out_reference(x.reshape(B * L, D), o_tilde.reshape(B * L, -1), W_g, W_o)
    return c, o_tilde, y.reshape(B, L, -1)

