"""GPU parity of the decoupled-RoPE prefill (gmla_prefill with W_kr, W_qr)
against the fp64 oracle: the cache rows [c ; RoPE(k^R, s)] and o~, plus the
consistency of a RoPE prefill's cache with the RoPE decode that follows it."""
import numpy as np
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, dev, f64, full_size_rows, rel_err, row_err, say

pytestmark = pytest.mark.gpu


def _np(t):
    return None if t is None else t.float().numpy()


def _run(inp):
    return ops.prefill(dev(inp.x), dev(inp.W_c), dev(inp.W_q), dev(inp.W_uk), dev(inp.W_uv), inp.sm_scale,
                       W_dq=None if inp.W_dq is None else dev(inp.W_dq), W_kr=dev(inp.W_kr), W_qr=dev(inp.W_qr),
                       rope_base=inp.rope_base)


def _check(inp, rows=None):
    rows_gpu, ot = _run(inp)
    torch.cuda.synchronize()
    _, rot, _ = O.prefill_reference(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    inp.sm_scale, rows=rows, W_dq=_np(inp.W_dq), W_kr=_np(inp.W_kr),
                                    W_qr=_np(inp.W_qr), rope_base=inp.rope_base)
    # the cache rows [c ; RoPE(W_kr x_s, s)] of every token, from the oracle's
    # decode-step projections at the token's own position
    e_rows = []
    for b in range(inp.B):
        ref_rows, _ = O.decode_prepare_reference(_np(inp.x[b]), _np(inp.W_c), _np(inp.W_kr), _np(inp.W_q),
                                                 _np(inp.W_qr), _np(inp.W_uk), np.arange(inp.L), inp.rope_base,
                                                 W_dq=_np(inp.W_dq))
        e_rows.append(rel_err(rows_gpu[b].float(), ref_rows))
    sel = slice(None) if rows is None else rows
    e_o = rel_err(ot[:, sel].float(), rot)
    say(f"  rel err cache rows {max(e_rows):.2e}  o~ {e_o:.2e} (per row {row_err(ot[:, sel].float(), rot):.2e})")
    assert max(e_rows) <= BF16_TOL and e_o <= BF16_TOL
    return rows_gpu


@pytest.mark.parametrize("B,L,D,H,d_c,d", [(2, 300, 256, 4, 128, 128), (1, 517, 512, 3, 64, 64),
                                           (3, 33, 256, 5, 128, 64), (1, 64, 128, 2, 64, 128),
                                           (1, 1, 128, 2, 64, 128)])
def test_rope_prefill_matches_oracle(B, L, D, H, d_c, d):
    say(f"[rope prefill] B={B} L={L} D={D} H={H} d_c={d_c} d={d} d_r=64")
    _check(W.make_prefill(B, L, D, H, d_c, d, d, seed=41, d_r=64))


def test_rope_prefill_score_range_forces_redo_pass():
    """The redo path of the RoPE attention kernel (192-wide scores): the
    content part as in the NoPE redo test (c = K = V = x with W_c, W_UK,
    W_UV identities, each head's W_q a permutation, tokens from 64 on shifted
    by 4 in every feature, so later scores lie hundreds of log2 units above
    the first key tile's maximum) plus a small rotated RoPE part. The pass
    at the first tile's reference overflows its bound and the workgroup must
    redo it with the true maxima."""
    say("[rope prefill redo]")
    L, D, H, d_r = 300, 128, 2, 64
    g = torch.Generator().manual_seed(29)
    x = torch.randn(1, L, D, generator=g)
    x[:, 64:] += 4.0
    eye = torch.eye(D)
    W_q = torch.cat([eye[torch.randperm(D, generator=g)] for _ in range(H)], 0)
    bf = lambda t: t.to(torch.bfloat16).contiguous()
    inp = W.PrefillInputs(B=1, L=L, d_model=D, H=H, d_c=D, d_k=D, d_v=D, sm_scale=1.0 / (D + d_r) ** 0.5,
                          dtype=torch.bfloat16, x=bf(x), W_c=bf(eye), W_q=bf(W_q), W_uk=bf(eye.expand(H, D, D)),
                          W_uv=bf(eye.expand(H, D, D)), W_g=bf(torch.zeros(H * D, D)), W_o=bf(torch.zeros(D, H * D)),
                          name="rope redo", d_r=d_r, rope_base=10000.0,
                          W_kr=bf(torch.randn(d_r, D, generator=g) * 0.05),
                          W_qr=bf(torch.randn(H * d_r, D, generator=g) * 0.05))
    _check(inp)


def test_rope_prefill_with_low_rank_query():
    say("[rope prefill + low-rank q]")
    _check(W.make_prefill(2, 200, 256, 3, 128, 128, 128, seed=42, d_r=64, d_cq=192))


def test_rope_prefill_base_zero_is_unrotated():
    say("[rope prefill, base 0]")
    _check(W.make_prefill(1, 130, 256, 2, 64, 64, 64, seed=43, d_r=64, rope_base=0.0))


def test_rope_prefill_far_positions():
    """Positions past 4096 (the fp64 angle reduction): rows sampled."""
    say("[rope prefill, L=5000, sampled rows]")
    inp = W.make_prefill(1, 5000, 128, 2, 64, 64, 64, seed=44, d_r=64)
    _check(inp, rows=[0, 1, 2047, 4096, 4999])


def test_rope_prefill_cache_feeds_rope_decode():
    """The RoPE prefill's cache rows and the decode-step projection of the
    next token, attended by the RoPE decode kernel, give the oracle's result
    for that token."""
    say("[rope prefill -> decode]")
    H, d_c, d, D, L = 16, 512, 128, 256, 257
    inp = W.make_prefill(1, L + 1, D, H, d_c, d, d, seed=45, d_r=64)
    rows, _ = ops.prefill(dev(inp.x[:, :L]), dev(inp.W_c), dev(inp.W_q), dev(inp.W_uk), dev(inp.W_uv),
                          inp.sm_scale, W_kr=dev(inp.W_kr), W_qr=dev(inp.W_qr), rope_base=inp.rope_base)
    cache = torch.zeros((L + 1, d_c + 64), dtype=torch.bfloat16, device="cuda")
    cache[:L] = rows[0]
    seq_start = torch.zeros(1, dtype=torch.int64, device="cuda")
    seq_len = torch.full((1,), L, dtype=torch.int32, device="cuda")
    q_abs = ops.decode_prepare(dev(inp.x[0, L:]), dev(inp.W_c), dev(inp.W_kr), dev(inp.W_q), dev(inp.W_qr),
                               dev(inp.W_uk), cache, seq_start, seq_len, inp.rope_base)
    o_lat, _ = ops.decode(q_abs, cache, seq_start, seq_len + 1, d_c, 64, inp.rope_base, inp.sm_scale)
    torch.cuda.synchronize()
    o = O.value_up_projection(f64(o_lat), _np(inp.W_uv))
    _, rot, _ = O.prefill_reference(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    inp.sm_scale, rows=[L], W_kr=_np(inp.W_kr), W_qr=_np(inp.W_qr),
                                    rope_base=inp.rope_base)
    e = rel_err(torch.from_numpy(o[0]), rot[0, 0])
    say(f"  rel err {e:.2e} (per head {row_err(torch.from_numpy(o[0]).reshape(H, d), rot[0, 0].reshape(H, d)):.2e})")
    assert e <= BF16_TOL


@pytest.mark.slow
def test_rope_prefill_full_size_sampled_rows():
    """The RoPE prefill workload at full size (B=2, L=8192, d_model=7168,
    H=64, d_k=d_v=128, d_r=64) as the benchmark launches it: the cache rows
    and o~ of 256 tokens of every sequence and head (the first three, the
    last and 252 seeded random ones)."""
    say("[rope prefill full] generating")
    inp = W.prefill_rope_b2_l8192()
    rows_gpu, ot = _run(inp)
    torch.cuda.synchronize()
    rows = full_size_rows(inp.L)
    say(f"  oracle on {len(rows)} rows")
    _, rot, _ = O.prefill_reference(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    inp.sm_scale, rows=rows, W_kr=_np(inp.W_kr), W_qr=_np(inp.W_qr),
                                    rope_base=inp.rope_base)
    e_rows = []
    for b in range(inp.B):
        ref_rows, _ = O.decode_prepare_reference(_np(inp.x[b, rows]), _np(inp.W_c), _np(inp.W_kr), _np(inp.W_q),
                                                 _np(inp.W_qr), _np(inp.W_uk), np.asarray(rows), inp.rope_base)
        e_rows.append(rel_err(rows_gpu[b, rows].float(), ref_rows))
    e_o = rel_err(ot[:, rows].float(), rot)
    say(f"  rel err cache rows {max(e_rows):.2e}  o~ {e_o:.2e} (per row {row_err(ot[:, rows].float(), rot):.2e})")
    assert max(e_rows) <= BF16_TOL and e_o <= BF16_TOL


def _rope_sweep(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 4)), int(rng.integers(1, 420)), 64 * int(rng.integers(2, 17)),
             int(rng.integers(1, 9)), 64 * int(rng.integers(1, 9)), int(rng.choice([64, 128]))) for _ in range(n)]


@pytest.mark.parametrize("B,L,D,H,d_c,d", _rope_sweep(8, 17))
def test_rope_prefill_shape_sweep(B, L, D, H, d_c, d):
    """Seeded decoupled-RoPE prefill shapes (d_r = 64), ragged L."""
    say(f"[rope prefill sweep] B={B} L={L} D={D} H={H} d_c={d_c} d={d} d_r=64")
    _check(W.make_prefill(B, L, D, H, d_c, d, d, seed=B * 1013 + L, d_r=64))
