"""GPU parity of gmla_prefill and gmla_gate_out (through the C ABI) against
the fp64 oracle, plus the prefill/decode consistency of the HIP path."""
import numpy as np
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, F32_TOL, dev, f64, full_size_rows, rel_err, row_err, say

pytestmark = pytest.mark.gpu


def _prefill(inp):
    c, ot = ops.prefill(dev(inp.x), dev(inp.W_c), dev(inp.W_q), dev(inp.W_uk), dev(inp.W_uv), inp.sm_scale)
    B, L, D = inp.x.shape
    y = ops.gate_out(dev(inp.x).reshape(B * L, D), ot.reshape(B * L, -1), dev(inp.W_g), dev(inp.W_o))
    torch.cuda.synchronize()
    return c, ot, y.reshape(B, L, D)


def _np(t):
    return t.float().numpy()


@pytest.mark.parametrize("B,L,D,H,d_c,d", [(2, 300, 256, 4, 128, 128), (1, 517, 512, 3, 64, 64),
                                           (1, 64, 128, 2, 64, 128), (3, 33, 256, 5, 128, 64),
                                           # 256 x 256 tiles for the query, key, value and gate GEMMs,
                                           # ragged token rows (2000) and V^T padded from 1000 to 1024 keys
                                           (2, 1000, 512, 64, 128, 128)])
def test_prefill_bf16_matches_oracle(B, L, D, H, d_c, d):
    say(f"[prefill bf16] B={B} L={L} D={D} H={H} d_c={d_c} d={d}")
    inp = W.make_prefill(B, L, D, H, d_c, d, d, seed=21)
    c, ot, y = _prefill(inp)
    rc, rot, ry = O.gated_mla_layer(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    _np(inp.W_g), _np(inp.W_o), inp.sm_scale)
    e = (rel_err(c.float(), rc), rel_err(ot.float(), rot), rel_err(y.float(), ry))
    say(f"  rel err c {e[0]:.2e}  o~ {e[1]:.2e}  y {e[2]:.2e} (o~ per row {row_err(ot.float(), rot):.2e})")
    assert max(e) <= BF16_TOL


def test_prefill_score_range_forces_redo_pass():
    """Scores whose range defeats the first-tile reference of the attention
    kernel, with operands that bf16 holds exactly, so that the oracle's
    scores are the kernel's up to fp32 summation and the bf16 rounding of
    the scaled queries: d_model = d_c = d_k = d_v
    = 128, W_c, W_UK and W_UV identities, each head's W_q a permutation
    (entries 0 and 1), so c = K = V = x and q = P_h x exactly. Tokens from 64
    on get 4 added to every feature; the ones direction is left unchanged by
    the permutations, so for every query past the first key tile the largest
    score lies 242 to 275 log2 units above the first tile's maximum (a pass
    that kept that reference would overflow fp32 and give inf or NaN), while
    among the later keys the softmax still mixes several (median weight of
    the top key 0.49). The exact redo pass must run and match the oracle."""
    say("[prefill redo]")
    L, D, H = 300, 128, 2
    g = torch.Generator().manual_seed(23)
    x = torch.randn(1, L, D, generator=g)
    x[:, 64:] += 4.0
    eye = torch.eye(D)
    W_q = torch.cat([eye[torch.randperm(D, generator=g)] for _ in range(H)], 0)
    W_g = torch.randn(H * D, D, generator=g) / D ** 0.5
    W_o = torch.randn(D, H * D, generator=g) / (H * D) ** 0.5
    bf = lambda t: t.to(torch.bfloat16).contiguous()
    inp = W.PrefillInputs(B=1, L=L, d_model=D, H=H, d_c=D, d_k=D, d_v=D, sm_scale=1.0 / D ** 0.5,
                          dtype=torch.bfloat16, x=bf(x), W_c=bf(eye), W_q=bf(W_q), W_uk=bf(eye.expand(H, D, D)),
                          W_uv=bf(eye.expand(H, D, D)), W_g=bf(W_g), W_o=bf(W_o), name="redo")
    c, ot, y = _prefill(inp)
    rc, rot, ry = O.gated_mla_layer(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    _np(inp.W_g), _np(inp.W_o), inp.sm_scale)
    e = (rel_err(c.float(), rc), rel_err(ot.float(), rot), rel_err(y.float(), ry))
    say(f"  rel err c {e[0]:.2e}  o~ {e[1]:.2e}  y {e[2]:.2e} (o~ per row {row_err(ot.float(), rot):.2e})")
    assert max(e) <= BF16_TOL


def test_prefill_fp32_tiny_config():
    """The tiny fp32 workload at its full size (B=1, L=128, d_model=256, H=4,
    d_c=64, d_k=d_v=32), against the whole-layer oracle at 1e-4."""
    say("[prefill fp32 tiny config]")
    inp = W.prefill_f32_tiny()
    c, ot, y = _prefill(inp)
    rc, rot, ry = O.gated_mla_layer(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    _np(inp.W_g), _np(inp.W_o), inp.sm_scale)
    e = (rel_err(c, rc), rel_err(ot, rot), rel_err(y, ry))
    say(f"  rel err c {e[0]:.2e}  o~ {e[1]:.2e}  y {e[2]:.2e}")
    assert max(e) <= F32_TOL


@pytest.mark.parametrize("T,D,H,d_c,d_v", [(32, 1024, 64, 512, 128), (64, 512, 16, 256, 64), (8, 256, 8, 128, 32),
                                           (5, 512, 4, 64, 128), (100, 512, 4, 128, 64),
                                           # 64-column skinny workgroups (gate and value up-projection) and
                                           # split-K W_o, at 33..64 and at <= 32 rows
                                           (64, 512, 128, 512, 128), (20, 512, 128, 128, 128),
                                           (37, 256, 136, 64, 128),
                                           # workgroups narrower than 32 columns: W_o over 7168 columns
                                           # as 256 x 28, and 2240 columns as 12-wide ones with an
                                           # 8-column tail (gate and value up-projection 8 wide)
                                           (32, 7168, 8, 128, 64), (24, 2240, 16, 128, 128),
                                           # shared-activation workgroups of 128 columns at 33..64
                                           # rows, K split: W_o and the gate (gate epilogue in the
                                           # split-K reduce); 4160 columns end in a partial group
                                           (64, 7168, 32, 512, 128), (40, 4160, 40, 256, 64),
                                           # ... and batched: the value up-projection over d_c = 2048
                                           # (one 128-column group per head, K split in two)
                                           (48, 512, 64, 2048, 128),
                                           # even shares of W_o's 36 groups x 64 chunks over 256
                                           # workgroups of 9 chunks: shares that end one group and
                                           # start the next, up to 8 slots per group
                                           (64, 4608, 64, 512, 128), (40, 4608, 64, 512, 128)])
def test_gate_out_with_value_up_projection(T, D, H, d_c, d_v):
    say(f"[gate_out decode-side] T={T} D={D} H={H} d_c={d_c} d_v={d_v}")
    g = torch.Generator().manual_seed(5)
    o_lat = torch.randn(T, H, d_c, generator=g).to(torch.bfloat16)
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    W_uv = (torch.randn(H, d_v, d_c, generator=g) / d_c ** 0.5).to(torch.bfloat16)
    W_g = (torch.randn(H * d_v, D, generator=g) / D ** 0.5).to(torch.bfloat16)
    W_o = (torch.randn(D, H * d_v, generator=g) / (H * d_v) ** 0.5).to(torch.bfloat16)
    y = ops.gate_out(dev(x), dev(o_lat), dev(W_g), dev(W_o), W_uv=dev(W_uv))
    torch.cuda.synchronize()
    ot = O.value_up_projection(_np(o_lat), _np(W_uv))
    ry = O.gate_out_reference(_np(x), ot, _np(W_g), _np(W_o))
    e = rel_err(y.float(), ry)
    say(f"  rel err y {e:.2e}")
    assert e <= BF16_TOL


@pytest.mark.parametrize("T,H,d_v", [(1, 64, 128), (5, 64, 128), (32, 64, 128), (33, 24, 128), (37, 24, 128),
                                     (64, 24, 128),
                                     # 17 heads: a grid that is not a multiple of the 8 XCDs keeps
                                     # the plain workgroup order
                                     (40, 17, 128), (64, 17, 128)])
def test_gate_out_fused_value_up_gated_elementwise(T, H, d_v):
    """d_c = 512 with a wide enough gate GEMM computes o~ inside the gate
    GEMM's workgroups (no separate value up-projection launch). W_o = I
    makes y the gated product itself, compared element by element."""
    d_c = 512
    HV = H * d_v
    say(f"[gate_out fused value up] T={T} H={H} d_v={d_v}")
    g = torch.Generator().manual_seed(11)
    o_lat = torch.randn(T, H, d_c, generator=g).to(torch.bfloat16)
    x = torch.randn(T, HV, generator=g).to(torch.bfloat16)
    W_uv = (torch.randn(H, d_v, d_c, generator=g) / d_c ** 0.5).to(torch.bfloat16)
    W_g = (torch.randn(HV, HV, generator=g) / HV ** 0.5).to(torch.bfloat16)
    W_o = torch.eye(HV, dtype=torch.bfloat16)
    ops.trace_begin(64)
    y = ops.gate_out(dev(x), dev(o_lat), dev(W_g), dev(W_o), W_uv=dev(W_uv))
    torch.cuda.synchronize()
    ops.trace_end()
    kernels = ops.trace_kernels()
    ops.trace_reset()
    assert "gemm_value_up" not in kernels, kernels
    _, gated = O.gate_out_reference(_np(x), O.value_up_projection(_np(o_lat), _np(W_uv)), _np(W_g), _np(W_o),
                                    return_gated=True)
    e = rel_err(y.float(), gated)
    say(f"  rel err gated {e:.2e}")
    assert e <= BF16_TOL


@pytest.mark.parametrize("T,D,HV", [(4133, 4224, 4096), (2144, 4160, 8192)])
def test_gate_out_large_tiles_sampled_rows(T, D, HV):
    """gate_out at sizes whose GEMMs take the 256 x 256 tile kernels (at least
    256 output tiles), with ragged row and column edges and both even and odd
    counts of 64-wide k-steps; the oracle checks a seeded sample of rows that
    always holds the first, last and tile-boundary rows."""
    say(f"[gate_out large tiles] T={T} D={D} H*d_v={HV}")
    g = torch.Generator().manual_seed(9)
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    o = torch.randn(T, HV, generator=g).to(torch.bfloat16)
    W_g = (torch.randn(HV, D, generator=g) / D ** 0.5).to(torch.bfloat16)
    W_o = (torch.randn(D, HV, generator=g) / HV ** 0.5).to(torch.bfloat16)
    y = ops.gate_out(dev(x), dev(o), dev(W_g), dev(W_o))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, 255, 256, T // 256 * 256 - 1, T - 2, T - 1} | set(rng.choice(T, 24, replace=False).tolist()))
    ry = O.gate_out_reference(_np(x)[rows], _np(o)[rows], _np(W_g), _np(W_o))
    e = rel_err(y[rows].float(), ry)
    say(f"  rel err y {e:.2e}")
    assert e <= BF16_TOL


def test_gate_out_fp32_with_value_up_projection():
    say("[gate_out fp32]")
    g = torch.Generator().manual_seed(6)
    T, D, H, d_c, d_v = 7, 96, 3, 40, 24
    o_lat, x = torch.randn(T, H, d_c, generator=g), torch.randn(T, D, generator=g)
    W_uv, W_g, W_o = torch.randn(H, d_v, d_c, generator=g), torch.randn(H * d_v, D, generator=g), torch.randn(D, H * d_v, generator=g)
    y = ops.gate_out(dev(x), dev(o_lat), dev(W_g), dev(W_o), W_uv=dev(W_uv))
    torch.cuda.synchronize()
    ry = O.gate_out_reference(x.double().numpy(), O.value_up_projection(o_lat.numpy(), W_uv.numpy()),
                              W_g.numpy(), W_o.numpy())
    assert rel_err(y, ry) <= F32_TOL


def test_prefill_last_row_equals_decode_on_its_latent():
    """HIP prefill's last position and a HIP decode step over the latent that
    prefill wrote agree once the query is absorbed on the host."""
    say("[prefill vs decode]")
    B, L, D, H, d_c, d = 2, 130, 256, 64, 512, 128
    inp = W.make_prefill(B, L, D, H, d_c, d, d, seed=8)
    c, ot, _ = _prefill(inp)
    q = (inp.x[:, -1].double() @ inp.W_q.double().T).reshape(B, H, d)
    q_abs = torch.einsum("bhk,hkc->bhc", q, inp.W_uk.double()).to(torch.bfloat16).contiguous()
    seq_start = torch.arange(B, dtype=torch.int64) * L
    seq_len = torch.full((B,), L, dtype=torch.int32)
    o_lat, lse = ops.decode(dev(q_abs), c.reshape(B * L, d_c), dev(seq_start), dev(seq_len), d_c, 0, 0.0,
                            inp.sm_scale)
    torch.cuda.synchronize()
    o_dec = O.value_up_projection(f64(o_lat), _np(inp.W_uv))
    e = rel_err(ot[:, -1].float(), o_dec)
    say(f"  rel diff {e:.2e} (per row {row_err(ot[:, -1].float(), o_dec):.2e})")
    assert e <= BF16_TOL


@pytest.mark.slow
def test_prefill_full_size_sampled_rows():
    """The B=2, L=8192, d_model=7168, H=64 prefill at full size, as the
    benchmark launches it; the oracle checks the latent in full and o~, y on
    256 query rows of every sequence and head (the first three, the last and
    252 seeded random ones)."""
    say("[prefill full] generating")
    inp = W.prefill_b2_l8192()
    c, ot, y = _prefill(inp)
    rows = full_size_rows(inp.L)
    say(f"  oracle on {len(rows)} rows")
    rc, rot, _ = O.prefill_reference(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                     inp.sm_scale, rows=rows)
    xr = _np(inp.x)[:, rows].reshape(-1, inp.d_model)
    ry = O.gate_out_reference(xr, rot.reshape(xr.shape[0], -1), _np(inp.W_g), _np(inp.W_o))
    e = (rel_err(c.float(), rc), rel_err(ot[:, rows].float(), rot),
         rel_err(y[:, rows].float().reshape(xr.shape[0], -1), ry))
    say(f"  rel err c {e[0]:.2e}  o~ {e[1]:.2e}  y {e[2]:.2e} (o~ per row {row_err(ot[:, rows].float(), rot):.2e}, "
        f"y per row {row_err(y[:, rows].float().reshape(xr.shape[0], -1), ry):.2e})")
    assert max(e) <= BF16_TOL


@pytest.mark.slow
def test_decode_output_side_full_size_h128():
    """gate_out on the RoPE decode workload's output side at full size (T =
    64, d_model = 7168, H = 128, d_c = 512, d_v = 128): W_o runs as shared-
    activation workgroups with K split four ways."""
    say("[gate_out full decode-side H=128]")
    g = torch.Generator().manual_seed(2)
    T, D, H, d_c, d_v = 64, 7168, 128, 512, 128
    o_lat = torch.randn(T, H, d_c, generator=g).to(torch.bfloat16)
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    W_uv = (torch.randn(H, d_v, d_c, generator=g) / d_c ** 0.5).to(torch.bfloat16)
    W_g = (torch.randn(H * d_v, D, generator=g) / D ** 0.5).to(torch.bfloat16)
    W_o = (torch.randn(D, H * d_v, generator=g) / (H * d_v) ** 0.5).to(torch.bfloat16)
    y = ops.gate_out(dev(x), dev(o_lat), dev(W_g), dev(W_o), W_uv=dev(W_uv))
    torch.cuda.synchronize()
    ry = O.gate_out_reference(_np(x), O.value_up_projection(_np(o_lat), _np(W_uv)), _np(W_g), _np(W_o))
    e = rel_err(y.float(), ry)
    say(f"  rel err y {e:.2e} (per row {row_err(y.float(), ry):.2e})")
    assert e <= BF16_TOL


@pytest.mark.slow
def test_decode_output_side_full_size():
    """gate_out on the decode workload's output side at full size (T = 32,
    d_model = 7168, H = 64, d_c = 512, d_v = 128)."""
    say("[gate_out full decode-side]")
    inp = W.decode_nope_b32_h64()
    g = torch.Generator().manual_seed(1)
    o_lat = torch.randn(inp.B, inp.H, inp.d_c, generator=g).to(torch.bfloat16)
    y = ops.gate_out(dev(inp.x), dev(o_lat), dev(inp.W_g), dev(inp.W_o), W_uv=dev(inp.W_uv))
    torch.cuda.synchronize()
    ry = O.gate_out_reference(_np(inp.x), O.value_up_projection(_np(o_lat), _np(inp.W_uv)), _np(inp.W_g), _np(inp.W_o))
    e = rel_err(y.float(), ry)
    say(f"  rel err y {e:.2e}")
    assert e <= BF16_TOL


def _sweep_shapes(n, seed):
    """Seeded bf16 gate_out shapes over the decode-side paths: the skinny
    per-wave form (with and without K split), the shared-activation form at
    33..64 rows (even shares), the value up-projection batched or inside the
    gate GEMM (d_c = 512), ragged row counts."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.integers(1, 65))
        H = int(rng.choice([4, 8, 16, 24, 32, 48, 64]))
        d_v = int(rng.choice([32, 64, 128]))
        d_c = int(rng.choice([64, 128, 256, 512, 512]))
        D = int(rng.choice([256, 512, 1024, 2048, 3072, 4096, 4608]))
        if (H * d_v) % 64 == 0 and H * d_v * D <= 6 * 2 ** 25:
            out.append((T, D, H, d_c, d_v))
    return out


@pytest.mark.parametrize("T,D,H,d_c,d_v", _sweep_shapes(24, 7))
def test_gate_out_shape_sweep(T, D, H, d_c, d_v):
    say(f"[gate_out sweep] T={T} D={D} H={H} d_c={d_c} d_v={d_v}")
    g = torch.Generator().manual_seed(T * 7919 + D + H * 31 + d_c + d_v)
    o_lat = torch.randn(T, H, d_c, generator=g).to(torch.bfloat16)
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    W_uv = (torch.randn(H, d_v, d_c, generator=g) / d_c ** 0.5).to(torch.bfloat16)
    W_g = (torch.randn(H * d_v, D, generator=g) / D ** 0.5).to(torch.bfloat16)
    W_o = (torch.randn(D, H * d_v, generator=g) / (H * d_v) ** 0.5).to(torch.bfloat16)
    y = ops.gate_out(dev(x), dev(o_lat), dev(W_g), dev(W_o), W_uv=dev(W_uv))
    torch.cuda.synchronize()
    ry = O.gate_out_reference(_np(x), O.value_up_projection(_np(o_lat), _np(W_uv)), _np(W_g), _np(W_o))
    e = rel_err(y.float(), ry)
    say(f"  rel err y {e:.2e}")
    assert e <= BF16_TOL


def _prefill_sweep(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        L = int(rng.integers(1, 420))
        D = 64 * int(rng.integers(2, 17))
        H = int(rng.integers(1, 9))
        d_c = 64 * int(rng.integers(1, 9))
        d = int(rng.choice([64, 128]))
        out.append((B, L, D, H, d_c, d))
    return out


@pytest.mark.parametrize("B,L,D,H,d_c,d", _prefill_sweep(10, 13))
def test_prefill_shape_sweep(B, L, D, H, d_c, d):
    """Seeded prefill shapes: ragged L (query and key tiles cut anywhere,
    L below one 256-query tile), several batches, both head widths."""
    say(f"[prefill sweep] B={B} L={L} D={D} H={H} d_c={d_c} d={d}")
    inp = W.make_prefill(B, L, D, H, d_c, d, d, seed=B * 1009 + L)
    c, ot, y = _prefill(inp)
    rc, rot, ry = O.gated_mla_layer(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                    _np(inp.W_g), _np(inp.W_o), inp.sm_scale)
    e = (rel_err(c.float(), rc), rel_err(ot.float(), rot), rel_err(y.float(), ry))
    say(f"  rel err c {e[0]:.2e}  o~ {e[1]:.2e}  y {e[2]:.2e}")
    assert max(e) <= BF16_TOL
