"""GPU parity of the low-rank query (c^Q = W^DQ x, q = W^UQ c^Q) in
gmla_prefill and gmla_decode_prepare against the fp64 oracle."""
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, F32_TOL, dev, f64, rel_err, say

pytestmark = pytest.mark.gpu


def _np(t):
    return None if t is None else t.float().numpy()


@pytest.mark.parametrize("B,L,D,H,d_c,d_cq,d,dtype", [
    (2, 300, 256, 4, 128, 192, 128, torch.bfloat16),
    (1, 129, 512, 3, 64, 64, 64, torch.bfloat16),
    (1, 70, 64, 2, 32, 48, 16, torch.float32),
])
def test_prefill_low_rank_query_matches_oracle(B, L, D, H, d_c, d_cq, d, dtype):
    say(f"[prefill low-rank q] B={B} L={L} D={D} H={H} d_c={d_c} d_cq={d_cq} d={d} {dtype}")
    inp = W.make_prefill(B, L, D, H, d_c, d, d, seed=33, d_cq=d_cq, dtype=dtype)
    c, ot = ops.prefill(dev(inp.x), dev(inp.W_c), dev(inp.W_q), dev(inp.W_uk), dev(inp.W_uv), inp.sm_scale,
                        W_dq=dev(inp.W_dq))
    torch.cuda.synchronize()
    rc, rot, _ = O.prefill_reference(_np(inp.x), _np(inp.W_c), _np(inp.W_q), _np(inp.W_uk), _np(inp.W_uv),
                                     inp.sm_scale, W_dq=_np(inp.W_dq))
    e = (rel_err(c.float(), rc), rel_err(ot.float(), rot))
    say(f"  rel err c {e[0]:.2e}  o~ {e[1]:.2e}")
    assert max(e) <= (BF16_TOL if dtype == torch.bfloat16 else F32_TOL)


@pytest.mark.parametrize("B,H,d_r,d_model,d_cq", [(37, 64, 64, 512, 192), (5, 16, 0, 256, 128),
                                                  (70, 32, 64, 256, 64)])
def test_decode_prepare_low_rank_query_matches_oracle(B, H, d_r, d_model, d_cq):
    """B <= 64 runs two grouped launches (x, then c^Q); B = 70 the tile GEMMs."""
    say(f"[decode_prepare low-rank q] B={B} H={H} d_r={d_r} d_model={d_model} d_cq={d_cq}")
    dec = W.make_decode(B, H, 512, d_r, 1, 200, gap_rows=1, seed=5, d_k_scale=128, name="prepare")
    st = W.make_decode_step(dec, d_model, 128, seed=5, d_cq=d_cq)
    cache = dev(dec.cache)
    q_abs = ops.decode_prepare(dev(st.x), dev(st.W_c), None if st.W_kr is None else dev(st.W_kr), dev(st.W_q),
                               None if st.W_qr is None else dev(st.W_qr), dev(st.W_uk), cache, dev(dec.seq_start),
                               dev(dec.seq_len), dec.rope_base, W_dq=dev(st.W_dq))
    torch.cuda.synchronize()
    row_ref, q_ref = O.decode_prepare_reference(_np(st.x), _np(st.W_c), _np(st.W_kr), _np(st.W_q), _np(st.W_qr),
                                                _np(st.W_uk), dec.seq_len.numpy(), dec.rope_base, W_dq=_np(st.W_dq))
    tgt = (dec.seq_start + dec.seq_len.to(torch.int64)).to(cache.device)
    e_row = rel_err(cache[tgt].float(), row_ref)
    e_q = rel_err(q_abs[..., :512].float(), q_ref[..., :512])
    msg = f"  cache row {e_row:.2e}, absorbed q {e_q:.2e}"
    errs = [e_row, e_q]
    if d_r:
        errs.append(rel_err(q_abs[..., 512:].float(), q_ref[..., 512:]))
        msg += f", rope query {errs[-1]:.2e}"
    say(msg)
    assert max(errs) <= BF16_TOL
