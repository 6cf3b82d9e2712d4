"""GPU parity of gmla_head_gate_out (per-head scalar gate, bias, W_o; with or
without the value up-projection) against the fp64 oracle."""
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, dev, rel_err, say

pytestmark = pytest.mark.gpu


def _np(t):
    return None if t is None else t.float().numpy()


def _check(g):
    y = ops.head_gate_out(dev(g.x), dev(g.o), dev(g.W_g), dev(g.W_o), b_g=None if g.b_g is None else dev(g.b_g),
                          W_uv=None if g.W_uv is None else dev(g.W_uv))
    torch.cuda.synchronize()
    ot = _np(g.o) if g.W_uv is None else O.value_up_projection(_np(g.o), _np(g.W_uv))
    ry = O.head_gate_out_reference(_np(g.x), ot, _np(g.W_g), _np(g.b_g), _np(g.W_o))
    e = rel_err(y.float(), ry)
    say(f"  T={g.T} D={g.d_model} H={g.H} d_v={g.d_v} d_c={g.d_c}: y rel err {e:.2e}")
    assert e <= BF16_TOL


@pytest.mark.parametrize("T,D,H,d_v,d_c,bias", [
    (300, 256, 4, 128, 0, True),     # prefill form, tile GEMMs
    (1000, 512, 8, 64, 0, False),
    (32, 1024, 64, 128, 512, True),  # decode form: value up-projection, split-K logits
    (7, 512, 16, 64, 128, True),
    (64, 7168, 128, 128, 512, True),  # the RoPE decode workload's output side
])
def test_head_gate_out_matches_oracle(T, D, H, d_v, d_c, bias):
    say(f"[head gate] T={T} D={D} H={H} d_v={d_v} d_c={d_c} bias={bias}")
    _check(W.make_head_gate(T, D, H, d_v, d_c, with_bias=bias, seed=9))


def test_head_gate_rejects_bad_shapes():
    g = W.make_head_gate(4, 256, 4, 64, 0, seed=1)
    with pytest.raises(ops.GmlaError):  # H % 4 != 0
        ops.head_gate_out(dev(g.x), dev(g.o)[:, :192].contiguous(), dev(g.W_g)[:3].contiguous(),
                          dev(g.W_o)[:, :192].contiguous())
    with pytest.raises(ops.GmlaError):  # fp32 is not supported
        ops.head_gate_out(dev(g.x).float(), dev(g.o).float(), dev(g.W_g).float(), dev(g.W_o).float())
