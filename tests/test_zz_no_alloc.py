"""gmla_decode_noalloc (the decode entry point that allocates nothing and
takes no workspace; its scratch is the library's static device array)
against gmla_decode with a caller workspace: two calls in a row, the second
with a smaller input, must give the same bits; a request past the scratch
size is refused before any launch."""
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, dev, rel_err, say

pytestmark = pytest.mark.gpu


def _args(inp):
    return (dev(inp.q_abs), dev(inp.cache), dev(inp.seq_start), dev(inp.seq_len), inp.d_c, inp.d_r, inp.rope_base,
            inp.sm_scale)


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    big = W.make_decode(40, 128, 512, 64, 1, 3000, seed=31, name="noalloc-big")
    small = W.make_decode(6, 64, 512, 0, 1, 500, seed=32, name="noalloc-small")
    ref = [ops.decode(*_args(i)) for i in (big, small)]
    torch.cuda.synchronize()
    # two calls in a row on the library's scratch, the second smaller
    got = [ops.decode_noalloc(*_args(i)) for i in (big, small)]
    torch.cuda.synchronize()
    for inp, (o_r, l_r), (o_n, l_n) in zip((big, small), ref, got):
        say(f"[noalloc] {inp.name} B={inp.B} H={inp.H} d_r={inp.d_r}: max |diff| o "
            f"{float((o_n.float() - o_r.float()).abs().max()):.1e}, lse {float((l_n - l_r).abs().max()):.1e}")
        assert torch.equal(o_n, o_r) and torch.equal(l_n, l_r)
    # and the oracle agrees (the parity bar of the workspace entry point)
    ro, _ = O.decode_reference(small.q_abs.float().numpy(), small.cache.float().numpy(), small.seq_start.numpy(),
                               small.seq_len.numpy(), small.d_c, small.d_r, small.rope_base, small.sm_scale)
    assert rel_err(got[1][0].float(), ro) <= BF16_TOL


def test_noalloc_decode_with_explicit_splits_and_refusal():
    inp = W.make_decode(5, 96, 512, 64, 10, 900, seed=33, name="noalloc-splits")
    o_r, l_r = ops.decode(*_args(inp), num_splits=37)
    o_n, l_n = ops.decode_noalloc(*_args(inp), num_splits=37)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_r) and torch.equal(l_n, l_r)
    # 65535 slices of 96 heads need ~13 GB of partial outputs: refused
    with pytest.raises(ops.GmlaError) as e:
        ops.decode_noalloc(*_args(inp), num_splits=65535)
    assert e.value.status == 2 and "scratch" in e.value.detail
