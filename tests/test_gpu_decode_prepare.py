"""GPU parity of gmla_decode_prepare (through the C ABI) against the fp64
oracle: the appended cache row, the absorbed query, the rows left alone, and
the step chained into gmla_decode."""
import numpy as np
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, dev, f64, rel_err, say

pytestmark = pytest.mark.gpu


def _inputs(B, H, d_c, d_r, d_model, d_k, lengths=None, lo=1, hi=300, seed=3, rope_base=10000.0):
    dec = W.make_decode(B, H, d_c, d_r, lo, hi, lengths=lengths, gap_rows=2, seed=seed, rope_base=rope_base,
                        d_k_scale=d_k, name="prepare")
    return dec, W.make_decode_step(dec, d_model, d_k, seed=seed)


def _prepare(dec, st):
    g = dict(x=dev(st.x), W_c=dev(st.W_c), W_kr=None if st.W_kr is None else dev(st.W_kr), W_q=dev(st.W_q),
             W_qr=None if st.W_qr is None else dev(st.W_qr), W_uk=dev(st.W_uk))
    cache = dev(dec.cache)
    seq_start, seq_len = dev(dec.seq_start), dev(dec.seq_len)
    q_abs = ops.decode_prepare(g["x"], g["W_c"], g["W_kr"], g["W_q"], g["W_qr"], g["W_uk"], cache, seq_start,
                               seq_len, dec.rope_base)
    torch.cuda.synchronize()
    return cache, q_abs


def _oracle(dec, st):
    return O.decode_prepare_reference(st.x.float().numpy(), st.W_c.float().numpy(),
                                      None if st.W_kr is None else st.W_kr.float().numpy(),
                                      st.W_q.float().numpy(), None if st.W_qr is None else st.W_qr.float().numpy(),
                                      st.W_uk.float().numpy(), dec.seq_len.numpy(), dec.rope_base)


def _check_prepare(dec, st, cache, q_abs):
    row_ref, q_ref = _oracle(dec, st)
    tgt = (dec.seq_start + dec.seq_len.to(torch.int64)).numpy()
    got = f64(cache[torch.from_numpy(tgt).to(cache.device)])
    d_c = dec.d_c
    e_c = rel_err(got[:, :d_c], row_ref[:, :d_c])
    e_q = rel_err(q_abs[..., :d_c].float(), q_ref[..., :d_c])
    msg = f"  B={dec.B} H={dec.H} d_c={d_c} d_r={dec.d_r}: latent {e_c:.2e}, absorbed q {e_q:.2e}"
    assert e_c <= BF16_TOL and e_q <= BF16_TOL
    if dec.d_r:
        e_kr = rel_err(got[:, d_c:], row_ref[:, d_c:])
        e_qr = rel_err(q_abs[..., d_c:].float(), q_ref[..., d_c:])
        msg += f", rope key {e_kr:.2e}, rope query {e_qr:.2e}"
        assert e_kr <= BF16_TOL and e_qr <= BF16_TOL
    say(msg)
    # every other row keeps its bits
    keep = np.ones(dec.cache.shape[0], bool)
    keep[tgt] = False
    before = dec.cache.view(torch.int16).numpy()
    after = cache.view(torch.int16).cpu().numpy()
    assert np.array_equal(before[keep], after[keep])


@pytest.mark.parametrize("B,H,d_c,d_r,d_model,d_k", [
    (37, 64, 512, 0, 512, 128),     # NoPE, ragged batch (two LDS row blocks, partial tile)
    (37, 128, 512, 64, 1024, 128),  # decoupled RoPE
    (40, 32, 512, 64, 2176, 128),   # 33..64 rows, K = 17 x 128: shared-activation workgroups of 128
                                    # columns over the segments (the 64-wide RoPE key one partial)
    (5, 16, 256, 64, 256, 64),
    (1, 8, 128, 4, 192, 32),
    (70, 32, 64, 64, 128, 128),
    (300, 8, 512, 64, 256, 128),    # B > 64 (tile GEMMs); several cache appends per absorb workgroup
])
def test_prepare_matches_oracle(B, H, d_c, d_r, d_model, d_k):
    say(f"[decode_prepare] B={B} H={H} d_c={d_c} d_r={d_r} d_model={d_model} d_k={d_k}")
    dec, st = _inputs(B, H, d_c, d_r, d_model, d_k)
    cache, q_abs = _prepare(dec, st)
    _check_prepare(dec, st, cache, q_abs)


def test_prepare_positions_zero_and_far():
    """Empty sequences append at their first row; a far position keeps the
    rotation angle accurate (reduced in fp64)."""
    say("[decode_prepare] positions 0 .. 70000")
    lengths = [0, 1, 0, 63, 64, 4095, 70000, 2]
    dec, st = _inputs(len(lengths), 16, 512, 64, 256, 128, lengths=lengths)
    cache, q_abs = _prepare(dec, st)
    _check_prepare(dec, st, cache, q_abs)


def test_prepare_rope_base_zero_leaves_key_unrotated():
    say("[decode_prepare] rope_base 0")
    dec, st = _inputs(9, 16, 512, 64, 256, 128, rope_base=0.0)
    cache, q_abs = _prepare(dec, st)
    _check_prepare(dec, st, cache, q_abs)


@pytest.mark.parametrize("d_r", [0, 64])
def test_prepare_then_decode_matches_oracle(d_r):
    """prepare -> seq_len + 1 -> gmla_decode equals the oracle's chain (its
    appended row and absorbed query fed to its decode reference)."""
    say(f"[decode_prepare -> decode] d_r={d_r}")
    lengths = [0, 1, 31, 64, 65, 300, 1000]
    H, d_c, d_k, D = 64, 512, 128, 512
    dec, st = _inputs(len(lengths), H, d_c, d_r, D, d_k, lengths=lengths)
    cache, q_abs = _prepare(dec, st)
    new_len = dec.seq_len + 1
    o, lse = ops.decode(q_abs, cache, dev(dec.seq_start), dev(new_len), d_c, d_r, dec.rope_base, dec.sm_scale)
    torch.cuda.synchronize()
    row_ref, q_ref = _oracle(dec, st)
    cache_ref = dec.cache.double().numpy().copy()
    cache_ref[(dec.seq_start + dec.seq_len.to(torch.int64)).numpy()] = row_ref
    ro, rl = O.decode_reference(q_ref, cache_ref, dec.seq_start.numpy(), new_len.numpy(), d_c, d_r, dec.rope_base,
                                dec.sm_scale)
    e_o = rel_err(o.float(), ro)
    e_l = float(np.abs(f64(lse) - rl).max())
    say(f"  o rel err {e_o:.2e}, lse abs err {e_l:.2e}")
    assert e_o <= BF16_TOL
    # lse in absolute natural-log units: this chain also rounds the absorbed
    # query q~ to bf16 (the dtype it is handed over in), which the fp64
    # oracle does not; that moves each score by up to 2^-9 of the sum of
    # |q~_i c_i| (measured 7.1e-3 and 8.3e-3)
    assert e_l <= 2e-2


def test_prepare_full_size_rope_b64_h128():
    """DeepSeek-V2-shaped step: B=64, d_model=7168, H=128, d_k=128,
    d_c=512 + d_r=64, positions U[1024, 16384]."""
    say("[decode_prepare] full size B=64 H=128 d_model=7168")
    dec, st = _inputs(64, 128, 512, 64, 7168, 128, lo=1024, hi=16384, seed=0)
    cache, q_abs = _prepare(dec, st)
    _check_prepare(dec, st, cache, q_abs)


def test_prepare_rejects_fp32_and_short_workspace():
    dec, st = _inputs(4, 16, 512, 64, 256, 128)
    with pytest.raises(ops.GmlaError):  # fp32 is not supported by this entry point
        ops.decode_prepare(dev(st.x).float(), dev(st.W_c).float(), dev(st.W_kr).float(), dev(st.W_q).float(),
                           dev(st.W_qr).float(), dev(st.W_uk).float(), dev(dec.cache).float(), dev(dec.seq_start),
                           dev(dec.seq_len), dec.rope_base)
    need = ops.lib().gmla_decode_prepare_workspace_size(4, 256, 16, 512, 0, 128, 64, ops.GMLA_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.GmlaError):
        ops.decode_prepare(dev(st.x), dev(st.W_c), dev(st.W_kr), dev(st.W_q), dev(st.W_qr), dev(st.W_uk),
                           dev(dec.cache), dev(dec.seq_start), dev(dec.seq_len), dec.rope_base, workspace=ws[:need - 1])
