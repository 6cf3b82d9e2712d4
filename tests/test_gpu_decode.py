"""GPU parity of gmla_decode (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gated_mla_latent_amd import ops
from gated_mla_latent_amd import workloads as W
from tests.gpu_util import BF16_TOL, F32_TOL, dev, f64, rel_err, row_err, say

pytestmark = pytest.mark.gpu


def _run(inp, num_splits=0):
    o, lse = ops.decode(dev(inp.q_abs), dev(inp.cache), dev(inp.seq_start), dev(inp.seq_len), inp.d_c, inp.d_r,
                        inp.rope_base, inp.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def _oracle(inp, batches=None):
    return O.decode_reference(inp.q_abs.float().numpy(), inp.cache.float().numpy(), inp.seq_start.numpy(),
                              inp.seq_len.numpy(), inp.d_c, inp.d_r, inp.rope_base, inp.sm_scale, batches=batches)


def _check(inp, o, lse, tol=BF16_TOL, batches=None):
    ro, rl = _oracle(inp, batches)
    bs = list(range(inp.B)) if batches is None else list(batches)
    e_o = rel_err(o[bs].float(), ro[bs])
    e_r = row_err(o[bs].float(), ro[bs])
    e_l = float(np.abs(f64(lse)[bs] - rl[bs]).max())
    say(f"  {inp.name or 'decode'} B={inp.B} H={inp.H} d_c={inp.d_c} d_r={inp.d_r}: o rel err {e_o:.2e} "
        f"(per row {e_r:.2e}), lse abs err {e_l:.2e}")
    assert e_o <= tol
    # lse in absolute natural-log units. Scores are fp32 sums of exact bf16
    # products; the one rounding the oracle does not share is the RoPE query,
    # rotated in fp32 and rounded to bf16 before the MFMA (measured at most
    # 4.8e-3 over these cases, 1e-6 without RoPE)
    assert e_l <= 1e-2
    return e_o


# ragged lengths covering 1, tile-1, tile, tile+1 and several tiles
RAGGED = [1, 31, 32, 33, 63, 64, 65, 200, 257, 600]


@pytest.mark.parametrize("H,d_c,d_r", [(64, 512, 0), (128, 512, 64), (128, 512, 0), (64, 512, 64),
                                       (16, 512, 0), (96, 512, 64), (200, 512, 64)])
def test_decode_ragged_matches_oracle(H, d_c, d_r):
    say(f"[decode ragged] H={H} d_c={d_c} d_r={d_r}")
    inp = W.make_decode(len(RAGGED), H, d_c, d_r, 0, lengths=RAGGED, seed=11, name="ragged")
    o, lse = _run(inp)
    _check(inp, o, lse)


@pytest.mark.parametrize("d_c,d_r", [(256, 0), (256, 64), (128, 0), (64, 64), (384, 64), (512, 32)])
def test_decode_other_latent_widths(d_c, d_r):
    """Latent and RoPE widths outside the MFMA kernel's (d_c = 512 with
    d_r in {0, 64}) run the generic bf16 decode."""
    say(f"[decode generic] d_c={d_c} d_r={d_r}")
    inp = W.make_decode(len(RAGGED), 64, d_c, d_r, 0, lengths=RAGGED, seed=11, name="generic")
    o, lse = _run(inp)
    _check(inp, o, lse)


def test_decode_unsupported_latent_widths_are_rejected():
    for d_c, d_r in [(96, 0), (576, 0), (512, 600)]:
        inp = W.make_decode(2, 8, d_c, d_r, 5, 9, seed=1)
        with pytest.raises(ops.GmlaError) as e:
            _run(inp)
        assert e.value.status == 2


@pytest.mark.parametrize("num_splits", [1, 2, 7, 36, 64, 0])
def test_decode_split_invariance(num_splits):
    say(f"[decode splits] num_splits={num_splits}")
    inp = W.make_decode(6, 128, 512, 64, 1, 700, seed=3, name="splits")
    o, lse = _run(inp, num_splits)
    _check(inp, o, lse)
    o1, l1 = _run(inp, 1)
    # the same answer up to fp32 rounding of the partial merge and bf16 output rounding
    assert rel_err(o.float(), f64(o1)) <= 8e-3
    assert float((lse - l1).abs().max()) <= 1e-4


def test_decode_more_slices_than_cost_units():
    """Two short sequences cut into 1000 slices: the slices' cost ranges hold
    fewer units than there are slices, so many slices are empty and many
    hold only the start cost of a sequence (no tokens)."""
    say("[decode 1000 slices]")
    inp = W.make_decode(2, 64, 512, 64, 0, lengths=[3, 5], seed=6, name="slices")
    o, lse = _run(inp, 1000)
    _check(inp, o, lse)


@pytest.mark.parametrize("B,H", [(130, 64), (1100, 64), (600, 16)])
def test_decode_many_sequences(B, H):
    """More sequences than one wave (or one workgroup) of the prefix scan
    holds, with empty ones among them."""
    say(f"[decode many] B={B} H={H}")
    rng = np.random.default_rng(B)
    lengths = rng.integers(0, 41, size=B).tolist()
    lengths[0] = 0
    lengths[-1] = 33
    inp = W.make_decode(B, H, 512, 64, 0, lengths=lengths, seed=4, name="many")
    o, lse = _run(inp)
    nonempty = [b for b in range(B) if lengths[b] > 0]
    empty = [b for b in range(B) if lengths[b] == 0]
    assert torch.all(o[empty] == 0)
    assert torch.all(torch.isneginf(lse[empty]))
    _check(inp, o, lse, batches=nonempty)


def test_decode_honours_seq_start_with_gaps():
    say("[decode gaps]")
    inp = W.make_decode(5, 64, 512, 64, 10, 300, seed=5, gap_rows=13, name="gaps")
    o, lse = _run(inp, 3)
    _check(inp, o, lse)


def test_decode_empty_sequence_gives_zero_and_minus_inf():
    say("[decode empty]")
    inp = W.make_decode(3, 64, 512, 0, 0, lengths=[40, 0, 70], seed=2, name="empty")
    o, lse = _run(inp)
    assert torch.all(o[1] == 0)
    assert torch.all(torch.isneginf(lse[1]))
    _check(inp, o, lse, batches=[0, 2])


def test_decode_long_rope_positions():
    """One long sequence: RoPE angles at position ~1e5 and a many-slice split."""
    say("[decode long]")
    inp = W.make_decode(2, 128, 512, 64, 0, lengths=[100_003, 5], seed=7, name="long")
    o, lse = _run(inp)
    _check(inp, o, lse)


def test_decode_score_range_forces_redo_pass():
    """Scores that grow by far more than the kernel's first-tile reference
    (keys scaled up 40x after token 64) exercise the exact redo path: later
    scores then sit about 300 log2 units above the first tile's maximum, so
    a pass that kept that reference would overflow fp32 (2^128) and give
    inf or NaN."""
    say("[decode redo]")
    inp = W.make_decode(2, 64, 512, 0, 0, lengths=[300, 129], seed=9, name="redo")
    c = inp.cache.float()
    s0 = int(inp.seq_start[0])
    c[s0 + 64:s0 + 300] *= 40.0
    inp.cache = c.to(torch.bfloat16)
    o, lse = _run(inp, 1)
    _check(inp, o, lse)


def test_decode_fp32_path():
    say("[decode fp32]")
    inp = W.make_decode(4, 8, 64, 16, 1, 90, dtype=torch.float32, seed=4, name="f32")
    o, lse = _run(inp)
    _check(inp, o, lse, tol=F32_TOL)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", ["decode_nope_b32_h64", "decode_rope_b64_h128", "decode_rope_b8_l131072"])
def test_decode_full_size_workloads(cfg):
    """Full workload sizes in the launch configuration the benchmark times
    (num_splits = 0); the oracle checks every sequence and head."""
    say(f"[decode full] {cfg}")
    inp = getattr(W, cfg)(with_output_side=False)
    o, lse = _run(inp)
    _check(inp, o, lse)


def _decode_sweep(n, seed):
    """Seeded decode batches: head counts that are and are not multiples of
    the 64-head chunks, NoPE and RoPE, lengths from 0 (empty) to a few
    thousand with ragged mixes, explicit and automatic slice counts."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 40))
        H = int(rng.choice([8, 16, 32, 64, 80, 128, 160]))
        d_r = int(rng.choice([0, 64]))
        lengths = [int(v) for v in rng.integers(0, 3000, size=B)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, B))] = 0
        splits = int(rng.choice([0, 0, 1, 7, 64]))
        out.append((H, d_r, tuple(lengths), splits))
    return out


@pytest.mark.parametrize("H,d_r,lengths,splits", _decode_sweep(10, 19))
def test_decode_shape_sweep(H, d_r, lengths, splits):
    say(f"[decode sweep] B={len(lengths)} H={H} d_r={d_r} splits={splits} total={sum(lengths)}")
    inp = W.make_decode(len(lengths), H, 512, d_r, 0, lengths=list(lengths), seed=len(lengths) * 31 + H,
                        name="sweep")
    o, lse = _run(inp, num_splits=splits)
    empty = [b for b in range(len(lengths)) if lengths[b] == 0]
    assert torch.all(o[empty] == 0) and torch.all(torch.isneginf(lse[empty]))
    nonempty = [b for b in range(len(lengths)) if lengths[b] > 0]
    if nonempty:
        _check(inp, o, lse, batches=nonempty)
