"""Seeded synthetic inputs for the Gated-MLA kernels.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. The test suite feeds the very same tensors to the HIP
library and to the fp64 CPU oracle, and the benchmark uses them too.

Recipe (shared by every workload):
  * one `torch.Generator('cpu')` seeded with `seed` (default 0) per workload;
  * values are drawn in fp32 with `torch.randn`, scaled, then rounded to the
    workload dtype (bf16 is round-to-nearest-even, i.e. `.to(torch.bfloat16)`);
  * activations, latents and queries are N(0, 1); every weight is
    N(0, 1/fan_in), fan_in being the input width of that projection;
  * draw order: sequence lengths (`randint(lo, hi + 1)`), cache, query, then
    x, W_c, W_q, W_UK, W_UV, W_g, W_o as the workload needs them;
  * weights use the [out, in] layout; W_UK is [H, d_k, d_c], W_UV [H, d_v, d_c];
  * the decode cache packs the sequences back to back unless `gap_rows` asks
    for unused rows between them (filled with a large constant so that a
    kernel reading outside its sequence is caught).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16
F32 = torch.float32


def _randn(gen, shape, std, dtype):
    t = torch.randn(shape, generator=gen, dtype=F32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _weight(gen, out_f, in_f, dtype, lead=()):
    return _randn(gen, tuple(lead) + (out_f, in_f), 1.0 / math.sqrt(in_f), dtype)


@dataclass
class DecodeInputs:
    B: int
    H: int
    d_c: int
    d_r: int
    rope_base: float
    sm_scale: float
    dtype: torch.dtype
    seq_len: torch.Tensor  # int32 [B]
    seq_start: torch.Tensor  # int64 [B]
    cache: torch.Tensor  # [rows, d_c + d_r]
    q_abs: torch.Tensor  # [B, H, d_c + d_r]
    # output side (optional): x [B, d_model], W_uv [H, d_v, d_c],
    # W_g [H*d_v, d_model], W_o [d_model, H*d_v]
    d_model: int = 0
    d_v: int = 0
    x: torch.Tensor | None = None
    W_uv: torch.Tensor | None = None
    W_g: torch.Tensor | None = None
    W_o: torch.Tensor | None = None
    name: str = ""


@dataclass
class PrefillInputs:
    B: int
    L: int
    d_model: int
    H: int
    d_c: int
    d_k: int
    d_v: int
    sm_scale: float
    dtype: torch.dtype
    x: torch.Tensor  # [B, L, d_model]
    W_c: torch.Tensor  # [d_c, d_model]
    W_q: torch.Tensor  # [H*d_k, d_model]
    W_uk: torch.Tensor  # [H, d_k, d_c]
    W_uv: torch.Tensor  # [H, d_v, d_c]
    W_g: torch.Tensor  # [H*d_v, d_model]
    W_o: torch.Tensor  # [d_model, H*d_v]
    name: str = ""
    # low-rank query (d_cq > 0): W_dq [d_cq, d_model]; W_q is then W^UQ [H*d_k, d_cq]
    d_cq: int = 0
    W_dq: torch.Tensor | None = None
    # decoupled RoPE (d_r > 0): W_kr [d_r, d_model], W_qr [H*d_r, d_in]
    d_r: int = 0
    rope_base: float = 0.0
    W_kr: torch.Tensor | None = None
    W_qr: torch.Tensor | None = None


def make_decode(B, H, d_c, d_r, len_lo, len_hi=None, *, rope_base=10000.0,
                sm_scale=None, d_k_scale=128, dtype=BF16, seed=0,
                with_output_side=False, d_model=7168, d_v=128, gap_rows=0,
                lengths=None, name="") -> DecodeInputs:
    """Decode-step inputs. Sequence lengths are drawn U[len_lo, len_hi]
    (or given explicitly by `lengths`)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    if lengths is not None:
        seq_len = torch.tensor(list(lengths), dtype=torch.int32)
    else:
        hi = len_lo if len_hi is None else len_hi
        seq_len = torch.randint(len_lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    starts = []
    pos = gap_rows
    for L in seq_len.tolist():
        starts.append(pos)
        pos += L + gap_rows
    rows = pos
    seq_start = torch.tensor(starts, dtype=torch.int64)
    W = d_c + d_r
    cache = torch.empty((rows, W), dtype=dtype)
    if gap_rows:
        cache.fill_(1.0e4)
    for b, L in enumerate(seq_len.tolist()):
        s0 = starts[b]
        cache[s0:s0 + L] = _randn(gen, (L, W), 1.0, dtype)
    q_abs = _randn(gen, (B, H, W), 1.0, dtype)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_k_scale + d_r)
    inp = DecodeInputs(B=B, H=H, d_c=d_c, d_r=d_r, rope_base=(rope_base if d_r else 0.0),
                       sm_scale=sm_scale, dtype=dtype, seq_len=seq_len, seq_start=seq_start,
                       cache=cache, q_abs=q_abs, name=name)
    if with_output_side:
        inp.d_model, inp.d_v = d_model, d_v
        inp.x = _randn(gen, (B, d_model), 1.0, dtype)
        inp.W_uv = _weight(gen, d_v, d_c, dtype, lead=(H,))
        inp.W_g = _weight(gen, H * d_v, d_model, dtype)
        inp.W_o = _weight(gen, d_model, H * d_v, dtype)
    return inp


def make_prefill(B, L, d_model, H, d_c, d_k, d_v, *, dtype=BF16, seed=0,
                 sm_scale=None, name="", d_cq=0, d_r=0, rope_base=10000.0) -> PrefillInputs:
    """Prefill inputs. With d_cq > 0 the query is low-rank: W_dq is drawn
    from a generator of its own (seed + 4099) and W_q has fan-in d_cq. With
    d_r > 0, W_kr and W_qr (fan-in d_model, and d_cq or d_model) come from
    another (seed + 8191), and the default scale is 1/sqrt(d_k + d_r). The
    other tensors are drawn exactly as without them."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = _randn(gen, (B, L, d_model), 1.0, dtype)
    W_c = _weight(gen, d_c, d_model, dtype)
    W_q = _weight(gen, H * d_k, d_cq if d_cq else d_model, dtype)
    W_uk = _weight(gen, d_k, d_c, dtype, lead=(H,))
    W_uv = _weight(gen, d_v, d_c, dtype, lead=(H,))
    W_g = _weight(gen, H * d_v, d_model, dtype)
    W_o = _weight(gen, d_model, H * d_v, dtype)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_k + d_r)
    W_dq = None
    if d_cq:
        W_dq = _weight(torch.Generator("cpu").manual_seed(seed + 4099), d_cq, d_model, dtype)
    W_kr = W_qr = None
    if d_r:
        g2 = torch.Generator("cpu").manual_seed(seed + 8191)
        W_kr = _weight(g2, d_r, d_model, dtype)
        W_qr = _weight(g2, H * d_r, d_cq if d_cq else d_model, dtype)
    return PrefillInputs(B=B, L=L, d_model=d_model, H=H, d_c=d_c, d_k=d_k, d_v=d_v,
                         sm_scale=sm_scale, dtype=dtype, x=x, W_c=W_c, W_q=W_q,
                         W_uk=W_uk, W_uv=W_uv, W_g=W_g, W_o=W_o, name=name, d_cq=d_cq, W_dq=W_dq,
                         d_r=d_r, rope_base=rope_base if d_r else 0.0, W_kr=W_kr, W_qr=W_qr)


# The five workloads, with their full sizes.
def prefill_f32_tiny(seed=0):
    """Tiny fp32 causal prefill: B=1, L=128, d_model=256, H=4, d_c=64,
    d_k=d_v=32, NoPE, full-rank gate 256 -> H*d_v."""
    return make_prefill(1, 128, 256, 4, 64, 32, 32, dtype=F32, seed=seed, name="prefill_f32_tiny")


def decode_nope_b32_h64(seed=0, with_output_side=True):
    """bf16 decode, NoPE: B=32, H=64, d_c=512, L_b ~ U[1024, 8192]."""
    return make_decode(32, 64, 512, 0, 1024, 8192, d_k_scale=128, seed=seed,
                       with_output_side=with_output_side, name="decode_nope_b32_h64")


def decode_rope_b64_h128(seed=0, with_output_side=True):
    """bf16 decode with decoupled RoPE: B=64, H=128, d_c=512 + d_r=64,
    base 10000, L_b ~ U[1024, 16384]."""
    return make_decode(64, 128, 512, 64, 1024, 16384, rope_base=10000.0, d_k_scale=128,
                       seed=seed, with_output_side=with_output_side, name="decode_rope_b64_h128")


def prefill_b2_l8192(seed=0):
    """bf16 causal prefill: B=2, L=8192, d_model=7168, H=64, d_c=512,
    d_k=d_v=128, NoPE, gate 7168 -> 8192 before W_o 8192 -> 7168."""
    return make_prefill(2, 8192, 7168, 64, 512, 128, 128, seed=seed, name="prefill_b2_l8192")


def prefill_rope_b2_l8192(seed=0):
    """bf16 causal prefill with decoupled RoPE: the prefill workload's shape
    plus d_r = 64 (RoPE key shared by the heads, base 10000), scale
    1/sqrt(128 + 64)."""
    return make_prefill(2, 8192, 7168, 64, 512, 128, 128, seed=seed, d_r=64, name="prefill_rope_b2_l8192")


def decode_rope_b8_l131072(seed=0, with_output_side=True):
    """bf16 long-context decode: B=8, H=128, d_c=512 + 64, L=131072 each."""
    return make_decode(8, 128, 512, 64, 131072, 131072, rope_base=10000.0, d_k_scale=128,
                       seed=seed, with_output_side=with_output_side, name="decode_rope_b8_l131072")


@dataclass
class DecodeStepInputs:
    """The new token of every sequence and the projections that feed one
    decode step: x [B, d_model], W_c [d_c, d_model], W_kr [d_r, d_model],
    W_q [H*d_k, d_model], W_qr [H*d_r, d_model], W_uk [H, d_k, d_c]
    (W_kr and W_qr are None when d_r == 0). With d_cq > 0 the query is
    low-rank: W_dq [d_cq, d_model], and W_q, W_qr have fan-in d_cq."""
    d_model: int
    d_k: int
    x: torch.Tensor
    W_c: torch.Tensor
    W_kr: torch.Tensor | None
    W_q: torch.Tensor
    W_qr: torch.Tensor | None
    W_uk: torch.Tensor
    d_cq: int = 0
    W_dq: torch.Tensor | None = None


def make_decode_step(dec: DecodeInputs, d_model: int, d_k: int, *, seed=0, d_cq=0) -> DecodeStepInputs:
    """Inputs of the decode-step projections for the sequences of `dec`.
    Drawn from their own generator (seed + 7919) in the order x, W_c, W_kr,
    W_q, W_qr, W_uk (then W_dq), so that `dec` is the same tensor set with or
    without them. Build `dec` with gap_rows >= 1 so that row seq_start +
    seq_len, the one the step appends, is free."""
    gen = torch.Generator("cpu").manual_seed(seed + 7919)
    B, H, d_c, d_r, dt = dec.B, dec.H, dec.d_c, dec.d_r, dec.dtype
    d_in = d_cq if d_cq else d_model
    x = _randn(gen, (B, d_model), 1.0, dt)
    W_c = _weight(gen, d_c, d_model, dt)
    W_kr = _weight(gen, d_r, d_model, dt) if d_r else None
    W_q = _weight(gen, H * d_k, d_in, dt)
    W_qr = _weight(gen, H * d_r, d_in, dt) if d_r else None
    W_uk = _weight(gen, d_k, d_c, dt, lead=(H,))
    W_dq = _weight(gen, d_cq, d_model, dt) if d_cq else None
    return DecodeStepInputs(d_model=d_model, d_k=d_k, x=x, W_c=W_c, W_kr=W_kr, W_q=W_q, W_qr=W_qr, W_uk=W_uk,
                            d_cq=d_cq, W_dq=W_dq)


@dataclass
class HeadGateInputs:
    """Inputs of the per-head scalar gate and output projection: x [T, d_model],
    o (o~ [T, H*d_v], or o_lat [T, H, d_c] with W_uv [H, d_v, d_c]),
    W_g [H, d_model], b_g [H] (or None), W_o [d_model, H*d_v]."""
    T: int
    d_model: int
    H: int
    d_v: int
    d_c: int
    x: torch.Tensor
    o: torch.Tensor
    W_uv: torch.Tensor | None
    W_g: torch.Tensor
    b_g: torch.Tensor | None
    W_o: torch.Tensor


def make_head_gate(T, d_model, H, d_v, d_c=0, *, with_bias=True, dtype=BF16, seed=0) -> HeadGateInputs:
    """Drawn in the order x, o, W_uv (d_c > 0: the decode form), W_g, b_g,
    W_o; o and the bias are N(0, 1), weights N(0, 1/fan_in)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = _randn(gen, (T, d_model), 1.0, dtype)
    o = _randn(gen, (T, H, d_c) if d_c else (T, H * d_v), 1.0, dtype)
    W_uv = _weight(gen, d_v, d_c, dtype, lead=(H,)) if d_c else None
    W_g = _weight(gen, H, d_model, dtype)
    b_g = _randn(gen, (H,), 1.0, dtype) if with_bias else None
    W_o = _weight(gen, d_model, H * d_v, dtype)
    return HeadGateInputs(T=T, d_model=d_model, H=H, d_v=d_v, d_c=d_c, x=x, o=o, W_uv=W_uv, W_g=W_g, b_g=b_g, W_o=W_o)
