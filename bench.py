#!/usr/bin/env python3
"""Benchmark of the Gated-MLA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 60] [--workload all]

A step is one pass of the hot path over one batch of synthetic input:
  decode_*  : gmla_decode (attention over the latent cache + split combine)
              followed by gmla_gate_out (value up-projection, sigmoid gate,
              W_o) for the B query tokens; the step's input side,
              gmla_decode_prepare (latent, RoPE key and query projections,
              cache append, query absorption, d_k = 128), is timed in a
              region of its own and reported as decode_prepare;
  prefill   : gmla_prefill (latent, query, K/V reconstruction, causal
              attention) followed by gmla_gate_out over all B*L tokens;
  prefill_rope: the same with decoupled RoPE (RoPE key and query
              projections, their rotation, 192-wide scores);
  tiny_fp32 : the same as prefill for the tiny fp32 workload.
Inputs are resident in HBM before timing starts; several copies of every
input that is read in the step rotate so that the 256 MB Infinity Cache
cannot serve a step from the previous one. The library is called through
its C ABI (argument tuples marshalled once). ms_per_step comes from events
around the timed steps alone; per-kernel device times come from a second
pass over as many steps with the library's event trace on (hipEvents
recorded on the launch stream around every kernel), since those events add
work to the stream themselves.

By default every workload of the path runs, one after the other, and one
JSON line carries them all: the top-level value, roofline and cpu_baseline
are those of the causal prefill (B=2, L=8192, d_model=7168, H=64), the
largest single-GPU workload by work, and "configs" holds the same record
for each workload (the three decode workloads and the tiny fp32 prefill
too). --workload NAME runs one workload alone. The fp64 CPU oracle is
timed on a bounded sample of each workload on the host cores
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + HBM GB/s (or MFMA %) of roofline; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
# The fp32 path runs plain (non-packed) fp32 FMAs on the vector ALUs: 256
# compute units x 64 FMA lanes x 2 flops x 2.4 GHz = 78.6 TFLOP/s. The
# published 157.3 TFLOP/s fp32 vector figure counts packed fp32 (two FMAs per
# lane and instruction), which this library never emits.
F32_FMA_PEAK_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12

ALL_WORKLOADS = ["prefill", "decode_nope", "decode_rope", "decode_long", "tiny_fp32"]
HEADLINE = "prefill"

WORKLOADS = {
    "decode_nope": ("decode_nope_b32_h64", "decode NoPE, B=32, H=64, d_c=512, L_b~U[1024,8192], bf16 + gate/W_o (d_model 7168, d_v 128)"),
    "decode_rope": ("decode_rope_b64_h128", "decode RoPE, B=64, H=128, d_c=512+d_r=64, L_b~U[1024,16384], bf16 + gate/W_o (d_model 7168, d_v 128)"),
    "decode_long": ("decode_rope_b8_l131072", "decode RoPE, B=8, H=128, d_c=512+64, L=131072 each, bf16 + gate/W_o (d_model 7168, d_v 128)"),
    "prefill": ("prefill_b2_l8192", "causal prefill B=2, L=8192, d_model=7168, H=64, d_c=512, d_k=d_v=128, bf16 + gate/W_o"),
    "prefill_rope": ("prefill_rope_b2_l8192", "causal prefill with decoupled RoPE B=2, L=8192, d_model=7168, H=64, d_c=512, d_k=d_v=128, d_r=64, bf16 + gate/W_o"),
    "tiny_fp32": ("prefill_f32_tiny", "causal prefill B=1, L=128, d_model=256, H=4, d_c=64, d_k=d_v=32, fp32 + gate/W_o"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 10 warmup steps left the first timed region of the decode workloads
    # 6-8% slower than later ones (318 against 293 us per RoPE step); from
    # about 60 steps on the timed regions agree
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=3, help="rotating input copies (cache-defeating)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of each oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--no-measured-peak", action="store_true",
                    help="skip the measured reference peaks (read-only streaming kernel, library GEMM)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (reference for HBM byte counters)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- accounting
def decode_bytes(inp):
    W = inp.d_c + inp.d_r
    tokens = int(inp.seq_len.clamp(min=0).sum())
    cache = tokens * W * 2
    q = inp.B * inp.H * W * 2
    out = inp.B * inp.H * inp.d_c * 2 + inp.B * inp.H * 4
    return {"cache": cache, "q": q, "out": out, "tokens": tokens}


def decode_attn_flops(inp):
    tokens = int(inp.seq_len.clamp(min=0).sum())
    return tokens * inp.H * (2 * (inp.d_c + inp.d_r) + 2 * inp.d_c)


def gate_out_bytes(inp):
    T, D, H, dv, dc = inp.B, inp.d_model, inp.H, inp.d_v, inp.d_c
    HV = H * dv
    return {
        "gemm_value_up": H * dv * dc * 2 + T * H * dc * 2 + T * HV * 2,
        "gemm_gate": HV * D * 2 + T * D * 2 + 2 * T * HV * 2,
        "gemm_out": D * HV * 2 + T * HV * 2 + T * D * 2,
    }


DECODE_D_K = 128  # per-head query width of the decode workloads' input side


def prepare_bytes(inp, d_k=DECODE_D_K):
    """Algorithmic HBM bytes of gmla_decode_prepare: x and every weight read
    once, the new cache rows and the absorbed queries written once."""
    B, D, H, dc, dr = inp.B, inp.d_model, inp.H, inp.d_c, inp.d_r
    W = dc + dr
    weights = (dc + dr + H * d_k + H * dr) * D * 2 + H * d_k * dc * 2
    return B * D * 2 + weights + B * W * 2 + B * H * W * 2


def head_gate_bytes(inp):
    """Algorithmic HBM bytes of gmla_head_gate_out at decode: W_UV, W_g
    [H, d_model], b_g, W_o and x read once, o_lat read once, y written once."""
    T, D, H, dv, dc = inp.B, inp.d_model, inp.H, inp.d_v, inp.d_c
    return (H * dv * dc + H * D + H + D * H * dv + T * D + T * H * dc + T * D) * 2


def gate_out_flops(inp):
    T, D, H, dv, dc = inp.B, inp.d_model, inp.H, inp.d_v, inp.d_c
    return {"gemm_value_up": 2 * T * H * dv * dc, "gemm_gate": 2 * T * D * H * dv, "gemm_out": 2 * T * D * H * dv}


def prefill_flops(p):
    T = p.B * p.L
    pairs = p.B * p.L * (p.L + 1) // 2  # unmasked (t, s <= t) pairs per head
    f = {
        "gemm_latent": 2 * T * p.d_model * p.d_c,
        "gemm_query": 2 * T * p.d_model * p.H * p.d_k,
        "gemm_key_recon": 2 * T * p.d_c * p.H * p.d_k,
        "gemm_value_recon": 2 * T * p.d_c * p.H * p.d_v,
        "prefill_attn": 2 * pairs * p.H * (p.d_k + p.d_r + p.d_v),
        "gemm_gate": 2 * T * p.d_model * p.H * p.d_v,
        "gemm_out": 2 * T * p.H * p.d_v * p.d_model,
    }
    if p.d_r:
        f["gemm_rope_key"] = 2 * T * p.d_model * p.d_r
        f["gemm_rope_query"] = 2 * T * p.d_model * p.H * p.d_r
    return f


# ----------------------------------------------------------------------------- runners
def _vp(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def build_decode(args, inp, torch, ops):
    dev = "cuda"
    L = ops.lib()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    q = inp.q_abs.to(dev)
    seq_start, seq_len = inp.seq_start.to(dev), inp.seq_len.to(dev)
    x = inp.x.to(dev)
    from gated_mla_latent_amd import workloads
    stp = workloads.make_decode_step(inp, inp.d_model, DECODE_D_K)
    copies = []
    for i in range(args.copies):
        copies.append(dict(cache=inp.cache.to(dev), W_uv=inp.W_uv.to(dev), W_g=inp.W_g.to(dev), W_o=inp.W_o.to(dev),
                           W_c=stp.W_c.to(dev), W_q=stp.W_q.to(dev), W_uk=stp.W_uk.to(dev),
                           W_kr=None if stp.W_kr is None else stp.W_kr.to(dev),
                           W_qr=None if stp.W_qr is None else stp.W_qr.to(dev)))
        log(f"  copy {i} resident")
    # the input side appends each new row to a [B, d_c + d_r] buffer of its
    # own (row b, at the sequence's true position seq_len[b]) so that the
    # timed caches stay as generated
    x_new = stp.x.to(dev)
    rows_new = torch.empty((inp.B, inp.d_c + inp.d_r), dtype=torch.bfloat16, device=dev)
    start_new = (torch.arange(inp.B, dtype=torch.int64) - inp.seq_len.to(torch.int64)).to(dev)
    q_new = torch.empty((inp.B, inp.H, inp.d_c + inp.d_r), dtype=torch.bfloat16, device=dev)
    wsp_n = L.gmla_decode_prepare_workspace_size(inp.B, inp.d_model, inp.H, inp.d_c, 0, DECODE_D_K, inp.d_r, 1)
    wsp = torch.empty(wsp_n, dtype=torch.uint8, device=dev)
    # the per-head scalar gate variant of the output side (W_g [H, d_model], b_g [H])
    hg = workloads.make_head_gate(1, inp.d_model, inp.H, inp.d_v, seed=3)
    W_gh, b_gh = hg.W_g.to(dev), hg.b_g.to(dev)
    wsh_n = L.gmla_head_gate_out_workspace_size(inp.B, inp.d_model, inp.H, inp.d_c, inp.d_v, 1, 1)
    wsh = torch.empty(wsh_n, dtype=torch.uint8, device=dev)
    o_lat = torch.empty((inp.B, inp.H, inp.d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.B, inp.H), dtype=torch.float32, device=dev)
    y = torch.empty((inp.B, inp.d_model), dtype=torch.bfloat16, device=dev)
    wsd_n = L.gmla_decode_workspace_size(inp.B, inp.H, inp.d_c, args.num_splits, 1)
    wsg_n = L.gmla_gate_out_workspace_size(inp.B, inp.d_model, inp.H, inp.d_c, inp.d_v, 1, 1)
    wsd = torch.empty(wsd_n, dtype=torch.uint8, device=dev)
    wsg = torch.empty(wsg_n, dtype=torch.uint8, device=dev)
    calls = []
    for c in copies:
        dec = (_vp(q), _vp(c["cache"]), _vp(seq_start), _vp(seq_len), _vp(o_lat), _vp(lse), _vp(wsd), C.c_size_t(wsd_n),
               inp.B, inp.H, inp.d_c, inp.d_r, C.c_float(inp.rope_base), C.c_float(inp.sm_scale), args.num_splits, 1,
               stream)
        go = (_vp(x), _vp(o_lat), _vp(c["W_uv"]), _vp(c["W_g"]), _vp(c["W_o"]), _vp(y), _vp(wsg), C.c_size_t(wsg_n),
              inp.B, inp.d_model, inp.H, inp.d_c, inp.d_v, 1, stream)
        pre = (_vp(x_new), _vp(c["W_c"]), _vp(c["W_kr"]), C.c_void_p(0), _vp(c["W_q"]), _vp(c["W_qr"]), _vp(c["W_uk"]),
               _vp(rows_new), _vp(start_new), _vp(seq_len), _vp(q_new), _vp(wsp), C.c_size_t(wsp_n), inp.B,
               inp.d_model, inp.H, inp.d_c, 0, DECODE_D_K, inp.d_r, C.c_float(inp.rope_base), 1, stream)
        hgo = (_vp(x), _vp(o_lat), _vp(c["W_uv"]), _vp(W_gh), _vp(b_gh), _vp(c["W_o"]), _vp(y), _vp(wsh),
               C.c_size_t(wsh_n), inp.B, inp.d_model, inp.H, inp.d_c, inp.d_v, 1, stream)
        calls.append((dec, go, pre, hgo))
    keep = (q, seq_start, seq_len, x, copies, o_lat, lse, y, wsd, wsg, x_new, rows_new, start_new, q_new, wsp,
            W_gh, b_gh, wsh)

    def step(i):
        dec, go = calls[i % len(calls)][:2]
        s = L.gmla_decode(*dec)
        if s:
            raise RuntimeError(L.gmla_last_error().decode())
        s = L.gmla_gate_out(*go)
        if s:
            raise RuntimeError(L.gmla_last_error().decode())

    def prepare(i):
        s = L.gmla_decode_prepare(*calls[i % len(calls)][2])
        if s:
            raise RuntimeError(L.gmla_last_error().decode())

    def head_gate(i):
        s = L.gmla_head_gate_out(*calls[i % len(calls)][3])
        if s:
            raise RuntimeError(L.gmla_last_error().decode())

    return step, (keep, {"decode_prepare": prepare, "head_gate_out": head_gate})


def build_prefill(args, p, torch, ops):
    dev = "cuda"
    L = ops.lib()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = 1 if p.dtype == torch.bfloat16 else 0
    T = p.B * p.L
    copies = []
    for i in range(args.copies):
        copies.append({k: (None if getattr(p, k) is None else getattr(p, k).to(dev))
                       for k in ("x", "W_c", "W_q", "W_uk", "W_uv", "W_g", "W_o", "W_kr", "W_qr")})
        log(f"  copy {i} resident")
    lat = torch.empty((p.B, p.L, p.d_c + p.d_r), dtype=p.dtype, device=dev)
    ot = torch.empty((p.B, p.L, p.H * p.d_v), dtype=p.dtype, device=dev)
    y = torch.empty((T, p.d_model), dtype=p.dtype, device=dev)
    wsp_n = L.gmla_prefill_workspace_size(p.B, p.L, p.H, 0, p.d_k, p.d_r, p.d_v, dt)
    wsg_n = L.gmla_gate_out_workspace_size(T, p.d_model, 1, 0, p.H * p.d_v, 0, dt)
    wsp = torch.empty(wsp_n, dtype=torch.uint8, device=dev)
    wsg = torch.empty(wsg_n, dtype=torch.uint8, device=dev)
    calls = []
    for c in copies:
        nul = C.c_void_p(0)
        pre = (_vp(c["x"]), _vp(c["W_c"]), nul, _vp(c["W_q"]), _vp(c["W_kr"]), _vp(c["W_qr"]), _vp(c["W_uk"]),
               _vp(c["W_uv"]), _vp(lat), _vp(ot), _vp(wsp), C.c_size_t(wsp_n), p.B, p.L, p.d_model, p.H, p.d_c, 0,
               p.d_k, p.d_r, p.d_v, C.c_float(p.sm_scale), C.c_float(p.rope_base), dt, stream)
        go = (_vp(c["x"]), _vp(ot), C.c_void_p(0), _vp(c["W_g"]), _vp(c["W_o"]), _vp(y), _vp(wsg), C.c_size_t(wsg_n),
              T, p.d_model, 1, 0, p.H * p.d_v, dt, stream)
        calls.append((pre, go))
    keep = (copies, lat, ot, y, wsp, wsg)

    def step(i):
        pre, go = calls[i % len(calls)]
        s = L.gmla_prefill(*pre)
        if s:
            raise RuntimeError(L.gmla_last_error().decode())
        s = L.gmla_gate_out(*go)
        if s:
            raise RuntimeError(L.gmla_last_error().decode())

    return step, keep


# ----------------------------------------------------------------------------- cpu baseline
def _oracle_threads():
    """Threads the oracle's numpy work can use: the BLAS pool (matrix
    products); elementwise numpy runs on one thread."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline_decode(inp, budget_s):
    import numpy as np
    import oracle as O
    threads = _oracle_threads()
    q = inp.q_abs.float().numpy()
    cache = inp.cache  # bf16 torch; rows are upcast per sequence inside the oracle
    # whole sequences until the budget is spent (or the batch is done)
    done, tokens, t0 = [], 0, time.perf_counter()
    for b in range(inp.B):
        s0, Lb = int(inp.seq_start[b]), int(inp.seq_len[b])
        rows = cache[s0:s0 + Lb].float().numpy()
        O.decode_reference(q[b:b + 1], rows, np.array([0]), np.array([Lb]), inp.d_c, inp.d_r, inp.rope_base,
                           inp.sm_scale)
        done.append(b)
        tokens += Lb
        if time.perf_counter() - t0 > budget_s:
            break
    t_dec = time.perf_counter() - t0
    # output side for the sampled query tokens
    t1 = time.perf_counter()
    o_lat = np.random.default_rng(0).standard_normal((len(done), inp.H, inp.d_c))
    ot = O.value_up_projection(o_lat, inp.W_uv.float().numpy())
    O.gate_out_reference(inp.x[done].float().numpy(), ot, inp.W_g.float().numpy(), inp.W_o.float().numpy())
    t_go = time.perf_counter() - t1
    secs = t_dec + t_go
    return {"value": len(done) / secs, "unit": "tokens/s", "cores": threads, "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"fp64 oracle: decode of {len(done)} of {inp.B} sequences ({tokens} cached tokens) plus "
                      f"gate/W_o for those {len(done)} query tokens; {secs:.1f} s on the host"}


def cpu_baseline_prefill(p, budget_s):
    import numpy as np
    import oracle as O
    threads = _oracle_threads()
    # sample: the first Ls positions of sequence 0; Ls doubles until the
    # oracle run takes about a third of the budget (or covers the sequence)
    Ls = min(p.L, 64)
    W = {k: (None if getattr(p, k) is None else getattr(p, k).float().numpy())
         for k in ("W_c", "W_q", "W_uk", "W_uv", "W_g", "W_o", "W_kr", "W_qr")}
    while True:
        x = p.x[:1, :Ls].float().numpy()
        reps, t0 = 0, time.perf_counter()
        while True:
            _, ot, _ = O.prefill_reference(x, W["W_c"], W["W_q"], W["W_uk"], W["W_uv"], p.sm_scale, W_kr=W["W_kr"],
                                           W_qr=W["W_qr"], rope_base=p.rope_base)
            O.gate_out_reference(x[0], ot[0], W["W_g"], W["W_o"])
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= min(1.0, budget_s / 3):
                break
        if secs / reps >= budget_s / 3 or Ls >= p.L:
            break
        Ls = min(p.L, Ls * 2)
    fl = prefill_flops(p.__class__(**{**p.__dict__, "B": 1, "L": Ls}))
    per = secs / reps
    return {"value": sum(fl.values()) / per / 1e12, "unit": "TFLOP/s", "cores": threads, "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"fp64 oracle: whole layer on the first {Ls} positions of one sequence "
                      f"({sum(fl.values()) / 1e9:.2f} GFLOP), {reps} run(s) in {secs:.1f} s on the host"}


def measured_peaks(torch, ops):
    """Measured references beside the published peaks, labelled separately:
    HBM: the library's read-bandwidth probe streaming 2 GiB (read-only, the
    access the HBM-bound kernels make); MFMA: torch.matmul (the vendor GEMM
    library) on an 8192^3 bf16 product A B^T with B stored [N, K] row-major,
    the operand layout of the library's GEMMs (C = A W^T); the vendor library
    runs that layout about 20% faster than A B with B stored [K, N]."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    out = {}
    n = 2 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(ops.PROBE_BLOCKS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        ops.probe_read(src, sink)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        ops.probe_read(src, sink)
    e1.record()
    torch.cuda.synchronize()
    out["hbm"] = {"value": n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, "unit": "GB/s",
                  "how": "read-only streaming kernel (16-byte loads) over 2 GiB"}
    del src, sink
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    bt = b.t()  # [N, K] storage read as B^T: the layout of the library's weights
    for _ in range(3):
        torch.matmul(a, bt)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, bt)
    e1.record()
    torch.cuda.synchronize()
    out["mfma"] = {"value": 2 * m ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, "unit": "TFLOP/s",
                   "how": "torch.matmul (vendor library) bf16 8192 x 8192 x 8192, A B^T with B stored [N, K]"}
    del a, b
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- main

# HBM traffic of a kernel, from a committed rocprofv3 counter summary
# (profiles/<kernel>_<workload>_traffic.md): FETCH_SIZE and WRITE_SIZE per
# dispatch, scaled by what the same counters read for a plain device copy of
# known size. The record names the SHA-256 of the kernel's sources when the
# counters were taken; if the sources changed since, the figure is stale and
# traffic is reported as null.
KERNEL_SOURCES = {
    "decode_attn": ["decode.hip", "common.h"],
    "prefill_attn": ["attn_prefill.hip", "common.h"],
}


def kernel_source_sha(kernel: str):
    import hashlib
    files = KERNEL_SOURCES.get(kernel)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_mla_latent_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip().lstrip("-").strip()
            if ":" in line and not line.startswith("|"):
                k, v = line.split(":", 1)
                rec[k.strip().strip("`")] = v.strip().strip("`")
    if rec.get("source_sha256") != kernel_source_sha(kernel):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None

def time_region(torch, fn, n, first):
    """Mean ms per call of fn(first), ..., fn(first + n - 1), from events
    around the calls alone."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(n):
        fn(first + i)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n


def trace_region(torch, ops, fn, n, first):
    """Per-kernel launch counts and mean device times (us) over n calls, from
    the library's launch trace (events recorded by each kernel's dispatch)."""
    kern = {}
    ops.trace_begin(16 * n + 64)
    for i in range(n):
        fn(first + i)
    torch.cuda.synchronize()
    ops.trace_end()
    for k in ops.trace_kernels():
        cnt, ms = ops.trace_summary(k)
        kern[k] = {"launches_per_step": cnt / n, "avg_us": ms * 1e3}
    ops.trace_reset()
    return kern


def run_workload(name, args, torch, ops, W):
    """Time one workload; returns its record (value, unit, ms_per_step,
    config, roofline, kernels, cpu_baseline, ...)."""
    cfg_name, desc = WORKLOADS[name]
    log(f"[bench] {name}: generating ({desc})")
    inp = getattr(W, cfg_name)()
    is_decode = name.startswith("decode")
    step, keep = (build_decode if is_decode else build_prefill)(args, inp, torch, ops)

    log(f"[bench] {name}: warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1: the steps alone (this gives ms_per_step and value)
    t0 = time.perf_counter()
    ms_step = time_region(torch, step, args.steps, args.warmup)
    wall = (time.perf_counter() - t0) / args.steps
    log(f"[bench] {name}: {ms_step * 1e3:.1f} us/step (wall {wall * 1e6:.1f} us/step)")
    # timed region 2: the same steps again with the library's launch trace on;
    # the events add work to the stream, so the step time comes from region 1
    kern = {} if args.no_trace else trace_region(torch, ops, step, args.steps, args.warmup + args.steps)

    rec = {"workload": name, "ms_per_step": ms_step, "steps": args.steps, "warmup": args.warmup,
           "dtype": "f32" if name == "tiny_fp32" else "bf16"}
    if is_decode:
        # timed regions 3, 4: the step's input side alone, and the per-head
        # gate variant of its output side, each then with its kernels
        extra = {}
        for xname, fn in keep[1].items():
            for i in range(args.warmup):
                fn(i)
            us = time_region(torch, fn, args.steps, args.warmup) * 1e3
            log(f"[bench] {name}: {xname} {us:.1f} us")
            extra[xname] = (us, {} if args.no_trace else trace_region(torch, ops, fn, args.steps, 0))
        db = decode_bytes(inp)
        gb = gate_out_bytes(inp)
        gf = gate_out_flops(inp)
        alg = {"decode_attn": db["cache"] + db["q"] + db["out"], **gb}
        flops = {"decode_attn": decode_attn_flops(inp), **gf}
        step_bytes = sum(alg.values())
        rec.update({"value": inp.B / (ms_step * 1e-3), "unit": "tokens/s",
                    "config": {"workload": desc, "batch": inp.B, "heads": inp.H, "d_c": inp.d_c, "d_r": inp.d_r,
                               "cached_tokens": db["tokens"], "num_splits": args.num_splits or "auto",
                               "input_copies": args.copies},
                    "step_hbm_gbs": step_bytes / (ms_step * 1e-3) / 1e9,
                    "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS})
        for k, v in kern.items():
            if k in alg:
                v["alg_bytes"] = alg[k]
                v["gbs"] = alg[k] / (v["avg_us"] * 1e-6) / 1e9
                v["tflops"] = flops[k] / (v["avg_us"] * 1e-6) / 1e12
        if "decode_attn" in kern:
            # the roofline kernel: the attention over the latent cache (HBM-bound)
            a = alg["decode_attn"] / (kern["decode_attn"]["avg_us"] * 1e-6) / 1e9
            rec["roofline"] = {"bound": "hbm", "kernel": "decode_attn", "achieved": a, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": a / HBM_PEAK_GBS, "traffic": traffic_record("decode_attn", name),
                               "alg_bytes_per_launch": alg["decode_attn"],
                               "mfma_tflops": kern["decode_attn"]["tflops"],
                               "mfma_frac": kern["decode_attn"]["tflops"] / BF16_PEAK_TFLOPS}
        rec["kernels"] = kern
        if "decode_attn" in kern and "decode_combine" in kern:
            # the attention part of the step alone (latent-cache attention and
            # the split-L combine, per launch), as tokens/s for one layer
            t_att = sum(kern[k]["avg_us"] * kern[k]["launches_per_step"] for k in ("decode_attn", "decode_combine"))
            rec["attention_only"] = {"us": t_att, "tokens_per_s": inp.B / (t_att * 1e-6),
                                     "hbm_frac": (db["cache"] + db["q"] + db["out"]) / (t_att * 1e-6) / 1e9
                                     / HBM_PEAK_GBS}
        go_us = sum(kern[k]["avg_us"] for k in gb if k in kern)
        if go_us:
            rec["gate_out"] = {"us": go_us, "alg_bytes": sum(gb.values()),
                               "hbm_frac": sum(gb.values()) / (go_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        pb = prepare_bytes(inp)
        prep_us, prep_kern = extra["decode_prepare"]
        rec["decode_prepare"] = {"us": prep_us, "alg_bytes": pb, "hbm_gbs": pb / (prep_us * 1e-6) / 1e9,
                                 "hbm_frac": pb / (prep_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "d_k": DECODE_D_K,
                                 "kernels": prep_kern,
                                 "layer_us": ms_step * 1e3 + prep_us,
                                 "layer_tokens_per_s": inp.B / ((ms_step * 1e3 + prep_us) * 1e-6)}
        hb = head_gate_bytes(inp)
        hg_us, hg_kern = extra["head_gate_out"]
        rec["head_gate_out"] = {"us": hg_us, "alg_bytes": hb, "hbm_gbs": hb / (hg_us * 1e-6) / 1e9,
                                "hbm_frac": hb / (hg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "kernels": hg_kern,
                                "per_channel_gate_out_us": go_us}
        if not args.no_cpu_baseline:
            log(f"[bench] {name}: cpu baseline (fp64 oracle)")
            rec["cpu_baseline"] = cpu_baseline_decode(inp, args.cpu_seconds)
    else:
        fl = prefill_flops(inp)
        total = sum(fl.values())
        f32 = inp.dtype == torch.float32
        peak = F32_FMA_PEAK_TFLOPS if f32 else BF16_PEAK_TFLOPS
        rec.update({"value": total / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
                    "config": {"workload": desc, "batch": inp.B, "seq_len": inp.L, "heads": inp.H,
                               "gflop_per_step": total / 1e9, "input_copies": args.copies},
                    "step_peak_frac": total / (ms_step * 1e-3) / 1e12 / peak})
        # the projections of x may run as one grouped launch (gemm_input)
        kfl = dict(fl, gemm_input=sum(fl.get(k, 0) for k in ("gemm_latent", "gemm_query", "gemm_rope_key",
                                                              "gemm_rope_query")))
        for k, v in kern.items():
            if k in kfl:
                v["tflops"] = kfl[k] / (v["avg_us"] * 1e-6) / 1e12
        # the roofline kernel: the causal attention, one launch per step
        # (every GEMM of the step is listed under kernels with its TFLOP/s)
        rk = "prefill_attn_f32" if f32 else "prefill_attn"
        if rk in kern:
            a = fl["prefill_attn"] / (kern[rk]["avg_us"] * 1e-6) / 1e12
            rec["roofline"] = {"bound": "alu" if f32 else "mfma", "kernel": rk, "achieved": a, "peak": peak,
                               "unit": "TFLOP/s", "frac": a / peak, "traffic": traffic_record(rk, name),
                               "alg_flops_per_launch": fl["prefill_attn"]}
            if f32:
                rec["roofline"]["peak_how"] = "non-packed fp32 FMA: 256 CUs x 64 lanes x 2 flops x 2.4 GHz"
        gemm_us = sum(v["avg_us"] * v["launches_per_step"] for k, v in kern.items() if k.startswith("gemm"))
        if gemm_us:
            gemm_fl = sum(v for k, v in fl.items() if k.startswith("gemm"))
            rec["gemms"] = {"us": gemm_us, "tflops": gemm_fl / (gemm_us * 1e-6) / 1e12,
                            "frac": gemm_fl / (gemm_us * 1e-6) / 1e12 / peak}
        rec["kernels"] = kern
        if not args.no_cpu_baseline:
            log(f"[bench] {name}: cpu baseline (fp64 oracle)")
            rec["cpu_baseline"] = cpu_baseline_prefill(inp, args.cpu_seconds)
    del step, keep, inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU layout is described in the design notes, not benchmarked.", file=sys.stderr)
        sys.exit(2)
    import numpy as np  # noqa: F401
    import torch
    from gated_mla_latent_amd import ops, workloads as W
    from gated_mla_latent_amd.build import LIB_PATH, build
    if not os.path.exists(LIB_PATH):
        build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    names = ALL_WORKLOADS if args.workload == "all" else [args.workload]
    recs = {n: run_workload(n, args, torch, ops, W) for n in names}
    # measured reference peaks, after the workloads (their long library GEMM
    # would otherwise warm the GPU before the first workload is timed)
    if not args.no_measured_peak:
        log("[bench] measured reference peaks")
        peaks = measured_peaks(torch, ops)
        for rec in recs.values():
            roof = rec.get("roofline")
            if roof and roof["bound"] in peaks:
                roof["measured_peak"] = peaks[roof["bound"]]
                roof["frac_of_measured"] = roof["achieved"] / peaks[roof["bound"]]["value"]
    head = recs[HEADLINE] if HEADLINE in recs else recs[names[0]]
    out = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": head["dtype"],
           "data": "synthetic (seeded; random-init weights of the stated shapes)",
           "config": head["config"]}
    for k in ("roofline", "cpu_baseline", "kernels", "gemms", "step_peak_frac"):
        if k in head:
            out[k] = head[k]
    if len(recs) > 1:
        out["configs"] = recs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
