"""Host-side checks of libgmla.so (no GPU needed): the library loads, exports
every function include/gmla.h declares, and rejects bad arguments with the
documented status before anything reaches the GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from gated_mla_latent_amd import build, ops
    if not os.path.exists(ops.LIB_PATH):
        build.build()
    return ops.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "gmla.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gmla_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.gmla_status_string(0) == b"ok"
    assert L.gmla_status_string(3) == b"workspace too small"
    assert L.gmla_version() >= 10000


OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
A = 0x100000  # an aligned fake device address; never dereferenced (validation fails first)


def _dec(L, **kw):
    a = dict(q=A, cache=A, start=A, len_=A, o=A, lse=0, ws=A, wsb=1 << 40, B=4, H=64, d_c=512, d_r=0,
             base=10000.0, scale=0.1, splits=8, dt=1)
    a.update(kw)
    return L.gmla_decode(a["q"], a["cache"], a["start"], a["len_"], a["o"], a["lse"], a["ws"], a["wsb"], a["B"],
                         a["H"], a["d_c"], a["d_r"], a["base"], a["scale"], a["splits"], a["dt"], None)


def test_decode_argument_checks(L):
    assert _dec(L, q=0) == INVALID
    assert _dec(L, cache=A + 8) == INVALID          # misaligned
    assert _dec(L, B=0) == INVALID
    assert _dec(L, d_r=3) == INVALID                # odd RoPE width
    assert _dec(L, splits=-1) == INVALID
    assert _dec(L, scale=float("nan")) == INVALID
    assert _dec(L, base=-1.0) == INVALID
    assert _dec(L, dt=7) == INVALID
    assert _dec(L, d_c=96) == UNSUPPORTED           # bf16 latent widths are multiples of 64 ...
    assert _dec(L, d_c=576) == UNSUPPORTED          # ... up to 512
    assert _dec(L, d_c=512, d_r=600) == UNSUPPORTED  # d_c + d_r <= 1024
    assert _dec(L, wsb=16) == WORKSPACE
    assert _dec(L, ws=0) == WORKSPACE
    assert b"workspace" in L.gmla_last_error()
    assert _dec(L, ws=A + 16) == INVALID            # workspace must be 256-byte aligned


def test_decode_noalloc_refuses_scratch_past_its_size(L):
    """The no-allocation decode refuses, before any HIP call, a request whose
    workspace would exceed the library's static scratch."""
    args = lambda B, H, splits: (A, A, A, A, A, 0, B, H, 512, 64, 10000.0, 0.1, splits, 1, None)
    big = L.gmla_decode_workspace_size(64, 128, 512, 65535, 1)
    assert big > 48 << 20
    assert L.gmla_decode_noalloc(*args(64, 128, 65535)) == UNSUPPORTED
    assert b"scratch" in L.gmla_last_error()
    assert L.gmla_decode_noalloc(*args(0, 128, 0)) == INVALID


def test_decode_workspace_size_formula(L):
    B, H, d_c, G = 4, 64, 512, 8
    up = lambda n: (n + 255) // 256 * 256
    assert L.gmla_decode_workspace_size(B, H, d_c, G, 1) == up(B * 8) + up(2 * G * H * 4) + up(2 * G * H * d_c * 2)
    # partial outputs are padded to whole groups of 16 heads
    assert L.gmla_decode_workspace_size(B, 20, d_c, G, 1) == up(B * 8) + up(2 * G * 20 * 4) + up(2 * G * 32 * d_c * 2)
    assert L.gmla_decode_workspace_size(B, H, d_c, G, 0) == 0  # fp32 path needs none
    assert L.gmla_decode_workspace_size(B, H, 256, G, 1) == 0  # nor the generic bf16 path
    assert L.gmla_decode_workspace_size(0, H, d_c, G, 1) == 0


def test_prefill_workspace_size_formula(L):
    up = lambda n: (n + 255) // 256 * 256
    for B, Lq, H, d in [(2, 100, 3, 64), (1, 8192, 64, 128), (3, 64, 1, 128)]:
        T, Lp = B * Lq, (Lq + 63) // 64 * 64
        # bf16: q and K as [T, H d], V transposed per sequence as [B, H d, Lp]
        assert L.gmla_prefill_workspace_size(B, Lq, H, 0, d, 0, d, 1) == 2 * up(T * H * d * 2) + up(B * H * d * Lp * 2)
        assert L.gmla_prefill_workspace_size(B, Lq, H, 0, d, 0, d, 0) == 3 * up(T * H * d * 4)
        # q then the RoPE queries [T, H (d + d_r)], K, V^T, then c^Q [T, d_cq]
        assert (L.gmla_prefill_workspace_size(B, Lq, H, 192, d, 64, d, 1) ==
                up(T * H * (d + 64) * 2) + up(T * H * d * 2) + up(B * H * d * Lp * 2) + up(T * 192 * 2))
    assert L.gmla_prefill_workspace_size(0, 16, 2, 0, 64, 0, 64, 1) == 0


def _pre(L, **kw):
    a = dict(x=A, Wc=A, Wdq=0, Wq=A, Wkr=0, Wqr=0, Wuk=A, Wuv=A, lat=A, ot=A, ws=A, wsb=1 << 40, B=1, Lq=16, D=256,
             H=2, d_c=128, d_cq=0, d_k=128, d_r=0, d_v=128, scale=0.1, base=0.0, dt=1)
    a.update(kw)
    return L.gmla_prefill(a["x"], a["Wc"], a["Wdq"], a["Wq"], a["Wkr"], a["Wqr"], a["Wuk"], a["Wuv"], a["lat"], a["ot"],
                          a["ws"], a["wsb"], a["B"], a["Lq"], a["D"], a["H"], a["d_c"], a["d_cq"], a["d_k"], a["d_r"],
                          a["d_v"], a["scale"], a["base"], a["dt"], None)


def test_prefill_argument_checks(L):
    assert _pre(L, Wq=0) == INVALID
    assert _pre(L, x=A + 2) == INVALID
    assert _pre(L, Lq=0) == INVALID
    assert _pre(L, D=100) == UNSUPPORTED            # bf16 needs d_model % 64 == 0
    assert _pre(L, d_c=96) == UNSUPPORTED
    assert _pre(L, d_k=96, d_v=96) == UNSUPPORTED
    assert _pre(L, d_k=128, d_v=64) == UNSUPPORTED
    assert _pre(L, d_v=2048, d_k=2048, dt=0) == UNSUPPORTED
    assert _pre(L, Wdq=A) == INVALID                # W_dq without d_cq
    assert _pre(L, d_cq=64) == INVALID              # d_cq without W_dq
    assert _pre(L, Wdq=A, d_cq=96) == UNSUPPORTED   # bf16 needs d_cq % 64 == 0
    assert _pre(L, d_r=64) == INVALID               # d_r without W_kr / W_qr
    assert _pre(L, Wkr=A, d_r=64) == INVALID
    assert _pre(L, Wkr=A, Wqr=A, d_r=63) == INVALID
    assert _pre(L, Wkr=A, Wqr=A, d_r=32) == UNSUPPORTED      # bf16 RoPE prefill: d_r == 64
    assert _pre(L, Wkr=A, Wqr=A, d_r=64, dt=0) == UNSUPPORTED  # ... and bf16 only
    assert _pre(L, base=-1.0) == INVALID
    assert _pre(L, wsb=100) == WORKSPACE
    assert _pre(L, Wdq=A, d_cq=64, wsb=L.gmla_prefill_workspace_size(1, 16, 2, 0, 128, 0, 128, 1)) == WORKSPACE
    need = L.gmla_prefill_workspace_size(1, 16, 2, 0, 128, 0, 128, 1)
    assert need == 2 * 16 * 2 * 128 * 2 + 2 * 128 * 64 * 2  # q, K, and V^T padded to 64 keys


def test_prefill_rejects_token_counts_past_int(L):
    """B * L is a GEMM row count: a product past INT_MAX (with widths small
    enough for the 2^40 element bound) is rejected, not wrapped."""
    kw = dict(D=64, H=1, d_c=64, d_k=64, d_v=64, dt=0)
    assert _pre(L, B=2, Lq=1 << 30, **kw) == UNSUPPORTED
    assert b"INT_MAX" in L.gmla_last_error()
    assert _pre(L, B=1 << 16, Lq=1 << 15, **kw) == UNSUPPORTED
    assert _pre(L, B=1 << 15, Lq=1 << 16, **{**kw, "dt": 1}) == UNSUPPORTED


def _prep(L, **kw):
    a = dict(x=A, Wc=A, Wkr=A, Wdq=0, Wq=A, Wqr=A, Wuk=A, cache=A, start=A, len_=A, q=A, ws=A, wsb=1 << 40, B=4,
             D=256, H=16, d_c=512, d_cq=0, d_k=128, d_r=64, base=10000.0, dt=1)
    a.update(kw)
    return L.gmla_decode_prepare(a["x"], a["Wc"], a["Wkr"], a["Wdq"], a["Wq"], a["Wqr"], a["Wuk"], a["cache"],
                                 a["start"], a["len_"], a["q"], a["ws"], a["wsb"], a["B"], a["D"], a["H"], a["d_c"],
                                 a["d_cq"], a["d_k"], a["d_r"], a["base"], a["dt"], None)


def test_decode_prepare_argument_checks(L):
    assert _prep(L, Wq=0) == INVALID
    assert _prep(L, Wkr=0) == INVALID               # d_r > 0 needs the RoPE projections
    assert _prep(L, Wkr=0, Wqr=0, d_r=0, wsb=0) == WORKSPACE  # ... d_r == 0 does not
    assert _prep(L, cache=A + 4) == INVALID
    assert _prep(L, B=0) == INVALID
    assert _prep(L, d_r=3) == INVALID
    assert _prep(L, base=float("inf")) == INVALID
    assert _prep(L, dt=0) == UNSUPPORTED            # bf16 only
    assert _prep(L, D=200) == UNSUPPORTED
    assert _prep(L, d_c=96) == UNSUPPORTED
    assert _prep(L, d_k=256) == UNSUPPORTED
    assert _prep(L, d_k=24) == UNSUPPORTED
    assert _prep(L, d_r=2) == UNSUPPORTED
    assert _prep(L, wsb=100) == WORKSPACE
    assert _prep(L, ws=A + 16) == INVALID           # workspace must be 256-byte aligned
    assert _prep(L, Wdq=A) == INVALID                # W_dq without d_cq
    assert _prep(L, d_cq=128) == INVALID             # d_cq without W_dq
    assert _prep(L, Wdq=A, d_cq=100) == UNSUPPORTED


def _sk_first(grp, chunks, tot, wgs):
    return -(-((grp * chunks + 1) * wgs) // tot) - 1


def _sk_last(grp, chunks, tot, wgs):
    return -(-((grp + 1) * chunks * wgs) // tot) - 1


def _shared_even(N, K):
    """Even shares of the (128-column group, 128-wide K chunk) space over up
    to 256 workgroups of at least 8 chunks: (workgroups, slots), slots = the
    most workgroups whose shares touch one group."""
    G, C = -(-N // 128), K // 128
    tot = G * C
    w = min(tot // 8, 256)
    if w <= G:
        return 0, 1
    return w, max(_sk_last(g, C, tot, w) - _sk_first(g, C, tot, w) + 1 for g in range(G))


def _ksplit(M, N, K, batches):
    """The documented split-K rule of the skinny GEMM (M <= 64).
    33..64 rows with K a multiple of 128, K >= 2048, at least 32 workgroups
    of 128 columns and fewer than 256 of 64 columns take the
    shared-activation form: workgroups of 128 columns; one batch shares the
    (column group, K chunk) space evenly over up to 256 workgroups (the
    partial-sum slices are the most workgroups touching one group), several
    batches split each group towards 256 workgroups with at least eight
    128-wide K chunks per slice. Otherwise: split when the grid has fewer
    than 64 workgroups of 32 columns, towards 256 workgroups, keeping at
    least four 64-wide K chunks per workgroup. Never an empty slice."""
    if M > 64:
        return 1
    groups = -(-N // 128) * batches
    if 32 < M and K % 128 == 0 and K >= 2048 and groups >= 32 and -(-N // 64) * batches < 256:
        if batches == 1:
            return _shared_even(N, K)[1]
        z = min(256 // groups, K // 128 // 8)
        if z <= 1:
            return 1
        per = -(-(K // 128) // z)
        return -(-(K // 128) // per)
    wgs = (N + 31) // 32 * batches
    if wgs >= 64:
        return 1
    z = min(-(-256 // wgs), K // 64 // 4)
    if z <= 1:
        return 1
    per = -(-(K // 64) // z)
    return -(-(K // 64) // per)


def _part(M, N, K, batches=1):
    z = _ksplit(M, N, K, batches)
    return z * batches * M * ((N + 3) // 4 * 4) * 4 if z > 1 else 0


def test_split_k_rule_examples():
    assert _ksplit(64, 512, 7168, 1) == 16      # narrow: 16 workgroups of 32 columns -> 256
    assert _ksplit(64, 128, 7168, 1) == 28      # 4 workgroups, capped at 4 chunks of 64 each
    assert _ksplit(64, 64, 7168, 1) == 28
    assert _ksplit(64, 4096, 7168, 1) == 7      # shared form: 32 groups x 56 chunks over 224 workgroups of 8
    assert _ksplit(64, 16384, 7168, 1) == 1     # 256 workgroups of 64 columns already
    assert _shared_even(7168, 16384) == (256, 6)  # W_o at 64 rows: 56 groups x 128 chunks, 28 per workgroup
    assert _ksplit(64, 7168, 16384, 1) == 6
    assert _ksplit(32, 7168, 16384, 1) == 1     # 32 rows: 224 workgroups of 32 columns, not split
    assert _ksplit(64, 128, 512, 128) == 1      # batched value up-projection: short K, 512 workgroups
    assert _ksplit(65, 512, 7168, 1) == 1       # tile kernel, no split


@pytest.mark.parametrize("N,K", [(7168, 16384), (4096, 7168), (4160, 7168), (7168, 8192), (5120, 2048),
                                 (8064, 4096), (16256, 2048)])
def test_shared_even_shares_cover_every_chunk_once(N, K):
    """The even-share plan of the shared-activation GEMM, as the kernel walks
    it: workgroup w takes items [w T / W, (w + 1) T / W) and writes each
    piece to slot w - sk_first(group); the reduce reads slots 0 ..
    sk_last - sk_first of the group. Every (group, chunk) item is covered
    once, every slot the reduce reads is written exactly once, and no slot
    reaches past the planned slice count."""
    G, C = -(-N // 128), K // 128
    tot = G * C
    w, slots = _shared_even(N, K)
    assert w > G and w <= 256 and tot // w >= 8
    seen = [0] * tot
    written = {}
    for wg in range(w):
        lo, hi = wg * tot // w, (wg + 1) * tot // w
        assert hi > lo
        while lo < hi:
            grp = lo // C
            end = min(hi, (grp + 1) * C)
            slot = wg - _sk_first(grp, C, tot, w)
            assert 0 <= slot < slots
            assert (grp, slot) not in written
            written[(grp, slot)] = wg
            for it in range(lo, end):
                seen[it] += 1
            lo = end
    assert all(c == 1 for c in seen)
    for grp in range(G):
        n = _sk_last(grp, C, tot, w) - _sk_first(grp, C, tot, w) + 1
        assert n <= slots
        assert all((grp, s) in written for s in range(n))
        assert not any((grp, s) in written for s in range(n, slots))


def test_decode_prepare_workspace_size_formula(L):
    up = lambda n: (n + 255) // 256 * 256
    for B, D, H, d_c, d_cq, d_k, d_r in [(4, 256, 16, 512, 0, 128, 64), (37, 7168, 128, 512, 0, 128, 0),
                                         (1, 192, 3, 64, 0, 32, 4), (64, 7168, 128, 512, 1536, 128, 64)]:
        # new cache rows [B, d_c + d_r], queries [B, H d_k], RoPE queries [B, H d_r], c^Q [B, d_cq]
        want = up(B * (d_c + d_r) * 2) + up(B * H * d_k * 2) + up(B * H * d_r * 2) + up(B * d_cq * 2)
        assert L.gmla_decode_prepare_workspace_size(B, D, H, d_c, d_cq, d_k, d_r, 1) == want
    assert L.gmla_decode_prepare_workspace_size(4, 256, 16, 512, 0, 128, 64, 0) == 0
    assert L.gmla_decode_prepare_workspace_size(0, 256, 16, 512, 0, 128, 64, 1) == 0


def test_gate_out_workspace_size_formula(L):
    up = lambda n: (n + 255) // 256 * 256
    for T, D, H, d_c, d_v, vu in [(4, 256, 2, 512, 64, 1), (32, 7168, 64, 512, 128, 1), (64, 7168, 128, 512, 128, 1),
                                  (8, 7168, 128, 512, 128, 1), (16384, 7168, 1, 0, 8192, 0)]:
        HV = H * d_v
        part = max(_part(T, HV, D), _part(T, D, HV), _part(T, d_v, d_c, H) if vu else 0)
        want = (2 if vu else 1) * up(T * HV * 2) + up(part)
        assert L.gmla_gate_out_workspace_size(T, D, H, d_c, d_v, vu, 1) == want
    assert L.gmla_gate_out_workspace_size(4, 256, 2, 64, 64, 1, 0) == 2 * up(4 * 2 * 64 * 4)  # fp32: no split
    assert L.gmla_gate_out_workspace_size(4, 256, 2, 0, 64, 1, 1) == 0  # value up-projection needs d_c


def _gate(L, **kw):
    a = dict(x=A, o=A, Wuv=0, Wg=A, Wo=A, y=A, ws=A, wsb=1 << 40, T=4, D=256, H=2, d_c=0, d_v=64, dt=1)
    a.update(kw)
    return L.gmla_gate_out(a["x"], a["o"], a["Wuv"], a["Wg"], a["Wo"], a["y"], a["ws"], a["wsb"], a["T"], a["D"],
                           a["H"], a["d_c"], a["d_v"], a["dt"], None)


def test_gate_out_argument_checks(L):
    assert _gate(L, Wg=0) == INVALID
    assert _gate(L, T=0) == INVALID
    assert _gate(L, Wuv=A, d_c=0) == INVALID
    assert _gate(L, D=200) == UNSUPPORTED
    assert _gate(L, Wuv=A, d_c=100) == UNSUPPORTED
    assert _gate(L, wsb=10) == WORKSPACE


def _hg(L, **kw):
    a = dict(x=A, o=A, Wuv=0, Wg=A, bg=0, Wo=A, y=A, ws=A, wsb=1 << 40, T=4, D=256, H=4, d_c=0, d_v=64, dt=1)
    a.update(kw)
    return L.gmla_head_gate_out(a["x"], a["o"], a["Wuv"], a["Wg"], a["bg"], a["Wo"], a["y"], a["ws"], a["wsb"],
                                a["T"], a["D"], a["H"], a["d_c"], a["d_v"], a["dt"], None)


def test_head_gate_out_argument_checks_and_workspace(L):
    assert _hg(L, Wg=0) == INVALID
    assert _hg(L, bg=A + 2) == INVALID              # misaligned bias
    assert _hg(L, Wuv=A, d_c=0) == INVALID
    assert _hg(L, dt=0) == UNSUPPORTED              # bf16 only
    assert _hg(L, H=3) == UNSUPPORTED               # H % 4
    assert _hg(L, d_v=60, H=16) == UNSUPPORTED      # d_v % 8
    assert _hg(L, wsb=10) == WORKSPACE
    assert _hg(L, ws=A + 16) == INVALID             # workspace must be 256-byte aligned
    up = lambda n: (n + 255) // 256 * 256
    for T, D, H, d_c, d_v, vu in [(4, 256, 4, 0, 64, 0), (32, 1024, 64, 512, 128, 1), (300, 256, 4, 0, 128, 0)]:
        HV = H * d_v
        part = max(_part(T, H, D), _part(T, D, HV), _part(T, d_v, d_c, H) if vu else 0)
        want = (2 if vu else 1) * up(T * HV * 2) + up(T * H * 2) + up(part)
        assert L.gmla_head_gate_out_workspace_size(T, D, H, d_c, d_v, vu, 1) == want
    assert L.gmla_head_gate_out_workspace_size(4, 256, 4, 0, 64, 0, 0) == 0


def test_trace_api_without_launches(L):
    assert L.gmla_trace_begin(0) == INVALID
    n, ms = C.c_int(5), C.c_double(1.0)
    assert L.gmla_trace_summary(b"decode_attn", C.byref(n), C.byref(ms)) == OK
    assert n.value == 0 and ms.value == 0.0
    L.gmla_trace_reset()
