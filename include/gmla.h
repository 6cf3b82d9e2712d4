/*
 * gmla.h -- Gated Multi-head Latent Attention kernels for AMD Instinct MI355X
 * (gfx950). C ABI of libgmla.so.
 *
 * What the library computes (sources are web pages, cited by title and
 * section):
 *   [GF]  "Gated MLA 计算公式：输出门与 FFN 的区别" -- §一: each token caches a
 *         latent c_s = W_c x_s and every head reconstructs k = W_k^(h) c,
 *         v = W_v^(h) c; §二: per-head causal softmax attention over s <= t,
 *         head concatenation o~_t, and the per-channel output gate
 *         y_t = W_o [ Sigmoid(W_g x_t) (.) o~_t ]; NoPE in Kimi K3.
 *   [N03] "LLM 注意力与计算内核精读笔记 · 03 注意力头变体：MQA / GQA / MLA" --
 *         §5.1: W^UK folds into the query and W^UV moves past the weighted
 *         sum, so decode attends the latent directly, and the low-rank
 *         query c^Q = W^DQ x; §5.2: decoupled RoPE, a shared d_h^R-wide
 *         rotated key cached next to the latent.
 *   [CD]  "Gated Multi-head Latent Attention (Gated MLA)" (concept page) --
 *         Gating Mechanism, Mathematical Formulation: the per-head scalar
 *         gate g_h = Sigmoid(W_g x + b_g) scaling head h's output.
 *
 * Conventions shared by every entry point
 *   - Every tensor is dense and row-major (last index fastest). Weights use
 *     the [out_features, in_features] layout. Device pointers unless stated.
 *   - dtype GMLA_BF16: bf16 storage, fp32 accumulation, intermediates (c, q,
 *     K, V, P, o~, gated) rounded to bf16 (round to nearest even).
 *     dtype GMLA_F32: fp32 storage and true fp32 arithmetic throughout.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; nothing synchronises the host.
 *   - The caller owns every buffer. The library allocates no device memory in
 *     these calls and keeps no state between them (apart from the optional
 *     trace below). Scratch space is the caller's `workspace`, at least the
 *     size the matching *_workspace_size() returns, 256-byte aligned.
 *     Calls that share a workspace must not overlap in time.
 *   - Errors: arguments are checked on the host before anything is enqueued.
 *     A failed check returns a status != GMLA_OK and enqueues nothing.
 *     GMLA_ERR_HIP reports a HIP launch error. gmla_last_error() gives a
 *     human-readable reason for the calling thread's last failure.
 *     No function aborts or throws.
 *   - Every device pointer must be 16-byte aligned.
 */
#ifndef GMLA_H
#define GMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GMLA_OK = 0,
  GMLA_ERR_INVALID_ARG = 1, /* null pointer, misalignment, non-positive size */
  GMLA_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
  GMLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  GMLA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} gmla_status_t;

typedef enum { GMLA_F32 = 0, GMLA_BF16 = 1 } gmla_dtype_t;

/* ------------------------------------------------------------------------
 * Prefill: latent projection, explicit per-head K/V reconstruction and
 * causal attention ([GF] §一 and §二 first two equations), with an optional
 * low-rank query ([N03] §5.1: c^Q = W^DQ x, q = W^UQ c^Q) and optional
 * decoupled RoPE ([N03] §5.2).
 *
 *   x          [B, L, d_model]      input hidden states
 *   W_c        [d_c, d_model]       latent (down) projection
 *   W_dq       [d_cq, d_model]      low-rank query projection W^DQ, or NULL
 *                                   (d_cq == 0: the query side reads x)
 *   W_q        [H*d_k, d_in]        query projection (W^UQ with W_dq),
 *                                   head-major rows; d_in = d_cq or d_model
 *   W_kr       [d_r, d_model]       shared RoPE key projection, or NULL (d_r == 0)
 *   W_qr       [H*d_r, d_in]        per-head RoPE query projection, or NULL
 *   W_uk       [H, d_k, d_c]        per-head key up-projection
 *   W_uv       [H, d_v, d_c]        per-head value up-projection
 *   latent_out [B, L, d_c + d_r]    out: the cache rows [c_s ; RoPE(W_kr x_s, s)],
 *                                   c_s = W_c x_s
 *   o_tilde    [B, L, H*d_v]        out: o~_t = Concat_h o_t^(h), channel
 *                                   h*d_v + j; o_t^(h) = sum_{s<=t}
 *                                   softmax_s(sm_scale q_t^(h).k_s^(h)) v_s^(h)
 * With RoPE the score is q^C.k^C + RoPE(q^R, t).RoPE(k^R, s) (pairs
 * interleaved, theta_i = rope_base^(-2i/d_r); rope_base 0: unrotated).
 * The gate and output projection follow with gmla_gate_out(W_uv = NULL).
 * Sizes: all >= 1 (d_cq, d_r >= 0). BF16 needs d_model, d_c and d_cq
 * % 64 == 0, d_k == d_v in {64, 128} and d_r in {0, 64}; F32 needs
 * d_k <= 1024, d_v <= 512 and d_r == 0 (GMLA_ERR_UNSUPPORTED otherwise).
 * ---------------------------------------------------------------------- */
size_t gmla_prefill_workspace_size(int B, int L, int H, int d_cq, int d_k, int d_r, int d_v, gmla_dtype_t dtype);
gmla_status_t gmla_prefill(const void* x, const void* W_c, const void* W_dq, const void* W_q, const void* W_kr,
                           const void* W_qr, const void* W_uk, const void* W_uv, void* latent_out, void* o_tilde,
                           void* workspace, size_t workspace_bytes, int B, int L, int d_model, int H, int d_c,
                           int d_cq, int d_k, int d_r, int d_v, float sm_scale, float rope_base, gmla_dtype_t dtype,
                           void* stream);

/* ------------------------------------------------------------------------
 * Decode: one query token per sequence against the latent cache, with W_UK
 * already absorbed into the query ([N03] §5.1, exercise 4 answer) and an
 * optional decoupled RoPE part ([N03] §5.2).
 *
 *   q_abs     [B, H, d_c + d_r]  q~_h = (W_UK^(h))^T q_h, then the RoPE query
 *                                part (not yet rotated; rotated here to
 *                                position seq_len[b] - 1 unless rope_base == 0)
 *   cache     [rows, d_c + d_r]  row j = [c_j ; kR_j], kR_j already rotated
 *   seq_start [B] int64 (device) first cache row of sequence b
 *   seq_len   [B] int32 (device) L_b; rows seq_start[b] .. + L_b - 1
 *   o_lat     [B, H, d_c]        out: sum_j softmax_j(s) c_j with
 *                                s_j = sm_scale (q~_h . [c_j ; kR_j])
 *   lse       [B, H] fp32 or NULL  out: natural log of sum_j exp(s_j)
 * Every head shares one latent row per token (MQA-shaped), V is the latent
 * part c_j only. L_b >= 1 is required; a sequence with L_b <= 0 yields
 * o_lat = 0 and lse = -inf. The seq_* arrays are read on the device and
 * trusted (rows must lie inside `cache`).
 * num_splits (BF16): number of slices the concatenated token range of all
 * sequences is cut into, slices of equal cost where a token counts 1 and
 * the start of a nonempty sequence 384; each slice runs as ceil(H/64)
 * workgroups of up to 64 heads (one if H <= 32). 0 = automatic: compute
 * units / workgroups per slice, rounded down to a multiple of 8. F32 runs
 * one workgroup per sequence and head and ignores it.
 * The result does not depend on it beyond fp32 rounding.
 * BF16 with d_c == 512 and d_r in {0, 64} runs the MFMA kernel described
 * above; every other BF16 width with d_c % 64 == 0, d_c <= 512 and
 * d_c + d_r <= 1024 runs a generic kernel (one workgroup per sequence and
 * head, fp32 arithmetic, no workspace; num_splits ignored), as does F32
 * (d_c + d_r <= 1024, d_c <= 512). GMLA_ERR_UNSUPPORTED otherwise.
 * ---------------------------------------------------------------------- */
/* Workspace bytes: 0 for F32 and for BF16 with d_c != 512. */
size_t gmla_decode_workspace_size(int B, int H, int d_c, int num_splits, gmla_dtype_t dtype);
gmla_status_t gmla_decode(const void* q_abs, const void* cache, const int64_t* seq_start, const int32_t* seq_len,
                          void* o_lat, float* lse, void* workspace, size_t workspace_bytes, int B, int H, int d_c,
                          int d_r, float rope_base, float sm_scale, int num_splits, gmla_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Decode without allocation: gmla_decode for callers that cannot allocate
 * device memory or pass a workspace -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The arguments, checks,
 * kernels and results are those of gmla_decode (bit-identical for the same
 * num_splits); the split-L scratch (cost offsets and partial outputs) lives
 * in a library-owned static device array of GMLA_DECODE_SCRATCH_BYTES per
 * GPU, held by each GPU the library runs on until the process ends. No
 * device memory is allocated by the call. A call whose scratch need
 * (gmla_decode_workspace_size) exceeds GMLA_DECODE_SCRATCH_BYTES returns
 * GMLA_ERR_UNSUPPORTED and enqueues nothing (the automatic slice count fits
 * for every batch up to ~2^20 sequences with d_c = 512). Every call on a GPU
 * shares that GPU's array and leaves its contents behind (nothing in it
 * needs to start at zero): calls that overlap in time on one GPU, e.g. on
 * two streams, race on it and must be serialised by the caller.
 * ---------------------------------------------------------------------- */
#define GMLA_DECODE_SCRATCH_BYTES (48u << 20)
gmla_status_t gmla_decode_noalloc(const void* q_abs, const void* cache, const int64_t* seq_start,
                                  const int32_t* seq_len, void* o_lat, float* lse, int B, int H, int d_c, int d_r,
                                  float rope_base, float sm_scale, int num_splits, gmla_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Decode-step projections: the new token's cache row and its absorbed query,
 * the inputs of gmla_decode ([N03] §5.1 and exercise 4 answer for the
 * absorbed query, §5.2 for the decoupled RoPE key that is rotated once and
 * cached, the query's RoPE part being rotated by the attention).
 *
 *   x         [B, d_model]          hidden state of each sequence's new token
 *   W_c       [d_c, d_model]        latent (down) projection
 *   W_kr      [d_r, d_model]        shared RoPE key projection (NULL if d_r == 0)
 *   W_dq      [d_cq, d_model]       low-rank query projection W^DQ ([N03] §5.1),
 *                                   or NULL (d_cq == 0: the query side reads x)
 *   W_q       [H*d_k, d_in]         query projection (W^UQ with W_dq),
 *                                   head-major rows; d_in = d_cq or d_model
 *   W_qr      [H*d_r, d_in]         per-head RoPE query projection (NULL if d_r == 0)
 *   W_uk      [H, d_k, d_c]         per-head key up-projection
 *   cache     [rows, d_c + d_r]     in/out: row seq_start[b] + seq_len[b] is
 *                                   set to [W_c x_b ; RoPE(W_kr x_b, seq_len[b])];
 *                                   no other row is touched
 *   seq_start [B] int64 (device), seq_len [B] int32 (device): cached tokens
 *                                   before this step; not modified (the caller
 *                                   adds 1 before gmla_decode, which then
 *                                   rotates the query to position seq_len[b])
 *   q_abs     [B, H, d_c + d_r]     out: [(W_UK^(h))^T q_h ; W_qr^(h) u_b],
 *                                   q_h = W_q^(h) u_b with u_b = W_dq x_b (or
 *                                   x_b), the RoPE part unrotated
 * RoPE pairs are interleaved (2i, 2i+1), theta_i = rope_base^(-2i/d_r);
 * rope_base == 0 leaves the key unrotated. The target rows must lie inside
 * `cache` and differ between sequences (trusted, read on the device).
 * The workspace holds the projections of x before the append and the absorb.
 * Only GMLA_BF16 is supported (GMLA_ERR_UNSUPPORTED otherwise); it needs
 * d_model, d_c and d_cq % 64 == 0, d_k % 16 == 0, d_k <= 128 and
 * d_r % 4 == 0.
 * ---------------------------------------------------------------------- */
size_t gmla_decode_prepare_workspace_size(int B, int d_model, int H, int d_c, int d_cq, int d_k, int d_r,
                                          gmla_dtype_t dtype);
gmla_status_t gmla_decode_prepare(const void* x, const void* W_c, const void* W_kr, const void* W_dq, const void* W_q,
                                  const void* W_qr, const void* W_uk, void* cache, const int64_t* seq_start,
                                  const int32_t* seq_len, void* q_abs, void* workspace, size_t workspace_bytes, int B,
                                  int d_model, int H, int d_c, int d_cq, int d_k, int d_r, float rope_base,
                                  gmla_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Gate and output projection ([GF] §二 boxed equation):
 *   y_t = W_o [ Sigmoid(W_g x_t) (.) o~_t ]
 * With W_uv == NULL, `o` is o~ [T, H*d_v] (prefill output). With W_uv given,
 * `o` is the decode output o_lat [T, H, d_c] and o~_h = W_uv[h] o_lat_h is
 * formed first (W_UV moved to the output side, [N03] §5.1; it cannot be
 * pre-multiplied into W_o because the gate between them is per channel).
 *   x [T, d_model], W_g [H*d_v, d_model], W_o [d_model, H*d_v], y [T, d_model]
 * BF16 needs d_model % 64 == 0, (H*d_v) % 64 == 0, d_c % 64 == 0 and
 * d_v % 4 == 0. At decode sizes (bf16, T <= 64, d_c == 512, an unsplit
 * gate GEMM) the gate GEMM's workgroups form the o~ columns they gate from
 * o_lat and W_uv themselves. The workspace holds gated (and o~ when W_uv is
 * given, used when o~ is formed by a GEMM of its own) and,
 * for T <= 64 with bf16, the fp32 partial sums of GEMMs whose K is split
 * across workgroups; its size depends on every argument of the size query
 * (d_c is ignored without the value up-projection).
 * ---------------------------------------------------------------------- */
size_t gmla_gate_out_workspace_size(int T, int d_model, int H, int d_c, int d_v, int with_value_up,
                                    gmla_dtype_t dtype);
gmla_status_t gmla_gate_out(const void* x, const void* o, const void* W_uv, const void* W_g, const void* W_o,
                            void* y, void* workspace, size_t workspace_bytes, int T, int d_model, int H, int d_c,
                            int d_v, gmla_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Per-head scalar gate and output projection ("Gated Multi-head Latent
 * Attention (Gated MLA)" concept page [CD], Gating Mechanism and
 * Mathematical Formulation):
 *   g_t = Sigmoid(W_g x_t + b_g) in R^H,  y_t = W_o [ g_t[h] o~_t^(h) ]_h
 * head h's output block (channels h*d_v .. h*d_v + d_v - 1) scaled by one
 * scalar. `o` and W_uv as in gmla_gate_out (W_uv given: `o` is o_lat
 * [T, H, d_c] and o~_h = W_uv[h] o_lat_h first).
 *   x [T, d_model], W_g [H, d_model], b_g [H] or NULL (zero),
 *   W_o [d_model, H*d_v], y [T, d_model]
 * The logits x W_g^T are rounded to bf16 before the bias and the sigmoid.
 * Only GMLA_BF16 (GMLA_ERR_UNSUPPORTED otherwise); it needs
 * d_model % 64 == 0, (H*d_v) % 64 == 0, d_v % 8 == 0, H % 4 == 0 and, with
 * W_uv, d_c % 64 == 0. Workspace: 256-byte aligned, the size below.
 * ---------------------------------------------------------------------- */
size_t gmla_head_gate_out_workspace_size(int T, int d_model, int H, int d_c, int d_v, int with_value_up,
                                         gmla_dtype_t dtype);
gmla_status_t gmla_head_gate_out(const void* x, const void* o, const void* W_uv, const void* W_g, const void* b_g,
                                 const void* W_o, void* y, void* workspace, size_t workspace_bytes, int T, int d_model,
                                 int H, int d_c, int d_v, gmla_dtype_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics
 * ---------------------------------------------------------------------- */
const char* gmla_status_string(gmla_status_t status);
/* Reason for the calling thread's most recent failure ("" if none). */
const char* gmla_last_error(void);
/* Library version as 10000*major + 100*minor + patch. */
int gmla_version(void);

/* Read-bandwidth probe: streams `bytes` (a multiple of 16) of the device
 * buffer `src` with 16-byte loads in GMLA_PROBE_BLOCKS workgroups, each of
 * which writes one 32-bit word to `sink` (device, at least
 * GMLA_PROBE_BLOCKS * 4 bytes), so that no load can be dropped. Not part
 * of the attention path: the benchmark times it to measure the read-only
 * HBM rate that the bandwidth-bound kernels are compared against. */
#define GMLA_PROBE_BLOCKS 2048
gmla_status_t gmla_probe_read(const void* src, size_t bytes, void* sink, void* stream);

/* Kernel trace: while enabled, every kernel the library enqueues is bracketed
 * by a pair of HIP events recorded on the same stream, so per-kernel device
 * time can be read back without a profiler. gmla_trace_begin creates up to
 * max_launches event pairs (host-side HIP objects) and starts recording;
 * launches beyond that are not traced. gmla_trace_end stops recording.
 * gmla_trace_summary waits for the recorded events and returns, for kernel
 * `name`, the number of traced launches and their mean duration in
 * milliseconds (count 0 if none). gmla_trace_reset drops all records and
 * destroys the events. Not for concurrent use from several threads. */
gmla_status_t gmla_trace_begin(int max_launches);
gmla_status_t gmla_trace_end(void);
gmla_status_t gmla_trace_summary(const char* name, int* count, double* mean_ms);
/* Names of the kernels seen so far, separated by ';' (valid until the next
 * trace call). */
const char* gmla_trace_kernels(void);
void gmla_trace_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* GMLA_H */
