// C-ABI layer of libgmla: argument checks, workspace layout, dispatch to the
// kernels, and the optional per-kernel event trace. See include/gmla.h.
#include "../../include/gmla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

namespace gmla {
thread_local LaunchEvents* g_launch_events = nullptr;
}
using namespace gmla;

namespace {

thread_local std::string g_err;

gmla_status_t fail(gmla_status_t s, const std::string& msg) {
  g_err = msg;
  return s;
}
gmla_status_t ok() {
  g_err.clear();
  return GMLA_OK;
}
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }
size_t esize(gmla_dtype_t dt) { return dt == GMLA_F32 ? 4 : 2; }

#define REQUIRE(cond, status, msg) \
  do {                             \
    if (!(cond)) return fail(status, msg); \
  } while (0)

// ---------------------------------------------------------------- trace
struct TraceRec {
  const char* name;
  LaunchEvents ev;
};
std::mutex g_tr_mu;
bool g_tr_on = false;
std::vector<TraceRec> g_tr;
int g_tr_used = 0;
std::string g_tr_names;

// A traced call hands its event pair to launch() (which has the kernel's
// dispatch record it) through g_launch_events; a call that launched nothing
// leaves launched == 0 and is left out of the summary.
int trace_pre(const char* name, hipStream_t) {
  if (!g_tr_on) return -1;
  std::lock_guard<std::mutex> lk(g_tr_mu);
  if (g_tr_used >= (int)g_tr.size()) return -1;
  const int i = g_tr_used++;
  g_tr[i].name = name;
  g_tr[i].ev.launched = 0;
  g_launch_events = &g_tr[i].ev;
  return i;
}
void trace_post(int, hipStream_t) { g_launch_events = nullptr; }

template <class F>
gmla_status_t run(const char* name, hipStream_t st, F&& f) {
  const int tr = trace_pre(name, st);
  hipError_t e = f();
  trace_post(tr, st);
  if (e != hipSuccess) return fail(GMLA_ERR_HIP, std::string(name) + ": " + hipGetErrorString(e));
  return GMLA_OK;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// Slices of the token range: the caller's count, or one workgroup per compute
// unit counting every head chunk (a multiple of 8 so each XCD gets equal work).
// The decode kernel slices the flattened tokens by cost, counting a
// sequence start as this many tokens: a workgroup whose slice holds the
// start of a sequence runs a second segment (its query loads, first DMA
// round trip, softmax exchanges and output stores). Measured on the NoPE
// B=32 H=64 workload (attention + combine): 50.5 us at 0 (slices of equal
// tokens), 48.5 at 128, 45.0 at 256, 43.8 at 384, 43.9 at 512 and 768;
// at RoPE B=64 H=128 187 us at 0 and 180 at 384; no change at B=8, where
// sequence starts are few.
constexpr int kDecodeSegCost = 384;

int decode_slices(int num_splits, int H) {
  if (num_splits > 0) return num_splits;
  const int g = device_cus() / decode_head_chunks(H);
  return g >= 16 ? g / 8 * 8 : (g > 0 ? g : 1);
}

GemmArgs gemm(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int M, int N, int K,
              int epi = EPI_STORE, const void* O = nullptr, int64_t ldo = 0) {
  GemmArgs g{};
  g.A = (const bf16*)A; g.W = (const bf16*)W; g.C = (bf16*)C; g.O = (const bf16*)O;
  g.M = M; g.N = N; g.K = K; g.batches = 1;
  g.lda = lda; g.ldw = ldw; g.ldc = ldc; g.ldo = ldo;
  g.epi = epi;
  return g;
}
// Give a bf16 GEMM its split-K plan and partial-sum space (shared by the
// GEMMs of one call, which run one after another on its stream).
GemmArgs with_split(GemmArgs g, void* part) {
  g.ksplit = gemm_ksplit(g.M, g.N, g.K, g.batches, g.npad);
  g.part = g.ksplit > 1 ? (float*)part : nullptr;
  return g;
}

GemmF32Args gemm32(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int M, int N, int K,
                   int epi = EPI_STORE, const void* O = nullptr, int64_t ldo = 0) {
  GemmF32Args g{};
  g.A = (const float*)A; g.W = (const float*)W; g.C = (float*)C; g.O = (const float*)O;
  g.M = M; g.N = N; g.K = K; g.batches = 1;
  g.lda = lda; g.ldw = ldw; g.ldc = ldc; g.ldo = ldo;
  g.epi = epi;
  return g;
}

}  // namespace

extern "C" {

const char* gmla_status_string(gmla_status_t s) {
  switch (s) {
    case GMLA_OK: return "ok";
    case GMLA_ERR_INVALID_ARG: return "invalid argument";
    case GMLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GMLA_ERR_WORKSPACE: return "workspace too small";
    case GMLA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* gmla_last_error(void) { return g_err.c_str(); }

int gmla_version(void) { return 10000; }

// ============================================================ prefill
// bf16 keeps V transposed per (sequence, head): [B][H d_v][Lp], keys
// contiguous, rows padded with zeros to Lp = L rounded up to 64 (one key tile)
static size_t prefill_vt_ld(int L) { return ((size_t)L + 63) / 64 * 64; }

size_t gmla_prefill_workspace_size(int B, int L, int H, int d_cq, int d_k, int d_r, int d_v, gmla_dtype_t dtype) {
  if (B <= 0 || L <= 0 || H <= 0 || d_cq < 0 || d_k <= 0 || d_r < 0 || d_v <= 0) return 0;
  const size_t T = (size_t)B * L;
  const size_t es = esize(dtype);
  const size_t v_elems = dtype == GMLA_BF16 ? (size_t)B * H * d_v * prefill_vt_ld(L) : T * H * d_v;
  // q and the RoPE queries ([T, H d_k], [T, H d_r]), K [T, H d_k], V, then
  // the low-rank query c^Q [T, d_cq]
  return up256(T * H * (d_k + d_r) * es) + up256(T * H * d_k * es) + up256(v_elems * es) + up256(T * d_cq * es);
}

gmla_status_t gmla_prefill(const void* x, const void* W_c, const void* W_dq, const void* W_q, const void* W_kr,
                           const void* W_qr, const void* W_uk, const void* W_uv, void* latent_out, void* o_tilde,
                           void* workspace, size_t workspace_bytes, int B, int L, int d_model, int H, int d_c,
                           int d_cq, int d_k, int d_r, int d_v, float sm_scale, float rope_base, gmla_dtype_t dtype,
                           void* stream) {
  REQUIRE(dtype == GMLA_F32 || dtype == GMLA_BF16, GMLA_ERR_INVALID_ARG, "dtype must be GMLA_F32 or GMLA_BF16");
  REQUIRE(x && W_c && W_q && W_uk && W_uv && latent_out && o_tilde, GMLA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(B > 0 && L > 0 && d_model > 0 && H > 0 && d_c > 0 && d_k > 0 && d_v > 0 && d_cq >= 0 && d_r >= 0,
          GMLA_ERR_INVALID_ARG, "sizes must be positive (d_cq, d_r >= 0)");
  REQUIRE((W_dq != nullptr) == (d_cq > 0), GMLA_ERR_INVALID_ARG, "W_dq is given exactly when d_cq > 0");
  REQUIRE((W_kr != nullptr && W_qr != nullptr) == (d_r > 0) && (W_kr != nullptr) == (W_qr != nullptr),
          GMLA_ERR_INVALID_ARG, "W_kr and W_qr are given exactly when d_r > 0");
  REQUIRE(d_r % 2 == 0, GMLA_ERR_INVALID_ARG, "d_r must be even (RoPE pairs)");
  REQUIRE(std::isfinite(sm_scale) && std::isfinite(rope_base) && rope_base >= 0.f, GMLA_ERR_INVALID_ARG,
          "sm_scale must be finite and rope_base finite and >= 0");
  REQUIRE(al16(x) && al16(W_c) && (!W_dq || al16(W_dq)) && al16(W_q) && (!W_kr || al16(W_kr)) &&
              (!W_qr || al16(W_qr)) && al16(W_uk) && al16(W_uv) && al16(latent_out) && al16(o_tilde),
          GMLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE((long long)B * L * std::max({d_model, H * (d_k + d_r), H * d_v, d_cq}) < (1LL << 40), GMLA_ERR_UNSUPPORTED,
          "problem too large");
  // the token count B*L is a GEMM row count (int), and the bf16 attention
  // grid holds one workgroup per (b, h, pair of 128-query tiles)
  REQUIRE((long long)B * L <= INT_MAX, GMLA_ERR_UNSUPPORTED, "B * L must not exceed INT_MAX");
  REQUIRE((long long)H * std::max(d_k, d_v) <= INT_MAX && (long long)H * (d_k + d_r) <= INT_MAX, GMLA_ERR_UNSUPPORTED,
          "H * d_k and H * d_v must not exceed INT_MAX");
  REQUIRE(dtype != GMLA_BF16 || ((long long)L + 255) / 256 * B * H <= INT_MAX, GMLA_ERR_UNSUPPORTED,
          "prefill attention grid too large");
  REQUIRE(d_r == 0 || dtype == GMLA_BF16, GMLA_ERR_UNSUPPORTED, "decoupled RoPE in prefill is bf16 only");
  if (dtype == GMLA_BF16) {
    REQUIRE(d_r == 0 || d_r == 64, GMLA_ERR_UNSUPPORTED, "bf16 prefill needs d_r in {0, 64}");
    REQUIRE(d_model % 64 == 0, GMLA_ERR_UNSUPPORTED, "bf16 prefill needs d_model % 64 == 0");
    REQUIRE(d_c % 64 == 0, GMLA_ERR_UNSUPPORTED, "bf16 prefill needs d_c % 64 == 0");
    REQUIRE(d_cq % 64 == 0, GMLA_ERR_UNSUPPORTED, "bf16 prefill needs d_cq % 64 == 0");
    REQUIRE(d_k == d_v && (d_k == 64 || d_k == 128), GMLA_ERR_UNSUPPORTED,
            "bf16 prefill needs d_k == d_v in {64, 128}");
  } else {
    REQUIRE(d_k <= 1024 && d_v <= 512, GMLA_ERR_UNSUPPORTED, "fp32 prefill needs d_k <= 1024, d_v <= 512");
  }
  const size_t need = gmla_prefill_workspace_size(B, L, H, d_cq, d_k, d_r, d_v, dtype);
  REQUIRE(workspace && workspace_bytes >= need, GMLA_ERR_WORKSPACE,
          "prefill workspace needs " + std::to_string(need) + " bytes");
  REQUIRE(al16(workspace), GMLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  const int T = B * L;
  const size_t es = esize(dtype);
  char* ws = (char*)workspace;
  void* q = ws;
  void* qr = ws + (size_t)T * H * d_k * es;  // RoPE queries follow q
  void* k = ws + up256((size_t)T * H * (d_k + d_r) * es);
  void* v = (char*)k + up256((size_t)T * H * d_k * es);
  const size_t v_elems = dtype == GMLA_BF16 ? (size_t)B * H * d_v * prefill_vt_ld(L) : (size_t)T * H * d_v;
  void* cq = (char*)v + up256(v_elems * es);
  // the query side reads x, or the low-rank query c^Q = x W_dq^T
  const void* xq = d_cq > 0 ? cq : x;
  const int dq_in = d_cq > 0 ? d_cq : d_model;
  const int HK = H * d_k, HV = H * d_v;
  const int CW = d_c + d_r;  // cache row width: [c ; RoPE key]
  gmla_status_t s;
  if (dtype == GMLA_BF16) {
    // c = x W_c^T (cache rows), q = x W_q^T, K = c W_UK^T, V = c W_UV^T (W_UK as [H*d_k, d_c]);
    // with RoPE also k^R = x W_kr^T into the cache rows' tail and q^R = u W_qr^T.
    // The projections that read x go out as one grid on the 256 x 256 tile
    // kernel when the shape qualifies (the latent, 512 wide, then rides on
    // the query's waves instead of a grid of its own); else one by one.
    GemmGroup gx{};
    gx.base = gemm(x, d_model, nullptr, d_model, nullptr, 0, T, 0, d_model);
    auto add = [&](const void* Wt, void* Ct, int n, int64_t ldc) {
      gx.W[gx.count] = (const bf16*)Wt; gx.C[gx.count] = (bf16*)Ct; gx.N[gx.count] = n;
      gx.ldw[gx.count] = d_model; gx.ldc[gx.count] = ldc; ++gx.count;
    };
    add(W_c, latent_out, d_c, CW);
    if (d_r > 0) add(W_kr, (bf16*)latent_out + d_c, d_r, CW);
    if (d_cq > 0) add(W_dq, cq, d_cq, d_cq);
    else {
      add(W_q, q, HK, HK);
      if (d_r > 0) add(W_qr, qr, H * d_r, (int64_t)H * d_r);
    }
    bool grouped = false;
    {
      const int tr = trace_pre("gemm_input", st);
      const hipError_t e = launch_gemm_group_big(gx, st);
      trace_post(tr, st);
      if (e == hipSuccess) grouped = true;
      else if (e != hipErrorNotSupported) return fail(GMLA_ERR_HIP, std::string("gemm_input: ") + hipGetErrorString(e));
      else (void)hipGetLastError();
    }
    if (!grouped) {
      if ((s = run("gemm_latent", st, [&] { return launch_gemm_bf16(gemm(x, d_model, W_c, d_model, latent_out, CW, T, d_c, d_model), st); }))) return s;
      if (d_cq > 0 &&
          (s = run("gemm_query_down", st, [&] { return launch_gemm_bf16(gemm(x, d_model, W_dq, d_model, cq, d_cq, T, d_cq, d_model), st); })))
        return s;
      if (d_r > 0 &&
          (s = run("gemm_rope_key", st, [&] { return launch_gemm_bf16(gemm(x, d_model, W_kr, d_model, (bf16*)latent_out + d_c, CW, T, d_r, d_model), st); })))
        return s;
    }
    if (!grouped || d_cq > 0) {
      if ((s = run("gemm_query", st, [&] { return launch_gemm_bf16(gemm(xq, dq_in, W_q, dq_in, q, HK, T, HK, dq_in), st); }))) return s;
      if (d_r > 0 &&
          (s = run("gemm_rope_query", st, [&] { return launch_gemm_bf16(gemm(xq, dq_in, W_qr, dq_in, qr, (int64_t)H * d_r, T, H * d_r, dq_in), st); })))
        return s;
    }
    if (d_r > 0) {
      // k^R = RoPE(x W_kr^T, s) in the cache rows' tail, q^R = RoPE(u W_qr^T, t), in place
      RopeRowsArgs rk{(bf16*)latent_out + d_c, CW, T, 1, d_r, L, rope_base};
      RopeRowsArgs rq{(bf16*)qr, (int64_t)H * d_r, T, H, d_r, L, rope_base};
      if ((s = run("rope_rows", st, [&] { return launch_rope_rows(rk, st); }))) return s;
      if ((s = run("rope_rows", st, [&] { return launch_rope_rows(rq, st); }))) return s;
    }
    if ((s = run("gemm_key_recon", st, [&] { return launch_gemm_bf16(gemm(latent_out, CW, W_uk, d_c, k, HK, T, HK, d_c), st); }))) return s;
    // V^T per sequence: [H d_v, Lp] = W_UV c^T (the operands swapped), the
    // columns past L written as zeros
    const int64_t Lp = (int64_t)prefill_vt_ld(L);
    if ((s = run("gemm_value_recon", st, [&] {
           GemmArgs g = gemm(W_uv, d_c, latent_out, CW, v, Lp, HV, L, d_c);
           g.batches = B; g.sA = 0; g.sW = (int64_t)L * CW; g.sC = (int64_t)HV * Lp; g.npad = (int)Lp;
           return launch_gemm_bf16(g, st);
         }))) return s;
    AttnArgs a{};
    a.q = (const bf16*)q; a.k = (const bf16*)k; a.v = (const bf16*)v; a.o = (bf16*)o_tilde;
    a.B = B; a.L = L; a.H = H; a.D = d_k;
    a.sqb = (int64_t)L * HK; a.sqt = HK; a.sqh = d_k;
    a.skb = (int64_t)L * HK; a.skt = HK; a.skh = d_k;
    a.svb = (int64_t)HV * Lp; a.svj = Lp; a.svh = (int64_t)d_v * Lp;
    a.sob = (int64_t)L * HV; a.sot = HV; a.soh = d_v;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    if (d_r > 0) {
      a.D_R = d_r;
      a.qr = (const bf16*)qr; a.sqrb = (int64_t)L * H * d_r; a.sqrt_ = (int64_t)H * d_r; a.sqrh = d_r;
      a.kr = (const bf16*)latent_out + d_c; a.skrb = (int64_t)L * CW; a.skrt = CW;
    }
    if ((s = run("prefill_attn", st, [&] { return launch_prefill_attn_bf16(a, st); }))) return s;
  } else {
    if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(x, d_model, W_c, d_model, latent_out, d_c, T, d_c, d_model), st); }))) return s;
    if (d_cq > 0 &&
        (s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(x, d_model, W_dq, d_model, cq, d_cq, T, d_cq, d_model), st); })))
      return s;
    if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(xq, dq_in, W_q, dq_in, q, HK, T, HK, dq_in), st); }))) return s;
    if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(latent_out, d_c, W_uk, d_c, k, HK, T, HK, d_c), st); }))) return s;
    if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(latent_out, d_c, W_uv, d_c, v, HV, T, HV, d_c), st); }))) return s;
    AttnF32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v; a.o = (float*)o_tilde;
    a.B = B; a.L = L; a.H = H; a.Dk = d_k; a.Dv = d_v;
    a.sqb = (int64_t)L * HK; a.sqt = HK; a.sqh = d_k;
    a.skb = (int64_t)L * HK; a.skt = HK; a.skh = d_k;
    a.svb = (int64_t)L * HV; a.svt = HV; a.svh = d_v;
    a.sob = (int64_t)L * HV; a.sot = HV; a.soh = d_v;
    a.scale = sm_scale;
    if ((s = run("prefill_attn_f32", st, [&] { return launch_prefill_attn_f32(a, st); }))) return s;
  }
  return ok();
}

// ============================================================ decode
size_t gmla_decode_workspace_size(int B, int H, int d_c, int num_splits, gmla_dtype_t dtype) {
  if (B <= 0 || H <= 0 || d_c <= 0 || num_splits < 0) return 0;
  // the fp32 path and the generic bf16 path (d_c != 512) need none
  if (dtype == GMLA_F32 || d_c != 512) return 0;
  const size_t G = (size_t)decode_slices(num_splits, H);
  const size_t H16 = ((size_t)H + 15) / 16 * 16;  // partial outputs are kept per group of 16 heads
  return up256((size_t)B * 8) + up256(2 * G * H * 4) + up256(2 * G * H16 * (size_t)d_c * 2);
}

gmla_status_t gmla_decode(const void* q_abs, const void* cache, const int64_t* seq_start, const int32_t* seq_len,
                          void* o_lat, float* lse, void* workspace, size_t workspace_bytes, int B, int H, int d_c,
                          int d_r, float rope_base, float sm_scale, int num_splits, gmla_dtype_t dtype,
                          void* stream) {
  REQUIRE(dtype == GMLA_F32 || dtype == GMLA_BF16, GMLA_ERR_INVALID_ARG, "dtype must be GMLA_F32 or GMLA_BF16");
  REQUIRE(q_abs && cache && seq_start && seq_len && o_lat, GMLA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(B > 0 && H > 0 && d_c > 0 && d_r >= 0, GMLA_ERR_INVALID_ARG, "sizes must be positive (d_r >= 0)");
  REQUIRE(d_r % 2 == 0, GMLA_ERR_INVALID_ARG, "d_r must be even (RoPE pairs)");
  REQUIRE(num_splits >= 0 && num_splits <= 65535, GMLA_ERR_INVALID_ARG, "num_splits must be in [0, 65535]");
  REQUIRE(std::isfinite(sm_scale) && std::isfinite(rope_base) && rope_base >= 0.f, GMLA_ERR_INVALID_ARG,
          "sm_scale must be finite and rope_base finite and >= 0");
  REQUIRE(al16(q_abs) && al16(cache) && al16(seq_start) && al16(seq_len) && al16(o_lat) && (!lse || al16(lse)),
          GMLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (dtype == GMLA_F32) {
    REQUIRE(d_c + d_r <= 1024 && d_c <= 512, GMLA_ERR_UNSUPPORTED, "fp32 decode needs d_c + d_r <= 1024, d_c <= 512");
    DecodeF32Args a{};
    a.q = q_abs; a.cache = cache; a.seq_start = seq_start; a.seq_len = seq_len;
    a.o_lat = o_lat; a.lse = lse; a.B = B; a.H = H; a.d_c = d_c; a.d_r = d_r;
    a.scale = sm_scale; a.rope_base = d_r > 0 ? rope_base : 0.f;
    gmla_status_t s = run("decode_f32", st, [&] { return launch_decode_f32(a, st); });
    return s ? s : ok();
  }
  if (!decode_bf16_supported(d_c, d_r)) {
    // latent and RoPE widths outside the MFMA kernel's: the generic bf16
    // decode (one workgroup per sequence and head, no workspace)
    REQUIRE(d_c % 64 == 0 && d_c <= 512 && d_c + d_r <= 1024, GMLA_ERR_UNSUPPORTED,
            "bf16 decode needs d_c % 64 == 0, d_c <= 512 and d_c + d_r <= 1024");
    REQUIRE((long long)B * H <= INT_MAX, GMLA_ERR_UNSUPPORTED, "B * H must not exceed INT_MAX");
    DecodeF32Args a{};
    a.q = q_abs; a.cache = cache; a.seq_start = seq_start; a.seq_len = seq_len;
    a.o_lat = o_lat; a.lse = lse; a.B = B; a.H = H; a.d_c = d_c; a.d_r = d_r;
    a.scale = sm_scale; a.rope_base = d_r > 0 ? rope_base : 0.f;
    gmla_status_t s = run("decode_generic", st, [&] { return launch_decode_generic_bf16(a, st); });
    return s ? s : ok();
  }
  const int G = decode_slices(num_splits, H);
  const size_t need = gmla_decode_workspace_size(B, H, d_c, num_splits, dtype);
  REQUIRE(workspace && workspace_bytes >= need, GMLA_ERR_WORKSPACE,
          "decode workspace needs " + std::to_string(need) + " bytes");
  REQUIRE(((uintptr_t)workspace & 255u) == 0, GMLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* ws = (char*)workspace;
  DecodeArgs a{};
  a.q = (const bf16*)q_abs; a.cache = (const bf16*)cache; a.seq_start = seq_start; a.seq_len = seq_len;
  a.o_lat = (bf16*)o_lat; a.lse = lse;
  a.prefix = (long long*)ws;
  a.part_lse = (float*)(ws + up256((size_t)B * 8));
  a.part_o = (bf16*)(ws + up256((size_t)B * 8) + up256(2 * (size_t)G * H * 4));
  a.B = B; a.H = H; a.d_c = d_c; a.d_r = d_r; a.G = G;
  a.seg_cost = kDecodeSegCost;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.rope_base = d_r > 0 ? rope_base : 0.f;
  gmla_status_t s;
  if ((s = run("decode_attn", st, [&] { return launch_decode_attn(a, st); }))) return s;
  if ((s = run("decode_combine", st, [&] { return launch_decode_combine(a, st); }))) return s;
  return ok();
}

// ============================================================ decode without allocation
// The scratch of gmla_decode_noalloc: one library-owned device array per GPU
// (each device holds its own copy, at its own address, until the process
// ends). Host code never uses the array's name as an address: it takes the
// device address from hipGetSymbolAddress once per device.
static __device__ __align__(256) unsigned char scratch[GMLA_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
gmla_status_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GMLA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GMLA_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GMLA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GMLA_OK;
}
}  // namespace

gmla_status_t gmla_decode_noalloc(const void* q_abs, const void* cache, const int64_t* seq_start,
                                  const int32_t* seq_len, void* o_lat, float* lse, int B, int H, int d_c, int d_r,
                                  float rope_base, float sm_scale, int num_splits, gmla_dtype_t dtype, void* stream) {
  REQUIRE(dtype == GMLA_F32 || dtype == GMLA_BF16, GMLA_ERR_INVALID_ARG, "dtype must be GMLA_F32 or GMLA_BF16");
  REQUIRE(B > 0 && H > 0 && d_c > 0 && num_splits >= 0, GMLA_ERR_INVALID_ARG, "sizes must be positive");
  const size_t need = gmla_decode_workspace_size(B, H, d_c, num_splits, dtype);
  REQUIRE(need <= (size_t)GMLA_DECODE_SCRATCH_BYTES, GMLA_ERR_UNSUPPORTED,
          "gmla_decode_noalloc: this call needs " + std::to_string(need) + " bytes of scratch, more than the " +
              std::to_string((size_t)GMLA_DECODE_SCRATCH_BYTES) + " the library holds per GPU");
  void* ws = nullptr;
  if (need > 0) {
    gmla_status_t s = scratch_address(&ws);
    if (s) return s;
  }
  // the same checks and kernels as gmla_decode, on the library's scratch
  return gmla_decode(q_abs, cache, seq_start, seq_len, o_lat, lse, ws, need > 0 ? (size_t)GMLA_DECODE_SCRATCH_BYTES : 0,
                     B, H, d_c, d_r, rope_base, sm_scale, num_splits, dtype, stream);
}

// ============================================================ decode-step projections
size_t gmla_decode_prepare_workspace_size(int B, int d_model, int H, int d_c, int d_cq, int d_k, int d_r,
                                          gmla_dtype_t dtype) {
  if (B <= 0 || d_model <= 0 || H <= 0 || d_c <= 0 || d_cq < 0 || d_k <= 0 || d_r < 0 || dtype != GMLA_BF16) return 0;
  return up256((size_t)B * (d_c + d_r) * 2) + up256((size_t)B * H * d_k * 2) + up256((size_t)B * H * d_r * 2) +
         up256((size_t)B * d_cq * 2);
}

gmla_status_t gmla_decode_prepare(const void* x, const void* W_c, const void* W_kr, const void* W_dq, const void* W_q,
                                  const void* W_qr, const void* W_uk, void* cache, const int64_t* seq_start,
                                  const int32_t* seq_len, void* q_abs, void* workspace, size_t workspace_bytes, int B,
                                  int d_model, int H, int d_c, int d_cq, int d_k, int d_r, float rope_base,
                                  gmla_dtype_t dtype, void* stream) {
  REQUIRE(dtype == GMLA_F32 || dtype == GMLA_BF16, GMLA_ERR_INVALID_ARG, "dtype must be GMLA_F32 or GMLA_BF16");
  REQUIRE(x && W_c && W_q && W_uk && cache && seq_start && seq_len && q_abs, GMLA_ERR_INVALID_ARG,
          "null tensor pointer");
  REQUIRE(B > 0 && d_model > 0 && H > 0 && d_c > 0 && d_k > 0 && d_r >= 0 && d_cq >= 0, GMLA_ERR_INVALID_ARG,
          "sizes must be positive (d_cq, d_r >= 0)");
  REQUIRE(d_r == 0 || (W_kr && W_qr), GMLA_ERR_INVALID_ARG, "d_r > 0 needs W_kr and W_qr");
  REQUIRE((W_dq != nullptr) == (d_cq > 0), GMLA_ERR_INVALID_ARG, "W_dq is given exactly when d_cq > 0");
  REQUIRE(d_r % 2 == 0, GMLA_ERR_INVALID_ARG, "d_r must be even (RoPE pairs)");
  REQUIRE(std::isfinite(rope_base) && rope_base >= 0.f, GMLA_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
  REQUIRE(al16(x) && al16(W_c) && (!d_r || (al16(W_kr) && al16(W_qr))) && (!W_dq || al16(W_dq)) && al16(W_q) &&
              al16(W_uk) && al16(cache) && al16(seq_start) && al16(seq_len) && al16(q_abs),
          GMLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(dtype == GMLA_BF16, GMLA_ERR_UNSUPPORTED, "decode_prepare is bf16 only");
  REQUIRE(d_model % 64 == 0 && d_c % 64 == 0 && d_cq % 64 == 0 && d_k <= 128 && d_k % 16 == 0 && d_r % 4 == 0,
          GMLA_ERR_UNSUPPORTED,
          "bf16 decode_prepare needs d_model, d_c and d_cq % 64 == 0, d_k % 16 == 0, d_k <= 128, d_r % 4 == 0");
  const size_t need = gmla_decode_prepare_workspace_size(B, d_model, H, d_c, d_cq, d_k, d_r, dtype);
  REQUIRE(workspace && workspace_bytes >= need, GMLA_ERR_WORKSPACE,
          "decode_prepare workspace needs " + std::to_string(need) + " bytes");
  REQUIRE(((uintptr_t)workspace & 255u) == 0, GMLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const int W = d_c + d_r;
  char* ws = (char*)workspace;
  bf16* row = (bf16*)ws;
  bf16* q = (bf16*)(ws + up256((size_t)B * W * 2));
  bf16* qr = (bf16*)(ws + up256((size_t)B * W * 2) + up256((size_t)B * H * d_k * 2));
  bf16* cq = (bf16*)(ws + up256((size_t)B * W * 2) + up256((size_t)B * H * d_k * 2) + up256((size_t)B * H * d_r * 2));
  // the query side reads x, or the low-rank query c^Q = x W_dq^T
  const void* xq = d_cq > 0 ? (const void*)cq : x;
  const int dq_in = d_cq > 0 ? d_cq : d_model;
  gmla_status_t s;
  if (B <= 64) {
    // the projections of x in one weight-streaming launch, then (low-rank
    // query) those of c^Q in a second
    struct Seg { const void* w; bf16* c; int n; int64_t ldc; };
    Seg from_x[4], from_q[2];
    int nx = 0, nq = 0;
    from_x[nx++] = {W_c, row, d_c, W};
    if (d_r > 0) from_x[nx++] = {W_kr, row + d_c, d_r, W};
    if (d_cq > 0) from_x[nx++] = {W_dq, cq, d_cq, d_cq};
    Seg* qs = d_cq > 0 ? from_q : from_x;
    int& nqs = d_cq > 0 ? nq : nx;
    qs[nqs++] = {W_q, q, H * d_k, (int64_t)H * d_k};
    if (d_r > 0) qs[nqs++] = {W_qr, qr, H * d_r, (int64_t)H * d_r};
    auto group = [&](const void* A, int K, const Seg* sg, int n) {
      GemmGroup gg{};
      gg.base = gemm(A, K, nullptr, K, nullptr, 0, B, 0, K);
      gg.count = n;
      for (int i = 0; i < n; ++i) {
        gg.W[i] = (const bf16*)sg[i].w; gg.C[i] = sg[i].c; gg.N[i] = sg[i].n; gg.ldw[i] = K; gg.ldc[i] = sg[i].ldc;
      }
      return launch_gemm_group_bf16(gg, st);
    };
    if ((s = run("gemm_input", st, [&] { return group(x, d_model, from_x, nx); }))) return s;
    if (nq > 0 && (s = run("gemm_query_up", st, [&] { return group(cq, d_cq, from_q, nq); }))) return s;
  } else {
    if ((s = run("gemm_latent", st, [&] { return launch_gemm_bf16(gemm(x, d_model, W_c, d_model, row, W, B, d_c, d_model), st); }))) return s;
    if (d_r > 0 &&
        (s = run("gemm_rope_key", st, [&] { return launch_gemm_bf16(gemm(x, d_model, W_kr, d_model, row + d_c, W, B, d_r, d_model), st); })))
      return s;
    if (d_cq > 0 &&
        (s = run("gemm_query_down", st, [&] { return launch_gemm_bf16(gemm(x, d_model, W_dq, d_model, cq, d_cq, B, d_cq, d_model), st); })))
      return s;
    if ((s = run("gemm_query", st, [&] { return launch_gemm_bf16(gemm(xq, dq_in, W_q, dq_in, q, H * d_k, B, H * d_k, dq_in), st); }))) return s;
    if (d_r > 0 &&
        (s = run("gemm_rope_query", st, [&] { return launch_gemm_bf16(gemm(xq, dq_in, W_qr, dq_in, qr, H * d_r, B, H * d_r, dq_in), st); })))
      return s;
  }
  PrepareArgs a{};
  a.row = row; a.q = q; a.q_r = qr; a.W_uk = (const bf16*)W_uk; a.cache = (bf16*)cache;
  a.seq_start = seq_start; a.seq_len = seq_len; a.q_abs = (bf16*)q_abs;
  a.B = B; a.H = H; a.d_c = d_c; a.d_k = d_k; a.d_r = d_r;
  a.rope_base = d_r > 0 ? rope_base : 0.f;
  if ((s = run("decode_absorb", st, [&] { return launch_decode_absorb(a, st); }))) return s;
  return ok();
}

// ============================================================ gate + output
// Split-K partial sums of the gate_out GEMMs (bf16, T <= 64): the largest.
static size_t gate_out_part_bytes(int T, int d_model, int H, int d_c, int d_v, int with_value_up) {
  const int HV = H * d_v;
  size_t p = std::max(gemm_part_bytes(T, HV, d_model, 1), gemm_part_bytes(T, d_model, HV, 1));
  if (with_value_up) p = std::max(p, gemm_part_bytes(T, d_v, d_c, H));
  return up256(p);
}

size_t gmla_gate_out_workspace_size(int T, int d_model, int H, int d_c, int d_v, int with_value_up,
                                    gmla_dtype_t dtype) {
  if (T <= 0 || d_model <= 0 || H <= 0 || d_v <= 0 || (with_value_up && d_c <= 0)) return 0;
  const size_t one = up256((size_t)T * H * d_v * esize(dtype));
  const size_t base = with_value_up ? 2 * one : one;
  if (dtype != GMLA_BF16) return base;
  return base + gate_out_part_bytes(T, d_model, H, d_c, d_v, with_value_up);
}

gmla_status_t gmla_gate_out(const void* x, const void* o, const void* W_uv, const void* W_g, const void* W_o, void* y,
                            void* workspace, size_t workspace_bytes, int T, int d_model, int H, int d_c, int d_v,
                            gmla_dtype_t dtype, void* stream) {
  REQUIRE(dtype == GMLA_F32 || dtype == GMLA_BF16, GMLA_ERR_INVALID_ARG, "dtype must be GMLA_F32 or GMLA_BF16");
  REQUIRE(x && o && W_g && W_o && y, GMLA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(T > 0 && d_model > 0 && H > 0 && d_v > 0 && (!W_uv || d_c > 0), GMLA_ERR_INVALID_ARG,
          "sizes must be positive");
  REQUIRE(al16(x) && al16(o) && (!W_uv || al16(W_uv)) && al16(W_g) && al16(W_o) && al16(y), GMLA_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  const int HV = H * d_v;
  if (dtype == GMLA_BF16) {
    REQUIRE(d_model % 64 == 0 && HV % 64 == 0 && d_v % 4 == 0, GMLA_ERR_UNSUPPORTED,
            "bf16 gate_out needs d_model % 64 == 0, H*d_v % 64 == 0, d_v % 4 == 0");
    REQUIRE(!W_uv || d_c % 64 == 0, GMLA_ERR_UNSUPPORTED, "bf16 value up-projection needs d_c % 64 == 0");
  }
  const size_t need = gmla_gate_out_workspace_size(T, d_model, H, d_c, d_v, W_uv != nullptr, dtype);
  REQUIRE(workspace && workspace_bytes >= need, GMLA_ERR_WORKSPACE,
          "gate_out workspace needs " + std::to_string(need) + " bytes");
  REQUIRE(al16(workspace), GMLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const size_t es = esize(dtype);
  char* ws = (char*)workspace;
  void* gated = ws;
  const void* ot = o;
  gmla_status_t s;
  if (dtype == GMLA_BF16) {
    void* part = ws + (W_uv ? 2 : 1) * up256((size_t)T * HV * es);
    if (W_uv && gemm_gate_vu_supported(T, HV, d_model, d_c, d_v)) {
      // the value up-projection folded into the gate GEMM: each workgroup
      // computes the o~ columns it gates from o_lat and W_uv itself
      GemmArgs g = gemm(x, d_model, W_g, d_model, gated, HV, T, HV, d_model, EPI_GATE_VU);
      g.vo = (const bf16*)o; g.vw = (const bf16*)W_uv; g.vdc = d_c; g.vdv = d_v; g.ldvo = (int64_t)H * d_c;
      if ((s = run("gemm_gate", st, [&] { return launch_gemm_bf16(g, st); }))) return s;
      if ((s = run("gemm_out", st, [&] { return launch_gemm_bf16(with_split(gemm(gated, HV, W_o, HV, y, d_model, T, d_model, HV), part), st); }))) return s;
      return ok();
    }
    if (W_uv) {
      void* otw = ws + up256((size_t)T * HV * es);
      GemmArgs g = gemm(o, (int64_t)H * d_c, W_uv, d_c, otw, HV, T, d_v, d_c);
      g.batches = H; g.sA = d_c; g.sW = (int64_t)d_v * d_c; g.sC = d_v;
      g = with_split(g, part);
      if ((s = run("gemm_value_up", st, [&] { return launch_gemm_bf16(g, st); }))) return s;
      ot = otw;
    }
    if ((s = run("gemm_gate", st, [&] { return launch_gemm_bf16(with_split(gemm(x, d_model, W_g, d_model, gated, HV, T, HV, d_model, EPI_GATE, ot, HV), part), st); }))) return s;
    if ((s = run("gemm_out", st, [&] { return launch_gemm_bf16(with_split(gemm(gated, HV, W_o, HV, y, d_model, T, d_model, HV), part), st); }))) return s;
  } else {
    if (W_uv) {
      void* otw = ws + up256((size_t)T * HV * es);
      GemmF32Args g = gemm32(o, (int64_t)H * d_c, W_uv, d_c, otw, HV, T, d_v, d_c);
      g.batches = H; g.sA = d_c; g.sW = (int64_t)d_v * d_c; g.sC = d_v;
      if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(g, st); }))) return s;
      ot = otw;
    }
    if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(x, d_model, W_g, d_model, gated, HV, T, HV, d_model, EPI_GATE, ot, HV), st); }))) return s;
    if ((s = run("gemm_f32", st, [&] { return launch_gemm_f32(gemm32(gated, HV, W_o, HV, y, d_model, T, d_model, HV), st); }))) return s;
  }
  return ok();
}

// ============================================================ per-head gate + output
size_t gmla_head_gate_out_workspace_size(int T, int d_model, int H, int d_c, int d_v, int with_value_up,
                                         gmla_dtype_t dtype) {
  if (T <= 0 || d_model <= 0 || H <= 0 || d_v <= 0 || (with_value_up && d_c <= 0) || dtype != GMLA_BF16) return 0;
  const int HV = H * d_v;
  size_t part = std::max(gemm_part_bytes(T, H, d_model, 1), gemm_part_bytes(T, d_model, HV, 1));
  if (with_value_up) part = std::max(part, gemm_part_bytes(T, d_v, d_c, H));
  const size_t one = up256((size_t)T * HV * 2);
  return (with_value_up ? 2 : 1) * one + up256((size_t)T * H * 2) + up256(part);
}

gmla_status_t gmla_head_gate_out(const void* x, const void* o, const void* W_uv, const void* W_g, const void* b_g,
                                 const void* W_o, void* y, void* workspace, size_t workspace_bytes, int T, int d_model,
                                 int H, int d_c, int d_v, gmla_dtype_t dtype, void* stream) {
  REQUIRE(dtype == GMLA_F32 || dtype == GMLA_BF16, GMLA_ERR_INVALID_ARG, "dtype must be GMLA_F32 or GMLA_BF16");
  REQUIRE(x && o && W_g && W_o && y, GMLA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(T > 0 && d_model > 0 && H > 0 && d_v > 0 && (!W_uv || d_c > 0), GMLA_ERR_INVALID_ARG,
          "sizes must be positive");
  REQUIRE(al16(x) && al16(o) && (!W_uv || al16(W_uv)) && al16(W_g) && (!b_g || al16(b_g)) && al16(W_o) && al16(y),
          GMLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(dtype == GMLA_BF16, GMLA_ERR_UNSUPPORTED, "head_gate_out is bf16 only");
  const int HV = H * d_v;
  REQUIRE(d_model % 64 == 0 && HV % 64 == 0 && d_v % 8 == 0 && H % 4 == 0 && (!W_uv || d_c % 64 == 0),
          GMLA_ERR_UNSUPPORTED,
          "bf16 head_gate_out needs d_model % 64 == 0, H*d_v % 64 == 0, d_v % 8 == 0, H % 4 == 0, d_c % 64 == 0");
  const size_t need = gmla_head_gate_out_workspace_size(T, d_model, H, d_c, d_v, W_uv != nullptr, dtype);
  REQUIRE(workspace && workspace_bytes >= need, GMLA_ERR_WORKSPACE,
          "head_gate_out workspace needs " + std::to_string(need) + " bytes");
  REQUIRE(((uintptr_t)workspace & 255u) == 0, GMLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const size_t one = up256((size_t)T * HV * 2);
  void* gated = ws;
  void* otw = ws + one;
  void* z = ws + (W_uv ? 2 : 1) * one;
  void* part = (char*)z + up256((size_t)T * H * 2);
  const void* ot = o;
  gmla_status_t s;
  if (W_uv) {
    GemmArgs g = gemm(o, (int64_t)H * d_c, W_uv, d_c, otw, HV, T, d_v, d_c);
    g.batches = H; g.sA = d_c; g.sW = (int64_t)d_v * d_c; g.sC = d_v;
    g = with_split(g, part);
    if ((s = run("gemm_value_up", st, [&] { return launch_gemm_bf16(g, st); }))) return s;
    ot = otw;
  }
  if ((s = run("gemm_gate_logits", st, [&] { return launch_gemm_bf16(with_split(gemm(x, d_model, W_g, d_model, z, H, T, H, d_model), part), st); }))) return s;
  HeadGateArgs hg{(const bf16*)z, (const bf16*)b_g, (const bf16*)ot, (bf16*)gated, T, H, d_v, H, HV, HV};
  if ((s = run("head_gate", st, [&] { return launch_head_gate(hg, st); }))) return s;
  if ((s = run("gemm_out", st, [&] { return launch_gemm_bf16(with_split(gemm(gated, HV, W_o, HV, y, d_model, T, d_model, HV), part), st); }))) return s;
  return ok();
}

// ============================================================ probe
gmla_status_t gmla_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  REQUIRE(src && sink, GMLA_ERR_INVALID_ARG, "null pointer");
  REQUIRE(al16(src) && al16(sink) && bytes % 16 == 0, GMLA_ERR_INVALID_ARG,
          "src and sink must be 16-byte aligned and bytes a multiple of 16");
  hipStream_t st = (hipStream_t)stream;
  gmla_status_t s = run("probe_read", st, [&] { return launch_probe_read(src, bytes, (unsigned*)sink, GMLA_PROBE_BLOCKS, st); });
  return s ? s : ok();
}

// ============================================================ trace
gmla_status_t gmla_trace_begin(int max_launches) {
  REQUIRE(max_launches > 0 && max_launches <= (1 << 20), GMLA_ERR_INVALID_ARG, "max_launches out of range");
  std::lock_guard<std::mutex> lk(g_tr_mu);
  while ((int)g_tr.size() < max_launches) {
    TraceRec r{nullptr, {nullptr, nullptr, 0}};
    if (hipEventCreate(&r.ev.start) != hipSuccess || hipEventCreate(&r.ev.stop) != hipSuccess)
      return fail(GMLA_ERR_HIP, "hipEventCreate failed");
    g_tr.push_back(r);
  }
  g_tr_on = true;
  return ok();
}

gmla_status_t gmla_trace_end(void) {
  std::lock_guard<std::mutex> lk(g_tr_mu);
  g_tr_on = false;
  return ok();
}

gmla_status_t gmla_trace_summary(const char* name, int* count, double* mean_ms) {
  REQUIRE(name && count && mean_ms, GMLA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> lk(g_tr_mu);
  int n = 0;
  double sum = 0;
  for (int i = 0; i < g_tr_used; ++i) {
    if (!g_tr[i].name || std::strcmp(g_tr[i].name, name) != 0 || g_tr[i].ev.launched == 0) continue;
    if (hipEventSynchronize(g_tr[i].ev.stop) != hipSuccess) return fail(GMLA_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_tr[i].ev.start, g_tr[i].ev.stop) != hipSuccess)
      return fail(GMLA_ERR_HIP, "hipEventElapsedTime failed");
    sum += ms;
    ++n;
  }
  *count = n;
  *mean_ms = n ? sum / n : 0.0;
  return ok();
}

const char* gmla_trace_kernels(void) {
  std::lock_guard<std::mutex> lk(g_tr_mu);
  g_tr_names.clear();
  for (int i = 0; i < g_tr_used; ++i) {
    const std::string nm = g_tr[i].name ? g_tr[i].name : "";
    if ((";" + g_tr_names + ";").find(";" + nm + ";") == std::string::npos) {
      if (!g_tr_names.empty()) g_tr_names += ";";
      g_tr_names += nm;
    }
  }
  return g_tr_names.c_str();
}

void gmla_trace_reset(void) {
  std::lock_guard<std::mutex> lk(g_tr_mu);
  for (auto& r : g_tr) {
    if (r.ev.start) hipEventDestroy(r.ev.start);
    if (r.ev.stop) hipEventDestroy(r.ev.stop);
  }
  g_tr.clear();
  g_tr_used = 0;
  g_tr_on = false;
  g_launch_events = nullptr;
}

}  // extern "C"
