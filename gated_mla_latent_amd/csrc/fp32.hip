// fp32 path: the same operations in true fp32 arithmetic (FMA on the vector
// ALU, no reduced-precision matrix emulation). Used when callers ask for
// GMLA_F32; sized for small models, not tuned.
//
//  * gemm_f32: C = epi(A . W^T) with the same epilogues as the bf16 GEMM
//    (store, or Sigmoid(acc) * O -- "Gated MLA 计算公式" §二 boxed equation).
//  * attn_row: one workgroup per attention row (fp32 elements, or bf16
//    elements widened to fp32 for the generic bf16 decode). Prefill rows attend keys
//    s <= t of their own (b, h) ("Gated MLA 计算公式" §二 first equation);
//    decode rows attend all L_b cached rows with the latent as value and the
//    query's RoPE part rotated to position L_b - 1 ("LLM 注意力与计算内核精读笔记 · 03"
//    §5.2). Scores are computed 256 keys at a time into LDS, then every thread
//    folds them into its own output channels with an exact online softmax.
#include "common.h"
#include "kernels.h"

namespace gmla {

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args g) {
  // 64-wide k-steps: the workload's GEMMs are a few tiles each, so their
  // time is the chain of load-then-multiply round trips (four per K = 256)
  constexpr int T = 64, KT = 64;
  __shared__ float As[KT][T + 1];
  __shared__ float Ws[KT][T + 1];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  const int batch = blockIdx.z;
  const float* A = g.A + batch * g.sA;
  const float* W = g.W + batch * g.sW;
  float* C = g.C + batch * g.sC;
  const float* O = g.O ? g.O + batch * g.sO : nullptr;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += KT) {
    for (int i = threadIdx.x; i < T * KT; i += 256) {
      const int r = i / KT, kk = i % KT;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < g.M && k < g.K) ? A[(int64_t)m * g.lda + k] : 0.f;
      Ws[kk][r] = (n < g.N && k < g.K) ? W[(int64_t)n * g.ldw + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KT; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[kk][ty * 4 + i], Ws[kk][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m >= g.M || n >= g.N) continue;
      float v = acc[i][j];
      if (g.epi == EPI_GATE) v = (1.0f / (1.0f + expf(-v))) * O[(int64_t)m * g.ldo + n];
      C[(int64_t)m * g.ldc + n] = v;
    }
}

hipError_t launch_gemm_f32(const GemmF32Args& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batches <= 0) return hipSuccess;
  const dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batches);
  return launch(gemm_f32_kernel, grid, dim3(256), 0, st, g);
}

// --------------------------------------------------------------------------
// element loads and stores of the row kernels: fp32, or bf16 widened to fp32
// (the generic bf16 decode below)
__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const bf16* p) { return (float)*p; }
__device__ __forceinline__ void st_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_f(bf16* p, float v) { *p = __builtin_bit_cast(bf16, f32_to_bf16_bits(v)); }

template <typename E>
struct RowJob {
  const float* q;     // Dk floats (already rotated)
  const E* k;         // key s at k + s * ks
  const E* v;         // value s at v + s * vs
  int64_t ks, vs;
  int n;              // keys 0 .. n-1
  E* o;               // Dv elements
  float* lse;         // or null
};

constexpr int kMaxDk = 1024, kMaxDv = 512;

template <typename E>
__device__ void attn_row(const RowJob<E>& j, int Dk, int Dv, float scale, float* qs, float* zs) {
  const int tid = threadIdx.x;
  // each thread owns output channels tid and tid + 256
  float o0 = 0.f, o1 = 0.f, m = -INFINITY, l = 0.f;
  for (int s0 = 0; s0 < j.n; s0 += 256) {
    const int s = s0 + tid;
    float z = -INFINITY;
    if (s < j.n) {
      const E* kr = j.k + s * j.ks;
      float acc = 0.f;
      for (int d = 0; d < Dk; ++d) acc = fmaf(qs[d], ld_f(kr + d), acc);
      z = acc * scale;
    }
    zs[tid] = z;
    __syncthreads();
    const int cnt = (j.n - s0) < 256 ? (j.n - s0) : 256;
    float cm = -INFINITY;
    for (int i = 0; i < cnt; ++i) cm = fmaxf(cm, zs[i]);
    const float m_new = fmaxf(m, cm);
    const float alpha = expf(m - m_new);  // m = -inf on the first chunk -> 0
    o0 *= alpha; o1 *= alpha; l *= alpha;
    for (int i = 0; i < cnt; ++i) {
      const float p = expf(zs[i] - m_new);
      l += p;
      const E* vr = j.v + (s0 + i) * j.vs;
      if (tid < Dv) o0 = fmaf(p, ld_f(vr + tid), o0);
      if (tid + 256 < Dv) o1 = fmaf(p, ld_f(vr + tid + 256), o1);
    }
    m = m_new;
    __syncthreads();
  }
  if (j.n <= 0) { m = -INFINITY; l = 0.f; }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (tid < Dv) st_f(j.o + tid, o0 * inv);
  if (tid + 256 < Dv) st_f(j.o + tid + 256, o1 * inv);
  if (tid == 0 && j.lse) j.lse[0] = (l > 0.f) ? m + logf(l) : -INFINITY;
}

__global__ __launch_bounds__(256) void prefill_attn_f32_kernel(AttnF32Args a) {
  __shared__ float qs[kMaxDk];
  __shared__ float zs[256];
  const int t = blockIdx.x % a.L;
  const int bh = blockIdx.x / a.L;
  const int b = bh / a.H, h = bh % a.H;
  const float* qp = a.q + b * a.sqb + t * a.sqt + h * a.sqh;
  for (int d = threadIdx.x; d < a.Dk; d += 256) qs[d] = qp[d];
  __syncthreads();
  RowJob<float> j;
  j.q = qs;
  j.k = a.k + b * a.skb + h * a.skh; j.ks = a.skt;
  j.v = a.v + b * a.svb + h * a.svh; j.vs = a.svt;
  j.n = t + 1;
  j.o = a.o + b * a.sob + t * a.sot + h * a.soh;
  j.lse = nullptr;
  attn_row(j, a.Dk, a.Dv, a.scale, qs, zs);
}

// One workgroup per (sequence, head): fp32 decode, and the generic bf16
// decode for latent and RoPE widths the MFMA decode kernel does not take
// (element type E of q, cache and o_lat; fp32 arithmetic either way).
template <typename E>
__global__ __launch_bounds__(256) void decode_row_kernel(DecodeF32Args a) {
  __shared__ float qs[kMaxDk];
  __shared__ float zs[256];
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int W = a.d_c + a.d_r;
  const int Lb = a.seq_len[b];
  const E* qp = (const E*)a.q + ((int64_t)b * a.H + h) * W;
  for (int d = threadIdx.x; d < W; d += 256) {
    float v = ld_f(qp + d);
    if (d >= a.d_c && a.rope_base != 0.f) {
      // interleaved pairs (2i, 2i+1), theta_i = base^(-2i/d_r), position Lb-1
      const int col = d - a.d_c, i = col >> 1;
      const double theta = exp2(-(2.0 * i / a.d_r) * log2((double)a.rope_base));
      double ang = (double)(Lb - 1) * theta;
      ang -= 6.283185307179586 * floor(ang * 0.15915494309189535);
      float sn, cs;
      sincosf((float)ang, &sn, &cs);
      const float x0 = ld_f(qp + a.d_c + 2 * i), x1 = ld_f(qp + a.d_c + 2 * i + 1);
      v = (col & 1) ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
    }
    qs[d] = v;
  }
  __syncthreads();
  RowJob<E> j;
  j.q = qs;
  j.k = (const E*)a.cache + a.seq_start[b] * W; j.ks = W;
  j.v = j.k; j.vs = W;
  j.n = Lb > 0 ? Lb : 0;
  j.o = (E*)a.o_lat + ((int64_t)b * a.H + h) * a.d_c;
  j.lse = a.lse ? a.lse + (int64_t)b * a.H + h : nullptr;
  attn_row(j, W, a.d_c, a.scale, qs, zs);
}

hipError_t launch_prefill_attn_f32(const AttnF32Args& a, hipStream_t st) {
  if (a.Dk > kMaxDk || a.Dv > kMaxDv) return hipErrorInvalidValue;
  return launch(prefill_attn_f32_kernel, dim3(a.B * a.H * a.L), dim3(256), 0, st, a);
}

hipError_t launch_decode_f32(const DecodeF32Args& a, hipStream_t st) {
  if (a.d_c + a.d_r > kMaxDk || a.d_c > kMaxDv) return hipErrorInvalidValue;
  if ((long long)a.B * a.H > 2147483647LL) return hipErrorInvalidValue;
  return launch(decode_row_kernel<float>, dim3(a.B * a.H), dim3(256), 0, st, a);
}

hipError_t launch_decode_generic_bf16(const DecodeF32Args& a, hipStream_t st) {
  if (a.d_c + a.d_r > kMaxDk || a.d_c > kMaxDv) return hipErrorInvalidValue;
  if ((long long)a.B * a.H > 2147483647LL) return hipErrorInvalidValue;
  return launch(decode_row_kernel<bf16>, dim3(a.B * a.H), dim3(256), 0, st, a);
}

}  // namespace gmla
