// Internal launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

namespace gmla {

// Every kernel goes out through launch(). While the C-ABI layer traces a
// call it points g_launch_events at a pair of events, and launch() has the
// kernel's own dispatch record them (hipExtLaunchKernelGGL), so the pair
// brackets that kernel alone rather than also the queue work around it. When
// one traced call launches several kernels, the first records the start and
// each records the stop: the pair spans all of them.
struct LaunchEvents {
  hipEvent_t start, stop;
  int launched;
};
extern thread_local LaunchEvents* g_launch_events;

// Let kernel `fn` use `bytes` of dynamic LDS on the current device. The
// attribute belongs to a device, so it is set once per (kernel, device).
inline hipError_t lds_opt_in(const void* fn, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}

template <typename K, typename... Args>
inline hipError_t launch(K kern, dim3 grid, dim3 block, unsigned shmem, hipStream_t st, Args... args) {
  if (LaunchEvents* ev = g_launch_events) {
    hipExtLaunchKernelGGL(kern, grid, block, shmem, st, ev->launched == 0 ? ev->start : nullptr, ev->stop, 0,
                          args...);
    ++ev->launched;
  } else {
    hipLaunchKernelGGL(kern, grid, block, shmem, st, args...);
  }
  return hipGetLastError();
}

typedef __bf16 bf16;

// ---------------------------------------------------------------- decode
struct DecodeArgs {
  const bf16* q;            // [B, H, d_c + d_r]
  const bf16* cache;        // [rows, d_c + d_r]
  const int64_t* seq_start; // [B] first cache row of each sequence
  const int32_t* seq_len;   // [B]
  bf16* o_lat;              // [B, H, d_c]
  float* lse;               // [B, H] or null
  bf16* part_o;             // [2G, H/16 head groups, 16 x d_c] partial outputs of cut sequences (wave order)
  float* part_lse;          // [2G, H]
  long long* prefix;        // [B] cost offsets: exclusive prefix sums of seq_len[b] + seg_cost (nonempty b)
  int B, H, d_c, d_r, G;
  int seg_cost;             // slicing cost of a sequence start, in tokens (0: slices of equal tokens)
  float scale_log2;         // sm_scale * log2(e)
  float rope_base;          // 0 = no rotation of the query's RoPE part
};
// decode-step projections after the input GEMMs: cache append, query absorb
struct PrepareArgs {
  const bf16* row;          // [B, d_c + d_r] latent and unrotated k^R of the new tokens
  const bf16* q;            // [B, H, d_k] per-head queries
  const bf16* q_r;          // [B, H, d_r] per-head RoPE queries (unrotated)
  const bf16* W_uk;         // [H, d_k, d_c]
  bf16* cache;              // [rows, d_c + d_r], row seq_start[b] + seq_len[b] is written
  const int64_t* seq_start; // [B]
  const int32_t* seq_len;   // [B] (the new token's position)
  bf16* q_abs;              // [B, H, d_c + d_r] out
  int B, H, d_c, d_k, d_r;
  float rope_base;          // 0: no rotation
};
// in-place RoPE rotation of row-major rows (prefill): row r holds nvec
// vectors of d_r elements at p + r ld + v d_r, position r % L; base 0: none
struct RopeRowsArgs {
  bf16* p;
  int64_t ld;
  int rows, nvec, d_r, L;
  float base;
};
hipError_t launch_rope_rows(const RopeRowsArgs& a, hipStream_t st);
// the query absorption, with the cache append of the new rows on the same launch
hipError_t launch_decode_absorb(const PrepareArgs& a, hipStream_t st);

// per-head scalar gate: gated[t, h d_v + j] = sigmoid(z[t, h] + bias[h]) o[t, h d_v + j]
struct HeadGateArgs {
  const bf16* z;     // [T, ldz] gate logits x W_g^T
  const bf16* bias;  // [H] or null
  const bf16* o;     // [T, ldo] o~
  bf16* gated;       // [T, ldg]
  int T, H, d_v;
  int64_t ldz, ldo, ldg;
};
hipError_t launch_head_gate(const HeadGateArgs& a, hipStream_t st);

hipError_t launch_decode_attn(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st);
bool decode_bf16_supported(int d_c, int d_r);
// workgroups per slice (head chunks) of the bf16 decode kernel for H heads
int decode_head_chunks(int H);

// read-bandwidth probe: `blocks` workgroups stream `bytes` (a multiple of 16)
// of src and write one word each to sink[0 .. blocks - 1]
hipError_t launch_probe_read(const void* src, size_t bytes, unsigned* sink, int blocks, hipStream_t st);

// ---------------------------------------------------------------- GEMM
// C[m, n] = epi( sum_k A[m, k] * W[n, k] ), all bf16 with fp32 accumulation.
// A is [M, K] (row stride lda), W is [N, K] (row stride ldw), C is [M, N]
// (row stride ldc). Batches advance every pointer by its batch stride.
// EPI_GATE_VU: EPI_GATE whose O is the value up-projection of o_lat,
// computed in the epilogue (skinny GEMMs whose column block lies in one head)
enum GemmEpilogue { EPI_STORE = 0, EPI_GATE = 1, EPI_GATE_VU = 2 };
struct GemmArgs {
  const bf16* A;
  const bf16* W;
  bf16* C;
  const bf16* O;            // EPI_GATE: C = sigmoid(acc) * O[m, n]
  int M, N, K, batches;
  int64_t lda, ldw, ldc, ldo;
  int64_t sA, sW, sC, sO;   // batch strides (elements)
  int epi;
  int npad;                 // EPI_STORE: columns N .. npad - 1 of C are written as zeros (<= N: none)
  float* part;              // split-K partial sums (gemm_ksplit(...) > 1): gemm_part_bytes(...) bytes
  int ksplit;               // K slices of the skinny kernel (<= 1: none)
  int cw;                   // skinny kernel: output columns per workgroup (set by the launcher)
  int sk_wgs;               // shared-activation form: workgroups sharing the (column group, K chunk)
                            // space evenly (0: K slices of equal length per group; set by the launcher)
  // EPI_GATE_VU: O[m, h d_v + j] = sum_c vo[m, h, c] vw[h, j, c] (bf16-rounded),
  // vo [M, H, d_c] with row stride ldvo, vw [H, d_v, d_c]
  const bf16* vo;
  const bf16* vw;
  int vdc, vdv;
  int64_t ldvo;
};
// Whether gemm_bf16 with EPI_GATE_VU runs for this product (M rows, N = H d_v
// columns, K, value up-projection width d_c and head width d_v): the skinny
// per-wave form without K split, 32- or 64-column workgroups that divide d_v,
// d_c = 512.
bool gemm_gate_vu_supported(int M, int N, int K, int d_c, int d_v);
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st);
// Split-K plan of the skinny kernel (M <= 64) for an under-filled grid, and
// the fp32 partial-sum space it needs (0 when it does not split).
int gemm_ksplit(int M, int N, int K, int batches, int npad = 0);
size_t gemm_part_bytes(int M, int N, int K, int batches, int npad = 0);
// Up to four plain-store GEMMs C_s = A W_s^T sharing A, M <= 64 and K, in one
// launch (base gives A, lda, M, K; segment s its W, ldw, C, ldc, N;
// first_wg is filled by the launcher; count 1..4).
struct GemmGroup {
  GemmArgs base;
  const bf16* W[4];
  bf16* C[4];
  int N[4];
  int64_t ldw[4], ldc[4];
  int first_wg[4];   // first workgroup (skinny) or first n-tile (big tiles) of each segment
  int count;
  int tiles_n;       // big tiles: n-tiles over all segments (set by the launcher)
};
hipError_t launch_gemm_group_bf16(GemmGroup gg, hipStream_t st);
// The same with M >= 65 on the 256 x 256 tile kernel, when it applies (grid
// of >= 256 tiles, K >= 2048, 32-bit offsets): one launch whose n-tiles run
// over the segments side by side. Returns hipErrorNotSupported (and
// launches nothing) when the shape does not qualify.
hipError_t launch_gemm_group_big(GemmGroup gg, hipStream_t st);

// ---------------------------------------------------------------- prefill attention
// Causal flash attention, one head per (b, h): q,k,v rows of width D.
// Element (b, t, h, j) of q, k and o lives at X + b*sXb + t*sXt + h*sXh + j. V is transposed:
// element (b, key t, h, j) at b svb + h svh + j svj + t, each row (b, h, j)
// holding at least L rounded up to 64 keys, zeros past L.
// Decoupled RoPE (D_R > 0): every head's score gains q^R_(b,t,h) . k^R_(b,s), both
// already rotated; q^R at qr + b sqrb + t sqrt + h sqrh, the shared k^R at
// kr + b skrb + s skrt (D_R elements each).
struct AttnArgs {
  const bf16* q; const bf16* k; const bf16* v; bf16* o;
  int B, L, H, D;
  int64_t sqb, sqt, sqh, skb, skt, skh, svb, svj, svh, sob, sot, soh;
  float scale_log2;
  const bf16* qr; const bf16* kr;
  int D_R;
  int64_t sqrb, sqrt_, sqrh, skrb, skrt;
};
hipError_t launch_prefill_attn_bf16(const AttnArgs& a, hipStream_t st);

// ---------------------------------------------------------------- fp32 path
struct GemmF32Args {
  const float* A; const float* W; float* C; const float* O;
  int M, N, K, batches;
  int64_t lda, ldw, ldc, ldo, sA, sW, sC, sO;
  int epi;
};
hipError_t launch_gemm_f32(const GemmF32Args& g, hipStream_t st);
struct AttnF32Args {
  const float* q; const float* k; const float* v; float* o;
  int B, L, H, Dk, Dv;
  int64_t sqb, sqt, sqh, skb, skt, skh, svb, svt, svh, sob, sot, soh;
  float scale;
};
hipError_t launch_prefill_attn_f32(const AttnF32Args& a, hipStream_t st);
// one workgroup per (sequence, head); q, cache and o_lat are fp32
// (launch_decode_f32) or bf16 (launch_decode_generic_bf16: latent and RoPE
// widths outside the MFMA decode kernel's), fp32 arithmetic either way
struct DecodeF32Args {
  const void* q; const void* cache; const int64_t* seq_start; const int32_t* seq_len;
  void* o_lat; float* lse;
  int B, H, d_c, d_r;
  float scale, rope_base;
};
hipError_t launch_decode_f32(const DecodeF32Args& a, hipStream_t st);
hipError_t launch_decode_generic_bf16(const DecodeF32Args& a, hipStream_t st);

}  // namespace gmla
