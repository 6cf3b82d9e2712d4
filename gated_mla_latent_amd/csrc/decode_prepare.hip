// RoPE rotation kernels (bf16, gfx950): the decode step's cache append and
// query absorption, and the in-place rotation of prefill's RoPE rows.
//
// The projections around one decode step, after the input GEMMs (x W_c^T,
// x W^KR^T, x W_q^T, x W^QR^T) have run:
//
//   * append: the new token's cache row [c ; RoPE(k^R, pos)] goes to row
//     seq_start[b] + seq_len[b] of the cache, pos = seq_len[b]
//     ("LLM 注意力与计算内核精读笔记 · 03", §5.2: the shared RoPE key is
//     rotated before it is cached);
//   * absorb: q~^(h) = (W_UK^(h))^T q^(h) (same page, §5.1 and the answer to
//     exercise 4), written next to the per-head RoPE query, which stays
//     unrotated (the decode kernel rotates it at its position).
//
// Both are small next to the weight-streaming GEMMs; the absorb reads W_UK
// once (H d_k d_c bf16) for the whole batch.
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

// The new row of sequence b: the latent copied in 16-byte pieces (4-byte
// ones when d_c + d_r is not a multiple of 8), then the RoPE part rotated
// pair by pair, by the threads of one workgroup.
__device__ void append_row(const PrepareArgs& a, int b) {
  const int W = a.d_c + a.d_r;
  const int pos = a.seq_len[b];
  const int64_t row = a.seq_start[b] + pos;
  const bf16* src = a.row + (int64_t)b * W;
  bf16* dst = a.cache + row * W;
  if (W % 8 == 0) {  // rows 16-byte aligned
    for (int i = threadIdx.x; i < a.d_c / 8; i += blockDim.x)
      *(u32x4*)(dst + 8 * i) = *(const u32x4*)(src + 8 * i);
  } else {  // W is even: rows 4-byte aligned
    for (int i = threadIdx.x; i < a.d_c / 2; i += blockDim.x)
      *(unsigned*)(dst + 2 * i) = *(const unsigned*)(src + 2 * i);
  }
  if (a.d_r > 0) {
    const double lb = a.rope_base != 0.0f ? log2((double)a.rope_base) : 0.0;
    for (int i = threadIdx.x; i < a.d_r / 2; i += blockDim.x) {
      const unsigned v = *(const unsigned*)(src + a.d_c + 2 * i);
      float x0 = bf16_bits_to_f32((unsigned short)(v & 0xffff)), x1 = bf16_bits_to_f32((unsigned short)(v >> 16));
      if (a.rope_base != 0.0f) rope_pair(x0, x1, i, a.d_r, lb, (double)pos);
      *(unsigned*)(dst + a.d_c + 2 * i) = pack_bf16x2(x0, x1);
    }
  }
}

// Workgroup (head h, 64 latent columns c0 ..): q~[b, h, c0 + j] =
// sum_k q[b, h, k] W_UK[h, k, c0 + j], a [B x d_k] . [d_k x 64] product on
// v_mfma_f32_32x32x16_bf16. W_UK's block is staged in LDS transposed
// (column-major, so that the B operand is one 16-byte read per lane); the
// queries of head h follow in blocks of 64 rows, zero past B. Wave w computes
// the 32 x 32 tile (rows 32 (w >> 1), columns 32 (w & 1)) of each block. The
// workgroup with c0 = 0 also copies the head's RoPE query into q_abs. The
// workgroups also append the new cache rows, one sequence each in turn (the
// append rides on this launch instead of one of its own: 4 us less per
// step).
constexpr int kAbsorbRows = 64;  // batch rows per block
__device__ __forceinline__ int absorb_ld(int d_k) { return d_k + 8; }  // LDS row length (bf16), 16-byte rows
__global__ __launch_bounds__(256) void decode_absorb_kernel(PrepareArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int KP = absorb_ld(a.d_k);
  bf16* sw = (bf16*)smem_raw;       // [64 columns][KP]: W_UK^T block
  bf16* sq = sw + 64 * KP;          // [kAbsorbRows][KP]: queries
  const int h = blockIdx.x, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = a.d_c + a.d_r, KC = a.d_k / 8;  // 16-byte chunks per query row
  const bf16* wuk = a.W_uk + (int64_t)h * a.d_k * a.d_c + c0;
  for (int i = tid; i < a.d_k * 8; i += 256) {  // row k, 8 columns 8 ch ..
    const int k = i >> 3, ch = i & 7;
    const u32x4 v = *(const u32x4*)(wuk + (int64_t)k * a.d_c + 8 * ch);
    const bf16x8 e = as_bf16x8(v);
#pragma unroll
    for (int j = 0; j < 8; ++j) sw[(8 * ch + j) * KP + k] = e[j];
  }
  const int rt = wave >> 1, ct = wave & 1;
  const int r32 = lane & 31, k8 = 8 * (lane >> 5);
  for (int b0 = 0; b0 < a.B; b0 += kAbsorbRows) {
    const int nb = (a.B - b0) < kAbsorbRows ? (a.B - b0) : kAbsorbRows;
    __syncthreads();  // the previous block is consumed (and W_UK is staged)
    for (int i = tid; i < kAbsorbRows * KC; i += 256) {
      const int r = i / KC, ch = i % KC;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nb) v = *(const u32x4*)(a.q + ((int64_t)(b0 + r) * a.H + h) * a.d_k + 8 * ch);
      *(u32x4*)(sq + r * KP + 8 * ch) = v;
    }
    __syncthreads();
    if (32 * rt < nb) {
      floatx16 acc = {};
      const bf16* pa = sq + (32 * rt + r32) * KP + k8;
      const bf16* pb = sw + (32 * ct + r32) * KP + k8;
      for (int k0 = 0; k0 < a.d_k; k0 += 16)
        acc = mfma32(as_bf16x8(*(const u32x4*)(pa + k0)), as_bf16x8(*(const u32x4*)(pb + k0)), acc);
      const int col = c0 + 32 * ct + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < nb) a.q_abs[((int64_t)(b0 + row) * a.H + h) * W + col] = (bf16)acc[r];
      }
    }
  }
  // the cache appends, dealt round robin over all H x (d_c / 64) workgroups
  for (int b = (int)blockIdx.y * a.H + h; b < a.B; b += a.H * (int)gridDim.y) append_row(a, b);
  if (blockIdx.y == 0 && a.d_r > 0) {
    const int P = a.d_r / 2;
    for (int i = tid; i < a.B * P; i += 256) {
      const int b = i / P, j = i % P;
      *(unsigned*)(a.q_abs + ((int64_t)b * a.H + h) * W + a.d_c + 2 * j) =
          *(const unsigned*)(a.q_r + ((int64_t)b * a.H + h) * a.d_r + 2 * j);
    }
  }
}

// Rotate in place every RoPE vector of a row-major buffer: row r holds nvec
// vectors of d_r elements (vector v at p + r ld + v d_r), at position r % L
// (rows are sequence-major, L tokens each). One thread per pair.
__global__ __launch_bounds__(256) void rope_rows_kernel(RopeRowsArgs a) {
  const int P = a.d_r / 2;
  const int64_t n = (int64_t)a.rows * a.nvec * P;
  const double lb = log2((double)a.base);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int pi = (int)(i % P);
    const int64_t rv = i / P;
    const int v = (int)(rv % a.nvec);
    const int64_t r = rv / a.nvec;
    unsigned* w = (unsigned*)(a.p + r * a.ld + (int64_t)v * a.d_r + 2 * pi);
    const unsigned u = *w;
    float x0 = bf16_bits_to_f32((unsigned short)(u & 0xffff)), x1 = bf16_bits_to_f32((unsigned short)(u >> 16));
    rope_pair(x0, x1, pi, a.d_r, lb, (double)(r % a.L));
    *w = pack_bf16x2(x0, x1);
  }
}

}  // namespace

hipError_t launch_rope_rows(const RopeRowsArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.nvec <= 0 || a.d_r <= 0 || a.base == 0.0f) return hipSuccess;
  if (a.d_r % 2 != 0 || a.ld % 2 != 0 || a.L <= 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.rows * a.nvec * (a.d_r / 2);
  const int64_t blocks = (n + 255) / 256;
  return launch(rope_rows_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, st, a);
}

hipError_t launch_decode_absorb(const PrepareArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (a.d_c % 64 != 0 || a.d_k <= 0 || a.d_k > 128 || a.d_k % 16 != 0 || a.d_r % 2 != 0 || a.H <= 0)
    return hipErrorInvalidValue;
  const size_t lds = (size_t)(64 + kAbsorbRows) * (a.d_k + 8) * 2;  // <= 34 KiB
  return launch(decode_absorb_kernel, dim3(a.H, a.d_c / 64), dim3(256), lds, st, a);
}

}  // namespace gmla
