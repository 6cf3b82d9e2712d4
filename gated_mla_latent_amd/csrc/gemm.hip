// bf16 GEMMs with fp32 accumulation on gfx950 MFMA, with the gate epilogue.
//
//   C[m, n] = epi( sum_k A[m, k] W[n, k] )          (W in the [out, in] layout)
//   EPI_STORE: C = acc                                (projections W_c, W_q,
//                                                      W_UK, W_UV, W_o)
//   EPI_GATE:  C = Sigmoid(acc) * O[m, n]            ("Gated MLA 计算公式" §二:
//                                                      the per-channel gate
//                                                      applied to o~ before W_o)
//
// Both operands are K-contiguous, so every MFMA fragment is a 16-byte read.
// The weight is the MFMA "A" side: the accumulator layout then gives each lane
// four consecutive output columns, which become one 8-byte store.
//
// Two kernels:
//  * gemm_tile: LDS-tiled (BN x BM x 64 tiles, 2 stages, direct-to-LDS
//    16-byte loads, XOR-swizzled rows) for token counts >= 65.
//  * gemm_skinny: M <= 64 (decode-step projections). Weight-streaming bound:
//    each workgroup owns 32 output columns, its 4 waves split K, fragments go
//    straight from global memory to VGPRs (64 contiguous bytes per lane, with
//    K permuted identically on both operands), partial sums meet in LDS.
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

__device__ __forceinline__ float sigmoidf_fast(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Store 4 consecutive columns (n .. n+3) of row m, applying the epilogue.
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs& g, bf16* C, const bf16* O, int m, int n, float v0, float v1,
                                      float v2, float v3) {
  if (m >= g.M || n >= g.N) return;
  if constexpr (EPI == EPI_GATE) {
    u32x2 ov = *(const u32x2*)(O + (int64_t)m * g.ldo + n);
    v0 = sigmoidf_fast(v0) * bf16_bits_to_f32((unsigned short)(ov[0] & 0xffff));
    v1 = sigmoidf_fast(v1) * bf16_bits_to_f32((unsigned short)(ov[0] >> 16));
    v2 = sigmoidf_fast(v2) * bf16_bits_to_f32((unsigned short)(ov[1] & 0xffff));
    v3 = sigmoidf_fast(v3) * bf16_bits_to_f32((unsigned short)(ov[1] >> 16));
  }
  *(u32x2*)(C + (int64_t)m * g.ldc + n) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

}  // namespace

// ----------------------------------------------------------------------------
template <int BN, int BM, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int TN = BN / 64, TM = BM / 64;
  constexpr int W_BYTES = BN * BK * 2, A_BYTES = BM * BK * 2, STAGE = W_BYTES + A_BYTES;
  constexpr int W_ROUNDS = BN * 8 / 256, A_ROUNDS = BM * 8 / 256;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int tiles_n = (g.N + BN - 1) / BN, tiles_m = (g.M + BM - 1) / BM;
  const int total = tiles_n * tiles_m;
  int pid = blockIdx.x;
  // XCD-contiguous tile ranges, then grouped rasterisation (8 m-tiles per group)
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int grp = pid / group_size;
  const int first_m = grp * GROUP;
  const int gm = (tiles_m - first_m) < GROUP ? (tiles_m - first_m) : GROUP;
  const int tile_m = first_m + (pid % group_size) % gm;
  const int tile_n = (pid % group_size) / gm;
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  const int batch = blockIdx.y;
  const bf16* A = g.A + batch * g.sA;
  const bf16* W = g.W + batch * g.sW;
  bf16* Cp = g.C + batch * g.sC;
  const bf16* Op = (EPI == EPI_GATE) ? g.O + batch * g.sO : nullptr;

  auto load_stage = [&](int s, int k0) {
    LDS_AS char* wt = smem + s * STAGE;
    LDS_AS char* at = wt + W_BYTES;
#pragma unroll
    for (int r = 0; r < W_ROUNDS; ++r) {
      const int p = r * 256 + wave * 64 + lane;
      const int row = p >> 3, c = (p & 7) ^ swz8(row);
      int gr = n0 + row;
      gr = gr < g.N ? gr : g.N - 1;
      g2lds16(W + (int64_t)gr * g.ldw + k0 + c * 8, wt + (r * 256 + wave * 64) * 16);
    }
#pragma unroll
    for (int r = 0; r < A_ROUNDS; ++r) {
      const int p = r * 256 + wave * 64 + lane;
      const int row = p >> 3, c = (p & 7) ^ swz8(row);
      int gr = m0 + row;
      gr = gr < g.M ? gr : g.M - 1;
      g2lds16(A + (int64_t)gr * g.lda + k0 + c * 8, at + (r * 256 + wave * 64) * 16);
    }
  };

  floatx16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = floatx16{};

  const int ktiles = g.K / BK;
  load_stage(0, 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    wait_vmcnt<0>();
    lds_barrier();
    if (kt + 1 < ktiles) load_stage((kt + 1) & 1, (kt + 1) * BK);
    const LDS_AS char* wt = smem + (kt & 1) * STAGE;
    const LDS_AS char* at = wt + W_BYTES;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8 wf[TN], af[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int row = wn * (BN / 2) + i * 32 + (lane & 31);
        wf[i] = as_bf16x8(lds_read16(wt + row * 128 + ((c ^ swz8(row)) << 4)));
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int row = wm * (BM / 2) + j * 32 + (lane & 31);
        af[j] = as_bf16x8(lds_read16(at + row * 128 + ((c ^ swz8(row)) << 4)));
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32(wf[i], af[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * (BM / 2) + j * 32 + (lane & 31);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = n0 + wn * (BN / 2) + i * 32 + 8 * r4 + 4 * (lane >> 5);
        store4<EPI>(g, Cp, Op, m, n, acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                    acc[i][j][4 * r4 + 3]);
      }
    }
}

// ----------------------------------------------------------------------------
template <int MT, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  __shared__ float red[4][MT][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 32;
  const int batch = blockIdx.y;
  const bf16* A = g.A + batch * g.sA;
  const bf16* W = g.W + batch * g.sW;
  bf16* Cp = g.C + batch * g.sC;
  const bf16* Op = (EPI == EPI_GATE) ? g.O + batch * g.sO : nullptr;

  int wr = n0 + (lane & 31);
  wr = wr < g.N ? wr : g.N - 1;
  const bf16* wrow = W + (int64_t)wr * g.ldw + 32 * (lane >> 5);
  const bf16* arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    int ar = t * 32 + (lane & 31);
    ar = ar < g.M ? ar : g.M - 1;
    arow[t] = A + (int64_t)ar * g.lda + 32 * (lane >> 5);
  }

  floatx16 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx16{};

  const int chunks = g.K / 64;
  u32x4 wv[2][4], av[2][MT][4];
  auto fetch = [&](int buf, int j) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) wv[buf][kk] = *(const u32x4*)(wrow + 64 * j + 8 * kk);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) av[buf][t][kk] = *(const u32x4*)(arow[t] + 64 * j + 8 * kk);
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma32(as_bf16x8(wv[buf][kk]), as_bf16x8(av[buf][t][kk]), acc[t]);
  };
  int j = wave;
  if (j < chunks) fetch(0, j);
  for (; j < chunks; j += 8) {
    if (j + 4 < chunks) fetch(1, j + 4);
    compute(0);
    if (j + 4 >= chunks) break;
    if (j + 8 < chunks) fetch(0, j + 8);
    compute(1);
  }

#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][t][r][lane] = acc[t][r];
  __syncthreads();
  // wave w finishes register group r4 = w (4 consecutive columns per lane)
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * wave + e;
      v[e] = red[0][t][r][lane] + red[1][t][r][lane] + red[2][t][r][lane] + red[3][t][r][lane];
    }
    const int m = t * 32 + (lane & 31);
    const int n = n0 + 8 * wave + 4 * (lane >> 5);
    store4<EPI>(g, Cp, Op, m, n, v[0], v[1], v[2], v[3]);
  }
}

// ----------------------------------------------------------------------------
template <int BN, int BM, int EPI>
static hipError_t launch_tile(const GemmArgs& g, hipStream_t st) {
  constexpr int LDS = 2 * (BN + BM) * 64 * 2;
  auto kern = gemm_tile_kernel<BN, BM, EPI>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tiles = ((g.N + BN - 1) / BN) * ((g.M + BM - 1) / BM);
  hipLaunchKernelGGL(kern, dim3(tiles, g.batches), dim3(256), LDS, st, g);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 64) {
    const dim3 grid((g.N + 31) / 32, g.batches);
    if (g.M <= 32) hipLaunchKernelGGL((gemm_skinny_kernel<1, EPI>), grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_skinny_kernel<2, EPI>), grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  const long long big_tiles = (long long)((g.N + 255) / 256) * ((g.M + 255) / 256) * g.batches;
  if (big_tiles >= 256) return launch_tile<256, 256, EPI>(g, st);
  return launch_tile<128, 128, EPI>(g, st);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batches <= 0) return hipSuccess;
  if (g.K % 64 != 0 || g.N % 4 != 0) return hipErrorInvalidValue;
  return g.epi == EPI_GATE ? launch_epi<EPI_GATE>(g, st) : launch_epi<EPI_STORE>(g, st);
}

}  // namespace gmla
