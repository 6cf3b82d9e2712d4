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
//    16-byte loads, XOR-swizzled rows, 8 waves) for token counts >= 65.
//  * gemm_skinny: M <= 64 (decode-step projections). Weight-streaming bound:
//    each workgroup owns 32 output columns, its 4 waves split K and stream
//    their chunks through private LDS rings (several chunks in flight per
//    wave, no barrier in the loop), partial sums meet in LDS. A grid of
//    fewer than 512 workgroups (narrow N) also splits K across workgroups:
//    fp32 partial sums, then gemm_splitk_reduce applies the epilogue.
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

__device__ __forceinline__ float sigmoidf_fast(float x) { return 1.0f / (1.0f + __expf(-x)); }

constexpr int EPI_LDS_MAX = 163840;

// Columns of C that are written: N, or npad with zeros past N (plain store).
template <int EPI>
__device__ __forceinline__ int c_cols(const GemmArgs& g) { return (EPI == EPI_STORE && g.npad > g.N) ? g.npad : g.N; }

// Store 4 consecutive columns (n .. n+3) of row m, applying the epilogue.
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs& g, bf16* C, const bf16* O, int m, int n, float v0, float v1,
                                      float v2, float v3) {
  if (m >= g.M || n >= c_cols<EPI>(g)) return;
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
// 8 waves, two per SIMD (a wave held up issuing its share of the next
// stage's loads leaves its SIMD to the other); wave (wn, wm) of a 2 x 4 grid
// owns BN/2 x BM/4 of the output tile.
template <int BN, int BM, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void gemm_tile_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int TN = BN / 64, TM = BM / 128;
  constexpr int W_BYTES = BN * BK * 2, A_BYTES = BM * BK * 2, STAGE = W_BYTES + A_BYTES;
  constexpr int W_ROUNDS = BN * 8 / 512, A_ROUNDS = BM * 8 / 512;
  static_assert(TM >= 1 && W_ROUNDS >= 1 && A_ROUNDS >= 1, "tile too small for 8 waves");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int tiles_n = (c_cols<EPI>(g) + BN - 1) / BN, tiles_m = (g.M + BM - 1) / BM;
  const int total = tiles_n * tiles_m;
  int pid = blockIdx.x;
  // XCD-contiguous tile ranges, then grouped rasterisation (4 m-tiles per group:
  // the 32 tiles that run at once on an XCD are 4 m-tiles x 8 n-tiles, so each
  // activation line serves 8 of them; measured 4% faster than 8 x 4)
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  constexpr int GROUP = 4;
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
      const int p = r * 512 + wave * 64 + lane;
      const int row = p >> 3, c = (p & 7) ^ swz8(row);
      int gr = n0 + row;
      gr = gr < g.N ? gr : g.N - 1;
      g2lds16(W + (int64_t)gr * g.ldw + k0 + c * 8, wt + (r * 512 + wave * 64) * 16);
    }
#pragma unroll
    for (int r = 0; r < A_ROUNDS; ++r) {
      const int p = r * 512 + wave * 64 + lane;
      const int row = p >> 3, c = (p & 7) ^ swz8(row);
      int gr = m0 + row;
      gr = gr < g.M ? gr : g.M - 1;
      g2lds16(A + (int64_t)gr * g.lda + k0 + c * 8, at + (r * 512 + wave * 64) * 16);
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
    // the next stage's loads: the first wave of each SIMD right away, the
    // second after a quarter of the MFMAs, so that a wave held up by a full
    // memory queue leaves the SIMD to the other (measured 1-2% faster)
    const bool more = kt + 1 < ktiles;
    const int s1 = (kt + 1) & 1, k1 = (kt + 1) * BK;
    if (more && wave < 4) load_stage(s1, k1);
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
        const int row = wm * (BM / 4) + j * 32 + (lane & 31);
        af[j] = as_bf16x8(lds_read16(at + row * 128 + ((c ^ swz8(row)) << 4)));
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32(wf[i], af[j], acc[i][j]);
      if (more && kk == 0 && wave >= 4) load_stage(s1, k1);
    }
  }

  // Epilogue through LDS, one column half (BN/2) at a time: the waves that
  // own the half write their fp32 accumulators as [BM][BN/2] rows (padded by
  // 16 bytes), then every thread takes 8 consecutive columns of a row, applies
  // the epilogue and stores 16 contiguous bytes, so C (and O) move in whole
  // cache lines instead of 16-byte pieces of 32 rows.
  constexpr int HN = BN / 2, RS = HN * 4 + 16;  // half width, row stride in bytes
  static_assert(BM * RS <= EPI_LDS_MAX, "epilogue tile fits in LDS");
  LDS_AS float* ct = (LDS_AS float*)smem;
  // 16-byte row segments need 16-byte aligned row starts
  const bool vec16 = g.ldc % 8 == 0 && g.sC % 8 == 0 && (EPI != EPI_GATE || (g.ldo % 8 == 0 && g.sO % 8 == 0));
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    lds_barrier();  // the ring (or the previous half) is free
    if (wn == half) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int ml = wm * (BM / 4) + j * 32 + (lane & 31);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int nl = i * 32 + 8 * r4 + 4 * (lane >> 5);
            *(LDS_AS floatx4*)((LDS_AS char*)ct + ml * RS + nl * 4) =
                floatx4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
          }
        }
    }
    lds_barrier();
    constexpr int ITEMS = BM * HN / 8;  // 8 columns per item
    const int ncols = c_cols<EPI>(g);
#pragma unroll
    for (int it = tid; it < ITEMS; it += 512) {
      const int ml = it / (HN / 8), nl = (it % (HN / 8)) * 8;
      const int m = m0 + ml, n = n0 + half * HN + nl;
      if (m >= g.M || n >= ncols) continue;
      const floatx4 v0 = *(const LDS_AS floatx4*)((const LDS_AS char*)ct + ml * RS + nl * 4);
      const floatx4 v1 = *(const LDS_AS floatx4*)((const LDS_AS char*)ct + ml * RS + nl * 4 + 16);
      float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      if (n + 8 > g.N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = n + e < g.N ? v[e] : 0.f;  // padding columns
      }
      if (vec16 && n + 8 <= ncols) {
        if constexpr (EPI == EPI_GATE) {
          const u32x4 ov = *(const u32x4*)(Op + (int64_t)m * g.ldo + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = sigmoidf_fast(v[2 * e]) * bf16_bits_to_f32((unsigned short)(ov[e] & 0xffff));
            v[2 * e + 1] = sigmoidf_fast(v[2 * e + 1]) * bf16_bits_to_f32((unsigned short)(ov[e] >> 16));
          }
        }
        *(u32x4*)(Cp + (int64_t)m * g.ldc + n) =
            u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      } else {
        store4<EPI>(g, Cp, Op, m, n, v[0], v[1], v[2], v[3]);  // the written width is a multiple of 4
        store4<EPI>(g, Cp, Op, m, n + 4, v[4], v[5], v[6], v[7]);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Skinny GEMM (M <= 64): pure weight streaming. A workgroup owns 32 output
// columns and all M rows; its 4 waves split K into 64-wide chunks (wave w
// takes chunks w, w + 4, ...). Each wave streams its chunks HBM -> LDS
// through a private ring of NBUF buffers with 1 KiB direct-to-LDS loads
// (4 KiB of weights + 32 MT rows of A per chunk), so up to NBUF chunks per
// wave are in flight and no barrier is needed until the final reduction.
// Rows are 128 bytes; the 16-byte piece p of row r is stored at piece
// p ^ ((r >> 2) & 7), which makes the fragment reads (32 rows at one piece
// per half-wave) hit 32 distinct bank groups.
// NT = 2: a workgroup owns 64 columns, so each activation chunk in LDS
// serves two weight tiles (half the activation bytes per weight byte) at the
// price of one buffer less per wave.
template <int MT, int NT>
struct SkinnyCfg {
  static constexpr int NBUF = (MT == 1 ? 4 : 3) - (NT - 1);
  static constexpr int W_BYTES = NT * 32 * 128;      // 32 NT weight rows x 64 K
  static constexpr int A_BYTES = MT * 32 * 128;      // 32 MT rows of A x 64 K
  static constexpr int BUF_BYTES = W_BYTES + A_BYTES;
  static constexpr int WAVE_BYTES = NBUF * BUF_BYTES;
  static constexpr int RPC = (W_BYTES + A_BYTES) / 1024;  // DMA instructions per chunk
  static constexpr int LDS_BYTES = 4 * WAVE_BYTES;
  static_assert(NT == 1 || NT == 2, "32 or 64 columns per workgroup");
  static_assert(LDS_BYTES <= 163840, "LDS budget");
  static_assert(LDS_BYTES >= 4 * NT * MT * 16 * 64 * 4, "reduction fits in the ring");
  static_assert((NBUF - 1) * RPC < 64, "vmcnt range");
};
// use 64-column workgroups when the grid still has a workgroup per CU
constexpr bool kSkinnyNT2 = true;

template <int RPC, int MAXP>
__device__ __forceinline__ void skinny_wait(int pending) {
  if constexpr (MAXP >= 3) { if (pending >= 3) { wait_vmcnt<3 * RPC>(); return; } }
  if constexpr (MAXP >= 2) { if (pending >= 2) { wait_vmcnt<2 * RPC>(); return; } }
  if constexpr (MAXP >= 1) { if (pending >= 1) { wait_vmcnt<RPC>(); return; } }
  wait_vmcnt<0>();
}

// Columns n0 .. n0 + cw - 1 (cw <= 32 NT, a multiple of 4) of batch `batch`,
// K slice zi of nz. Weight rows from n0 + cw on are not this workgroup's: the
// tile re-reads its last row there (a cache hit) and those columns are not
// stored, so each workgroup streams exactly its own cw rows.
template <int MT, int NT, int EPI>
__device__ __forceinline__ void skinny_body(const GemmArgs& g, int n0, int cw, int batch, int zi, int nz) {
  using C = SkinnyCfg<MT, NT>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bf16* A = g.A + batch * g.sA;
  const bf16* W = g.W + batch * g.sW;
  bf16* Cp = g.C + batch * g.sC;
  const bf16* Op = (EPI == EPI_GATE) ? g.O + batch * g.sO : nullptr;
  LDS_AS char* ring = smem + wave * C::WAVE_BYTES;
  // K slice of this workgroup: chunks c_lo .. c_hi - 1 (all of K without split)
  const int all_chunks = g.K / 64;
  const int per = (all_chunks + nz - 1) / nz;
  const int c_lo = zi * per;
  const int c_hi = (c_lo + per) < all_chunks ? (c_lo + per) : all_chunks;
  const unsigned ring_addr = (unsigned)(uintptr_t)ring;

  // DMA: instruction q of a 32-row tile moves rows 8q .. 8q + 7; lane l
  // writes physical piece l % 8 of row 8q + l / 8, i.e. logical piece
  // (l % 8) ^ ((row >> 2) & 7). Rows past the workgroup's last re-read it.
  const int lr = lane >> 3;
  const int n_end = (n0 + cw) < g.N ? (n0 + cw) : g.N;
  auto piece_off = [&](int row) { return ((lane & 7) ^ ((row >> 2) & 7)) * 16; };
  auto issue = [&](int b, int j) {
    const unsigned dst = ring_addr + b * C::BUF_BYTES;
#pragma unroll
    for (int q = 0; q < 4 * NT; ++q) {
      int row = n0 + 8 * q + lr;
      row = row < n_end ? row : n_end - 1;
      const unsigned long long base = (unsigned long long)(uintptr_t)(W + (int64_t)j * 64);
      g2lds16_s(base, (unsigned)(row * g.ldw * 2 + piece_off(8 * q + lr)), dst + q * 1024);
    }
#pragma unroll
    for (int q = 0; q < 4 * MT; ++q) {
      int row = 8 * q + lr;
      row = row < g.M ? row : g.M - 1;
      const unsigned long long base = (unsigned long long)(uintptr_t)(A + (int64_t)j * 64);
      g2lds16_s(base, (unsigned)(row * g.lda * 2 + piece_off(8 * q + lr)), dst + C::W_BYTES + q * 1024);
    }
  };
  // fragment read: row r (32 rows per MFMA operand), logical piece p
  auto frag = [&](const LDS_AS char* tile, int r, int p) -> bf16x8 {
    return as_bf16x8(lds_read16(tile + r * 128 + ((p ^ ((r >> 2) & 7)) << 4)));
  };

  floatx16 acc[NT][MT];
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[u][t] = floatx16{};
  const int span = c_hi > c_lo ? c_hi - c_lo : 0;
  const int nmy = span > wave ? (span - wave + 3) / 4 : 0;  // this wave's chunks: c_lo + wave, + 4, ...
#pragma unroll
  for (int b = 0; b < C::NBUF; ++b)
    if (b < nmy) issue(b, c_lo + wave + 4 * b);
  const int r32 = lane & 31, hk = lane >> 5;
  for (int i = 0; i < nmy; ++i) {
    const int b = i % C::NBUF;
    int pend = nmy - 1 - i;
    pend = pend < C::NBUF - 1 ? pend : C::NBUF - 1;
    skinny_wait<C::RPC, C::NBUF - 1>(pend);
    const LDS_AS char* wt = ring + b * C::BUF_BYTES;
    const LDS_AS char* at = wt + C::W_BYTES;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) af[t] = frag(at, 32 * t + r32, 2 * kk + hk);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const bf16x8 wf = frag(wt + u * 4096, r32, 2 * kk + hk);
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[u][t] = mfma32(wf, af[t], acc[u][t]);
      }
    }
    if (i + C::NBUF < nmy) {
      wait_lgkm0();  // this buffer's fragments are in registers before it is refilled
      issue(b, c_lo + wave + 4 * (i + C::NBUF));
    }
  }

  __syncthreads();  // every wave is done with its ring: reuse it for the reduction
  constexpr int NA = NT * MT;  // accumulators per wave
  LDS_AS float* red = (LDS_AS float*)smem;  // [4 waves][NT MT][16][64]
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wave * NA + u * MT + t) * 16 + r) * 64 + lane] = acc[u][t][r];
  __syncthreads();
  // wave w finishes register group r4 = w (4 consecutive columns per lane)
#pragma unroll
  for (int ut = 0; ut < NA; ++ut) {
    const int u = ut / MT, t = ut % MT;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * wave + e;
      v[e] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v[e] += red[((w * NA + ut) * 16 + r) * 64 + lane];
    }
    const int m = 32 * t + (lane & 31);
    const int n = n0 + 32 * u + 8 * wave + 4 * (lane >> 5);
    if (n >= n0 + cw) continue;  // another workgroup's columns
    if (nz > 1) {  // partial sums [slice][batch][M][N rounded up to 4]
      const int ldp = (g.N + 3) & ~3;
      if (m < g.M && n < g.N)
        *(float4*)(g.part + (((int64_t)zi * g.batches + batch) * g.M + m) * ldp + n) =
            make_float4(v[0], v[1], v[2], v[3]);
    } else {
      store4<EPI>(g, Cp, Op, m, n, v[0], v[1], v[2], v[3]);
    }
  }
}

template <int MT, int NT, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  skinny_body<MT, NT, EPI>(g, blockIdx.x * g.cw, g.cw, blockIdx.y, blockIdx.z, gridDim.z);
}

// Several plain-store GEMMs that share A, M and K in one grid: segment s
// owns workgroups first_wg[s] .. first_wg[s + 1] - 1.
template <int MT, int NT>
__global__ __launch_bounds__(256) void gemm_skinny_group_kernel(GemmGroup gg) {
  const int x = blockIdx.x;
  const int s = (x >= gg.first_wg[1]) + (x >= gg.first_wg[2]) + (x >= gg.first_wg[3]);
  GemmArgs g = gg.base;
  g.W = s == 0 ? gg.W[0] : s == 1 ? gg.W[1] : s == 2 ? gg.W[2] : gg.W[3];
  g.C = s == 0 ? gg.C[0] : s == 1 ? gg.C[1] : s == 2 ? gg.C[2] : gg.C[3];
  g.N = s == 0 ? gg.N[0] : s == 1 ? gg.N[1] : s == 2 ? gg.N[2] : gg.N[3];
  g.ldw = s == 0 ? gg.ldw[0] : s == 1 ? gg.ldw[1] : s == 2 ? gg.ldw[2] : gg.ldw[3];
  g.ldc = s == 0 ? gg.ldc[0] : s == 1 ? gg.ldc[1] : s == 2 ? gg.ldc[2] : gg.ldc[3];
  const int first = s == 0 ? 0 : s == 1 ? gg.first_wg[1] : s == 2 ? gg.first_wg[2] : gg.first_wg[3];
  skinny_body<MT, NT, EPI_STORE>(g, (x - first) * g.cw, g.cw, 0, 0, 1);
}

// Sum the split-K partial sums of 4 consecutive columns and apply the
// epilogue. Eight threads share one (batch, m, 4 columns) quad: thread j adds
// slices j, j + 8, ..., keeping the loads of four slices in flight at once,
// and a butterfly over the eight threads completes the sum, so a deep split
// costs a few memory latencies instead of one per slice.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(GemmArgs g) {
  const int ldp = (g.N + 3) & ~3, q4 = ldp / 4;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  const bool ok = i < (int64_t)g.batches * g.M * q4;
  const int64_t slice = (int64_t)g.batches * g.M * ldp;
  const int64_t bm = i / q4;
  const int n = (int)(i % q4) * 4;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const float* p = g.part + bm * ldp + n;
    for (int z0 = j; z0 < g.ksplit; z0 += 32) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int z = z0 + 8 * u;
        v[u] = z < g.ksplit ? *(const float4*)(p + z * slice) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
      }
    }
  }
  // every thread of the wave takes part in the exchange
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  if (!ok || j != 0) return;
  const int m = (int)(bm % g.M), batch = (int)(bm / g.M);
  bf16* Cp = g.C + batch * g.sC;
  const bf16* Op = (EPI == EPI_GATE) ? g.O + batch * g.sO : nullptr;
  store4<EPI>(g, Cp, Op, m, n, acc.x, acc.y, acc.z, acc.w);
}

template <int MT, int NT, int EPI>
static hipError_t launch_skinny(const GemmArgs& g, hipStream_t st) {
  using C = SkinnyCfg<MT, NT>;
  auto kern = gemm_skinny_kernel<MT, NT, EPI>;
  {
    hipError_t e = lds_opt_in((const void*)kern, C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const int z = g.ksplit > 1 ? g.ksplit : 1;
  if (z > 1 && !g.part) return hipErrorInvalidValue;
  if (g.cw <= 0 || g.cw > 32 * NT || g.cw % 4 != 0) return hipErrorInvalidValue;
  hipError_t e = launch(kern, dim3((g.N + g.cw - 1) / g.cw, g.batches, z), dim3(256), C::LDS_BYTES, st, g);
  if (e != hipSuccess || z == 1) return e;
  const int64_t n4 = (int64_t)g.batches * g.M * (((g.N + 3) & ~3) / 4);  // output quads, 8 threads each
  return launch(gemm_splitk_reduce_kernel<EPI>, dim3((unsigned)((8 * n4 + 255) / 256)), dim3(256), 0, st, g);
}


// ----------------------------------------------------------------------------
template <int BN, int BM, int EPI>
static hipError_t launch_tile(const GemmArgs& g, hipStream_t st) {
  constexpr int RING = 2 * (BN + BM) * 64 * 2, EPIL = BM * ((BN / 2) * 4 + 16);
  constexpr int LDS = RING > EPIL ? RING : EPIL;
  auto kern = gemm_tile_kernel<BN, BM, EPI>;
  {
    hipError_t e = lds_opt_in((const void*)kern, LDS);
    if (e != hipSuccess) return e;
  }
  const int ncols = (EPI == EPI_STORE && g.npad > g.N) ? g.npad : g.N;
  const int tiles = ((ncols + BN - 1) / BN) * ((g.M + BM - 1) / BM);
  return launch(kern, dim3(tiles, g.batches), dim3(512), LDS, st, g);
}

static bool skinny_path(int M, int N, int npad) { return M <= 64 && !(npad > N); }

// Columns per skinny workgroup. With up to 32 rows the kernel streams
// weight rows at one workgroup per compute unit, so its time follows the
// rows the busiest unit streams: (columns per workgroup) x (rounds of the
// grid). Pick the width (a multiple of 4 up to 64; above 32 the 64-column
// form) that minimises it, the widest among equals (fewer workgroups
// re-read the activations): e.g. 7168 columns run as 256 workgroups of 28
// rather than 224 of 32 (measured 29.5 -> 25.4 us at K = 8192). With 33..64
// rows (two 32-row blocks, fewer ring buffers per wave) narrower
// workgroups measured slower: there the widths stay 32, or 64 while that
// still gives a workgroup per compute unit.
static int skinny_cols(const int* N, int nseg, int batches, int M) {
  if (M > 32) {
    long long wide = 0;
    for (int s = 0; s < nseg; ++s) wide += (long long)((N[s] + 63) / 64) * batches;
    return kSkinnyNT2 && wide >= 256 ? 64 : 32;
  }
  int best = 32;
  long long best_cost = -1;
  for (int cw = 64; cw >= 4; cw -= 4) {
    if (cw > 32 && !kSkinnyNT2) continue;
    long long wgs = 0;
    for (int s = 0; s < nseg; ++s) wgs += (long long)((N[s] + cw - 1) / cw) * batches;
    const long long cost = (long long)cw * ((wgs + 255) / 256);
    if (best_cost < 0 || cost < best_cost) {
      best = cw;
      best_cost = cost;
    }
  }
  return best;
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t st) {
  if (skinny_path(g.M, g.N, EPI == EPI_STORE ? g.npad : 0)) {
    // the DMA offsets are 32-bit: every row start must be below 4 GiB
    if ((long long)g.N * g.ldw * 2 >= (1LL << 32) || (long long)g.M * g.lda * 2 >= (1LL << 32))
      return hipErrorInvalidValue;
    GemmArgs h = g;
    if (g.ksplit > 1) {
      h.cw = 32;
    } else {
      const int n1[1] = {g.N};
      h.cw = skinny_cols(n1, 1, g.batches, g.M);
    }
    const bool nt2 = h.cw > 32;
    if (g.M <= 32) return nt2 ? launch_skinny<1, 2, EPI>(h, st) : launch_skinny<1, 1, EPI>(h, st);
    return nt2 ? launch_skinny<2, 2, EPI>(h, st) : launch_skinny<2, 1, EPI>(h, st);
  }
  const long long big_tiles = (long long)((g.N + 255) / 256) * ((g.M + 255) / 256) * g.batches;
  if (big_tiles >= 256) return launch_tile<256, 256, EPI>(g, st);
  return launch_tile<128, 128, EPI>(g, st);
}

// Split K when the skinny grid has fewer than 64 workgroups (a quarter of
// the compute units; a grid of a few hundred loses more to the extra pass
// than it gains), up to 256 workgroups, keeping at least 4 chunks of 64 per
// workgroup (one per wave).
int gemm_ksplit(int M, int N, int K, int batches, int npad) {
  if (M <= 0 || N <= 0 || K <= 0 || batches <= 0 || !skinny_path(M, N, npad)) return 1;
  const long long wgs = (long long)((N + 31) / 32) * batches;
  if (wgs >= 64) return 1;
  const int want = (int)((256 + wgs - 1) / wgs);
  const int most = K / 64 / 4;
  const int z = want < most ? want : most;
  if (z <= 1) return 1;
  const int per = (K / 64 + z - 1) / z;  // no empty slice
  return (K / 64 + per - 1) / per;
}

size_t gemm_part_bytes(int M, int N, int K, int batches, int npad) {
  const int z = gemm_ksplit(M, N, K, batches, npad);
  return z > 1 ? (size_t)z * batches * M * (size_t)((N + 3) & ~3) * 4 : 0;
}

template <int MT, int NT>
static hipError_t launch_group(const GemmGroup& gg, int wgs, hipStream_t st) {
  using C = SkinnyCfg<MT, NT>;
  auto kern = gemm_skinny_group_kernel<MT, NT>;
  {
    hipError_t e = lds_opt_in((const void*)kern, C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  return launch(kern, dim3(wgs), dim3(256), C::LDS_BYTES, st, gg);
}

hipError_t launch_gemm_group_bf16(GemmGroup gg, hipStream_t st) {
  const GemmArgs& b = gg.base;
  if (gg.count < 1 || gg.count > 4 || b.M <= 0 || b.M > 64 || b.K % 64 != 0) return hipErrorInvalidValue;
  if ((long long)b.M * b.lda * 2 >= (1LL << 32)) return hipErrorInvalidValue;
  int first = 0;
  for (int s = 0; s < gg.count; ++s)
    if (gg.N[s] <= 0) return hipErrorInvalidValue;
  const int cols = skinny_cols(gg.N, gg.count, 1, b.M);
  for (int s = 0; s < 4; ++s) {
    if (s < gg.count) {
      if (gg.N[s] <= 0 || gg.N[s] % 4 != 0 || (long long)gg.N[s] * gg.ldw[s] * 2 >= (1LL << 32))
        return hipErrorInvalidValue;
      if (s > 0) gg.first_wg[s] = first;
      first += (gg.N[s] + cols - 1) / cols;
    } else {
      gg.first_wg[s] = INT32_MAX;  // no workgroup reaches an unused segment
    }
  }
  gg.first_wg[0] = 0;
  gg.base.batches = 1;
  gg.base.ksplit = 1;
  gg.base.epi = EPI_STORE;
  gg.base.npad = 0;
  gg.base.cw = cols;
  if (b.M <= 32) return cols > 32 ? launch_group<1, 2>(gg, first, st) : launch_group<1, 1>(gg, first, st);
  return cols > 32 ? launch_group<2, 2>(gg, first, st) : launch_group<2, 1>(gg, first, st);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batches <= 0) return hipSuccess;
  if (g.npad > g.N && (g.epi != EPI_STORE || g.npad % 4 != 0)) return hipErrorInvalidValue;
  if (g.K % 64 != 0 || (g.npad > g.N ? g.npad : g.N) % 4 != 0) return hipErrorInvalidValue;
  return g.epi == EPI_GATE ? launch_epi<EPI_GATE>(g, st) : launch_epi<EPI_STORE>(g, st);
}

}  // namespace gmla
