// bf16 GEMMs with fp32 accumulation on gfx950 MFMA, with the gate epilogue.
//
//   C[m, n] = epi( sum_k A[m, k] W[n, k] )          (W in the [out, in] layout)
//   EPI_STORE: C = acc                                (projections W_c, W_q,
//                                                      W_UK, W_UV, W_o)
//   EPI_GATE:  C = Sigmoid(acc) * O[m, n]            ("Gated MLA 计算公式" §二:
//                                                      the per-channel gate
//                                                      applied to o~ before W_o)
//   EPI_GATE_VU: the same with O[m, h d_v + j] = sum_c o_lat[m, h, c] W_UV[h, j, c]
//              formed by the skinny workgroup that gates it ("LLM 注意力与计算
//              内核精读笔记 · 03" §5.2: the value up-projection applied once
//              to the latent-space output)
//
// Both operands are K-contiguous, so every MFMA fragment is a 16-byte read.
// The weight is the MFMA "A" side: the accumulator layout then gives each lane
// four consecutive output columns, which become one 8-byte store.
//
// Three kernels:
//  * gemm_big: 256 x 256 x 64 tiles for grids of at least 256 tiles and
//    K >= 2048 (the prefill projections of x and of o~): 4 waves, one per
//    SIMD, each owning 128 x 128 of the tile (accumulators in AGPRs);
//    operands staged through registers two k-tiles ahead with buffer loads,
//    then into a double-buffered LDS tile with padded rows.
//  * gemm_tile: LDS-tiled (BN x BM x 64 tiles, 2 stages, direct-to-LDS
//    16-byte loads, XOR-swizzled rows, 8 waves) for the other token counts
//    >= 65.
//  * gemm_skinny: M <= 64 (decode-step projections). Weight-streaming bound:
//    each workgroup owns 32 output columns, its 4 waves split K and stream
//    their chunks through private LDS rings (several chunks in flight per
//    wave, no barrier in the loop), partial sums meet in LDS. A grid of
//    fewer than 512 workgroups (narrow N) also splits K across workgroups:
//    fp32 partial sums, then gemm_splitk_reduce applies the epilogue.
//  * gemm_skinny_shared: 33..64 rows where 64-column workgroups would not
//    fill the grid: a workgroup owns 128 columns and shares each activation
//    chunk among its 4 waves (a quarter of the activation bytes per weight
//    byte), 256-byte row pieces, K split across workgroups (even shares of
//    the column groups' chunks over the grid).
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
// 256 x 256 tiles, 4 waves (one per SIMD), wave (wn, wm) owns 128 weight rows
// x 128 activation rows of the tile: 16 accumulators of 32 x 32 (AGPRs), and
// each 16-wide k-step reads 8 fragments for 16 MFMAs (half the LDS reads per
// MFMA of two waves per SIMD with 128 x 64 each).
//
// Loads: every thread moves 16 chunks of 16 bytes per 64-wide k-tile with
// buffer loads into registers (two register sets: tiles t + 1 and t + 2 are
// in flight while tile t is multiplied), and writes them to the LDS stage of
// tile t + 1 a quarter at a time between the MFMAs of tile t; the refill of
// the freed registers with tile t + 3 follows each quarter. The buffer
// descriptors cover exactly the operand bytes, so rows past N (or M) read as
// zeros and edge tiles need no clamping. LDS rows are 144 bytes (128 of data,
// 16 of padding): the fragment reads (32 consecutive rows at one 16-byte
// chunk per half-wave) fall on distinct banks, and every k-step is a
// compile-time offset from one base address per operand.
//
// Measured at 16384 x 8192 x 7168 and 16384 x 7168 x 8192 (interleaved
// medians, same box): 1462-1477 us against 1590 us for gemm_tile, with the
// same bits. The shader clock during these GEMMs reads 1.6-1.7 GHz (s_memtime
// against s_memrealtime), so power, not the MFMA issue rate, bounds them.
namespace big {
constexpr int BN = 256, BM = 256, BK = 64;
constexpr int TN = 4, TM = 4;         // 32 x 32 blocks per wave (weights x activations)
constexpr int RSB = 144;              // LDS row stride in bytes
constexpr int STAGE = (BN + BM) * RSB;
constexpr int LDS = 2 * STAGE;        // 144 KiB
constexpr int NS = 16;                // 16-byte chunks per thread per k-tile
constexpr int RS = (BN / 2) * 4 + 16; // epilogue row stride (fp32, half the columns)
static_assert(BM * RS <= LDS, "epilogue tile fits in the ring");
}  // namespace big

// Up to four GEMMs that share A, M and K run as one grid (GemmGroup): the
// n-tiles of the segments sit side by side, each workgroup takes its
// segment's weight, output, widths and strides. A single GEMM is a group of
// one (with npad: its zero columns).
template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_big_kernel(GemmGroup gg) {
  using namespace big;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  GemmArgs g = gg.base;
  const int tiles_n = gg.tiles_n, tiles_m = (g.M + BM - 1) / BM;
  const int total = tiles_n * tiles_m;
  // XCD-contiguous tile ranges, then groups of 4 m-tiles (as gemm_tile)
  int pid = blockIdx.x;
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  constexpr int GROUP = 4;
  const int group_size = GROUP * tiles_n;
  const int grp = pid / group_size;
  const int first_m = grp * GROUP;
  const int gm = (tiles_m - first_m) < GROUP ? (tiles_m - first_m) : GROUP;
  const int tile_m = first_m + (pid % group_size) % gm;
  const int tile_n = (pid % group_size) / gm;
  // this n-tile's segment (unused segments start at INT32_MAX)
  const int seg = (tile_n >= gg.first_wg[1]) + (tile_n >= gg.first_wg[2]) + (tile_n >= gg.first_wg[3]);
  const int seg_first = seg == 0 ? 0 : seg == 1 ? gg.first_wg[1] : seg == 2 ? gg.first_wg[2] : gg.first_wg[3];
  // every launch fills the segment arrays, a single GEMM as segment 0
  g.W = seg == 0 ? gg.W[0] : seg == 1 ? gg.W[1] : seg == 2 ? gg.W[2] : gg.W[3];
  g.C = seg == 0 ? gg.C[0] : seg == 1 ? gg.C[1] : seg == 2 ? gg.C[2] : gg.C[3];
  g.N = seg == 0 ? gg.N[0] : seg == 1 ? gg.N[1] : seg == 2 ? gg.N[2] : gg.N[3];
  g.ldw = seg == 0 ? gg.ldw[0] : seg == 1 ? gg.ldw[1] : seg == 2 ? gg.ldw[2] : gg.ldw[3];
  g.ldc = seg == 0 ? gg.ldc[0] : seg == 1 ? gg.ldc[1] : seg == 2 ? gg.ldc[2] : gg.ldc[3];
  const int n0 = (tile_n - seg_first) * BN, m0 = tile_m * BM;
  const int batch = blockIdx.y;
  const bf16* A = g.A + batch * g.sA;
  const bf16* W = g.W + batch * g.sW;
  bf16* Cp = g.C + batch * g.sC;
  const bf16* Op = (EPI == EPI_GATE) ? g.O + batch * g.sO : nullptr;

  // descriptors over this batch's operand bytes (raw buffers, 32-bit sizes;
  // the launcher checks that every offset fits)
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, (short)0, (int)(((int64_t)(g.N - 1) * g.ldw + g.K) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, (short)0, (int)(((int64_t)(g.M - 1) * g.lda + g.K) * 2), 0x00020000);
  // chunk slot r of a k-tile: row 32 r + tid / 8 of the weight tile (r < 8)
  // or of the activation tile (r >= 8), 16-byte piece tid % 8
  const int rsub = tid >> 3, piece = tid & 7;
  const int vW = ((n0 + rsub) * g.ldw + piece * 8) * 2;
  const int vA = ((m0 + rsub) * g.lda + piece * 8) * 2;
  const int sW = 32 * g.ldw * 2, sA = 32 * g.lda * 2;
  const unsigned dst0 = (unsigned)(rsub * RSB + piece * 16);
  const int ktiles = g.K / BK;
  u32x4 R0[NS], R1[NS];
  auto issue = [&](u32x4* R, int r, int kt) {
    if (r < 8) R[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, vW, kt * 128 + r * sW, 0));
    else R[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, vA, kt * 128 + (r - 8) * sA, 0));
  };
  auto put = [&](const u32x4* R, int r, int st) {
    *(LDS_AS u32x4*)(smem + st * STAGE + dst0 + r * 32 * RSB) = R[r];
  };

  floatx16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = floatx16{};
  // fragment rows: weights 128 wn + 32 i + lane % 32, activations 128 wm +
  // 32 j + lane % 32; k-step kk reads 16-byte chunk 2 kk + lane / 32
  const unsigned fw0 = (unsigned)((wn * (BN / 2) + (lane & 31)) * RSB + (lane >> 5) * 16);
  const unsigned fa0 = (unsigned)(BN * RSB + (wm * (BM / 2) + (lane & 31)) * RSB + (lane >> 5) * 16);
  auto read_frags = [&](bf16x8* wf, bf16x8* af, int st, int kk) {
#pragma unroll
    for (int i = 0; i < TN; ++i) wf[i] = as_bf16x8(lds_read16(smem + st * STAGE + fw0 + i * 32 * RSB + kk * 32));
#pragma unroll
    for (int j = 0; j < TM; ++j) af[j] = as_bf16x8(lds_read16(smem + st * STAGE + fa0 + j * 32 * RSB + kk * 32));
  };

  // prologue: tile 0 -> stage 0; tiles 1 and 2 in flight in R1 and R0
#pragma unroll
  for (int r = 0; r < NS; ++r) issue(R0, r, 0);
  if (ktiles > 1) {
#pragma unroll
    for (int r = 0; r < NS; ++r) issue(R1, r, 1);
  }
#pragma unroll
  for (int r = 0; r < NS; ++r) put(R0, r, 0);
  if (ktiles > 2) {
#pragma unroll
    for (int r = 0; r < NS; ++r) issue(R0, r, 2);
  }
  lds_barrier();

  // iteration t multiplies tile t (stage st = t % 2); quarter c reads the
  // fragments of k-step c + 1 ahead, runs the 16 MFMAs of k-step c, writes
  // chunk slots 4c .. 4c + 3 of tile t + 1 (register set R) to the other
  // stage and refills them with tile t + 3. The scheduling groups put the
  // fragment reads first and spread the writes and loads between the MFMAs.
  auto body = [&](u32x4* R, int t, int st, bool wr, bool rf) {
    bf16x8 wf[2][TN], af[2][TM];
    read_frags(wf[0], af[0], st, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < 3) read_frags(wf[(c + 1) & 1], af[(c + 1) & 1], st, c + 1);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32(wf[c & 1][i], af[c & 1][j], acc[i][j]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (wr) put(R, 4 * c + q, st ^ 1);
        if (rf) issue(R, 4 * c + q, t + 3);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // DS reads
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
  };
  // the register set alternates with the tile, so iterations go in pairs
  int t = 0;
  for (; t + 4 < ktiles; t += 2) {
    body(R1, t, 0, true, true);
    body(R0, t + 1, 1, true, true);
  }
  for (; t < ktiles; t += 2) {
    body(R1, t, 0, t + 1 < ktiles, t + 3 < ktiles);
    if (t + 1 < ktiles) body(R0, t + 1, 1, t + 2 < ktiles, t + 4 < ktiles);
  }

  // Epilogue through LDS, one column half (BN/2) at a time, as gemm_tile.
  // The gate's O values of both halves are loaded first, into the registers
  // the operand staging no longer needs, so their latency overlaps the
  // staging of the accumulators instead of following it.
  LDS_AS float* ct = (LDS_AS float*)smem;
  const bool vec16 = g.ldc % 8 == 0 && g.sC % 8 == 0 && (EPI != EPI_GATE || (g.ldo % 8 == 0 && g.sO % 8 == 0));
  constexpr int HN = BN / 2;
  constexpr int ITEMS = BM * HN / 8;      // 8 columns per item
  constexpr int IPT = ITEMS / 256;        // items per thread and half
  const int ncols = c_cols<EPI>(g);
  u32x4 ov[2][IPT];
  if constexpr (EPI == EPI_GATE) {
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int k = 0; k < IPT; ++k) {
        const int it = tid + 256 * k;
        const int m = m0 + it / (HN / 8), n = n0 + half * HN + (it % (HN / 8)) * 8;
        ov[half][k] = (vec16 && m < g.M && n + 8 <= ncols) ? *(const u32x4*)(Op + (int64_t)m * g.ldo + n)
                                                           : u32x4{0u, 0u, 0u, 0u};
      }
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    lds_barrier();
    if (wn == half) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int ml = wm * (BM / 2) + j * 32 + (lane & 31);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int nl = i * 32 + 8 * r4 + 4 * (lane >> 5);
            *(LDS_AS floatx4*)((LDS_AS char*)ct + ml * RS + nl * 4) =
                floatx4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
          }
        }
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int it = tid + 256 * k;
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
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = sigmoidf_fast(v[2 * e]) * bf16_bits_to_f32((unsigned short)(ov[half][k][e] & 0xffff));
            v[2 * e + 1] = sigmoidf_fast(v[2 * e + 1]) * bf16_bits_to_f32((unsigned short)(ov[half][k][e] >> 16));
          }
        }
        *(u32x4*)(Cp + (int64_t)m * g.ldc + n) =
            u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      } else {
        store4<EPI>(g, Cp, Op, m, n, v[0], v[1], v[2], v[3]);
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
  const int r32 = lane & 31, hk = lane >> 5;
  // EPI_GATE_VU: the operands of this workgroup's value up-projection (head
  // h = n0 / d_v, its rows j0 .. j0 + 32 NT - 1 of W_uv, all M rows of
  // o_lat), k-steps wave, wave + 4, ... of the 32 over d_c = 512. They are
  // loaded before the weight stream starts and multiplied after it ends:
  // their wait then holds nothing up (memory operations complete in issue
  // order, so a wait for loads issued after the weight DMA would drain it).
  constexpr int KV = 8;  // value up-projection k-steps per wave
  bf16x8 vwf[EPI == EPI_GATE_VU ? KV : 1][NT], vof[EPI == EPI_GATE_VU ? KV : 1][MT];
  if constexpr (EPI == EPI_GATE_VU) {
    const int h = n0 / g.vdv, j0 = n0 - h * g.vdv;
    const bf16* wv = g.vw + ((int64_t)h * g.vdv + j0 + r32) * g.vdc + 8 * hk;
    const bf16* ov = g.vo + (int64_t)h * g.vdc + 8 * hk;
#pragma unroll
    for (int x = 0; x < KV; ++x) {
      const int c = 16 * (wave + 4 * x);
#pragma unroll
      for (int u = 0; u < NT; ++u) vwf[x][u] = as_bf16x8(*(const u32x4*)(wv + (int64_t)32 * u * g.vdc + c));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        int m = 32 * t + r32;
        m = m < g.M ? m : g.M - 1;
        vof[x][t] = as_bf16x8(*(const u32x4*)(ov + (int64_t)m * g.ldvo + c));
      }
    }
  }
#pragma unroll
  for (int b = 0; b < C::NBUF; ++b)
    if (b < nmy) issue(b, c_lo + wave + 4 * b);
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

  floatx16 vacc[EPI == EPI_GATE_VU ? NT : 1][EPI == EPI_GATE_VU ? MT : 1];
  if constexpr (EPI == EPI_GATE_VU) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) vacc[u][t] = floatx16{};
#pragma unroll
    for (int x = 0; x < KV; ++x)
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t) vacc[u][t] = mfma32(vwf[x][u], vof[x][t], vacc[u][t]);
  }

  __syncthreads();  // every wave is done with its ring: reuse it for the reduction
  constexpr int NA = NT * MT;  // accumulators per wave
  LDS_AS float* red = (LDS_AS float*)smem;  // [4 waves][NT MT][16][64]
  LDS_AS float* vred = red + 4 * NA * 16 * 64;  // EPI_GATE_VU: the same for the value up-projection
  static_assert(EPI != EPI_GATE_VU || 2 * 4 * NA * 16 * 64 * 4 <= C::LDS_BYTES, "both reductions fit in the ring");
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[((wave * NA + u * MT + t) * 16 + r) * 64 + lane] = acc[u][t][r];
        if constexpr (EPI == EPI_GATE_VU) vred[((wave * NA + u * MT + t) * 16 + r) * 64 + lane] = vacc[u][t][r];
      }
  __syncthreads();
  // wave w finishes register group r4 = w (4 consecutive columns per lane)
#pragma unroll
  for (int ut = 0; ut < NA; ++ut) {
    const int u = ut / MT, t = ut % MT;
    float v[4], vo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * wave + e;
      v[e] = 0.f;
      vo[e] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[e] += red[((w * NA + ut) * 16 + r) * 64 + lane];
        if constexpr (EPI == EPI_GATE_VU) vo[e] += vred[((w * NA + ut) * 16 + r) * 64 + lane];
      }
    }
    const int m = 32 * t + (lane & 31);
    const int n = n0 + 32 * u + 8 * wave + 4 * (lane >> 5);
    if (n >= n0 + cw) continue;  // another workgroup's columns
    if constexpr (EPI == EPI_GATE_VU) {
      // o~ as the separate up-projection would store it (bf16), then the gate
      if (m < g.M && n < g.N) {
        u32x2 w;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const unsigned pk = pack_bf16x2(vo[2 * e], vo[2 * e + 1]);
          w[e] = pack_bf16x2(sigmoidf_fast(v[2 * e]) * bf16_bits_to_f32((unsigned short)(pk & 0xffff)),
                             sigmoidf_fast(v[2 * e + 1]) * bf16_bits_to_f32((unsigned short)(pk >> 16)));
        }
        *(u32x2*)(Cp + (int64_t)m * g.ldc + n) = w;
      }
      continue;
    }
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

// ----------------------------------------------------------------------------
// Skinny GEMM, 33..64 rows, with the activation chunk shared by the
// workgroup. A workgroup owns 128 output columns (wave w: columns 32 w ..
// 32 w + 31) and one K slice; its 4 waves walk the slice's 128-wide chunks
// together, each chunk one ring stage: the 128 weight rows (each wave DMAs
// its own 32) and the 32 MT activation rows (a quarter per wave), 256 bytes
// per row, with one barrier per stage. Sharing the activation chunk cuts
// the activation bytes per weight byte from M / 32 to M / 128, and the
// 256-byte row pieces stream faster than 128-byte ones. K is split across
// workgroups to fill the grid (one batch: the column groups' K chunks in
// even shares over the grid); fp32 partial sums go to the split-K reduce.
// Rows are 256 bytes; 16-byte piece p of row r sits at p ^ (r % 16).
template <int MT>
struct SharedCfg {
  static constexpr int KB = 128, ROWB = 256;
  static constexpr int W_BYTES = 128 * ROWB;
  static constexpr int A_BYTES = MT * 32 * ROWB;
  static constexpr int STAGE = W_BYTES + A_BYTES;
  static constexpr int NST = 163840 / STAGE;
  static constexpr int LDS_BYTES = NST * STAGE;
  static constexpr int WI = 8;           // weight DMA instructions per wave and stage
  static constexpr int AI = 2 * MT;      // activation DMA instructions per wave and stage
  static constexpr int IPS = WI + AI;
  static_assert(NST >= 3 && NST <= 4, "ring of 3 or 4 stages");
  static_assert((NST - 2) * IPS < 64, "vmcnt range");
};

// Even shares of the T = groups x chunks (column group, K chunk) items over
// W workgroups: workgroup w takes items [w T / W, (w + 1) T / W). The first
// and the last workgroup whose share touches group grp (its items
// grp C .. grp C + C - 1, C chunks per group): the largest w with
// w T / W rounded down <= item, for its first and its last item.
__host__ __device__ inline int sk_first(int grp, int chunks, long long tot, int wgs) {
  return (int)((((long long)grp * chunks + 1) * wgs + tot - 1) / tot) - 1;
}
__host__ __device__ inline int sk_last(int grp, int chunks, long long tot, int wgs) {
  return (int)((((long long)(grp + 1) * chunks) * wgs + tot - 1) / tot) - 1;
}

// Columns n0 .. n0 + 127 of batch `batch`, K chunks c_lo .. c_hi - 1 (of
// 128); partial: fp32 partial sums into slice `slot` of the split-K space,
// else the epilogue and the bf16 store.
template <int MT, int EPI>
__device__ __forceinline__ void shared_body(const GemmArgs& g, int n0, int batch, int c_lo, int c_hi, int slot,
                                            bool partial) {
  using C = SharedCfg<MT>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const unsigned smem_base = (unsigned)(uintptr_t)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bf16* A = g.A + batch * g.sA;
  const bf16* W = g.W + batch * g.sW;
  bf16* Cp = g.C + batch * g.sC;
  const bf16* Op = (EPI == EPI_GATE) ? g.O + batch * g.sO : nullptr;
  const int n = c_hi > c_lo ? c_hi - c_lo : 0;

  // DMA: instruction q of a wave moves 4 rows of 256 bytes; lane l writes
  // physical piece l % 16 of row 4 q + l / 16, i.e. logical piece
  // (l % 16) ^ (row % 16) of that row
  const int lr = lane >> 4, lp = lane & 15;
  auto issue = [&](int st, int j) {
    const unsigned dst = smem_base + st * C::STAGE;
    const unsigned long long wbase = (unsigned long long)(uintptr_t)(W + (int64_t)j * C::KB);
#pragma unroll
    for (int q = 0; q < C::WI; ++q) {
      const int trow = 32 * wave + 4 * q + lr;  // row of the weight tile
      int row = n0 + trow;
      row = row < g.N ? row : g.N - 1;
      g2lds16_s(wbase, (unsigned)(row * g.ldw * 2 + ((lp ^ (trow & 15)) << 4)), dst + (8 * wave + q) * 1024);
    }
    const unsigned long long abase = (unsigned long long)(uintptr_t)(A + (int64_t)j * C::KB);
#pragma unroll
    for (int q = 0; q < C::AI; ++q) {
      const int trow = 4 * (C::AI * wave + q) + lr;  // row of the activation tile
      const int row = trow < g.M ? trow : g.M - 1;
      g2lds16_s(abase, (unsigned)(row * g.lda * 2 + ((lp ^ (trow & 15)) << 4)),
                dst + C::W_BYTES + (C::AI * wave + q) * 1024);
    }
  };
  auto frag = [&](const LDS_AS char* tile, int r, int p) -> bf16x8 {
    return as_bf16x8(lds_read16(tile + r * C::ROWB + ((p ^ (r & 15)) << 4)));
  };

  floatx16 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx16{};
  const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
  for (int s = 0; s < C::NST - 1; ++s)
    if (s < n) issue(s, c_lo + s);
  for (int i = 0; i < n; ++i) {
    // stage i has landed once at most min(NST - 2, n - 1 - i) later stages
    // of this wave are in flight; the barrier then makes every wave's share
    // of it visible, and frees the stage of chunk i - 1 for chunk i + NST - 1
    const int later = (n - 1 - i) < C::NST - 2 ? (n - 1 - i) : C::NST - 2;
    if constexpr (C::NST == 4) {
      if (later >= 2) wait_vmcnt<2 * C::IPS>();
      else if (later == 1) wait_vmcnt<C::IPS>();
      else wait_vmcnt<0>();
    } else {
      if (later >= 1) wait_vmcnt<C::IPS>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    if (i + C::NST - 1 < n) issue((i + C::NST - 1) % C::NST, c_lo + i + C::NST - 1);
    const LDS_AS char* wt = smem + (i % C::NST) * C::STAGE;
    const LDS_AS char* at = wt + C::W_BYTES;
#pragma unroll
    for (int kk = 0; kk < C::KB / 16; ++kk) {
      const bf16x8 wf = frag(wt, 32 * wave + r32, 2 * kk + hk);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma32(wf, frag(at, 32 * t + r32, 2 * kk + hk), acc[t]);
    }
  }
  // register r of lane l: output row m = 32 t + l % 32, column
  // n0 + 32 wave + 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 32 * t + r32;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int col = n0 + 32 * wave + 8 * r4 + 4 * hk;
      const float v0 = acc[t][4 * r4], v1 = acc[t][4 * r4 + 1], v2 = acc[t][4 * r4 + 2], v3 = acc[t][4 * r4 + 3];
      if (partial) {
        const int ldp = (g.N + 3) & ~3;
        if (m < g.M && col < g.N)
          *(float4*)(g.part + (((int64_t)slot * g.batches + batch) * g.M + m) * ldp + col) = make_float4(v0, v1, v2, v3);
      } else {
        store4<EPI>(g, Cp, Op, m, col, v0, v1, v2, v3);
      }
    }
  }
}

template <int MT, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_shared_kernel(GemmArgs g) {
  const int chunks = g.K / SharedCfg<MT>::KB;
  if (g.sk_wgs > 0) {
    // even shares of the (column group, chunk) space: workgroup w takes
    // chunks [w T / W, (w + 1) T / W) of the T = groups x chunks in order,
    // which may end one group and start the next; each piece is a partial
    // sum in the slot of its group given by sk_first
    const int w = blockIdx.x;
    const long long tot = (long long)((g.N + 127) / 128) * chunks;
    int lo = (int)((long long)w * tot / g.sk_wgs);
    const int hi = (int)((long long)(w + 1) * tot / g.sk_wgs);
    bool first = true;
    while (lo < hi) {
      const int grp = lo / chunks;
      const int end = hi < (grp + 1) * chunks ? hi : (grp + 1) * chunks;
      if (!first) lds_barrier();  // every wave is done with the ring
      shared_body<MT, EPI>(g, grp * 128, 0, lo - grp * chunks, end - grp * chunks,
                           w - sk_first(grp, chunks, tot, g.sk_wgs), true);
      lo = end;
      first = false;
    }
    return;
  }
  const int nz = gridDim.z, zi = blockIdx.z;
  const int per = (chunks + nz - 1) / nz;
  const int c_lo = zi * per;
  const int c_hi = (c_lo + per) < chunks ? (c_lo + per) : chunks;
  shared_body<MT, EPI>(g, blockIdx.x * 128, blockIdx.y, c_lo, c_hi, zi, nz > 1);
}

// Several plain-store GEMMs that share A, M and K (one K slice each): segment
// s owns workgroups first_wg[s] .. first_wg[s + 1] - 1, 128 columns each.
template <int MT>
__global__ __launch_bounds__(256) void gemm_skinny_shared_group_kernel(GemmGroup gg) {
  const int x = blockIdx.x;
  const int s = (x >= gg.first_wg[1]) + (x >= gg.first_wg[2]) + (x >= gg.first_wg[3]);
  GemmArgs g = gg.base;
  g.W = s == 0 ? gg.W[0] : s == 1 ? gg.W[1] : s == 2 ? gg.W[2] : gg.W[3];
  g.C = s == 0 ? gg.C[0] : s == 1 ? gg.C[1] : s == 2 ? gg.C[2] : gg.C[3];
  g.N = s == 0 ? gg.N[0] : s == 1 ? gg.N[1] : s == 2 ? gg.N[2] : gg.N[3];
  g.ldw = s == 0 ? gg.ldw[0] : s == 1 ? gg.ldw[1] : s == 2 ? gg.ldw[2] : gg.ldw[3];
  g.ldc = s == 0 ? gg.ldc[0] : s == 1 ? gg.ldc[1] : s == 2 ? gg.ldc[2] : gg.ldc[3];
  const int first = s == 0 ? 0 : s == 1 ? gg.first_wg[1] : s == 2 ? gg.first_wg[2] : gg.first_wg[3];
  shared_body<MT, EPI_STORE>(g, (x - first) * 128, 0, 0, g.K / SharedCfg<MT>::KB, 0, false);
}

template <int MT, int NT, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  int x = blockIdx.x;
  if constexpr (EPI == EPI_GATE_VU) {
    // workgroups are dealt to the 8 XCDs in turn: give each XCD a run of
    // adjacent column blocks, so the workgroups of one head, which all read
    // that head's o_lat, share it through one L2
    const int G = gridDim.x;
    if (G % 8 == 0) x = (x % 8) * (G / 8) + x / 8;
  }
  skinny_body<MT, NT, EPI>(g, x * g.cw, g.cw, blockIdx.y, blockIdx.z, gridDim.z);
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
  // slices of this column: all of them, or with even shares the workgroups
  // whose shares touched its 128-column group
  int ns = g.ksplit;
  if (g.sk_wgs > 0) {
    const int chunks = g.K / 128, grp = n / 128;
    const long long tot = (long long)((g.N + 127) / 128) * chunks;
    ns = sk_last(grp, chunks, tot, g.sk_wgs) - sk_first(grp, chunks, tot, g.sk_wgs) + 1;
  }
  if (ok) {
    const float* p = g.part + bm * ldp + n;
    for (int z0 = j; z0 < ns; z0 += 32) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int z = z0 + 8 * u;
        v[u] = z < ns ? *(const float4*)(p + z * slice) : float4{0.f, 0.f, 0.f, 0.f};
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
// One batch: the (column group, chunk) space in even shares over up to 256
// workgroups of at least 8 chunks each, so the grid is full whatever the
// group count (W_o at 64 rows: 56 groups of 128 columns would fill 224
// workgroups with four equal K slices each); slots = the most workgroups
// that share one group, the partial-sum slices the reduce reads.
struct SharedPlan {
  int wgs, slots;
};
static SharedPlan shared_even(int N, int K) {
  const int G = (N + 127) / 128, C = K / 128;
  const long long tot = (long long)G * C;
  long long w = tot / 8;
  w = w < 256 ? w : 256;
  if (w <= G) return {0, 1};
  int smax = 1;
  for (int grp = 0; grp < G; ++grp) {
    const int sl = sk_last(grp, C, tot, (int)w) - sk_first(grp, C, tot, (int)w) + 1;
    smax = sl > smax ? sl : smax;
  }
  return {(int)w, smax};
}
template <int EPI>
static hipError_t launch_shared(const GemmArgs& g, hipStream_t st) {
  using C = SharedCfg<2>;
  auto kern = gemm_skinny_shared_kernel<2, EPI>;
  {
    hipError_t e = lds_opt_in((const void*)kern, C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const int z = g.ksplit > 1 ? g.ksplit : 1;
  if (z > 1 && !g.part) return hipErrorInvalidValue;
  GemmArgs h = g;
  h.sk_wgs = 0;
  dim3 grid((g.N + 127) / 128, g.batches, z);
  if (g.batches == 1 && z > 1) {
    const SharedPlan pl = shared_even(g.N, g.K);
    if (pl.wgs <= 0 || pl.slots != z) return hipErrorInvalidValue;  // not the plan the partial space is sized for
    h.sk_wgs = pl.wgs;
    grid = dim3(pl.wgs, 1, 1);
  }
  hipError_t e = launch(kern, grid, dim3(256), C::LDS_BYTES, st, h);
  if (e != hipSuccess || z == 1) return e;
  const int64_t n4 = (int64_t)g.batches * g.M * (((g.N + 3) & ~3) / 4);  // output quads, 8 threads each
  return launch(gemm_splitk_reduce_kernel<EPI>, dim3((unsigned)((8 * n4 + 255) / 256)), dim3(256), 0, st, h);
}

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

// The big-tile kernel addresses its operands with 32-bit buffer offsets:
// every row start of a batch's A and W (plus a tile of rows past the end,
// which read as zeros) and the descriptor sizes must stay below 2^31.
static bool big_fits_rows(long long rows, long long ld, long long K) {
  const long long lim = 1LL << 31;
  return (rows + 256) * ld * 2 < lim && ((rows - 1) * ld + K) * 2 < lim;
}
template <int EPI>
static bool big_fits(const GemmArgs& g) {
  return big_fits_rows(g.N, g.ldw, g.K) && big_fits_rows(g.M, g.lda, g.K);
}

template <int EPI>
static hipError_t launch_big_group(const GemmGroup& gg, hipStream_t st) {
  auto kern = gemm_big_kernel<EPI>;
  {
    hipError_t e = lds_opt_in((const void*)kern, big::LDS);
    if (e != hipSuccess) return e;
  }
  const int tiles = gg.tiles_n * ((gg.base.M + big::BM - 1) / big::BM);
  return launch(kern, dim3(tiles, gg.base.batches), dim3(256), big::LDS, st, gg);
}

template <int EPI>
static hipError_t launch_big(const GemmArgs& g, hipStream_t st) {
  GemmGroup gg{};
  gg.base = g;
  gg.count = 1;
  gg.W[0] = g.W; gg.C[0] = g.C; gg.N[0] = g.N; gg.ldw[0] = g.ldw; gg.ldc[0] = g.ldc;
  gg.first_wg[0] = 0;
  gg.first_wg[1] = gg.first_wg[2] = gg.first_wg[3] = INT32_MAX;
  const int ncols = (EPI == EPI_STORE && g.npad > g.N) ? g.npad : g.N;
  gg.tiles_n = (ncols + big::BN - 1) / big::BN;
  return launch_big_group<EPI>(gg, st);
}

hipError_t launch_gemm_group_big(GemmGroup gg, hipStream_t st) {
  const GemmArgs& b = gg.base;
  if (gg.count < 1 || gg.count > 4 || b.M <= 0 || b.K % 64 != 0 || b.K < 2048) return hipErrorNotSupported;
  if (!big_fits_rows(b.M, b.lda, b.K)) return hipErrorNotSupported;
  int tiles_n = 0;
  for (int s = 0; s < 4; ++s) {
    if (s < gg.count) {
      if (gg.N[s] <= 0 || gg.N[s] % 4 != 0 || !big_fits_rows(gg.N[s], gg.ldw[s], b.K)) return hipErrorNotSupported;
      gg.first_wg[s] = tiles_n;
      tiles_n += (gg.N[s] + big::BN - 1) / big::BN;
    } else {
      gg.first_wg[s] = INT32_MAX;
    }
  }
  if ((long long)tiles_n * ((b.M + big::BM - 1) / big::BM) < 256) return hipErrorNotSupported;
  gg.tiles_n = tiles_n;
  gg.base.batches = 1;
  gg.base.epi = EPI_STORE;
  gg.base.npad = 0;
  gg.base.sA = gg.base.sW = gg.base.sC = 0;
  return launch_big_group<EPI_STORE>(gg, st);
}

static bool skinny_path(int M, int N, int npad) { return M <= 64 && !(npad > N); }

// 33..64 rows over long K, where 64-column workgroups would not give one per
// compute unit: the shared-activation form, K split to fill the grid. It
// took W_o at 64 rows, 7168 x 16384, from 58.5 to 50.6 us (with the split-K
// reduce); at 32 rows or fewer, and where 64-column workgroups fill the
// grid, it measured slower than the per-wave rings.
static bool shared_path(int M, int N, int K, int batches) {
  if (M <= 32 || M > 64 || K % 128 != 0 || K < 2048) return false;
  const long long groups = (long long)((N + 127) / 128) * batches;
  // at least 32 workgroups before the split (narrow products keep the
  // per-wave form, whose split reaches more workgroups)
  return groups >= 32 && (long long)((N + 63) / 64) * batches < 256;
}
static int shared_split(int N, int K, int batches) {
  const long long groups = (long long)((N + 127) / 128) * batches;
  int z = (int)(256 / groups);
  const int most = K / 128 / 8;  // at least 8 chunks per slice
  z = z < most ? z : most;
  if (z <= 1) return 1;
  const int per = (K / 128 + z - 1) / z;  // no empty slice
  return (K / 128 + per - 1) / per;
}

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
  // the skinny kernels' DMA offsets are 32-bit: every row start below 4 GiB
  const bool offsets32 = (long long)g.N * g.ldw * 2 < (1LL << 32) && (long long)g.M * g.lda * 2 < (1LL << 32);
  if constexpr (EPI == EPI_GATE_VU) {
    if (!gemm_gate_vu_supported(g.M, g.N, g.K, g.vdc, g.vdv) || g.batches != 1 || !g.vo || !g.vw || !offsets32)
      return hipErrorInvalidValue;
    GemmArgs h = g;
    const int n1[1] = {g.N};
    h.cw = skinny_cols(n1, 1, 1, g.M);
    const bool nt2 = h.cw > 32;
    if (g.M <= 32) return nt2 ? launch_skinny<1, 2, EPI>(h, st) : launch_skinny<1, 1, EPI>(h, st);
    return nt2 ? launch_skinny<2, 2, EPI>(h, st) : launch_skinny<2, 1, EPI>(h, st);
  } else {
    if (skinny_path(g.M, g.N, EPI == EPI_STORE ? g.npad : 0)) {
      if (!offsets32) return hipErrorInvalidValue;
      if (shared_path(g.M, g.N, g.K, g.batches)) return launch_shared<EPI>(g, st);
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
    // the big-tile kernel's two-tile lookahead pays off over long K; at short
    // K (the K and V reconstruction, K = 512) its prologue dominates and
    // gemm_tile measured faster (182 against 230 us)
    if (big_tiles >= 256)
      return g.K >= 2048 && big_fits<EPI>(g) ? launch_big<EPI>(g, st) : launch_tile<256, 256, EPI>(g, st);
    return launch_tile<128, 128, EPI>(g, st);
  }
}

// Split K when the skinny grid has fewer than 64 workgroups (a quarter of
// the compute units; a grid of a few hundred loses more to the extra pass
// than it gains), up to 256 workgroups, keeping at least 4 chunks of 64 per
// workgroup (one per wave).
int gemm_ksplit(int M, int N, int K, int batches, int npad) {
  if (M <= 0 || N <= 0 || K <= 0 || batches <= 0 || !skinny_path(M, N, npad)) return 1;
  if (shared_path(M, N, K, batches)) return batches == 1 ? shared_even(N, K).slots : shared_split(N, K, batches);
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
    if (gg.N[s] <= 0 || gg.N[s] % 4 != 0 || (long long)gg.N[s] * gg.ldw[s] * 2 >= (1LL << 32))
      return hipErrorInvalidValue;
  gg.base.batches = 1;
  gg.base.ksplit = 1;
  gg.base.epi = EPI_STORE;
  gg.base.npad = 0;
  if (b.M > 32 && b.K % 128 == 0 && b.K >= 2048) {
    // 33..64 rows: shared-activation workgroups of 128 columns when they fit
    // one round of the grid (no K split here)
    long long groups = 0;
    for (int s = 0; s < gg.count; ++s) groups += (gg.N[s] + 127) / 128;
    if (groups >= 32 && groups <= 256) {
      for (int s = 0; s < 4; ++s) {
        if (s < gg.count) {
          gg.first_wg[s] = first;
          first += (gg.N[s] + 127) / 128;
        } else {
          gg.first_wg[s] = INT32_MAX;
        }
      }
      gg.base.cw = 128;
      using C = SharedCfg<2>;
      auto kern = gemm_skinny_shared_group_kernel<2>;
      hipError_t e = lds_opt_in((const void*)kern, C::LDS_BYTES);
      if (e != hipSuccess) return e;
      return launch(kern, dim3(first), dim3(256), C::LDS_BYTES, st, gg);
    }
  }
  const int cols = skinny_cols(gg.N, gg.count, 1, b.M);
  for (int s = 0; s < 4; ++s) {
    if (s < gg.count) {
      if (s > 0) gg.first_wg[s] = first;
      first += (gg.N[s] + cols - 1) / cols;
    } else {
      gg.first_wg[s] = INT32_MAX;  // no workgroup reaches an unused segment
    }
  }
  gg.first_wg[0] = 0;
  gg.base.cw = cols;
  if (b.M <= 32) return cols > 32 ? launch_group<1, 2>(gg, first, st) : launch_group<1, 1>(gg, first, st);
  return cols > 32 ? launch_group<2, 2>(gg, first, st) : launch_group<2, 1>(gg, first, st);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batches <= 0) return hipSuccess;
  if (g.npad > g.N && (g.epi != EPI_STORE || g.npad % 4 != 0)) return hipErrorInvalidValue;
  if (g.K % 64 != 0 || (g.npad > g.N ? g.npad : g.N) % 4 != 0) return hipErrorInvalidValue;
  if (g.epi == EPI_GATE_VU) return launch_epi<EPI_GATE_VU>(g, st);
  return g.epi == EPI_GATE ? launch_epi<EPI_GATE>(g, st) : launch_epi<EPI_STORE>(g, st);
}

bool gemm_gate_vu_supported(int M, int N, int K, int d_c, int d_v) {
  if (M <= 0 || M > 64 || N <= 0 || K <= 0 || K % 64 != 0 || N % 4 != 0 || d_c != 512 || d_v <= 0) return false;
  if (!skinny_path(M, N, 0) || shared_path(M, N, K, 1) || gemm_ksplit(M, N, K, 1, 0) > 1) return false;
  const int n1[1] = {N};
  const int cw = skinny_cols(n1, 1, 1, M);
  // whole 32- or 64-column workgroups, each inside one head
  return (cw == 32 || cw == 64) && d_v % cw == 0 && N % d_v == 0;
}

}  // namespace gmla
