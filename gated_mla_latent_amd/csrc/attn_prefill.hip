// Causal flash attention for prefill over explicitly reconstructed per-head
// K and V (bf16 in, fp32 accumulate, bf16 out), gfx950.
//
// What it computes ("Gated MLA 计算公式", §二 first equation): for every
// sequence b, head h and query position t,
//     o_t = sum_{s <= t} softmax_s( scale * q_t . k_s ) v_s
// with the inclusive causal boundary s <= t. The result goes straight into
// the head-major concatenation o~[b, t, h*D + j] ("Gated MLA 计算公式" §二
// second equation) when the output strides say so.
//
// Design (MI355X):
//  * One workgroup = (b, h, 128 queries), 4 waves, one per SIMD, and two
//    workgroups per compute unit (at most 80 KiB of LDS each, no static
//    LDS): wave w owns 32 queries. With O^T (D x 32) and the scores (64
//    keys x 32) per wave the registers fit two waves per SIMD, so one
//    wave's softmax arithmetic runs while the other wave's MFMAs do; the
//    two belong to different workgroups, so a barrier holds only one of
//    them.
//  * K and V tiles of 64 keys stream through a 2-stage LDS ring with 1 KiB
//    direct-to-LDS loads: one barrier per tile, after which the next tile
//    is loaded into the stage of the previous one.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query and
//    16 keys per 32-key block, so the first-tile max needs one exchange with
//    lane ^ 32. The K rows enter the MFMA in an order (bits 2 and 3 of the
//    key swapped within each 16) that leaves every lane's accumulator
//    holding runs of 8 consecutive keys.
//  * O^T += V^T . P^T: P^T is the S^T accumulator rounded to bf16, so each
//    MFMA k-step covers 16 consecutive keys. V arrives transposed (keys
//    contiguous, written so by the value reconstruction GEMM), so each V^T
//    fragment is one plain 16-byte LDS read: transposing LDS reads run at
//    half the rate and would make LDS, not the MFMAs, the bound.
//  * K and V^T rows are 16-byte-chunk XOR-swizzled so that neither read
//    conflicts in LDS.
//  * Softmax: the scale (log2 e included) is folded into the queries when
//    they are loaded (rounded to bf16), so scores are base-2 exponents. No
//    rescale of O inside the loop: each query's reference max m is fixed at
//    its first key tile, and from then on the S^T accumulators start at -m
//    (the MFMA's C operand), so a weight is exp2 of the accumulator with no
//    per-score arithmetic and no per-tile max. If the weights' sum exceeds
//    2^32 (a later score outgrew the reference by as much), the workgroup
//    sweeps the scores once for the true maxima and redoes the pass with
//    them (exact for any input).
//  * Without RoPE the P.V MFMAs of a tile run at raised wave priority, so
//    the two waves of a SIMD settle into opposite phases: one issues MFMAs
//    while the other computes its softmax.
//  * Each workgroup takes two query tiles, the k-th longest and the k-th
//    shortest, so all workgroups carry the same causal work. The work items
//    of one (b, h) are placed on one XCD, where they share its L2.
//  * Decoupled RoPE ([N03] "LLM 注意力与计算内核精读笔记 · 03" §5.2): the
//    score gains q^R . k^R over DR more features, the rotated RoPE query of
//    the head and the RoPE key shared by all heads. They are DR / 16 more
//    k-steps of S^T: the query fragments from their own rows, the key
//    fragments from a third tile of the stage (64 keys x DR); two stages
//    are then 80 KiB.
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

// LDS operand fragments read ahead of their MFMA (scheduling barriers keep
// the order): one LDS latency then hides behind several MFMAs
constexpr int kPFS = 4;  // k-steps of K fragments (two each) in flight in S^T
constexpr int kPFV = 4;  // V^T fragments in flight in P.V
constexpr int kSync = 1;  // key tiles per barrier; the ring holds 2 kSync tiles

template <int D, int DR>
struct FaCfg {
  // 128 queries and 4 waves, so that two workgroups share a compute unit
  // (measured against 256 queries and 8 waves, same bits: NoPE with a
  // 4-stage ring 1951 -> 1912 us, RoPE with a 3-stage ring 2437 -> 2354 us)
  static constexpr int BQ = 128, BK = 64, NW = 4;
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int ROWB = 2 * D;           // bytes per row
  static constexpr int TILE = BK * ROWB;       // one K tile (64 rows of D), or one V^T tile (D rows of 64)
  static constexpr int RTILE = BK * DR * 2;    // the RoPE key tile (64 rows of DR)
  static constexpr int STAGE = 2 * TILE + RTILE;
  static constexpr int NST = 2 * kSync;  // ring stages
  static constexpr int LDS = NST * STAGE;
  static constexpr int KSC = D / 16;           // k-steps of S^T over the content features
  static constexpr int KS = (D + DR) / 16;     // all k-steps of S^T
  static constexpr int DB = D / 32;            // 32-row blocks of O^T
  static constexpr int RND = BK * CH / (64 * NW);  // 1 KiB loads per wave per K (or V) tile
  static constexpr int RNDR = BK * DR / 8 / (64 * NW);  // ... per RoPE key tile
  static_assert(RND >= 1, "at least one load per wave");
  static_assert(DR == 0 || (DR == 64 && RNDR >= 1 && RNDR * 64 * NW * 8 == BK * DR), "RoPE key tile: whole loads per wave");
  static_assert(LDS <= 81920, "LDS budget: two workgroups per compute unit");
};

// Chunk swizzles (physical chunk = logical chunk ^ f(row)). The K and V^T
// tiles are read as 32 rows x one chunk per half-wave. The XORs were picked
// by measuring the LDS bank-conflict counter on probe kernels that replay
// this read pattern for sixteen candidate swizzles: these measured zero
// conflicts.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7); }
// V^T tiles have 128-byte rows (64 keys) read 32 rows x one chunk per
// half-wave, the pattern of the D = 64 K tile, so they take its swizzle
__device__ __forceinline__ int swz_vt(int r) { return (r >> 1) & 7; }

}  // namespace

template <int D, int DR>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * FaCfg<D, DR>::NW, 64 * FaCfg<D, DR>::NW), amdgpu_waves_per_eu(2, 2)))
void prefill_attn_kernel(AttnArgs a) {
  using C = FaCfg<D, DR>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const unsigned smem_base = (unsigned)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // work item = (b, h, pair of query tiles {nqt - 1 - p, p}): a long and a
  // short causal tile per workgroup, so every workgroup has the same work
  const int nqt = (a.L + C::BQ - 1) / C::BQ;
  const int npair = (nqt + 1) / 2;
  // XCD-contiguous order: the hardware deals workgroup i to XCD i % 8, so
  // XCD x takes the x-th eighth of the work items in order, and the
  // workgroups of one (b, h), which all stream the same K and V, share
  // that XCD's L2 instead of each XCD fetching them again
  int wid = (int)blockIdx.x;
  {
    const int nwg = (int)gridDim.x, per = nwg >> 3, extra = nwg & 7, x = wid & 7;
    wid = x * per + (x < extra ? x : extra) + (wid >> 3);
  }
  const int pair = wid % npair;
  const int bh = wid / npair;
  const int b = bh / a.H, h = bh % a.H;

  const bf16* qb = a.q + b * a.sqb + h * a.sqh;
  const bf16* kb = a.k + b * a.skb + h * a.skh;
  const bf16* vb = a.v + b * a.svb + h * a.svh;
  bf16* ob = a.o + b * a.sob + h * a.soh;
  const bf16* qrb = DR ? a.qr + b * a.sqrb + h * a.sqrh : nullptr;
  const bf16* krb = DR ? a.kr + b * a.skrb : nullptr;

  // the softmax scale (log2 e included) is folded into the queries, so the
  // scores come out in base-2 exponent units
  const float qs = a.scale_log2;
  auto scaled = [&](const u32x4 v) -> bf16x8 {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = pack_bf16x2(bf16_bits_to_f32((unsigned short)(v[e] & 0xffff)) * qs,
                         bf16_bits_to_f32((unsigned short)(v[e] >> 16)) * qs);
    return as_bf16x8(r);
  };

  for (int rep = 0; rep < 2; ++rep) {
  const int qt = rep == 0 ? nqt - 1 - pair : pair;
  if (rep == 1 && qt == nqt - 1 - pair) break;  // odd tile count: the middle tile alone
  const int q0 = qt * C::BQ;
  const int wq0 = q0 + 32 * wave;                    // this wave's first query
  // this wave's queries as the B operand of S^T: query wq0 + lane % 32,
  // features 16 kk + 8 (lane / 32) .. + 7
  bf16x8 qf[C::KS];
  {
    int t = wq0 + (lane & 31);
    t = t < a.L ? t : a.L - 1;
    const bf16* qp = qb + (int64_t)t * a.sqt + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < C::KSC; ++kk) qf[kk] = scaled(*(const u32x4*)(qp + 16 * kk));
    if constexpr (DR > 0) {
      const bf16* qrp = qrb + (int64_t)t * a.sqrt_ + 8 * (lane >> 5);
#pragma unroll
      for (int kk = C::KSC; kk < C::KS; ++kk) qf[kk] = scaled(*(const u32x4*)(qrp + 16 * (kk - C::KSC)));
    }
  }

  // DMA of key tile kt into stage s. K: 1 KiB load n covers chunks 64 n +
  // lane, i.e. physical chunk p % CH of key row p / CH (logical chunk
  // p % CH ^ swz_k(row)). V^T: load n covers feature rows 8 n .. 8 n + 7,
  // physical chunk lane % 8 of row 8 n + lane / 8 (logical chunk ^ swz_vt);
  // the padded V^T rows hold every key of the last tile.
  auto load_tile = [&](int s, int kt) {
    const unsigned kdst = smem_base + s * C::STAGE;
    const unsigned vdst = kdst + C::TILE;
    const int t0 = kt * C::BK;
    const unsigned long long kbase = (unsigned long long)(uintptr_t)(kb + (int64_t)t0 * a.skt);
    const unsigned long long vbase = (unsigned long long)(uintptr_t)(vb + t0);
#pragma unroll
    for (int r = 0; r < C::RND; ++r) {
      const int n = r * C::NW + wave;
      const int p = 64 * n + lane;
      const int row = p / C::CH, pc = p % C::CH;
      int rr = t0 + row;
      rr = (rr < a.L ? rr : a.L - 1) - t0;
      g2lds16_s(kbase, (unsigned)((rr * a.skt + (pc ^ swz_k<D>(row)) * 8) * 2), kdst + n * 1024);
      const int vrow = 8 * n + (lane >> 3);
      g2lds16_s(vbase, (unsigned)((vrow * a.svj + ((lane & 7) ^ swz_vt(vrow)) * 8) * 2), vdst + n * 1024);
    }
    if constexpr (DR > 0) {
      // RoPE key rows 8 wave .. 8 wave + 7 (128-byte rows, the V^T swizzle)
      const unsigned rdst = kdst + 2 * C::TILE;
      const unsigned long long rbase = (unsigned long long)(uintptr_t)(krb + (int64_t)t0 * a.skrt);
#pragma unroll
      for (int r = 0; r < C::RNDR; ++r) {
        const int blk = r * C::NW + wave;  // 8 rows per 1 KiB load
        const int row = 8 * blk + (lane >> 3);
        int rr = t0 + row;
        rr = (rr < a.L ? rr : a.L - 1) - t0;
        g2lds16_s(rbase, (unsigned)((rr * a.skrt + ((lane & 7) ^ swz_vt(row)) * 8) * 2), rdst + blk * 1024);
      }
    }
  };

  floatx16 o[C::DB];
  float m = 0.f;               // reference max of this lane's query (scaled units)
  float m_true = -INFINITY;    // redo sweep: the largest score of this lane's keys
  float lsum = 0.f;
  // the S^T accumulators start at -m (the MFMA adds its C operand),
  // so the weights are exp2 of the accumulator with no arithmetic per score
  floatx16 negm = floatx16{};

  int last_q = q0 + C::BQ - 1;
  last_q = last_q < a.L - 1 ? last_q : a.L - 1;
  const int ntiles = last_q / C::BK + 1;                   // tiles the workgroup needs
  int my_last = wq0 + 31;
  my_last = my_last < a.L - 1 ? my_last : a.L - 1;
  const int my_tiles = wq0 < a.L ? my_last / C::BK + 1 : 0;  // tiles this wave needs
  const int tq = wq0 + (lane & 31);                          // this lane's query

  // key row this lane feeds into row lane % 32 of each 32-key S^T block:
  // bits 2 and 3 swapped, so accumulator register r of lane l holds key
  // 16 (r / 8) + 8 (l / 32) + r % 8 of the block
  const int krow = ((lane & 31) & 0x13) | ((lane & 4) << 1) | ((lane & 8) >> 1);

  // O^T (D x 32 queries) += V^T . P^T for the key tile in ring stage `st`.
  // k-step ks: P^T operand = accumulator registers 8 (ks % 2) .. + 7 of key
  // block ks / 2, i.e. keys 16 ks + 8 (lane / 32) + e; the V^T operand of
  // lane l is feature row 32 d + l % 32 at those same keys, chunk
  // 2 ks + l / 32 of the row.
  auto pv = [&](int st, const bf16x8* pw) {
    const LDS_AS char* vt_l = smem + st * C::STAGE + C::TILE;
    constexpr int NF = 4 * C::DB;  // fragment f: k-step f / DB, row block f % DB
    auto readV = [&](int f) -> bf16x8 {
      const int c = 2 * (f / C::DB) + (lane >> 5);
      const int row = 32 * (f % C::DB) + (lane & 31);
      return as_bf16x8(lds_read16(vt_l + row * 128 + ((c ^ swz_vt(row)) << 4)));
    };
    bf16x8 vf[kPFV];
#pragma unroll
    for (int x = 0; x < kPFV; ++x) vf[x] = readV(x);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      o[f % C::DB] = mfma32(vf[f % kPFV], pw[f / C::DB], o[f % C::DB]);
      if (f + kPFV < NF) vf[f % kPFV] = readV(f + kPFV);
      // LDS reads and MFMAs keep their order; the softmax arithmetic (VALU,
      // transcendental, SALU) may still move in between
      __builtin_amdgcn_sched_barrier(0x406);
    }
  };

  // pass 0: reference max from the first key tile; pass 1 (only if pass 0
  // overflowed its bound): the true maxima, tracked over a pass at
  // reference 0; pass 2: again with those
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const bool sweep = pass == 1;
#pragma unroll
    for (int d = 0; d < C::DB; ++d) o[d] = floatx16{};
    lsum = 0.f;
    lds_barrier();
    constexpr int PRE = kSync;  // tiles issued before the loop
#pragma unroll
    for (int j = 0; j < PRE; ++j)
      if (j < ntiles) load_tile(j, j);
    for (int it = 0; it < ntiles; ++it) {
      if (it % kSync == 0) {
        // tiles it .. it + kSync - 1 have landed; their successors go into
        // the stages of the previous kSync tiles, which every wave is done with
        wait_vmcnt<0>();
        lds_barrier();
#pragma unroll
        for (int j = kSync; j < 2 * kSync; ++j)
          if (it + j < ntiles) load_tile((it + j) % C::NST, it + j);
      }
      if (it >= my_tiles) continue;
      const LDS_AS char* kt_l = smem + (it % C::NST) * C::STAGE;

      // ---- S^T: 64 keys (2 blocks of 32) x 32 queries ----
      floatx16 s[2];
      s[0] = negm;
      s[1] = negm;
      auto readK = [&](int kk, int i) -> bf16x8 {
        const int row = 32 * i + krow;
        if (kk < C::KSC) {
          const int c = 2 * kk + (lane >> 5);
          return as_bf16x8(lds_read16(kt_l + row * C::ROWB + ((c ^ swz_k<D>(row)) << 4)));
        }
        const int c = 2 * (kk - C::KSC) + (lane >> 5);
        return as_bf16x8(lds_read16(kt_l + 2 * C::TILE + row * 128 + ((c ^ swz_vt(row)) << 4)));
      };
      {
        constexpr int PF = kPFS < C::KS ? kPFS : C::KS;
        bf16x8 kf[PF][2];
#pragma unroll
        for (int x = 0; x < PF; ++x)
#pragma unroll
          for (int i = 0; i < 2; ++i) kf[x][i] = readK(x, i);
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
#pragma unroll
          for (int i = 0; i < 2; ++i) s[i] = mfma32(kf[kk % PF][i], qf[kk], s[i]);
          if (kk + PF < C::KS) {
#pragma unroll
            for (int i = 0; i < 2; ++i) kf[kk % PF][i] = readK(kk + PF, i);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- softmax weights (lane owns query tq and keys
      //      it*64 + 32 i + 16 (r/8) + 8 (lane/32) + r%8) ----
      const bool diag = it * C::BK + C::BK - 1 > wq0;  // some key may lie past some query
      if (diag) {
        // a real branch (the empty asm cannot be speculated): the compiler
        // would otherwise turn the mask into selects on every tile
        asm volatile("");
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = it * C::BK + 32 * i + 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7);
            s[i][r] = key <= tq ? s[i][r] : -INFINITY;
          }
      }
      auto tile_max = [&]() {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[i][r]);
        return mx;
      };
      if (sweep) {
        // the redo's first pass also tracks the true maxima (its weights,
        // from a zero reference, are discarded)
        asm volatile("");
        m_true = fmaxf(m_true, tile_max());
      }
      if (pass == 0 && it == 0) {
        // the reference: this tile's max (key 0 is visible to every query)
        asm volatile("");
        const float mx = tile_max();
        m = fmaxf(mx, xor32(mx));
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[r] = -m;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[i][r] -= m;
      }
      bf16x8 pb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(s[i][r]);
          lsum += p[r];
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          pb[2 * i + hf] = as_bf16x8(u32x4{pack_bf16x2(p[8 * hf + 0], p[8 * hf + 1]), pack_bf16x2(p[8 * hf + 2], p[8 * hf + 3]),
                                           pack_bf16x2(p[8 * hf + 4], p[8 * hf + 5]), pack_bf16x2(p[8 * hf + 6], p[8 * hf + 7])});
      }
      // ---- O^T (D x 32 queries) += V^T . P^T ----
      // NoPE: raised wave priority for the P.V MFMAs. The SIMD's arbiter then
      // prefers this wave's MFMA and LDS issues while the other wave of the
      // SIMD, at normal priority, runs its softmax arithmetic in the gaps,
      // which keeps the two waves in opposite phases (measured 2-4% faster
      // than equal priorities; raising it for the score MFMAs as well, or for
      // the softmax instead, measured no gain, and with the RoPE k-steps and
      // one barrier per tile it measured 4% slower)
      if constexpr (DR == 0) __builtin_amdgcn_s_setprio(1);
      pv(it % C::NST, pb);
      if constexpr (DR == 0) __builtin_amdgcn_s_setprio(0);
    }
    if (pass == 0) {
      // every weight is at most the sum: a sum within 2^32 (and not NaN)
      // bounds each weight by 2^32, the bound the pass was made for
      const float l = lsum + xor32(lsum);
      // workgroup OR through the idle ring (every tile is consumed and no
      // load is in flight), which keeps the kernel free of static LDS
      const bool wover = __builtin_amdgcn_ballot_w64(!(l <= 0x1p32f)) != 0;
      lds_barrier();
      if (lane == 0) ((LDS_AS int*)smem)[wave] = wover ? 1 : 0;
      lds_barrier();
      int any = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) any |= ((const LDS_AS int*)smem)[w];
      if (!any) break;
      m = 0.f;
      negm = floatx16{};
    } else if (pass == 1) {
      m = fmaxf(m_true, xor32(m_true));
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m;
    }
  }

  // ---- write o~ ----
  const float l = lsum + xor32(lsum);
  if (tq < a.L) {
    const float inv = 1.0f / l;
    bf16* op = ob + (int64_t)tq * a.sot + 4 * (lane >> 5);
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(u32x2*)(op + 32 * d + 8 * r4) = u32x2{pack_bf16x2(o[d][4 * r4] * inv, o[d][4 * r4 + 1] * inv),
                                                pack_bf16x2(o[d][4 * r4 + 2] * inv, o[d][4 * r4 + 3] * inv)};
  }
  }
}

template <int D, int DR>
static hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  using C = FaCfg<D, DR>;
  auto kern = prefill_attn_kernel<D, DR>;
  {
    hipError_t e = lds_opt_in((const void*)kern, C::LDS);
    if (e != hipSuccess) return e;
  }
  // the loads use 32-bit offsets from a per-tile scalar base
  if ((long long)C::BK * a.skt * 2 >= (1LL << 31) || (long long)D * a.svj * 2 >= (1LL << 31) ||
      (long long)C::BK * a.skrt * 2 >= (1LL << 31))
    return hipErrorInvalidValue;
  const int npair = ((a.L + C::BQ - 1) / C::BQ + 1) / 2;
  return launch(kern, dim3(npair * a.B * a.H), dim3(64 * C::NW), C::LDS, st, a);
}

hipError_t launch_prefill_attn_bf16(const AttnArgs& a, hipStream_t st) {
  if (a.D_R == 0) {
    if (a.D == 128) return launch_d<128, 0>(a, st);
    if (a.D == 64) return launch_d<64, 0>(a, st);
  } else if (a.D_R == 64 && a.qr && a.kr) {
    if (a.D == 128) return launch_d<128, 64>(a, st);
    if (a.D == 64) return launch_d<64, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gmla
