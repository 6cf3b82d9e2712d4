// Decode attention over the latent cache (bf16, gfx950).
//
// What it computes ("LLM 注意力与计算内核精读笔记 · 03", §5.1 absorption and
// §5.2 decoupled RoPE; "Gated MLA 计算公式", §二 causal softmax): for each
// sequence b and head h,
//     s_j = scale * ( q~_h[:d_c] . c_j  +  RoPE_{L_b-1}(q~_h[d_c:]) . kR_j )
//     o_lat_h = sum_j softmax(s)_j c_j          (j over the L_b cached rows)
// The cache row j is [c_j ; kR_j] (d_c + d_r bf16), kR already rotated.
//
// Design (MI355X):
//  * The flattened token space of all sequences is cut into G equal slices,
//    so ragged lengths cost nothing in balance. A slice may hold pieces of
//    several sequences; a sequence cut across slices yields partial (o, lse)
//    pieces that the combine kernel merges.
//  * A workgroup takes one slice for up to 64 heads (more heads run as
//    further workgroups placed beside it on the same XCD). It has 8 waves,
//    two per SIMD, so one wave's memory-issue stalls leave its SIMD to the
//    other. Wave w computes the scores and softmax weights of head group
//    w % 4 (16 heads) for token half w / 4 (16 of a tile's 32 tokens); the
//    weights are exchanged through LDS and wave w accumulates O for all 64
//    heads over its eighth of the latent features (64 of 512).
//  * Latent tiles of 32 tokens stream HBM -> LDS through a ring of four
//    slots with 1 KiB direct-to-LDS loads (one per cache row; the row base
//    is scalar). Two slots are being read (scores of tile i, P.V of tile
//    i - 1) and two are in flight; each wave's share of the next slot's
//    loads is interleaved with its score MFMAs.
//  * S^T = C . Q^T on v_mfma_f32_16x16x32_bf16 (A = 16-byte LDS reads, B =
//    the wave's queries in VGPRs): each lane owns one head and 4 tokens.
//  * O^T += C^T . P^T on the same MFMA: P^T is the head group's weights read
//    back in exactly the B-operand lane layout; C^T fragments come from
//    ds_read_b64_tr_b16 (transposing LDS reads).
//  * Software pipeline with one barrier per tile: the P.V of tile i - 1 runs
//    between the scores and the softmax of tile i. LDS reads run ahead of
//    their MFMA, an order scheduling barriers keep (in the RoPE scores the
//    compiler's own order measured faster); the compiler inserts the MFMA
//    hazard wait states (inline-asm MFMAs would hide them from it).
//  * No rescale of O inside the loop: the reference max is fixed at a head's
//    first tile; a segment whose scores outgrow it by more than 2^32 is redone
//    once with its true max (exact for any input, and O never meets VALU).
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRedo = 32.0f;  // log2 headroom before a segment is redone
constexpr int kPF = 4;          // LDS operand fragments in flight ahead of the MFMA
constexpr bool kSpreadDMA = true;  // interleave the next slot's DMA with the score MFMAs
constexpr int kRing = 4;           // LDS ring slots (slots in flight = kRing - 2)

// LDS tile layout. A ring slot holds 32 cache rows.
// Bank conflicts on gfx950's LDS were measured (SQ_LDS_BANK_CONFLICT) on probe
// kernels that replay exactly the read patterns below; the layout is the one
// that measured zero for all of them.
// Latent part (d_c = 512 bf16 = 1 KiB per row): token t in row t, row stride
// 1056 bytes (32 bytes of padding; 1056 = 32 mod 512). Then
//   * score operand reads: 16 lanes read tokens t0..t0+15 at 16-byte chunk c,
//     the four 16-lane groups chunks c..c+3 -> bank groups 2t + c cover each
//     group twice;
//   * P.V operand reads (transposing): 64 lanes read 16 tokens x 4 units of
//     8 bytes -> 8-byte units 4t + u, all distinct.
// Each latent row is one 1 KiB direct-to-LDS load, so the padding costs
// nothing on the load side, and every k-step is a compile-time LDS offset.
// The RoPE part (d_r = 64 -> 8 chunks, 128-byte rows) follows the 32 latent
// rows with its chunks XOR-permuted by swr(t) = t mod 8; among the swizzles
// probed for this read pattern (16 tokens x 4 consecutive chunks per
// instruction) it is one of those that measured no bank conflict.
constexpr int kLatStride = 1056;
__device__ __forceinline__ int swr(int t) { return t & 7; }

template <int D_R, int HG, int R>
struct DecodeCfg {
  static constexpr int D_C = 512;
  static constexpr int RW = D_C + D_R;        // cache row width (elements)
  static constexpr int RWB = RW * 2;          // cache row bytes
  // wave w: head group w % HG (16 heads) for the scores of token half w / HG
  // (16 of the tile's 32 tokens), and features (512 / NW) w .. of P.V
  static constexpr int NW = 2 * HG;
  static constexpr int LAT_BYTES = 32 * kLatStride;
  static constexpr int SLOT_BYTES = LAT_BYTES + 32 * D_R * 2;
  static constexpr int ROWS_L = 32 / NW;                 // latent rows per wave per slot
  static constexpr int ROPE_ROWS = D_R ? 32 / NW : 0;    // RoPE rows per wave per slot (one instruction)
  static constexpr int ROUNDS = ROWS_L + (D_R ? 1 : 0);  // DMA instructions per wave per slot
  // slots in flight ahead of the one being read: the slot read for scores in
  // one iteration is read again for P.V in the next, so two stay resident
  static constexpr int PD = R - 2;
  static constexpr int KB = RW / 32;          // k-steps of the scores (32 features each)
  static constexpr int KB_C = D_C / 32;
  static constexpr int FBW = 32 / NW;         // 16-feature blocks of O per wave
  static constexpr int RING_BYTES = R * SLOT_BYTES;
  static constexpr int P_OFF = RING_BYTES;    // weights: 2 buffers x HG head groups x 1 KiB
  static constexpr int X_OFF = P_OFF + 2 * HG * 1024;  // per-head exchange: max and sum, [2 halves][16 HG]
  static constexpr int LDS_BYTES = X_OFF + 2 * 2 * 16 * HG * 4;
  static_assert(HG == 2 || HG == 4, "32 or 64 heads per workgroup");
  static_assert(D_R == 0 || D_R == 64, "RoPE rows are 8 chunks of 16 bytes");
  static_assert(ROPE_ROWS * 8 <= 64, "RoPE rows of a wave fit one instruction");
  static_assert(LDS_BYTES <= 163840, "LDS budget");
  static_assert(NW * 8 + 32 <= LDS_BYTES, "scan scratch fits in the ring");
  static_assert(PD >= 1 && PD <= 3, "ring of 3 to 5 slots");
  static_assert((PD - 1) * ROUNDS < 64, "vmcnt range");
};

// vmcnt(pending * ROUNDS) for a small runtime `pending`
template <int ROUNDS, int MAXP>
__device__ __forceinline__ void wait_slots(int pending) {
  if constexpr (MAXP >= 2) {
    if (pending >= 2) { wait_vmcnt<2 * ROUNDS>(); return; }
  }
  if constexpr (MAXP >= 1) {
    if (pending >= 1) { wait_vmcnt<ROUNDS>(); return; }
  }
  wait_vmcnt<0>();
}

// value of lane - off (any value where that is negative; callers mask it)
__device__ __forceinline__ long long shfl_up_ll(long long v, int off) {
  const int src = ((lane_id() - off) & 63) << 2;
  const unsigned lo = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)(unsigned)(v & 0xffffffffLL));
  const unsigned hi = (unsigned)__builtin_amdgcn_ds_bpermute(src, (int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane_id() ^ mask) << 2, __builtin_bit_cast(int, v)));
}

// max / sum over the four 16-lane groups (the lanes of one head)
__device__ __forceinline__ float head_max(float v) {
  v = fmaxf(v, shfl_xor_f(v, 16));
  return fmaxf(v, shfl_xor_f(v, 32));
}
__device__ __forceinline__ float head_sum(float v) {
  v += shfl_xor_f(v, 16);
  return v + shfl_xor_f(v, 32);
}

}  // namespace

template <int D_R, int HG, int R>
__global__ __attribute__((amdgpu_flat_work_group_size(128 * HG, 128 * HG), amdgpu_waves_per_eu(HG / 2, HG / 2)))
void decode_attn_kernel(DecodeArgs a) {
  using C = DecodeCfg<D_R, HG, R>;
  constexpr int D_C = C::D_C;
  constexpr int NT = 64 * C::NW;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const unsigned smem_base = (unsigned)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave % HG;   // head group of this wave's scores
  const int th = wave / HG;   // token half of this wave's scores
  const int G = a.G;

  // Work item = (slice, head chunk of 16 HG heads). XCD-aware order: the
  // hardware deals workgroups to the 8 XCDs round robin, so each XCD gets a
  // contiguous run of items, and the head chunks of one slice run side by
  // side on one XCD, where the second read of their cache rows hits its L2.
  const int chunks = (int)gridDim.x / G;
  int item = blockIdx.x;
  if (gridDim.x % 8 == 0) item = (item % 8) * ((int)gridDim.x / 8) + item / 8;
  const int g = item / chunks;
  const int head_base = (item % chunks) * (16 * HG);  // first head of this chunk

  // ---- slicing by cost (cooperative, any B); scratch in the ring ----
  // A nonempty sequence costs its length plus a.seg_cost tokens (its segment
  // start: query loads, the first DMA round trip, the softmax exchanges and
  // the output stores of a piece), and the G slices are equal ranges of
  // the total cost, so a slice that holds the start of a sequence gets
  // correspondingly fewer tokens. Sequence b occupies the cost range
  // [Q_b, Q_b + c + L_b): c units of start cost, then one per token.
  // Thread i sums the costs of sequences i*cb .. i*cb + cb - 1; a shuffle
  // scan inside each wave and one pass over the NW wave totals give every
  // thread its exclusive prefix with a single barrier.
  LDS_AS long long* s_wsum = (LDS_AS long long*)smem;  // [NW] wave totals
  LDS_AS long long* s_first = s_wsum + C::NW;          // [4] first sequence of the slice: index, cost offset, length, cache row
  const int B = a.B;
  const long long c = a.seg_cost;
  const int cb = (B + NT - 1) / NT;
  long long mysum = 0;
  int L0 = 0;         // the length of this thread's first sequence (the only one when B <= NT)
  long long S0 = 0;   // ... and its first cache row, loaded alongside so that the
                      // slice's first DMA needs no further round trip
  for (int i = 0; i < cb; ++i) {
    int bb = tid * cb + i;
    if (bb < B) {
      int L = a.seq_len[bb];
      if (i == 0) S0 = a.seq_start[bb];
      L = L > 0 ? L : 0;
      if (i == 0) L0 = L;
      mysum += L > 0 ? L + c : 0;
    }
  }
  long long incl = mysum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long up = shfl_up_ll(incl, off);
    if (lane >= off) incl += up;
  }
  if (lane == 63) s_wsum[wave] = incl;
  if (tid == 0) { s_first[0] = -1; s_first[1] = 0; }
  __syncthreads();
  long long Ctot = 0, before = 0;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) {
    const long long t = s_wsum[w];
    Ctot += t;
    before += w < wave ? t : 0;
  }
  const long long excl = before + incl - mysum;
  // this slice's cost range
  const long long lo_g = (long long)g * Ctot / G;
  const long long hi_g = (long long)(g + 1) * Ctot / G;
  {
    long long p = excl;
    for (int i = 0; i < cb; ++i) {
      int bb = tid * cb + i;
      if (bb >= B) break;
      int L = L0;
      if (i > 0) { L = a.seq_len[bb]; L = L > 0 ? L : 0; }
      if (blockIdx.x == 0) a.prefix[bb] = p;
      if (L > 0 && p <= lo_g && lo_g < p + c + L) {
        s_first[0] = bb;
        s_first[1] = p;
        s_first[2] = L;
        s_first[3] = i == 0 ? S0 : a.seq_start[bb];
      }
      p += L > 0 ? L + c : 0;
    }
  }
  __syncthreads();
  int b = (int)s_first[0];
  long long Q = s_first[1];  // cost offset of sequence b
  const int L_first = (int)s_first[2];
  const long long S_first = s_first[3];
  __syncthreads();  // the scan scratch becomes ring space
  if (b < 0 || lo_g >= hi_g) return;

  // ---- per-lane constants ----
  const float scale2 = a.scale_log2;
  const int G4 = lane >> 4;                       // 16-lane group
  const int j16 = lane & 15;
  const int h = head_base + hg * 16 + j16;        // this lane's head for the scores
  const bool h_ok = h < a.H;

  // DMA: latent row t of a slot is one instruction (lane l copies bytes
  // 16 l .. 16 l + 15); wave w loads rows w, w + NW, ... and RoPE rows
  // w * ROPE_ROWS .. + ROPE_ROWS - 1 (8 lanes per row) in one more.
  const unsigned offL = (unsigned)(lane << 4);
  const int rrow = wave * C::ROPE_ROWS + (lane >> 3);

  // score operand reads: token 16 th + j16, chunk 4 kb + G4 of its row
  const int t_s = 16 * th + j16;
  const int baseS = t_s * kLatStride + 16 * G4;
  int offR[2];                                    // RoPE part, k-steps KB_C, KB_C + 1
#pragma unroll
  for (int k = 0; k < 2; ++k) offR[k] = C::LAT_BYTES + t_s * (D_R * 2) + (((4 * k + G4) ^ swr(t_s)) << 4);
  // P.V operand reads (transposing): source lane j16 of group G4 reads token
  // 4 G4 + j16/4 (+16 for the second half), features fw + 16 fb + 4 (j16 % 4)
  // .. + 3, where wave w owns the features fw = (512 / NW) w .. + 512 / NW - 1
  const int fw = (D_C / C::NW) * wave;
  const int baseV = (4 * G4 + (j16 >> 2)) * kLatStride + 8 * (j16 & 3) + 2 * fw;
  LDS_AS float* s_mx = (LDS_AS float*)(smem + C::X_OFF);  // [2][16 HG] per-half head maxima
  LDS_AS float* s_ls = s_mx + 2 * 16 * HG;                  // [2][16 HG] per-half head sums
  const int xi = 16 * hg + j16;                             // this lane's head in the exchange arrays

  const unsigned long long cache_addr = (unsigned long long)(uintptr_t)a.cache;

  for (bool first_seg = true; b < B && Q < hi_g; ++b, first_seg = false) {
    const int Lb = first_seg ? L_first : a.seq_len[b];
    if (Lb <= 0) continue;
    const long long tok_c = Q + c;                // cost position of the sequence's first token
    const long long seg_lo = tok_c > lo_g ? tok_c : lo_g;
    const long long seg_hi = (tok_c + Lb) < hi_g ? (tok_c + Lb) : hi_g;
    const bool complete = (tok_c >= lo_g) && (tok_c + Lb <= hi_g);
    // a partial piece that follows another piece of the slice goes to slot
    // 2g + 1, the one that opens the slice to slot 2g
    const bool inside = lo_g < Q;
    Q += Lb + c;
    if (seg_lo >= seg_hi) continue;               // the slice ends within this sequence's start cost
    const int t0 = (int)(seg_lo - tok_c);         // first token of the segment in sequence b
    const int n = (int)(seg_hi - seg_lo);         // tokens in the segment
    const long long row0 = first_seg ? S_first : a.seq_start[b];
    const unsigned long long seg_addr = cache_addr + (unsigned long long)(row0 + t0) * C::RWB;

    const int nslots = (n + 31) >> 5;             // 32-token slots of the segment

    // DMA instruction k (< ROUNDS) of slot j (tokens 32 j .. 32 j + 31), into
    // ring position j % R: latent rows first, then the RoPE rows
    auto load_part = [&](int j, int k) {
      const unsigned sb = smem_base + (unsigned)((j % R) * C::SLOT_BYTES);
      const int tok0 = 32 * j;
      if (k < C::ROWS_L) {
        const int t = wave + C::NW * k;
        int row = tok0 + t;
        row = row < n ? row : n - 1;
        g2lds16_s(seg_addr + (unsigned long long)row * C::RWB, offL, sb + t * kLatStride);
      } else if constexpr (D_R > 0) {
        // a scalar base row plus a small per-lane row offset
        int row0 = tok0 + wave * C::ROPE_ROWS;
        row0 = row0 < n ? row0 : n - 1;
        int row = tok0 + rrow;
        row = row < n ? row : n - 1;
        const unsigned off = (unsigned)(D_C * 2 + (((lane & 7) ^ swr(rrow)) << 4));
        if (C::ROPE_ROWS * 8 == 64 || lane < C::ROPE_ROWS * 8)
          g2lds16_s(seg_addr + (unsigned long long)row0 * C::RWB, (unsigned)(row - row0) * C::RWB + off,
                    sb + C::LAT_BYTES + wave * C::ROPE_ROWS * 128);
      }
    };
    auto load_slot = [&](int j) {
#pragma unroll
      for (int k = 0; k < C::ROUNDS; ++k) load_part(j, k);
    };

    // the first slots of pass 0 go out before the queries are loaded, so the
    // two memory latencies overlap
#pragma unroll
    for (int j = 0; j < C::PD; ++j)
      if (j < nslots) load_slot(j);

    // queries of this lane's head: k-step kb holds features 32 kb + 8 G4 .. +7,
    // the RoPE part rotated to position Lb-1
    bf16x8 q[C::KB];
    {
      const bf16* qp = a.q + ((int64_t)b * a.H + (h_ok ? h : 0)) * C::RW + 8 * G4;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        u32x4 v = h_ok ? *(const u32x4*)(qp + 32 * kb) : u32x4{0, 0, 0, 0};
        q[kb] = as_bf16x8(v);
      }
      if constexpr (D_R > 0) {
        if (a.rope_base != 0.0f) {
          const double pos = (double)(Lb - 1);
          const double lb = log2((double)a.rope_base);
#pragma unroll
          for (int kb = C::KB_C; kb < C::KB; ++kb) {
            const int i0 = (32 * kb + 8 * G4 - D_C) / 2;  // first pair index
            bf16x8 r = q[kb];
            unsigned int w[4];
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              const double theta = exp2(-(2.0 * (i0 + pr) / D_R) * lb);
              double ang = pos * theta;
              ang -= 6.283185307179586 * floor(ang * 0.15915494309189535);
              float s, c;
              sincosf((float)ang, &s, &c);
              const float x0 = (float)r[2 * pr], x1 = (float)r[2 * pr + 1];
              w[pr] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
            }
            q[kb] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
          }
        }
      }
    }

    // O^T of every head of the workgroup over this wave's features:
    // o[fb * HG + hb] = features fw + 16 fb + 4 G4 + r, head 16 hb + j16
    floatx4 o[C::FBW * HG];
    float m = -INFINITY;     // reference max (log2 domain) of this lane's head
    float m_all = -INFINITY; // largest score of this lane (its head, its tokens) in the pass
    float lsum = 0.f;        // this lane's share of the softmax denominator

    // Pass 0 fixes each head's reference max at its first tile and never
    // rescales O. If a later score exceeds the reference by more than
    // 2^kRedo the pass may have lost range; the workgroup then repeats the
    // segment once with the true max as reference (pass 1), which cannot
    // overflow.
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int i = 0; i < C::FBW * HG; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      lsum = 0.f;
      m_all = -INFINITY;
      if (pass > 0) {
        lds_barrier();  // every wave is done with the ring
#pragma unroll
        for (int j = 0; j < C::PD; ++j)
          if (j < nslots) load_slot(j);
      }

      // O^T (this wave's features x all heads) += C^T . P^T for the tile in
      // ring slot `slot`, with the weights published in P buffer `pbi` (each
      // head group's B operand, written half by half by its two waves)
      auto pv = [&](int slot, int pbi) {
        const LDS_AS char* vbuf = smem + slot * C::SLOT_BYTES;
        const LDS_AS char* pbuf = smem + C::P_OFF + pbi * (HG * 1024);
        bf16x8 pt[HG];
#pragma unroll
        for (int hb = 0; hb < HG; ++hb) pt[hb] = as_bf16x8(lds_read16(pbuf + hb * 1024 + lane * 16));
        auto readV = [&](int fb) -> bf16x8 {
          u32x2 lo = lds_read_tr16(vbuf + baseV + 32 * fb);
          u32x2 hi2 = lds_read_tr16(vbuf + baseV + 16 * kLatStride + 32 * fb);
          return as_bf16x8(u32x4{lo[0], lo[1], hi2[0], hi2[1]});
        };
        constexpr int PFV = C::FBW < 4 ? C::FBW : 4;  // each fragment feeds HG MFMAs
        bf16x8 fr[PFV];
#pragma unroll
        for (int fb = 0; fb < PFV; ++fb) fr[fb] = readV(fb);
#pragma unroll
        for (int fb = 0; fb < C::FBW; ++fb) {
#pragma unroll
          for (int hb = 0; hb < HG; ++hb)
            o[fb * HG + hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[fb % PFV], pt[hb], o[fb * HG + hb], 0, 0, 0);
          if (fb + PFV < C::FBW) fr[fb % PFV] = readV(fb + PFV);
        }
      };

      // Software pipeline, one barrier per tile: iteration `it` computes the
      // scores and weights of tile it and the P.V product of tile it - 1
      // (whose weights the barrier has just made visible), so the softmax
      // arithmetic of one tile overlaps the P.V MFMAs of the previous one.
      for (int it = 0; it < nslots; ++it) {
        // slot it is read now; slots issued after it may stay in flight
        int issued = C::PD + it;
        issued = issued < nslots ? issued : nslots;
        wait_slots<C::ROUNDS, C::PD - 1>(issued - (it + 1));
        lds_barrier();
        // the next slot's DMA is issued one instruction at a time between the
        // score MFMAs: an issue that waits for room in the memory queue then
        // holds up this wave only, while the other wave of its SIMD computes
        const bool load_next = C::PD + it < nslots;
        if (!kSpreadDMA && load_next) load_slot(C::PD + it);

        const LDS_AS char* buf = smem + (it % R) * C::SLOT_BYTES;
        // ---- S^T (16 tokens x 16 heads) ----
        // LDS reads are issued kPF steps ahead of their MFMA
        auto readS = [&](int kb) -> bf16x8 {
          if (kb < C::KB_C) return as_bf16x8(lds_read16(buf + baseS + 64 * kb));
          return as_bf16x8(lds_read16(buf + offR[kb - C::KB_C]));
        };
        floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
        {
          constexpr int PF = kPF < C::KB ? kPF : C::KB;
          bf16x8 fr[PF];
#pragma unroll
          for (int x = 0; x < PF; ++x) fr[x] = readS(x);
#pragma unroll
          for (int x = 0; x < C::KB; ++x) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[x % PF], q[x], s, 0, 0, 0);
            if (x + PF < C::KB) fr[x % PF] = readS(x + PF);
            if constexpr (kSpreadDMA) {
              constexpr int SP = C::KB / C::ROUNDS;  // score steps per DMA instruction
              if (x % SP == 0 && x / SP < C::ROUNDS && load_next) load_part(C::PD + it, x / SP);
            }
            // the order is kept for the 16 k-steps of the NoPE scores; with
            // the RoPE k-steps the compiler's own order measured 1-2% faster
            if constexpr (D_R == 0) __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- P.V of the previous tile ----
        if (it > 0) pv((it - 1) % R, (it - 1) & 1);
        // ---- softmax weights; lane owns head j16, tokens 32 it + 16 th + 4 G4 + r ----
        const int tok_base = 32 * it + 16 * th + 4 * G4;
        float z[4];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[r] = tok_base + r < n ? s[r] * scale2 : -INFINITY;
          mx = fmaxf(mx, z[r]);
        }
        if (pass == 0 && it == 0) {
          // reference max: the head's max over the first tile, from both halves
          mx = head_max(mx);
          if (G4 == 0) s_mx[th * 16 * HG + xi] = mx;
          lds_barrier();
          m = fmaxf(s_mx[xi], s_mx[16 * HG + xi]);
        }
        m_all = fmaxf(m_all, mx);
        const float mref = (m == -INFINITY) ? 0.f : m;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(z[r] - mref);
          lsum += p[r];
        }
        // this half of the head group's P^T operand: k = 8 G4 + 4 th + r <->
        // token 16 th + 4 G4 + r
        *(LDS_AS u32x2*)(smem + C::P_OFF + (it & 1) * (HG * 1024) + hg * 1024 + lane * 16 + th * 8) =
            u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      }
      // ---- P.V of the last tile ----
      lds_barrier();
      if (nslots > 0) pv((nslots - 1) % R, (nslots - 1) & 1);
      // ---- overflow check: any head whose scores outgrew its reference ----
      m_all = head_max(m_all);
      const bool redo = (m != -INFINITY) && (m_all > m + kRedo);
      const bool wave_redo = __builtin_amdgcn_ballot_w64(redo) != 0;
      lds_barrier();  // every wave is done with the ring and the exchange arrays
      if (lane == 0) ((LDS_AS int*)smem)[wave] = wave_redo ? 1 : 0;
      if (G4 == 0) s_mx[th * 16 * HG + xi] = m_all;
      lds_barrier();
      int any = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) any |= ((const LDS_AS int*)smem)[w];
      if (!any) break;
      m = fmaxf(s_mx[xi], s_mx[16 * HG + xi]);
    }

    // ---- finish the segment ----
    // both halves publish their sums; every wave then scales and stores its
    // features of all heads
    lsum = head_sum(lsum);
    if (G4 == 0) s_ls[th * 16 * HG + xi] = lsum;
    lds_barrier();
    const long long slot = inside ? (2LL * g + 1) : (2LL * g);
    if (th == 0 && h_ok && G4 == 0) {
      const float lse_nat = m * kLn2 + __logf(s_ls[xi] + s_ls[16 * HG + xi]);
      if (!complete) a.part_lse[slot * a.H + h] = lse_nat;
      else if (a.lse) a.lse[(int64_t)b * a.H + h] = lse_nat;
    }
    const int H16 = (a.H + 15) >> 4;
#pragma unroll
    for (int hb = 0; hb < HG; ++hb) {
      const int hh = head_base + 16 * hb + j16;  // head of this lane's column in block hb
      if (hh < a.H) {
        const float inv = 1.0f / (s_ls[16 * hb + j16] + s_ls[16 * HG + 16 * hb + j16]);
        if (complete) {
          bf16* op = a.o_lat + ((int64_t)b * a.H + hh) * D_C + fw + 4 * G4;
#pragma unroll
          for (int fb = 0; fb < C::FBW; ++fb) {
            const floatx4 u = o[fb * HG + hb];
            *(u32x2*)(op + 16 * fb) = u32x2{pack_bf16x2(u[0] * inv, u[1] * inv), pack_bf16x2(u[2] * inv, u[3] * inv)};
          }
        } else {
          // partial piece, bf16, in register order: record K = fw / 32 + k of
          // head group hh / 16 holds features 32 K + 4 G4 + r and
          // 32 K + 16 + 4 G4 + r (r < 4) of head hh; one store writes 1 KiB
          bf16* op = a.part_o + ((slot * H16 + (hh >> 4)) * 16 + fw / 32) * (int64_t)512 + lane * 8;
#pragma unroll
          for (int k = 0; k < C::FBW / 2; ++k) {
            const floatx4 u = o[(2 * k) * HG + hb], v = o[(2 * k + 1) * HG + hb];
            *(u32x4*)(op + k * 512) = u32x4{pack_bf16x2(u[0] * inv, u[1] * inv), pack_bf16x2(u[2] * inv, u[3] * inv),
                                            pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
          }
        }
      }
    }
    lds_barrier();  // the exchange arrays are rewritten by the next segment
  }
}

// Merge the partial pieces of every sequence that was cut across slices, and
// define the result of an empty sequence (o = 0, lse = -inf): the log-sum-exp
// merge of split softmax sums. Workgroup = (sequence, group of 16 heads,
// quarter of the features); thread = one 16-byte lane record of one store
// index k of the pieces' wave-ordered layout (see the attention epilogue).
// The loads of NB pieces are issued together, so the merge costs one memory
// latency per NB pieces; the slot of every piece follows from the sequence's
// first and last slice (three divisions per thread, plus one per piece only
// when there are more slices than tokens and a slice can be empty).
template <int NB>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int D_C = 512;
  const int H16 = (a.H + 15) >> 4;
  const int b = blockIdx.x / (H16 * 4);
  const int hg = (blockIdx.x / 4) % H16;
  const int k = (blockIdx.x % 4) * 4 + (threadIdx.x >> 6);  // store index 0..15
  const int lane = threadIdx.x & 63;
  const int h = hg * 16 + (lane & 15);
  const int G4 = lane >> 4;
  if (h >= a.H) return;
  // every length and offset this thread needs, loaded together
  const int Lb = a.seq_len[b];
  const int Llast = a.seq_len[a.B - 1];
  const long long Qlast = a.prefix[a.B - 1];
  const long long Q = a.prefix[b];  // cost offset of sequence b (the attention kernel's slicing)
  bf16* op = a.o_lat + ((int64_t)b * a.H + h) * D_C + 32 * k + 4 * G4;  // features +0..3 and +16..19
  if (Lb <= 0) {
    *(u32x2*)op = u32x2{0u, 0u};
    *(u32x2*)(op + 16) = u32x2{0u, 0u};
    if (k == 0 && G4 == 0 && a.lse) a.lse[(int64_t)b * a.H + h] = -INFINITY;
    return;
  }
  const long long c = a.seg_cost;
  const long long N = Qlast + (Llast > 0 ? Llast + c : 0);  // total cost
  const int G = a.G;
  // slice whose cost range holds position x: the largest g with floor(g N / G) <= x;
  // the sequence's tokens hold the cost positions Q + c .. Q + c + Lb - 1
  const long long g_lo = ((Q + c + 1) * G - 1) / N;
  const long long g_hi = ((Q + c + Lb) * G - 1) / N;
  if (g_lo == g_hi) return;  // whole sequence inside one slice: already final
  // a piece that opens its slice sits in slot 2g, one that follows another
  // piece of the slice in 2g + 1; only the first piece can follow another
  const bool lo_inside = g_lo * N / G < Q;
  const bool may_empty = N < G;  // otherwise every slice holds at least one cost unit
  float M = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (long long g0 = g_lo; g0 <= g_hi; g0 += NB) {
    float l[NB];
    u32x4 raw[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const long long g = g0 + i;
      l[i] = -INFINITY;
      raw[i] = u32x4{0u, 0u, 0u, 0u};
      if (g <= g_hi && (!may_empty || g * N / G != (g + 1) * N / G)) {
        const long long slot = (g == g_lo && lo_inside) ? 2 * g + 1 : 2 * g;
        l[i] = a.part_lse[slot * a.H + h];
        raw[i] = *(const u32x4*)(a.part_o + ((slot * H16 + hg) * 16 + k) * (int64_t)512 + lane * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (l[i] == -INFINITY) continue;
      const float Mn = fmaxf(M, l[i]);
      const float c = __expf(M - Mn), w = __expf(l[i] - Mn);
      den = den * c + w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __builtin_bit_cast(float, raw[i][e] << 16), hi = __builtin_bit_cast(float, raw[i][e] & 0xffff0000u);
        acc[2 * e] = acc[2 * e] * c + w * lo;
        acc[2 * e + 1] = acc[2 * e + 1] * c + w * hi;
      }
      M = Mn;
    }
  }
  const float inv = 1.f / den;
  *(u32x2*)op = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *(u32x2*)(op + 16) = u32x2{pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  if (k == 0 && G4 == 0 && a.lse) a.lse[(int64_t)b * a.H + h] = M + __logf(den);
}

// ---------------------------------------------------------------------------
template <int D_R, int HG, int R>
static hipError_t launch_variant(const DecodeArgs& a, hipStream_t st) {
  using C = DecodeCfg<D_R, HG, R>;
  auto kern = decode_attn_kernel<D_R, HG, R>;
  {
    hipError_t e = lds_opt_in((const void*)kern, C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const int chunks = (a.H + 16 * HG - 1) / (16 * HG);
  return launch(kern, dim3(a.G * chunks), dim3(C::NW * 64), C::LDS_BYTES, st, a);
}

int decode_head_chunks(int H) { return H <= 32 ? 1 : (H + 63) / 64; }

hipError_t launch_decode_attn(const DecodeArgs& a, hipStream_t st) {
  // 32 or 64 heads per workgroup (4 or 8 waves); more heads run as chunks of 64
  if (a.d_c != 512) return hipErrorInvalidValue;
  if ((long long)a.G * decode_head_chunks(a.H) > 2147483647LL) return hipErrorInvalidValue;
  const bool small = a.H <= 32;
  if (a.d_r == 0) return small ? launch_variant<0, 2, kRing>(a, st) : launch_variant<0, 4, kRing>(a, st);
  if (a.d_r == 64) return small ? launch_variant<64, 2, kRing>(a, st) : launch_variant<64, 4, kRing>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st) {
  if (a.d_c != 512) return hipErrorInvalidValue;
  const long long blocks = (long long)a.B * ((a.H + 15) / 16) * 4;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  // pieces per sequence are about G / B + 1: issue the loads of that many
  // together (at most 16, which bounds the registers)
  const long long per_seq = a.B > 0 ? (long long)a.G / a.B + 1 : 1;
  if (per_seq > 8) return launch(decode_combine_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  if (per_seq > 4) return launch(decode_combine_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return launch(decode_combine_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, a);
}

// The MFMA kernel takes the d_c = 512 latent (1 KiB rows, one direct-to-LDS
// load each) with d_r in {0, 64}; other widths run the generic bf16 decode.
bool decode_bf16_supported(int d_c, int d_r) { return d_c == 512 && (d_r == 0 || d_r == 64); }

}  // namespace gmla
