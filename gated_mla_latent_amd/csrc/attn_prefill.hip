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
//  * One workgroup = (b, h, 256 queries); wave w owns 64 queries (two 32-row
//    MFMA blocks), so every K/V fragment read from LDS feeds two MFMAs.
//  * K and V tiles of 64 keys stream through a 2-stage LDS ring with 16-byte
//    direct-to-LDS loads, rows XOR-swizzled on 16-byte chunks.
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query and
//    16 keys, so the softmax max needs one exchange with lane ^ 32.
//  * O^T += V^T . P^T: P^T is the S^T accumulator (rounded to bf16) and V^T
//    fragments come from ds_read_b64_tr_b16 transposing reads.
//  * No rescale of O inside the loop: each query's reference max is fixed at
//    its first key tile; if a later score outgrows it by more than 2^32 the
//    workgroup redoes the pass once with the true maxima (exact for any input).
//  * Query tiles are issued longest-first (largest t first) to even out the
//    triangular work.
#include "common.h"
#include "kernels.h"

namespace gmla {

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void prefill_attn_kernel(AttnArgs a) {
  constexpr int BQ = 256, BKEY = 64;
  constexpr int ROWB = D * 2, CH = D / 8;       // bytes and 16-byte chunks per row
  constexpr int TILE = BKEY * ROWB;             // one K (or V) tile
  constexpr int STAGE = 2 * TILE;
  constexpr int ROUNDS = BKEY * CH / 256;
  constexpr int KS = D / 16;                    // k-steps of S^T
  constexpr int DB = D / 32;                    // output blocks of O^T
  static_assert(CH == 16 || CH == 8, "row of 8 or 16 chunks");
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nqt = (a.L + BQ - 1) / BQ;
  const int qt = nqt - 1 - (int)(blockIdx.x % nqt);  // longest first
  const int bh = blockIdx.x / nqt;
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qt * BQ;
  const int wq0 = q0 + 64 * wave;                    // this wave's first query

  const bf16* qb = a.q + b * a.sqb + h * a.sqh;
  const bf16* kb = a.k + b * a.skb + h * a.skh;
  const bf16* vb = a.v + b * a.svb + h * a.svh;
  bf16* ob = a.o + b * a.sob + h * a.soh;

  auto swz = [](int row) { return CH == 16 ? (row & 15) : ((row >> 1) & 7); };

  // queries of this wave: Q^T fragments for two 32-query blocks
  bf16x8 qf[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int t = wq0 + 32 * j + (lane & 31);
    t = t < a.L ? t : a.L - 1;
    const bf16* qp = qb + (int64_t)t * a.sqt + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[j][kk] = as_bf16x8(*(const u32x4*)(qp + 16 * kk));
  }

  auto load_tile = [&](int s, int kt) {
    LDS_AS char* kt_l = smem + s * STAGE;
    LDS_AS char* vt_l = kt_l + TILE;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int p = r * 256 + wave * 64 + lane;
      const int row = p / CH, c = (p % CH) ^ swz(p / CH);
      int t = kt * BKEY + row;
      t = t < a.L ? t : a.L - 1;
      g2lds16(kb + (int64_t)t * a.skt + c * 8, kt_l + (r * 256 + wave * 64) * 16);
      g2lds16(vb + (int64_t)t * a.svt + c * 8, vt_l + (r * 256 + wave * 64) * 16);
    }
  };

  floatx16 o[2][DB];
  float m[2] = {-INFINITY, -INFINITY};      // reference max per query (log2 domain)
  float m_all[2] = {-INFINITY, -INFINITY};  // largest score seen
  float lsum[2] = {0.f, 0.f};

  int last_q = q0 + BQ - 1;
  last_q = last_q < a.L - 1 ? last_q : a.L - 1;
  const int ntiles = last_q / BKEY + 1;                  // tiles the workgroup needs
  int my_last = wq0 + 63;
  my_last = my_last < a.L - 1 ? my_last : a.L - 1;
  const int my_tiles = wq0 < a.L ? my_last / BKEY + 1 : 0;  // tiles this wave needs

  // Pass 0 fixes each query's reference max at its first key tile and never
  // rescales O inside the loop; if a later score outgrows the reference by
  // more than 2^32 the workgroup repeats the pass with the true maxima.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int d = 0; d < DB; ++d) o[j][d] = floatx16{};
      lsum[j] = 0.f;
    }
    lds_barrier();
    load_tile(0, 0);
    for (int it = 0; it < ntiles; ++it) {
      wait_vmcnt<0>();
      lds_barrier();
      if (it + 1 < ntiles) load_tile((it + 1) & 1, it + 1);
      if (it >= my_tiles) continue;
      const LDS_AS char* kt_l = smem + (it & 1) * STAGE;
      const LDS_AS char* vt_l = kt_l + TILE;

      // ---- S^T: 64 keys (2 blocks) x 64 queries (2 blocks) ----
      floatx16 s[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) s[i][j] = floatx16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int c = 2 * kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = 32 * i + (lane & 31);
          bf16x8 kf = as_bf16x8(lds_read16(kt_l + row * ROWB + ((c ^ swz(row)) << 4)));
#pragma unroll
          for (int j = 0; j < 2; ++j) s[i][j] = mfma32(kf, qf[j][kk], s[i][j]);
        }
      }
      // ---- softmax weights per query (lane owns query 32j + lane%32) ----
      const bool diag = (it + 1) * BKEY > wq0;  // some key may lie past some query
      bf16x8 pb[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tq = wq0 + 32 * j + (lane & 31);
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = it * BKEY + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            float z = s[i][j][r] * a.scale_log2;
            if (diag) z = key <= tq ? z : -INFINITY;
            s[i][j][r] = z;
            mx = fmaxf(mx, z);
          }
        mx = fmaxf(mx, xor32(mx));
        m_all[j] = fmaxf(m_all[j], mx);
        if (m[j] == -INFINITY) m[j] = mx;  // O is still zero for this query
        const float mref = (m[j] == -INFINITY) ? 0.f : m[j];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(s[i][j][r] - mref);
            lsum[j] += p[r];
          }
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            pb[j][2 * i + hf] = as_bf16x8(u32x4{pack_bf16x2(p[8 * hf + 0], p[8 * hf + 1]),
                                                pack_bf16x2(p[8 * hf + 2], p[8 * hf + 3]),
                                                pack_bf16x2(p[8 * hf + 4], p[8 * hf + 5]),
                                                pack_bf16x2(p[8 * hf + 6], p[8 * hf + 7])});
        }
      }
      // ---- O^T (D x 64 queries) += V^T . P^T ----
      {
        const int G16 = lane >> 4, jj = lane & 15;
        const int trow = 4 * (G16 >> 1) + (jj >> 2);
        const int cpart = 2 * (G16 & 1) + ((jj & 3) >> 1);
        const int half = (jj & 1) << 3;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int ta = trow + 16 * ks, tb = ta + 8;
          const LDS_AS char* ra = vt_l + ta * ROWB + half;
          const LDS_AS char* rb = vt_l + tb * ROWB + half;
          const int sa = swz(ta), sb = swz(tb);
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const int c = 4 * d + cpart;
            u32x2 lo = lds_read_tr16(ra + ((c ^ sa) << 4));
            u32x2 hi = lds_read_tr16(rb + ((c ^ sb) << 4));
            bf16x8 vf = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
            for (int j = 0; j < 2; ++j) o[j][d] = mfma32(vf, pb[j][ks], o[j][d]);
          }
        }
      }
    }
    bool redo = false;
#pragma unroll
    for (int j = 0; j < 2; ++j) redo |= (m[j] != -INFINITY) && (m_all[j] > m[j] + 32.0f);
    if (!__syncthreads_or(redo)) break;
    m[0] = m_all[0];
    m[1] = m_all[1];
  }

  // ---- write o~ ----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float l = lsum[j] + xor32(lsum[j]);
    const int tq = wq0 + 32 * j + (lane & 31);
    if (tq >= a.L) continue;
    const float inv = 1.0f / l;
    bf16* op = ob + (int64_t)tq * a.sot + 4 * (lane >> 5);
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(u32x2*)(op + 32 * d + 8 * r4) = u32x2{pack_bf16x2(o[j][d][4 * r4] * inv, o[j][d][4 * r4 + 1] * inv),
                                                pack_bf16x2(o[j][d][4 * r4 + 2] * inv, o[j][d][4 * r4 + 3] * inv)};
  }
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  constexpr int LDS = 2 * 2 * 64 * D * 2;
  auto kern = prefill_attn_kernel<D>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int nqt = (a.L + 255) / 256;
  hipLaunchKernelGGL(kern, dim3(nqt * a.B * a.H), dim3(256), LDS, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn_bf16(const AttnArgs& a, hipStream_t st) {
  if (a.D == 128) return launch_d<128>(a, st);
  if (a.D == 64) return launch_d<64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace gmla
