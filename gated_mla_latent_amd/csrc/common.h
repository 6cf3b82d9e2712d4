// Shared device helpers for the gfx950 kernels of libgmla.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

// ---- bf16 conversion (round to nearest even; NaN stays NaN) -------------
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned int u = __builtin_bit_cast(unsigned int, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, (unsigned int)h << 16);
}
// two floats -> packed bf16x2 (lo = a), round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((float2_t){a, b}, bf16x2_t));
}

// Scheduling hints: keep `ahead` LDS reads in flight in front of a chain of
// `n` MFMAs that each consume `per` reads (reads and MFMAs otherwise free).
#define GMLA_SCHED_DS_MFMA(n, per, ahead)                                   \
  do {                                                                      \
    __builtin_amdgcn_sched_group_barrier(0x100, (ahead), 0);                \
    _Pragma("unroll") for (int _i = 0; _i < (n) - (ahead) / (per); ++_i) {  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    \
      __builtin_amdgcn_sched_group_barrier(0x100, (per), 0);                \
    }                                                                       \
    __builtin_amdgcn_sched_group_barrier(0x008, (ahead) / (per), 0);        \
  } while (0)

// ---- MFMA wrappers ---------------------------------------------------------
// D(32x32) += A(32x16) * B(16x32). Lane l holds A[l%32][8(l/32)+e], B[8(l/32)+e][l%32];
// accumulator register r of lane l is D[8(r/4) + 4(l/32) + r%4][l%32].
__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16). Lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16];
// accumulator register r of lane l is D[4(l/16) + r][l%16].
__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// ---- LDS access --------------------------------------------------------------
__device__ __forceinline__ u32x4 lds_read16(const LDS_AS void* p) {
  return *(const LDS_AS u32x4*)p;
}
// Transposing 8-byte LDS read: within each group of 16 lanes, lane i receives
// element i%4 of the 8 bytes read by lane 4e + i/4, as its element e.
__device__ __forceinline__ u32x2 lds_read_tr16(const LDS_AS void* p) {
  short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Direct global -> LDS copy of 16 bytes per lane. The 64 lanes of the wave
// write 1 KiB contiguously at byte address lds_wave_base (lane l at +16 l);
// lds_wave_base must be wave-uniform.
// Issued from inline asm on purpose: the compiler's wait-count pass cannot
// tell which LDS bytes a DMA load writes, so with the builtin it drains every
// outstanding load before each LDS read, which serialises a multi-buffered
// ring. Callers order the DMA with wait_vmcnt<>() and lds_barrier() instead.
// M0 carries the LDS base: it is written here (one wait state before the DMA,
// as the compiler's own lowering does) and left as is. The compiler keeps no
// value of its own in M0 in these kernels.
__device__ __forceinline__ void g2lds16(const void* gptr, const LDS_AS void* lds_wave_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_wave_base);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(base)
      : "memory", "m0");
}

// Same, with a 64-bit scalar base address plus a 32-bit per-lane byte offset
// (global_load_lds ... v_offset, s[base]): the base and the LDS destination
// are scalar, so a whole 1 KiB row costs no 64-bit vector address arithmetic.
// Five wait states precede the load: the scalar base may come straight from
// v_readfirstlane (a VALU write of an SGPR that a VMEM instruction then reads),
// a hazard the compiler cannot see inside asm; they also cover the M0 write.
__device__ __forceinline__ void g2lds16_s(unsigned long long sbase, unsigned voff, unsigned lds_wave_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_wave_base)
      : "memory", "m0");
}

// Workgroup barrier without the memory fence __syncthreads() implies (that
// fence waits for every outstanding global load, including in-flight DMA).
// LDS reads before the barrier complete first (lgkmcnt(0)).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");       // no compiler motion of memory ops across
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt unconstrained
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// value from lane l ^ 32
__device__ __forceinline__ float xor32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate the interleaved pair (x0, x1) with index i of a d_r-wide RoPE vector
// to position pos, theta_i = base^(-2i / d_r) ([N03] "LLM 注意力与计算内核精读笔记
// · 03" §5.2); the angle is formed and reduced modulo 2 pi in fp64 so that long
// positions keep their accuracy, then fp32 sine and cosine.
__device__ __forceinline__ void rope_pair(float& x0, float& x1, int i, int d_r, double log2_base, double pos) {
  const double theta = exp2(-(2.0 * i / d_r) * log2_base);
  double ang = pos * theta;
  ang -= 6.283185307179586 * floor(ang * 0.15915494309189535);
  float s, c;
  sincosf((float)ang, &s, &c);
  const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}

}  // namespace gmla
