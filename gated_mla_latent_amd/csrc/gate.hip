// Per-head scalar output gate (bf16, gfx950), the variant of the concept page
// "Gated Multi-head Latent Attention (Gated MLA)" (Gating Mechanism,
// Mathematical Formulation): g_(t,h) = Sigmoid(z_(t,h) + b_h) with the
// logits z = x W_g^T from a GEMM, and head h's output block scaled by it,
//     gated[t, h d_v + j] = g_(t,h) o~[t, h d_v + j],
// before the output projection. Elementwise and HBM-bound: one thread per 8
// channels of one head (16-byte loads and stores); the logit and the bias are
// re-read from L1/L2 by the d_v / 8 threads of a head.
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

__global__ __launch_bounds__(256) void head_gate_kernel(HeadGateArgs a) {
  const int per_row = a.H * a.d_v / 8;
  const int64_t n = (int64_t)a.T * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / per_row;
    const int c = (int)(i % per_row) * 8;  // channel h d_v + j, j % 8 == 0
    const int h = c / a.d_v;
    float z = (float)a.z[t * a.ldz + h];
    if (a.bias) z += (float)a.bias[h];
    const float g = 1.0f / (1.0f + __expf(-z));
    const u32x4 v = *(const u32x4*)(a.o + t * a.ldo + c);
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = pack_bf16x2(g * bf16_bits_to_f32((unsigned short)(v[e] & 0xffff)),
                         g * bf16_bits_to_f32((unsigned short)(v[e] >> 16)));
    *(u32x4*)(a.gated + t * a.ldg + c) = r;
  }
}

}  // namespace

hipError_t launch_head_gate(const HeadGateArgs& a, hipStream_t st) {
  if (a.T <= 0 || a.H <= 0) return hipSuccess;
  if (a.d_v % 8 != 0 || a.ldo % 8 != 0 || a.ldg % 8 != 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.T * a.H * a.d_v / 8;
  const int64_t blocks = (n + 255) / 256;
  return launch(head_gate_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, st, a);
}

}  // namespace gmla
