// Per-token int8 quantization of Q or K for the int8 QK product.
//
// "H3 SLA Attention", inputs table, use_int8_qk: Q and K are quantized to int8 per token
// with a dynamic scale before the QK product; PV stays in full precision. For each
// (row, head) vector x of head_dim values, in float32 with correct rounding:
//   s = amax / 127,  x8 = clamp(rint(x / s), -127, 127)  (rint: half to even),
// and s = 0 with x8 = 0 for a zero vector. HBM-bound: one read of x, one write of x8 and
// one float per (row, head).
#include "h3_internal.h"

namespace h3 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LPP = D / 8 lanes per (row, head), 8 values per lane (16 bytes of bf16, 32 of float).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void quant_int8_kernel(const void* __restrict__ x, int64_t pairs,
                                                         int8_t* __restrict__ x8,
                                                         float* __restrict__ sc) {
  constexpr int LPP = D / 8;
  // grid-stride over whole 256-thread rounds, so every lane of a (row, head) group runs
  // the same iterations and takes part in the shuffles
  const int64_t total = (pairs * LPP + 255) / 256 * 256;
  for (int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x; gl < total;
       gl += (int64_t)gridDim.x * 256) {
  const int64_t pair = gl / LPP;
  const int part = (int)(gl % LPP);
  const bool valid = pair < pairs;
  float v[8];
  if (valid) {
    const int64_t e0 = pair * D + part * 8;
    if (BF16) {
      const u32x4 u = *(const u32x4*)((const uint16_t*)x + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ((const float*)x)[e0 + i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = LPP / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = __fdiv_rn(amax, 127.0f);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qv = 0;
    if (s > 0.f) qv = (int)fminf(fmaxf(rintf(__fdiv_rn(v[i], s)), -127.f), 127.f);
    w[i >> 2] |= ((uint32_t)qv & 0xFFu) << (8 * (i & 3));
  }
  if (valid) {
    *(u32x2*)(x8 + pair * D + part * 8) = u32x2{w[0], w[1]};
    if (part == 0) sc[pair] = s;
  }
  }
}

}  // namespace

hipError_t launch_quant_int8(const void* x, bool bf16, int64_t pairs, int D, int8_t* x8,
                             float* sc, hipStream_t s) {
  const int64_t blocks = (pairs * (D / 8) + 255) / 256;
  const dim3 grid((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20)));
  if (D == 128) {
    if (bf16) quant_int8_kernel<128, true><<<grid, 256, 0, s>>>(x, pairs, x8, sc);
    else quant_int8_kernel<128, false><<<grid, 256, 0, s>>>(x, pairs, x8, sc);
  } else {
    if (bf16) quant_int8_kernel<64, true><<<grid, 256, 0, s>>>(x, pairs, x8, sc);
    else quant_int8_kernel<64, false><<<grid, 256, 0, s>>>(x, pairs, x8, sc);
  }
  return hipGetLastError();
}

}  // namespace h3
