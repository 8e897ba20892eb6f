// Stable log-sum-exp merge of partition results, and accumulator finalisation.
//
// "Flash Partitions for H3 native temporal alignment", section 4: each partition
// keeps its natural-log normaliser L_i; with multiplier w_i the merged result is
//   L = logsumexp(L_i + log w_i),  O = sum_i exp(L_i + log w_i - L) O_i.
// Successive merges use logaddexp; nothing subtracts two large outputs.
// Memory bound: one read of each operand and one write of the accumulator.
#include "h3_internal.h"

namespace h3 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// D/4 lanes own one (row, head) pair; all of them sit in one wave, so the pair's
// normaliser is read by every lane before the owning lane rewrites it.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(float* __restrict__ o_acc,
                                                        float* __restrict__ lse_acc,
                                                        const float* __restrict__ o_i,
                                                        const float* __restrict__ lse_i,
                                                        float log_w,
                                                        const float* __restrict__ log_w_rows,
                                                        int64_t pairs) {
  constexpr int LPP = D / 4;
  for (int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x; gt < pairs * LPP;
       gt += (int64_t)gridDim.x * 256) {
  const int64_t pair = gt / LPP;
  const int part = (int)(gt % LPP);
  const float a = lse_acc[pair];
  float b = lse_i[pair] + log_w;
  if (log_w_rows) b += log_w_rows[pair];
  if (!(b > -INFINITY)) continue;  // zero-weight part (or NaN normaliser): no-op
  const float m = fmaxf(a, b);
  const float L = m + log1pf(expf(-fabsf(a - b)));
  const float wa = expf(a - L);
  const float wb = expf(b - L);
  f32x4* po = (f32x4*)(o_acc + pair * D) + part;
  const f32x4 y = *((const f32x4*)(o_i + pair * D) + part);
  f32x4 x = *po;
  x = (a > -INFINITY) ? x * wa + y * wb : y * wb;
  *po = x;
  if (part == 0) lse_acc[pair] = L;
  }
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ o_acc,
                                                       const float* __restrict__ lse_acc,
                                                       void* __restrict__ o, int o_f32,
                                                       float* __restrict__ lse, int64_t pairs,
                                                       int D) {
  const int64_t n4 = pairs * D / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const f32x4 x = ((const f32x4*)o_acc)[i];
    if (o_f32)
      ((f32x4*)o)[i] = x;
    else
      ((bf16x4*)o)[i] = __builtin_convertvector(x, bf16x4);
  }
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pairs; i += stride)
    lse[i] = lse_acc[i];
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ o_acc,
                                                   float* __restrict__ lse_acc, int64_t pairs,
                                                   int D) {
  const int64_t n4 = pairs * D / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
    ((f32x4*)o_acc)[i] = z;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pairs; i += stride)
    lse_acc[i] = -INFINITY;
}

inline int grid_for(int64_t work) {
  const int64_t g = (work + 255) / 256;
  return (int)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_i, const float* lse_i,
                            float log_w, const float* log_w_rows, int64_t pairs, int D,
                            hipStream_t s) {
  const int64_t blocks = (pairs * (D / 4) + 255) / 256;
  const unsigned grid = (unsigned)(blocks < (1 << 20) ? blocks : (1 << 20));
  if (D == 128)
    lse_merge_kernel<128><<<grid, 256, 0, s>>>(o_acc, lse_acc, o_i, lse_i, log_w, log_w_rows, pairs);
  else
    lse_merge_kernel<64><<<grid, 256, 0, s>>>(o_acc, lse_acc, o_i, lse_i, log_w, log_w_rows, pairs);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* o_acc, const float* lse_acc, void* o, int o_f32,
                           float* lse, int64_t pairs, int D, hipStream_t s) {
  finalize_kernel<<<grid_for(pairs * D / 4), 256, 0, s>>>(o_acc, lse_acc, o, o_f32, lse, pairs, D);
  return hipGetLastError();
}

hipError_t launch_fill(float* o_acc, float* lse_acc, int64_t pairs, int D, hipStream_t s) {
  fill_kernel<<<grid_for(pairs * D / 4), 256, 0, s>>>(o_acc, lse_acc, pairs, D);
  return hipGetLastError();
}

}  // namespace h3
