// float32 attention (dense TARA and block-sparse) on the vector ALUs.
//
// Same score rule as the bf16 path ("Flash Partitions for H3 native temporal
// alignment", section 1) with every product, exponential and sum in float32, so
// float32 inputs are never rounded to bf16. One lane owns one query row; keys are
// staged 16 at a time in LDS and read as broadcasts. This path serves float32
// callers and small problems; the matrix-core path serves bf16.
#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int kSub = 16;

template <int D, bool SPARSE, bool PEN>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float ksh[kSub][D];
  __shared__ float vsh[kSub][D];
  __shared__ uint32_t sgs[kSub];
  __shared__ float tss[kSub];
  // sparse: the attended routing blocks (protected, routed, or all for a sink block) of
  // the workgroup's query blocks: one map, or two for 32-row blocks (lanes 0-31, 32-63)
  __shared__ uint32_t tile_bits[SPARSE ? 2 * kBitmapWords : 1];
  __shared__ int sink_map[2];

  const int lane = threadIdx.x;
  const int qblk = blockIdx.x;
  const int h = blockIdx.y;
  const int H = a.H;
  const float* __restrict__ qp = (const float*)a.q;
  const float* __restrict__ kp = (const float*)a.k;
  const float* __restrict__ vp = (const float*)a.v;
  const int qrow = qblk * 64 + lane;
  const bool qvalid = qrow < a.nq;

  float q[D];
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qvalid ? qp[((int64_t)qrow * H + h) * D + d] : 0.f;
    o[d] = 0.f;
  }
  const float qt = qvalid ? a.q_t[qrow] : 0.f;
  const bool q_out = PEN && qvalid && a.q_seg[qrow] == kSegOutput;
  float m = -INFINITY, l = 0.f;

  // key blocks of the routing size (dense: 64-key units)
  const int bs = SPARSE ? a.bs : 64;
  const int nkb = (a.nk + bs - 1) / bs;
  const int words = (nkb + 31) >> 5;
  const int nmaps = (SPARSE && bs == 32) ? 2 : 1;
  const int my_map = nmaps == 2 ? lane >> 5 : 0;
  if constexpr (SPARSE) {
    for (int i = lane; i < 2 * kBitmapWords; i += 64) tile_bits[i] = 0u;
    __syncthreads();
    for (int m = 0; m < nmaps; ++m) {
      const int row0 = qblk * 64 + m * 32;
      if (row0 >= a.nq) continue;
      const int qb = row0 / bs;
      // a sink block attends every key (its rows may extend past this workgroup's)
      const int lo = qb * bs, hi = min(a.nq, lo + bs);
      bool sink_row = false;
      for (int r = lo + lane; r < hi; r += 64) sink_row |= (a.sink_mask >> a.q_seg[r]) & 1u;
      const bool sink = __ballot(sink_row) != 0ull;
      if (lane == 0) sink_map[m] = sink;
      uint32_t* bm = tile_bits + m * kBitmapWords;
      if (sink) {
        for (int i = lane; i < words; i += 64) bm[i] = ~0u;
        continue;
      }
      const int32_t* rt = a.tiles + ((int64_t)h * a.nqb + qb) * a.k_sel;
      for (int i = lane; i < a.n_prot + a.k_sel; i += 64) {
        const int kb = i < a.n_prot ? a.prot[i] : rt[i - a.n_prot];
        if (kb >= 0 && kb < nkb) atomicOr(&bm[kb >> 5], 1u << (kb & 31));
      }
    }
    __syncthreads();
  }

  // key blocks in ascending order (sparse: those some lane attends; a lane masks the
  // blocks its own query block does not attend)
  for (int kb = 0; kb < nkb; ++kb) {
    bool mine = true;
    if constexpr (SPARSE) {
      const uint32_t w = (tile_bits[kb >> 5] | tile_bits[kBitmapWords + (kb >> 5)]) >> (kb & 31);
      if (w == 0u) {  // nothing further in this word
        kb = (kb | 31);
        continue;
      }
      kb += __builtin_ctz(w);
      mine = (tile_bits[my_map * kBitmapWords + (kb >> 5)] >> (kb & 31)) & 1u;
    }
    for (int sub = 0; sub < bs / kSub; ++sub) {
      const int k0 = kb * bs + sub * kSub;
      if (k0 >= a.nk) break;
      __syncthreads();
      for (int e = lane; e < kSub * D; e += 64) {
        const int j = e / D, d = e % D;
        const int key = k0 + j;
        const bool kv = key < a.nk;
        ksh[j][d] = kv ? kp[((int64_t)key * H + h) * D + d] : 0.f;
        vsh[j][d] = kv ? vp[((int64_t)key * H + h) * D + d] : 0.f;
      }
      if (lane < kSub) {
        const int key = k0 + lane;
        const bool kv = key < a.nk;
        sgs[lane] = kv ? (uint32_t)a.k_seg[key] : (uint32_t)kSegInvalid;
        tss[lane] = kv ? a.k_t[key] : 0.f;
      }
      __syncthreads();
      float sc[kSub];
      float smax = -INFINITY;
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(q[d], ksh[j][d], dot);
        float x = dot * a.scale;
        const uint32_t sg = sgs[j];
        if (sg == (uint32_t)kSegInvalid || !mine) {
          x = -INFINITY;
        } else if (PEN && q_out && sg == (uint32_t)kSegGuide) {
          const float dt = fabsf(qt - tss[j]);
          const float u = fmaxf(dt - a.window, 0.f) * a.inv_falloff;
          x -= fminf(a.strength * (u * u), a.cap);
        }
        sc[j] = x;
        smax = fmaxf(smax, x);
      }
      if (smax > m) {
        const float alpha = expf(m - smax);  // m = -inf gives 0
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        l *= alpha;
        m = smax;
      }
      if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
          const float p = expf(sc[j] - m);
          l += p;
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] = fmaf(p, vsh[j][d], o[d]);
        }
      }
    }
  }
  if (!qvalid) return;
  // optional tail key of the query block: one more softmax term with logit tail_lse
  // and value tail_v
  float tail_w = 0.f;
  const float* tail_v = nullptr;
  if (SPARSE && a.tail_lse && !sink_map[my_map]) {
    const int64_t tb = (int64_t)h * a.nqb + qrow / bs;
    const float lt = a.tail_lse[tb];
    if (lt != -INFINITY) {
      const float m_new = fmaxf(m, lt);
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
      tail_w = expf(lt - m_new);
      l = l * alpha + tail_w;
      m = m_new;
      tail_v = a.tail_v + tb * D;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t ob = ((int64_t)qrow * H + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float val = (tail_v ? o[d] + tail_w * tail_v[d] : o[d]) * inv;
    if (a.o_f32)
      ((float*)a.o)[ob + d] = val;
    else
      ((__bf16*)a.o)[ob + d] = (__bf16)val;
  }
  a.lse[(int64_t)qrow * H + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D, bool SPARSE, bool PEN>
hipError_t launch_f32_variant(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.nq + 63) / 64, a.H);
  attn_f32_kernel<D, SPARSE, PEN><<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int D, bool sparse, bool penalty, hipStream_t s) {
  if (D == 128) {
    if (sparse) return penalty ? launch_f32_variant<128, true, true>(a, s) : launch_f32_variant<128, true, false>(a, s);
    return penalty ? launch_f32_variant<128, false, true>(a, s) : launch_f32_variant<128, false, false>(a, s);
  }
  if (sparse) return penalty ? launch_f32_variant<64, true, true>(a, s) : launch_f32_variant<64, true, false>(a, s);
  return penalty ? launch_f32_variant<64, false, true>(a, s) : launch_f32_variant<64, false, false>(a, s);
}

}  // namespace h3
