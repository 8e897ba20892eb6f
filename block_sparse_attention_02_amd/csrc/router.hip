// Pooled block router for block-sparse attention.
//
// "H3 SLA Attention", "How it works": a single product of the block-mean queries with
// the block-mean keys rates each (query block, key block) pair, and a query block keeps
// the highest-rated (1 - sparsity) share of the key blocks; inputs table: blocks
// overlapping language or audio rows are always attended.
// "H3 sparse-attention breakpoints": the density is a fraction of the video KV tiles.
//
// Three kernels, all deterministic (no floating-point atomics):
//   1. flags   : protected / video classification of the blocks (32, 64 or 128 rows,
//                the same size for queries and keys) and their ascending lists (one
//                workgroup, ballot-based compaction);
//   2. pool    : per-block means of q and k, float32 sums in row order, one pass over
//                q and k in HBM (memory bound);
//   3. score+top-k: per head and group of query blocks, pooled scores against every
//                video tile in LDS (float32 products added in order of d, no fused
//                multiply-add), then an exact radix select of the k best per query block
//                with ties to the lower tile index, emitted in ascending tile order.
// With the tail term ("H3 SLA Attention", inputs table, tail_correction) the pool pass
// also takes the mean of V, and the top-k kernel folds the unrouted video tiles of each
// query block into one pooled key: logit ln sum_u n_u exp(scale * S[qb,u]) from the same
// float32 pooled scores, and normalised weights whose product with the V means (float32
// on the matrix cores) gives the key's value.
#include <atomic>

#include "h3_internal.h"

#pragma clang fp contract(off)

namespace h3 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTopkWaves = 4;

// ------------------------------------------------------------------ 1. flags
__global__ __launch_bounds__(1024) void router_flags_kernel(const uint8_t* __restrict__ seg,
                                                            int n, int prefix, int nb,
                                                            int bs, bool guide_protected,
                                                            int32_t* __restrict__ prot,
                                                            int prot_cap,
                                                            int32_t* __restrict__ video,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wsum_p[16], wsum_v[16];
  __shared__ int base_p, base_v;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  if (tid == 0) { base_p = 0; base_v = 0; }
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int start = 0; start < nb; start += 1024) {
    const int b = start + tid;
    const bool valid = b < nb;
    bool isp = false;
    if (valid) {
      const int lo = b * bs;
      const int hi = min(n, lo + bs);
      isp = lo < prefix;
      for (int r = lo; r < hi && !isp; ++r) {
        const int s = seg[r];
        isp = (s == kSegText) || (s == kSegAudio) || (guide_protected && s == kSegGuide);
      }
    }
    const bool isv = valid && !isp;
    isp = valid && isp;
    const uint64_t mp = __ballot(isp);
    const uint64_t mv = __ballot(isv);
    if (lane == 0) { wsum_p[w] = __popcll(mp); wsum_v[w] = __popcll(mv); }
    __syncthreads();
    int offp = base_p, offv = base_v;
    for (int j = 0; j < w; ++j) { offp += wsum_p[j]; offv += wsum_v[j]; }
    const int ip = offp + __popcll(mp & below);
    const int iv = offv + __popcll(mv & below);
    if (isp && ip < prot_cap) prot[ip] = b;
    if (isv) video[iv] = b;
    __syncthreads();
    if (tid == 0) {
      int tp = 0, tv = 0;
      for (int j = 0; j < 16; ++j) { tp += wsum_p[j]; tv += wsum_v[j]; }
      base_p += tp;
      base_v += tv;
    }
    __syncthreads();
  }
  if (tid == 0) { counts[0] = base_p; counts[1] = base_v; }
}

// ------------------------------------------------------------------ 2. pool
// Workgroup = kPoolBlocks waves, one per consecutive block of bs rows, over the same 512
// (head, d) elements (8 per lane). Each wave adds its block's rows in row order; the
// query (and value) means go straight to memory, row-major. The key means pass through
// LDS so that the workgroup writes them d-major as aligned runs of kPoolBlocks floats
// per (head, d): every store fills whole 64-byte lines (the d-major row stride is nb
// rounded up to kPoolBlocks).
constexpr int kPoolBlocks = 16;
constexpr int kPoolCols = 512;   // (head, d) elements per workgroup
constexpr int kPoolElems = 8;    // per lane

template <bool BF16, int D, bool TAIL>
__global__ __launch_bounds__(64 * kPoolBlocks) void router_pool_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, int n,
    int H, int nb, int nbk, int bs, float* __restrict__ qbar, float* __restrict__ kbar,
    float* __restrict__ vbar) {
  __shared__ float kt[kPoolBlocks][kPoolCols + 4];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b0 = blockIdx.x * kPoolBlocks;
  const int b = b0 + w;
  const int col0 = blockIdx.y * kPoolCols;
  const int e0 = col0 + lane * kPoolElems;
  const bool live = b < nb && e0 < H * D;
  float ak[kPoolElems];
#pragma unroll
  for (int i = 0; i < kPoolElems; ++i) ak[i] = 0.f;
  if (live) {
    const int h = e0 / D, d0 = e0 % D;
    const int lo = b * bs, hi = min(n, lo + bs);
    const int64_t rs = (int64_t)H * D;
    float aq[kPoolElems], av[kPoolElems];
#pragma unroll
    for (int i = 0; i < kPoolElems; ++i) { aq[i] = 0.f; av[i] = 0.f; }
#pragma unroll 8
    for (int r = lo; r < hi; ++r) {
      const int64_t off = (int64_t)r * rs + e0;
      float xq[8], xk[8], xv[8];
      if (BF16) {
        const u32x4 uq = *(const u32x4*)((const uint16_t*)q + off);
        const u32x4 uk = *(const u32x4*)((const uint16_t*)k + off);
        u32x4 uv = {0u, 0u, 0u, 0u};
        if (TAIL) uv = *(const u32x4*)((const uint16_t*)v + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xq[2 * i] = __uint_as_float(uq[i] << 16);
          xq[2 * i + 1] = __uint_as_float(uq[i] & 0xFFFF0000u);
          xk[2 * i] = __uint_as_float(uk[i] << 16);
          xk[2 * i + 1] = __uint_as_float(uk[i] & 0xFFFF0000u);
          xv[2 * i] = __uint_as_float(uv[i] << 16);
          xv[2 * i + 1] = __uint_as_float(uv[i] & 0xFFFF0000u);
        }
      } else {
        const f32x4* pq = (const f32x4*)((const float*)q + off);
        const f32x4* pk = (const f32x4*)((const float*)k + off);
        const f32x4 q0 = pq[0], q1 = pq[1], k0 = pk[0], k1 = pk[1];
        f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (TAIL) {
          const f32x4* pv = (const f32x4*)((const float*)v + off);
          v0 = pv[0];
          v1 = pv[1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xq[i] = q0[i]; xq[4 + i] = q1[i];
          xk[i] = k0[i]; xk[4 + i] = k1[i];
          xv[i] = v0[i]; xv[4 + i] = v1[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        aq[i] = __fadd_rn(aq[i], xq[i]);
        ak[i] = __fadd_rn(ak[i], xk[i]);
        if (TAIL) av[i] = __fadd_rn(av[i], xv[i]);
      }
    }
    const float cnt = (float)(hi - lo);
    f32x4 m0, m1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m0[i] = __fdiv_rn(aq[i], cnt);
      m1[i] = __fdiv_rn(aq[4 + i], cnt);
    }
    float* oq = qbar + ((int64_t)h * nb + b) * D + d0;   // [H][nb][D]
    *(f32x4*)oq = m0;
    *(f32x4*)(oq + 4) = m1;
    if (TAIL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m0[i] = __fdiv_rn(av[i], cnt);
        m1[i] = __fdiv_rn(av[4 + i], cnt);
      }
      float* ov = vbar + ((int64_t)h * nb + b) * D + d0;  // [H][nb][D]
      *(f32x4*)ov = m0;
      *(f32x4*)(ov + 4) = m1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ak[i] = __fdiv_rn(ak[i], cnt);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) kt[w][lane * kPoolElems + i] = ak[i];  // zero past the end
  __syncthreads();
  // [H][D][nbk]: thread t stores blocks 4p..4p+3 (p = t % 4) of column t / 4, so four
  // neighbouring threads fill one 64-byte run
  for (int idx = threadIdx.x; idx < kPoolCols * 4; idx += 64 * kPoolBlocks) {
    const int c = idx >> 2, p4 = (idx & 3) * 4;
    const int e = col0 + c;
    if (e >= H * D) continue;
    const int h = e / D, d = e % D;
    *(f32x4*)(kbar + ((int64_t)h * D + d) * nbk + b0 + p4) =
        f32x4{kt[p4][c], kt[p4 + 1][c], kt[p4 + 2][c], kt[p4 + 3][c]};
  }
}

// ------------------------------------------------------------------ 3. score + top-k
// float32 product rounded on its own: the empty asm makes the value opaque, so the
// following addition can never be contracted into a fused multiply-add (the file is
// also compiled with -ffp-contract=off).
__device__ __forceinline__ float mul_rounded(float a, float b) {
  float p = a * b;
  __asm__("" : "+v"(p));
  return p;
}

// Order-preserving map of a float32 score to an unsigned key: larger key = better;
// -0 and +0 map together; NaN maps below every number.
__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D, int QB, bool TAIL, bool REF = false>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar,
                                                          const int32_t* __restrict__ video,
                                                          const int32_t* __restrict__ counts,
                                                          int nb, int nbk, int k_sel,
                                                          int32_t* __restrict__ tiles,
                                                          TailArgs tail, RefQuota rq) {
  static_assert(QB == 1 || QB == 4, "query blocks per workgroup");
  static_assert(!(TAIL && REF), "the tail term is not combined with the reference quota");
  extern __shared__ float sc[];  // [QB][nv] pooled scores
  __shared__ int hist[kTopkWaves][256];
  // reference quota: the union of the selections of each query block, one bit per block
  __shared__ uint32_t chosen[REF ? QB : 1][REF ? kBitmapWords : 1];
  const int h = blockIdx.y;
  const int qb0 = blockIdx.x * QB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nv = counts[1];

  // The QB query means sit at workgroup-uniform addresses, so they arrive by scalar
  // loads into SGPRs and the score loop reads nothing from LDS. A query block past the
  // end reads the last block's means; its scores are never used.
  const float* qrow[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) qrow[j] = qbar + ((int64_t)h * nb + min(qb0 + j, nb - 1)) * D;
  // Lanes take consecutive video tiles, so each d reads one coalesced run of the
  // d-major kbar (row stride nbk).
  const float* kh = kbar + (int64_t)h * D * nbk;
  for (int vi = tid; vi < nv; vi += 256) {
    const int kb = video[vi];
    float acc[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) acc[j] = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const float kv = kh[(int64_t)d * nbk + kb];
#pragma unroll
      for (int j = 0; j < QB; ++j) acc[j] = acc[j] + mul_rounded(qrow[j][d], kv);
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) sc[j * nv + vi] = acc[j];
  }
  __syncthreads();

  const bool active = w < QB;
  const float* my = sc + (active ? w : 0) * nv;
  if constexpr (REF) {
    // Light reference protection: the ordinary top-k over every video tile, then each
    // reference range's quota of its best tiles (a contiguous run [lo, hi) of the
    // video list), all marked in one bitmap per query block; the union is written in
    // ascending block order and padded with -1 up to the list width k_sel.
    for (int i = tid; i < QB * kBitmapWords; i += 256) (&chosen[0][0])[i] = 0u;
    __syncthreads();
    const int nparts = 1 + rq.n;
    for (int part = 0; part < nparts; ++part) {
      const int lo = part ? min(rq.lo[part - 1], nv) : 0;
      const int hi = part ? min(rq.hi[part - 1], nv) : nv;
      const int cnt = hi - lo;
      const int kk = min(part ? rq.q[part - 1] : rq.k_ord, cnt);
      if (kk <= 0) continue;  // workgroup-uniform
      const bool all = kk == cnt;
      uint32_t prefix = 0u, pmask = 0u;
      int rem = kk;
      for (int pass = 0; pass < 4 && !all; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int j = lane; j < 256; j += 64) hist[w][j] = 0;
        __syncthreads();
        if (active) {
          for (int i = lo + lane; i < hi; i += 64) {
            const uint32_t key = order_key(my[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1);
          }
        }
        __syncthreads();
        if (active) {
          int c[4];
          int sum = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) { c[j] = hist[w][255 - 4 * lane - j]; sum += c[j]; }
          int incl = sum;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
          }
          const int excl = incl - sum;
          const bool here = excl < rem && rem <= incl;
          int digit = 0, above = 0;
          if (here) {
            int cum = excl;
            for (int j = 0; j < 4; ++j) {
              if (cum + c[j] >= rem) { digit = 255 - 4 * lane - j; above = cum; break; }
              cum += c[j];
            }
          }
          const uint64_t bm = __ballot(here);
          const int src = __ffsll((unsigned long long)bm) - 1;
          digit = __shfl(digit, src);
          above = __shfl(above, src);
          rem -= above;
          prefix |= (uint32_t)digit << shift;
          pmask |= 0xFFu << shift;
        }
        __syncthreads();
      }
      if (active) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int eq_seen = 0;
        for (int base = lo; base < hi; base += 64) {
          const int i = base + lane;
          const bool valid = i < hi;
          const uint32_t key = valid ? order_key(my[i]) : 0u;
          const bool gt = valid && (all || key > prefix);
          const bool eq = valid && !all && key == prefix;
          const uint64_t eqm = __ballot(eq);
          const bool sel = gt || (eq && eq_seen + __popcll(eqm & below) < rem);
          if (sel) {
            const int kb = video[i];
            atomicOr(&chosen[w][kb >> 5], 1u << (kb & 31));
          }
          eq_seen += __popcll(eqm);
        }
      }
    }
    __syncthreads();
    const int qb = qb0 + w;
    if (active && qb < nb && k_sel > 0) {
      int32_t* out = tiles + ((int64_t)h * nb + qb) * k_sel;
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int pos = 0;
      for (int base = 0; base < nb; base += 64) {
        const int kb = base + lane;
        const bool sel = kb < nb && ((chosen[w][kb >> 5] >> (kb & 31)) & 1u);
        const uint64_t selm = __ballot(sel);
        const int at = pos + __popcll(selm & below);
        if (sel && at < k_sel) out[at] = kb;
        pos += __popcll(selm);
      }
      for (int j = pos + lane; j < k_sel; j += 64) out[j] = -1;
    }
    return;
  }

  // ---- exact selection: radix select of the k-th best key, 8 bits per pass
  const int kk = min(k_sel, nv);
  const bool take_all = (kk == nv);
  uint32_t prefix = 0u, pmask = 0u;
  int rem = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = lane; j < 256; j += 64) hist[w][j] = 0;
    __syncthreads();
    if (active && !take_all && kk > 0) {
      for (int i = lane; i < nv; i += 64) {
        const uint32_t key = order_key(my[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (active && !take_all && kk > 0) {
      int c[4];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = hist[w][255 - 4 * lane - j]; sum += c[j]; }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const int excl = incl - sum;
      const bool here = excl < rem && rem <= incl;
      int digit = 0, above = 0;
      if (here) {
        int cum = excl;
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= rem) { digit = 255 - 4 * lane - j; above = cum; break; }
          cum += c[j];
        }
      }
      const uint64_t bm = __ballot(here);
      const int src = __ffsll((unsigned long long)bm) - 1;
      digit = __shfl(digit, src);
      above = __shfl(above, src);
      rem -= above;
      prefix |= (uint32_t)digit << shift;
      pmask |= 0xFFu << shift;
    }
    __syncthreads();
  }

  const int qb = qb0 + w;
  if (active && qb < nb && k_sel > 0) {
  int32_t* out = tiles + ((int64_t)h * nb + qb) * k_sel;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int pos = 0, eq_seen = 0;
  for (int base = 0; base < nv; base += 64) {
    const int i = base + lane;
    const bool valid = i < nv;
    const uint32_t key = valid ? order_key(my[i]) : 0u;
    bool gt, eq;
    if (take_all) {
      gt = valid;
      eq = false;
    } else {
      gt = valid && kk > 0 && key > prefix;
      eq = valid && kk > 0 && key == prefix;
    }
    const uint64_t eqm = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqm & below);
    const bool sel = gt || (eq && eq_rank < rem);
    const uint64_t selm = __ballot(sel);
    if (sel) {
      out[pos + __popcll(selm & below)] = video[i];
      if (TAIL) sc[w * nv + i] = -INFINITY;  // routed: not part of the tail
    }
    pos += __popcll(selm);
    eq_seen += __popcll(eqm);
  }
  for (int j = kk + lane; j < k_sel; j += 64) out[j] = -1;
  }
  if (!TAIL) return;

  // ---- tail term of each query block from the unrouted video tiles: weights in place
  // of the scores, logit to tail.lse, then the normalised weights to tail.wts
  __shared__ float tsum[QB];
  if (active) {
    float* my_w = sc + w * nv;
    float mx = -INFINITY;
    for (int i = lane; i < nv; i += 64) {
      const float s = my_w[i];
      if (s != -INFINITY) {
        const int kb = video[i];
        const float x = s * tail.scale + __logf((float)min(tail.bs, tail.n - kb * tail.bs));
        my_w[i] = x;
        mx = fmaxf(mx, x);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.f;
    for (int i = lane; i < nv; i += 64) {
      const float x = my_w[i];
      const float e = (x == -INFINITY) ? 0.f : __expf(x - mx);
      my_w[i] = e;
      sum += e;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) {
      tsum[w] = sum;
      if (qb < nb) tail.lse[(int64_t)h * nb + qb] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
    }
  }
  __syncthreads();
  // normalised weights as float32 rows [qb][nbp] (zero for routed tiles and past nv);
  // the weighted V means are one matrix product per head (tail_v_kernel)
  if (active && qb < nb) {
    const float* my_w = sc + w * nv;
    const float sm = tsum[w];
    const float inv = sm > 0.f ? 1.f / sm : 0.f;
    float* row = tail.wts + ((int64_t)h * nb + qb) * tail.nbp;
    for (int i = lane; i < tail.nbp; i += 64) row[i] = i < nv ? my_w[i] * inv : 0.f;
  }
}

// V means of the video tiles, transposed: vbt[h][d][i] = vbar[h][video[i]][d] for
// i < n_video, zero up to nbp.
template <int D>
__global__ __launch_bounds__(256) void tail_vbar_kernel(const float* __restrict__ vbar,
                                                        const int32_t* __restrict__ video,
                                                        const int32_t* __restrict__ counts,
                                                        int nb, int nbp,
                                                        float* __restrict__ vbt) {
  const int h = blockIdx.y;
  const int i = blockIdx.x * 64 + (threadIdx.x & 63);
  const int nv = counts[1];
  const bool live = i < nv;
  const int kb = live ? video[i] : 0;
  for (int d = threadIdx.x >> 6; d < D; d += 4) {
    const float x = live ? vbar[((int64_t)h * nb + kb) * D + d] : 0.f;
    if (i < nbp) vbt[((int64_t)h * D + d) * nbp + i] = x;
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// tail_v[h][qb][:] = sum_i wts[h][qb][i] * vbt[h][:][i]: a [nb x nv] x [nv x D] product per
// head on the matrix cores in float32 (v_mfma_f32_32x32x2_f32). Workgroup = 32 query
// blocks of one head; wave w takes the 32 output columns 32w..32w+31. The k index of a
// product step is a lane's own: lane half hh holds tiles k0 + 4hh + j for the four steps
// j of a group of eight tiles, so that every lane reads its operands as float4.
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void tail_v_kernel(const float* __restrict__ wts,
                                                               const float* __restrict__ vbt,
                                                               const int32_t* __restrict__ counts,
                                                               int nb, int nbp,
                                                               float* __restrict__ tail_v) {
  const int h = blockIdx.y;
  const int qb0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  // video tiles in steps of 32: nbp is a multiple of 32 and both operands are zero past
  // the video count, so the extra products are 0 x 0; four steps of loads are in flight
  const int kend = (counts[1] + 31) & ~31;
  const bool row_ok = qb0 + l32 < nb;
  const float* arow = wts + ((int64_t)h * nb + (row_ok ? qb0 + l32 : 0)) * nbp + 4 * hh;
  const float* brow = vbt + ((int64_t)h * D + 32 * w + l32) * nbp + 4 * hh;
  f32x16 acc = {};
  for (int k0 = 0; k0 < kend; k0 += 32) {
    f32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = *(const f32x4*)(arow + k0 + 8 * u);
      b[u] = *(const f32x4*)(brow + k0 + 8 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!row_ok) a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][j], b[u][j], acc, 0, 0, 0);
    }
  }
  // lane holds column 32w + l32 and rows 8(r/4) + 4hh + r%4
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qb = qb0 + 8 * (r >> 2) + 4 * hh + (r & 3);
    if (qb < nb) tail_v[((int64_t)h * nb + qb) * D + 32 * w + l32] = acc[r];
  }
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Row stride of the d-major key means: the block count rounded up to whole pool groups.
inline size_t kbar_stride(size_t nb) { return (nb + kPoolBlocks - 1) / kPoolBlocks * kPoolBlocks; }

size_t router_ws_bytes(int n, int H, int D, int bs, bool tail) {
  const size_t nb = (size_t)((n + bs - 1) / bs);
  const size_t nbp = (nb + 31) / 32 * 32;
  const size_t means = align256(nb * H * D * sizeof(float));
  const size_t kmeans = align256(kbar_stride(nb) * H * D * sizeof(float));
  size_t b = means + kmeans + align256(nb * sizeof(int32_t)) + 256;
  if (tail)
    b += means + align256((size_t)H * nb * nbp * 4) + align256((size_t)H * D * nbp * 4);
  return b;
}

RouterWs router_ws_carve(void* ws, int n, int H, int D, int bs, bool tail) {
  const size_t nb = (size_t)((n + bs - 1) / bs);
  const size_t means = align256(nb * H * D * sizeof(float));
  char* p = (char*)ws;
  RouterWs w;
  w.qbar = (float*)p;
  p += means;
  w.kbar = (float*)p;
  w.nbk = (int)kbar_stride(nb);
  p += align256((size_t)w.nbk * H * D * sizeof(float));
  w.video = (int32_t*)p;
  p += align256(nb * sizeof(int32_t));
  w.counts = (int32_t*)p;
  p += 256;
  w.vbar = nullptr;
  w.wts = nullptr;
  w.vbt = nullptr;
  w.nbp = (int)((nb + 31) / 32 * 32);
  if (tail) {
    w.vbar = (float*)p;
    p += means;
    w.wts = (float*)p;
    p += align256((size_t)H * nb * w.nbp * 4);
    w.vbt = (float*)p;
  }
  return w;
}

// Largest block count the score/top-k kernel keeps in LDS (QB x nb floats).
int router_max_blocks() { return kMaxBlocks; }

// The device's LDS limit per workgroup, queried once per device (64 KB if the query
// fails). The cache only ever holds that attribute, so concurrent first calls store the
// same value.
int max_lds_per_block() {
  constexpr int kDevices = 64;
  static std::atomic<int> cached[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 64 * 1024;
  if (dev < kDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      v <= 0)
    v = 64 * 1024;
  if (dev < kDevices) cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int D, int QB, bool TAIL, bool REF>
void launch_topk(dim3 grid, size_t lds, hipStream_t s, const RouterWs& w, int nb, int k_sel,
                 int32_t* tiles, const TailArgs& ta, const RefQuota& rq) {
  router_topk_kernel<D, QB, TAIL, REF><<<grid, 256, lds, s>>>(w.qbar, w.kbar, w.video, w.counts,
                                                              nb, w.nbk, k_sel, tiles, ta, rq);
}

template <int D, bool TAIL>
void launch_pool_topk(const void* q, const void* k, const void* v, bool bf16, int n, int H,
                      int nb, int bs, int k_sel, int32_t* tiles, const RouterWs& w,
                      const TailArgs& ta, const RefQuota* rq, hipStream_t s) {
  const int chunks = (H * D + kPoolCols - 1) / kPoolCols;
  dim3 pgrid((nb + kPoolBlocks - 1) / kPoolBlocks, chunks);
  if (bf16)
    router_pool_kernel<true, D, TAIL><<<pgrid, 64 * kPoolBlocks, 0, s>>>(
        q, k, v, n, H, nb, w.nbk, bs, w.qbar, w.kbar, w.vbar);
  else
    router_pool_kernel<false, D, TAIL><<<pgrid, 64 * kPoolBlocks, 0, s>>>(
        q, k, v, n, H, nb, w.nbk, bs, w.qbar, w.kbar, w.vbar);
  // four query blocks per workgroup when their scores fit in the LDS next to the
  // kernel's own arrays (about 12 KB, and 4 bitmaps of the reference quota)
  const size_t own = 12 * 1024 + (rq ? (size_t)4 * kBitmapWords * 4 : 0);
  const bool wide = (size_t)4 * nb * sizeof(float) + own <= (size_t)max_lds_per_block();
  const int qb = wide ? 4 : 1;
  dim3 tgrid((nb + qb - 1) / qb, H);
  const size_t lds = (size_t)qb * nb * sizeof(float);
  if (TAIL) tail_vbar_kernel<D><<<dim3(w.nbp / 64 + 1, H), 256, 0, s>>>(w.vbar, w.video, w.counts,
                                                                    nb, w.nbp, w.vbt);
  const RefQuota none{};
  if constexpr (!TAIL) {
    if (rq) {
      if (wide)
        launch_topk<D, 4, false, true>(tgrid, lds, s, w, nb, k_sel, tiles, ta, *rq);
      else
        launch_topk<D, 1, false, true>(tgrid, lds, s, w, nb, k_sel, tiles, ta, *rq);
      return;
    }
  }
  if (wide)
    launch_topk<D, 4, TAIL, false>(tgrid, lds, s, w, nb, k_sel, tiles, ta, none);
  else
    launch_topk<D, 1, TAIL, false>(tgrid, lds, s, w, nb, k_sel, tiles, ta, none);
  if (TAIL)
    tail_v_kernel<D><<<dim3((nb + 31) / 32, H), 64 * (D / 32), 0, s>>>(w.wts, w.vbt, w.counts, nb,
                                                                      w.nbp, ta.v);
}

hipError_t launch_router(const void* q, const void* k, const void* v, bool bf16, int n, int H,
                         int D, int bs, const uint8_t* seg, int prefix, int k_sel,
                         int32_t* tiles, int32_t* prot, int prot_cap, const RouterWs& w,
                         float scale, float* tail_lse, float* tail_v, hipStream_t s,
                         bool guide_protected, const RefQuota* rq) {
  const int nb = (n + bs - 1) / bs;
  router_flags_kernel<<<1, 1024, 0, s>>>(seg, n, prefix, nb, bs, guide_protected, prot,
                                         prot_cap, w.video, w.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool tail = tail_lse != nullptr;
  if (tail && rq) return hipErrorInvalidValue;
  const TailArgs ta{scale, n, bs, w.vbar, tail_lse, tail_v, w.wts, w.nbp};
  if (D == 128) {
    if (tail) launch_pool_topk<128, true>(q, k, v, bf16, n, H, nb, bs, k_sel, tiles, w, ta, rq, s);
    else launch_pool_topk<128, false>(q, k, v, bf16, n, H, nb, bs, k_sel, tiles, w, ta, rq, s);
  } else {
    if (tail) launch_pool_topk<64, true>(q, k, v, bf16, n, H, nb, bs, k_sel, tiles, w, ta, rq, s);
    else launch_pool_topk<64, false>(q, k, v, bf16, n, H, nb, bs, k_sel, tiles, w, ta, rq, s);
  }
  return hipGetLastError();
}

}  // namespace h3
