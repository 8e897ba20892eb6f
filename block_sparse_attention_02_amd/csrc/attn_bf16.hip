// bf16 attention for gfx950: dense TARA and block-sparse over 64-key tiles.
//
// Score rule ("Flash Partitions for H3 native temporal alignment", section 1):
//   s_ij = scale * q_i.k_j - p_ij, p_ij = min(strength*(max(|t_i-t_j|-window,0)/falloff)^2, cap)
//   only for (output-video query, guide-video key) pairs.
// The penalty is computed in registers per 64-key tile. A tile whose 64 keys are all
// guide rows of one frame gets a per-query scalar penalty (all spatial tokens of a
// frame share the same temporal correction, section 3); mixed and ragged tiles take a
// per-element path. No rows x rows bias is ever formed.
//
// Work decomposition: 8 waves of 64 lanes (two per SIMD), 256 query rows per
// workgroup; wave w owns rows 32w..32w+31 and all 64 keys of each tile, so each K/V
// tile load serves up to 256 queries.
//   dense : every key tile, in order;
//   sparse: the workgroup's rows are four 64-row query blocks. Their attended tiles
//           (the protected tiles plus each block's routed tiles) are collected as bitmaps
//           in LDS, and the workgroup walks the union in ascending tile order: every tile
//           is loaded once for all four blocks and each wave computes only the tiles its
//           own block attends. Routed lists of neighbouring blocks overlap heavily when
//           the blocks share a video frame, so most loads serve the whole workgroup.
// Matrix cores: S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, so each
// lane holds one query column; softmax row reductions stay in registers plus one
// exchange between lane halves.
// K and V^T tiles are double-buffered in LDS with an XOR swizzle on 16-byte chunks
// (bank-conflict-free operand reads) and loaded one tile ahead straight from global
// memory into LDS (global_load_lds_dwordx4), so the loads hold no registers.
// V^T comes from a transposed copy of v whose keys are permuted within 16-key groups
// (bits 2 and 3 of the key index swapped) so that the probability registers produced by
// the first product are directly the B operand of the second.
#include <type_traits>

#include "h3_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima are only raised when a tile exceeds them by more than this (log2
// units); probabilities then stay below 2^8 and most tiles skip the O rescale.
constexpr float kLazyRescale = 8.0f;
// Buffer descriptor word 3 for raw 32-bit-format loads on CDNA (out-of-range reads
// return zero).
constexpr int kBufferFlags = 0x00020000;

// Position of key `key` inside its 16-key group of the transposed v copy.
__host__ __device__ constexpr int key_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Lanes l and l^32 hold the two key halves of the same query column.
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

// One 16-byte chunk per lane from a raw buffer [base, base + nbytes) straight into LDS
// at lds + 16 * lane (the LDS address is wave-uniform); out-of-range lanes read zero.
__device__ __forceinline__ void buffer_to_lds16(const void* base, int nbytes, void* lds,
                                                uint32_t voffset) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}

__device__ __forceinline__ float tara_pen(float dt, float window, float inv_falloff,
                                          float strength, float cap) {
  float x = fmaxf(dt - window, 0.f) * inv_falloff;
  return fminf(strength * (x * x), cap);
}

// ------------------------------------------------------------------ v transpose
// vt[h][d][pos] = v[key][h][d] with pos = key_pos(key) inside each 16-key group;
// keys past nk are zero so padded tiles contribute nothing.
template <int D>
__global__ __launch_bounds__(256) void vt_transpose_kernel(const uint16_t* __restrict__ v,
                                                           uint16_t* __restrict__ vt, int nk,
                                                           int nkp, int H) {
  constexpr int LD = D + 2;  // padded row so the column reads spread over banks
  constexpr int CPR = D / 8;
  __shared__ uint16_t tile[64 * LD];
  const int k0 = blockIdx.x * 64;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  for (int c = tid; c < 64 * CPR; c += 256) {
    const int r = c / CPR, ch = c % CPR;
    const int key = k0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < nk) val = *(const u32x4*)(v + ((int64_t)key * H + h) * D + ch * 8);
    uint32_t* dst = (uint32_t*)(tile + r * LD + ch * 8);
    dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
  }
  __syncthreads();
  for (int c = tid; c < D * 8; c += 256) {
    const int d = c / 8, pc = c % 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = tile[key_pos(pc * 8 + 2 * j) * LD + d];
      const uint32_t hi = tile[key_pos(pc * 8 + 2 * j + 1) * LD + d];
      w[j] = lo | (hi << 16);
    }
    u32x4 out = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(vt + ((int64_t)h * D + d) * nkp + k0 + pc * 8) = out;
  }
}

// ------------------------------------------------------------------ tile info
// Per 64-key tile: bit0 any guide key, bit1 every key a guide row of one frame,
// bit2 all 64 keys present; .t = time of the tile's first key.
__global__ __launch_bounds__(64) void tile_info_kernel(const uint8_t* __restrict__ k_seg,
                                                       const float* __restrict__ k_t, int nk,
                                                       TileInfo* __restrict__ info) {
  const int kb = blockIdx.x;
  const int key = kb * 64 + threadIdx.x;
  const bool valid = key < nk;
  const uint32_t sg = valid ? (uint32_t)k_seg[key] : (uint32_t)kSegInvalid;
  const float tt = valid ? k_t[key] : 0.f;
  const uint64_t g = __ballot(sg == (uint32_t)kSegGuide);
  const uint64_t full = __ballot(valid);
  const float t0 = __shfl(tt, 0);
  const uint64_t same = __ballot(tt == t0);
  if (threadIdx.x == 0) {
    int f = 0;
    if (g) f |= kTileAnyGuide;
    if (g == ~0ull && same == ~0ull) f |= kTileUniformGuide;
    if (full == ~0ull) f |= kTileFull;
    info[kb] = TileInfo{f, t0};
  }
}

// ------------------------------------------------------------------ attention
// LDS layouts (bf16, 16-byte chunks, XOR-swizzled so that every 8- and 16-lane phase
// of a 128-bit operand read touches distinct banks):
//   K   : row = key (D*2 bytes); chunk c of key r sits at chunk c ^ (r & 15) (D = 128)
//         or c ^ (r & 7) (D = 64).
//   V^T : rows d and d+1 share a 256-byte line p = d/2; chunk c of row d sits at
//         (8*(d&1) + c) ^ ((p & 15) ^ 4*(d&1)).
template <int D>
__device__ __forceinline__ int k_lds_chunk(int r, int c) {
  return D == 128 ? (c ^ (r & 15)) : (c ^ (r & 7));
}
__device__ __forceinline__ int vt_lds_byte(int d, int c) {
  const int p = d >> 1, b = d & 1;
  return p * 256 + (((8 * b + c) ^ ((p & 15) ^ (4 * b))) * 16);
}

template <int D, bool SPARSE, bool PEN>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NW = 8;               // waves per workgroup (two per SIMD)
  constexpr int BM = 32 * NW;         // query rows per workgroup
  constexpr int QB = BM / kTile;      // query blocks per workgroup (sparse)
  constexpr int KW = 64;              // keys of a tile handled by one wave
  constexpr int NT = KW / 32;         // 32x32 score tiles per wave
  constexpr int NS = KW / 16;         // k-steps of the PV product
  constexpr int DK = D / 16;          // k-steps of the QK product
  constexpr int DT = D / 32;          // 32-row output tiles (over d)
  constexpr int TILE_ELEMS = 64 * D;  // bf16 elements of one K (or V^T) tile
  constexpr int DMA_PER_WAVE = TILE_ELEMS * 2 / 1024 / NW;  // 1 KB wave loads per wave
  constexpr int KROW_BYTES = D * 2;

  // Two stages, each its own LDS object so the compiler can tell the stage being
  // read from the stage being filled by the direct-to-LDS loads.
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t ks1[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t vs1[TILE_ELEMS];
  __shared__ uint8_t kseg0[64], kseg1[64];
  __shared__ float kt0[64], kt1[64];
  // sparse: bitmap 0 = protected tiles, bitmap 1 + j = routed tiles of query block j
  __shared__ uint32_t tile_bits[SPARSE ? (QB + 1) * kBitmapWords : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = wave;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int qblk = blockIdx.x;
  const int h = blockIdx.y;
  const int H = a.H;
  const uint16_t* __restrict__ qp = (const uint16_t*)a.q;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k;
  const uint16_t* __restrict__ vtp = a.vt;
  const TileInfo* __restrict__ tinfo = a.tinfo;
  const float c_log2 = a.scale * kLog2e;

  const int qrow = qblk * BM + rg * 32 + l32;
  const bool qvalid = qrow < a.nq;
  bf16x8 qreg[DK];
#pragma unroll
  for (int s = 0; s < DK; ++s) {
    if (qvalid) {
      qreg[s] = *(const bf16x8*)(qp + ((int64_t)qrow * H + h) * D + 16 * s + 8 * hh);
    } else {
      u32x4 z = {0u, 0u, 0u, 0u};
      qreg[s] = __builtin_bit_cast(bf16x8, z);
    }
  }
  const float qt = qvalid ? a.q_t[qrow] : 0.f;
  const bool q_out = PEN && qvalid && a.q_seg[qrow] == kSegOutput;
  // does any query row of this workgroup take the penalty?
  const bool pen_wg = PEN && __syncthreads_or(q_out);

  const int nkb = (a.nk + 63) / 64;
  const int ntiles = nkb;  // tiles are visited in ascending order; the cursor skips
                           // the ones no wave of this workgroup attends
  // query blocks of this workgroup that exist (bit j = block QB*qblk + j)
  int qb_valid = 0;
  // this wave's bit in a tile's attend mask
  const int my_qbit = 1 << (rg * 32 / kTile);
  if constexpr (SPARSE) {
    const int words = (nkb + 31) >> 5;  // the cursor reads no word past these
    for (int i = tid; i < (QB + 1) * words; i += 64 * NW)
      tile_bits[(i / words) * kBitmapWords + i % words] = 0u;
    __syncthreads();
    for (int i = tid; i < a.n_prot; i += 64 * NW) {
      const int kb = a.prot[i];
      if (kb >= 0 && kb < nkb) atomicOr(&tile_bits[kb >> 5], 1u << (kb & 31));
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int qb = qblk * QB + j;
      if (qb < a.nqb) {
        qb_valid |= 1 << j;
        const int32_t* lst = a.tiles + ((int64_t)h * a.nqb + qb) * a.k_sel;
        for (int i = tid; i < a.k_sel; i += 64 * NW) {
          const int kb = lst[i];
          if (kb >= 0 && kb < nkb)
            atomicOr(&tile_bits[(1 + j) * kBitmapWords + (kb >> 5)], 1u << (kb & 31));
        }
      }
    }
    __syncthreads();
  }

  // ---- per-lane byte offsets of this thread's DMA chunks inside a tile (fixed)
  uint32_t koff[DMA_PER_WAVE], voff[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int off = (wave * DMA_PER_WAVE + i) * 1024 + lane * 16;  // LDS byte offset
    const int r = off / KROW_BYTES, pc = (off % KROW_BYTES) / 16;    // key row, chunk slot
    koff[i] = (uint32_t)r * (uint32_t)(H * D * 2) + (uint32_t)(k_lds_chunk<D>(r, pc) * 16);
    // invert the V^T layout: slot -> (row d, logical chunk c)
    const int p = off / 256, slot = (off % 256) / 16;
    const int b = ((slot ^ (p & 15)) >> 3) & 1;
    const int c = (slot ^ ((p & 15) ^ (4 * b))) & 7;
    voff[i] = (uint32_t)(2 * p + b) * (uint32_t)(a.nkp * 2) + (uint32_t)(c * 16);
  }
  auto dma = [&](int kb, uint16_t* kdst, uint16_t* vdst) __attribute__((always_inline)) {
    const int k0 = kb * 64;
    const int rows = min(64, a.nk - k0);
    const void* kbase = kp + ((int64_t)k0 * H + h) * D;
    const int kbytes = (rows - 1) * H * D * 2 + D * 2;
    const void* vbase = vtp + (int64_t)h * D * a.nkp + k0;
    const int vbytes = (D - 1) * a.nkp * 2 + 128;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      buffer_to_lds16(kbase, kbytes, kdst + (wave * DMA_PER_WAVE + i) * 512, koff[i]);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      buffer_to_lds16(vbase, vbytes, vdst + (wave * DMA_PER_WAVE + i) * 512, voff[i]);
  };
  // row segment ids and times of a tile (per-key tiles only)
  uint32_t sreg = kSegInvalid;
  float treg = 0.f;
  auto small_load = [&](int kb) __attribute__((always_inline)) {
    if (tid < 64) {
      const int key = kb * 64 + tid;
      const bool kv = key < a.nk;
      sreg = kv ? (uint32_t)a.k_seg[key] : (uint32_t)kSegInvalid;
      treg = kv ? a.k_t[key] : 0.f;
    }
  };
  auto small_store = [&](uint8_t* sg, float* tt) __attribute__((always_inline)) {
    if (tid < 64) {
      sg[tid] = (uint8_t)sreg;
      tt[tid] = treg;
    }
  };

  // ---- tile classes: a tile is "fast" for this workgroup when all 64 keys are
  // present and its penalty is one scalar per query (no guide key, no query that takes
  // the penalty, or every key a guide row of one frame); every other tile is per-key.
  auto is_fast = [&](int flags) __attribute__((always_inline)) -> bool {
    return (flags & kTileFull) &&
           (!pen_wg || !(flags & kTileAnyGuide) || (flags & kTileUniformGuide));
  };
  // Walks the tile list in order, yielding the entries of one class. Each wave reads
  // 64 entries at a time and keeps a ballot mask of the matching ones.
  // Walks the key tiles in ascending order, yielding those of one class that some
  // wave attends. Each wave examines 64 tiles at a time and keeps a ballot mask of
  // the matching ones; .qmask says which query blocks attend the tile (sparse).
  struct Cursor { int chunk; uint64_t mask; int flags_lane; float t_lane; int qm_lane; };
  struct Tile { int kb; int flags; float t; int qmask; };
  auto cursor_next = [&](Cursor& cu, bool want_fast, Tile& tl) __attribute__((always_inline)) -> int {
    while (cu.mask == 0ull) {
      ++cu.chunk;
      if (cu.chunk * 64 >= ntiles) return ntiles;
      const int kb = cu.chunk * 64 + lane;
      int qm = 0;
      TileInfo ti{0, 0.f};
      if (kb < nkb) {
        if constexpr (SPARSE) {
          const int w = kb >> 5;
          const uint32_t b = 1u << (kb & 31);
          if (tile_bits[w] & b) {
            qm = qb_valid;
          } else {
#pragma unroll
            for (int j = 0; j < QB; ++j)
              if (tile_bits[(1 + j) * kBitmapWords + w] & b) qm |= 1 << j;
          }
        } else {
          qm = 1;
        }
        if (qm) ti = tinfo[kb];
      }
      cu.mask = __ballot(qm != 0 && (is_fast(ti.flags) == want_fast));
      cu.flags_lane = ti.flags;
      cu.t_lane = ti.t;
      cu.qm_lane = qm;
    }
    const int bit = __builtin_ctzll(cu.mask);
    cu.mask &= cu.mask - 1;
    tl.kb = cu.chunk * 64 + bit;
    tl.flags = __builtin_amdgcn_readfirstlane(__shfl(cu.flags_lane, bit));
    tl.t = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__shfl(cu.t_lane, bit))));
    tl.qmask = SPARSE ? __builtin_amdgcn_readfirstlane(__shfl(cu.qm_lane, bit)) : 1;
    return tl.kb;
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // ---- one tile: S^T = K Q^T, scores with the penalty, online softmax, O^T += V^T P^T.
  auto tile_body = [&](auto general_tag, const uint16_t* kst, const uint16_t* vst,
                       const uint8_t* ksg, const float* ktt, const Tile& tl) __attribute__((always_inline)) {
    constexpr bool GENERAL = decltype(general_tag)::value;
    if (SPARSE && !(tl.qmask & my_qbit)) return;  // this wave's block skips the tile
    f32x16 sacc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[c][r] = 0.f;
#pragma unroll
    for (int s = 0; s < DK; ++s) {
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int kr = 32 * c + l32;
        const bf16x8 ka = *(const bf16x8*)&kst[kr * D + k_lds_chunk<D>(kr, 2 * s + hh) * 8];
        sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], sacc[c], 0, 0, 0);
      }
    }
    float cc = c_log2, bb = 0.f, tmax;
    if constexpr (!GENERAL) {
      if (PEN && pen_wg && (tl.flags & kTileUniformGuide) && q_out)
        bb = -tara_pen(fabsf(qt - tl.t), a.window, a.inv_falloff, a.strength, a.cap) * kLog2e;
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          mx = __builtin_elementwise_maximum(
              __builtin_elementwise_maximum(mx, sacc[c][r]), sacc[c][r + 1]);
      tmax = mx * cc + bb;
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);
          const uint32_t sg = ksg[kl];
          float x = sacc[c][r] * cc;
          if (sg == (uint32_t)kSegInvalid) {
            x = -INFINITY;
          } else if (PEN && q_out && sg == (uint32_t)kSegGuide) {
            x -= tara_pen(fabsf(qt - ktt[kl]), a.window, a.inv_falloff, a.strength, a.cap) *
                 kLog2e;
          }
          sacc[c][r] = x;
          mx = __builtin_elementwise_maximum(mx, x);
        }
      }
      cc = 1.f;
      tmax = mx;
    }
    tmax = pair_max(tmax);
    if (__ballot(tmax > m_run + kLazyRescale) != 0ull) {
      const float m_new = __builtin_elementwise_maximum(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float mb = bb - (m_run == -INFINITY ? 0.f : m_run);
    bf16x8 pb[NS];
    float rs0 = 0.f, rs1 = 0.f;  // float32 row sums (two chains)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      f32x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][8 * (s & 1) + e], cc, mb));
        if (e & 1) rs1 += pv[e]; else rs0 += pv[e];
      }
      pb[s] = __builtin_convertvector(pv, bf16x8);
    }
    l_run += rs0 + rs1;
    const char* vsb = (const char*)vst;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dr = 32 * dt + l32;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int ch = 2 * s + hh;
        const bf16x8 va = *(const bf16x8*)(vsb + vt_lds_byte(dr, ch));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], oacc[dt], 0, 0, 0);
      }
    }
  };

  // ---- one pass over the tiles of one class, double-buffered: while stage s is
  // consumed, the next tile of the class streams into the other stage.
  auto run_pass = [&](auto general_tag) __attribute__((always_inline)) {
    constexpr bool GENERAL = decltype(general_tag)::value;
    Cursor cu{-1, 0ull, 0, 0.f, 0};
    Tile t_cur{-1, 0, 0.f, 0}, t_nxt{-1, 0, 0.f, 0}, t_nn{-1, 0, 0.f, 0};
    int cur = cursor_next(cu, !GENERAL, t_cur);
    if (cur < ntiles) {
      dma(t_cur.kb, ks0, vs0);
      if (GENERAL) { small_load(t_cur.kb); small_store(kseg0, kt0); }
    }
    __syncthreads();
    while (cur < ntiles) {
      const int nxt = cursor_next(cu, !GENERAL, t_nxt);
      if (nxt < ntiles) {
        dma(t_nxt.kb, ks1, vs1);
        if (GENERAL) small_load(t_nxt.kb);
      }
      tile_body(general_tag, ks0, vs0, kseg0, kt0, t_cur);
      if (GENERAL && nxt < ntiles) small_store(kseg1, kt1);
      __syncthreads();
      if (nxt >= ntiles) break;
      const int nn = cursor_next(cu, !GENERAL, t_nn);
      if (nn < ntiles) {
        dma(t_nn.kb, ks0, vs0);
        if (GENERAL) small_load(t_nn.kb);
      }
      tile_body(general_tag, ks1, vs1, kseg1, kt1, t_nxt);
      if (GENERAL && nn < ntiles) small_store(kseg0, kt0);
      __syncthreads();
      cur = nn;
      t_cur = t_nn;
    }
  };
  run_pass(std::false_type{});
  run_pass(std::true_type{});

  // ---- combine lane halves, then normalise
  const float l_tot = pair_sum(l_run);
  if (qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t obase = ((int64_t)qrow * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = oacc[dt][4 * g + j] * inv;
        const int d = 32 * dt + 8 * g + 4 * hh;
        if (a.o_f32) {
          *(f32x4*)((float*)a.o + obase + d) = ov;
        } else {
          *(bf16x4*)((__bf16*)a.o + obase + d) = __builtin_convertvector(ov, bf16x4);
        }
      }
    }
    if (hh == 0)
      a.lse[(int64_t)qrow * H + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool SPARSE, bool PEN>
hipError_t launch_variant(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.nq + 255) / 256, a.H);
  attn_bf16_kernel<D, SPARSE, PEN><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vt_transpose(const uint16_t* v, uint16_t* vt, int nk, int H, int D,
                               hipStream_t s) {
  const int nkp = (int)pad_keys(nk);
  dim3 grid(nkp / 64, H);
  if (D == 128)
    vt_transpose_kernel<128><<<grid, 256, 0, s>>>(v, vt, nk, nkp, H);
  else
    vt_transpose_kernel<64><<<grid, 256, 0, s>>>(v, vt, nk, nkp, H);
  return hipGetLastError();
}

hipError_t launch_tile_info(const uint8_t* k_seg, const float* k_t, int nk, TileInfo* info,
                            hipStream_t s) {
  tile_info_kernel<<<(nk + 63) / 64, 64, 0, s>>>(k_seg, k_t, nk, info);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int D, bool sparse, bool penalty, hipStream_t s) {
  if (D == 128) {
    if (sparse) return penalty ? launch_variant<128, true, true>(a, s) : launch_variant<128, true, false>(a, s);
    return penalty ? launch_variant<128, false, true>(a, s) : launch_variant<128, false, false>(a, s);
  }
  if (sparse) return penalty ? launch_variant<64, true, true>(a, s) : launch_variant<64, true, false>(a, s);
  return penalty ? launch_variant<64, false, true>(a, s) : launch_variant<64, false, false>(a, s);
}

}  // namespace h3
