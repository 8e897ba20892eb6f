// bf16 attention for gfx950: dense TARA and block-sparse attention over 64-key tiles.
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
//   sparse: the workgroup's rows are four 64-row query blocks (or halves of two 128-row
//           blocks, or eight 32-row blocks, one per wave). Their attended tiles (the
//           protected tiles plus each block's routed tiles, or every tile for a sink
//           block) are collected as bitmaps in LDS, and the workgroup walks the union in
//           ascending tile order: every tile is loaded once for all its blocks and each
//           wave computes only the tiles (or, for 32-row blocks, the tile halves) its own
//           block attends. Routed lists of neighbouring blocks overlap heavily when the
//           blocks share a video frame, so most loads serve the whole workgroup.
//           Optional: a pooled tail key merged in the epilogue, and an int8 QK product.
// Matrix cores: S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, so each
// lane holds one query column; softmax row reductions stay in registers plus one
// exchange between lane halves.
// K and V^T tiles sit in three LDS stages each, in rows padded by 16 bytes (bank-
// conflict-free operand reads, and every operand address is one base register plus an
// immediate), and are loaded ahead straight from global memory into LDS (buffer_load
// ... lds), so the loads hold no registers. The two waves of a SIMD run one slot apart:
// one wave's matrix products overlap the other's softmax.
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima are only raised when a tile exceeds them by more than this (log2
// units); probabilities then stay below 2^8 and most tiles skip the O rescale.
constexpr float kLazyRescale = 8.0f;
constexpr float kRescaleSum = 256.0f;  // 2^kLazyRescale
// Buffer descriptor word 3 for raw 32-bit-format loads on CDNA (out-of-range reads
// return zero).
constexpr int kBufferFlags = 0x00020000;

// Position of key `key` inside its 16-key group of the transposed v copy.
__host__ __device__ constexpr int key_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}


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
// Per 64-key tile: bit0 any guide key, bit1 every key a guide row of one frame, bit2 all
// 64 keys present, bit3 the 64 keys form exactly two runs of equal (segment, time), with
// bit4/bit5 marking which run is guide video, bits 8-15 the first key of the second run;
// .t = time of the first key, .t2 = time of the second run.
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
  // lanes where (segment, time) differs from the previous key
  const uint32_t sg_prev = __shfl_up(sg, 1);
  const float t_prev = __shfl_up(tt, 1);
  const uint64_t change = __ballot(threadIdx.x > 0 && (sg != sg_prev || tt != t_prev));
  const int split = change ? __builtin_ctzll(change) : 64;
  const float t2 = __shfl(tt, split & 63);
  if (threadIdx.x == 0) {
    int f = 0;
    if (g) f |= kTileAnyGuide;
    if (g == ~0ull && same == ~0ull) f |= kTileUniformGuide;
    if (full == ~0ull) {
      f |= kTileFull;
      if (__popcll(change) == 1) {
        f |= kTileTwoRun;
        if (g & 1ull) f |= kTileGuideA;
        if ((g >> split) & 1ull) f |= kTileGuideB;
      }
    }
    info[kb] = TileInfo{f | (split << 8), t0, t2, 0};
  }
}

// ------------------------------------------------------------------ attention
// LDS layouts (bf16): rows padded by one 16-byte slot, so 16 consecutive rows read at
// the same column start on 16 distinct bank groups (row stride = 16 bytes mod 256):
//   K   : row = key, D*2 + 16 bytes per row;
//   V^T : row = d, 64 keys = 128 + 16 bytes per row.
// A tile is filled by 1 KB direct-to-LDS wave loads over its contiguous bytes; lanes that
// land on a pad slot read out of range (zero).
template <int D>
struct Lds {
  static constexpr int KRS = D * 2 + 16;   // K row stride (bytes)
  static constexpr int KSL = D / 8 + 1;    // 16-byte slots per K row
  static constexpr int VRS = 128 + 16;     // V^T row stride (bytes)
  static constexpr int VSL = 9;            // 16-byte slots per V^T row
  static constexpr int KBYTES = 64 * KRS;  // one K tile
  static constexpr int VBYTES = D * VRS;   // one V^T tile
  static constexpr int KINS = KBYTES / 1024;  // 1 KB wave loads per K tile
  static constexpr int VINS = VBYTES / 1024;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "whole wave loads");
  // int8 K tiles (int8 QK product): rows of D bytes padded by 16
  static constexpr int KRS8 = D + 16;
  static constexpr int KSL8 = D / 16 + 1;
  static constexpr int KBYTES8 = 64 * KRS8;
  static constexpr int KINS8 = KBYTES8 / 1024;
  static_assert(KBYTES8 % 1024 == 0 && KBYTES8 <= KBYTES, "int8 K tile");
};
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // buffer offset that reads zero

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitAll0 = 0x0070;   // vmcnt(0) lgkmcnt(0)

// Scheduling order for a run of N MFMAs, each fed by one LDS operand read: AHEAD reads
// are issued first and one more after every MFMA, so AHEAD reads stay in flight and the
// MFMAs do not wait out each read's full LDS latency.
template <int N, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma() {
  constexpr int A = N > AHEAD ? AHEAD : N;  // a short run: every read first
  __builtin_amdgcn_sched_group_barrier(0x100, A, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}
constexpr int kLdsAhead = 4;

// Workgroup barrier without the memory-model fence of __syncthreads (that fence would
// also wait for the direct-to-LDS loads meant to stay in flight across it). WAIT is
// the s_waitcnt the caller needs before arriving; the empty asm statements keep the
// compiler from moving memory accesses across the barrier.
template <int WAIT>
__device__ __forceinline__ void slot_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(WAIT);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Lanes l and l^32 hold the two key halves of the same query column; one
// v_permlane32_swap gives every lane both halves.
__device__ __forceinline__ float pair_max_swap(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum_swap(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// FINE: block-sparse with 32-row routing blocks (per-wave lists, half tiles); a
// separate instance so the 64/128-row kernel carries none of that code.
// Q8: block-sparse with the int8 QK product ("H3 SLA Attention", inputs table,
// use_int8_qk): q and k come quantized per (row, head) (x8, scale); S = K8 Q8^T with
// v_mfma_i32_32x32x32_i8, then each score is the int32 sum times the key's scale, and
// the query's scale joins the exp factor. PV is unchanged (bf16 P, bf16 V).
template <int D, bool SPARSE, bool PEN, bool FINE = false, bool Q8 = false>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NW = 8;               // waves per workgroup (two per SIMD)
  constexpr int BM = 32 * NW;         // query rows per workgroup
  constexpr int QB = BM / kTile;      // query blocks per workgroup (sparse)
  constexpr int NT = 2;               // 32x32 score tiles per wave (64 keys)
  constexpr int NS = 4;               // k-steps of the PV product (64 keys / 16)
  constexpr int DK = D / 16;          // k-steps of the QK product
  constexpr int DT = D / 32;          // 32-row output tiles (over d)
  using L = Lds<D>;
  constexpr int KDMA = (L::KINS + NW - 1) / NW;  // wave loads per wave and K tile (at most)
  constexpr int VDMA = (L::VINS + NW - 1) / NW;

  // Three stages each for K and V^T, each stage its own LDS object so the compiler can
  // tell the stage being read from the stage being filled by the direct-to-LDS loads.
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[L::KBYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t ks1[L::KBYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t ks2[L::KBYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[L::VBYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t vs1[L::VBYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t vs2[L::VBYTES / 2];
  __shared__ uint8_t kseg0[64], kseg1[64], kseg2[64];
  __shared__ float kt0[64], kt1[64], kt2[64];
  // int8 QK: per-key scales of the staged tiles
  __shared__ __attribute__((aligned(16))) float ksc0[Q8 ? 64 : 4], ksc1[Q8 ? 64 : 4],
      ksc2[Q8 ? 64 : 4];
  __shared__ int simd_waves[4];
  __shared__ int sink_waves;  // sparse: bit w = wave w's rows hold a sink-segment row
  // sparse: bitmap 0 = protected blocks, bitmap 1 + j = routed blocks of map j (see below)
  __shared__ uint32_t tile_bits[SPARSE ? (NW + 1) * kBitmapWords : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int qblk = blockIdx.x;
  const int h = blockIdx.y;
  const int H = a.H;
  const uint16_t* __restrict__ qp = (const uint16_t*)a.q;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k;
  const uint16_t* __restrict__ vtp = a.vt;
  const TileInfo* __restrict__ tinfo = a.tinfo;
  float c_log2 = a.scale * kLog2e;

  const int qrow = qblk * BM + wave * 32 + l32;
  const bool qvalid = qrow < a.nq;
  bf16x8 qreg[Q8 ? 1 : DK];
  i32x4 q8reg[Q8 ? D / 32 : 1];
  if constexpr (Q8) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      q8reg[s] = qvalid ? *(const i32x4*)(a.q8 + ((int64_t)qrow * H + h) * D + 32 * s + 16 * hh)
                        : i32x4{0, 0, 0, 0};
    c_log2 *= qvalid ? a.qsc[(int64_t)qrow * H + h] : 0.f;  // the query's scale
  } else {
#pragma unroll
    for (int s = 0; s < DK; ++s) {
      if (qvalid) {
        qreg[s] = *(const bf16x8*)(qp + ((int64_t)qrow * H + h) * D + 16 * s + 8 * hh);
      } else {
        u32x4 z = {0u, 0u, 0u, 0u};
        qreg[s] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }
  const float qt = qvalid ? a.q_t[qrow] : 0.f;
  const bool q_out = PEN && qvalid && a.q_seg[qrow] == kSegOutput;

  // ---- the two waves that share a SIMD take opposite phases (group 0 / group 1):
  // while one runs its matrix-core slot the other runs its softmax slot.
  if (tid < 4) simd_waves[tid] = 0;
  if (SPARSE && tid == 0) sink_waves = 0;
  // does any query row of this workgroup take the penalty? (also orders the resets above)
  const bool pen_wg = __syncthreads_or(q_out);
  if constexpr (SPARSE) {
    const bool sink_row = qvalid && ((a.sink_mask >> a.q_seg[qrow]) & 1u);
    if (__ballot(sink_row) != 0ull && lane == 0) atomicOr(&sink_waves, 1 << wave);
  }
  int grp = 0;
  if (lane == 0) {
    const int simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);  // HW_ID.SIMD_ID
    grp = atomicAdd(&simd_waves[simd & 3], 1) & 1;
  }
  const bool grp_b = __builtin_amdgcn_readfirstlane(grp) != 0;

  const int nkb = (a.nk + 63) / 64;
  const int ntiles = nkb;  // tiles are visited in ascending order; the cursor skips
                           // the ones no wave of this workgroup attends
  // A tile's attend mask has two bits per wave: bit 2w for keys 0-31 of the tile, bit
  // 2w+1 for keys 32-63. Dense launches attend everything. Sparse launches keep one
  // bitmap of protected blocks and one per "map" of routed blocks:
  //   block size 64 / 128: map j = the 64-row block j of the workgroup (waves 2j, 2j+1),
  //     one bit per 64-key tile (a 128-row block sets both of its tiles, and its two
  //     64-row halves read the same list);
  //   block size 32: map j = wave j's 32-row block, one bit per 32 keys, so a wave may
  //     attend one half of a tile.
  // A query block holding a row of a sink segment attends every key.
  constexpr bool fine = SPARSE && FINE;
  int map_valid = 0;     // bit j: map j's query block exists
  bool my_sink = false;  // this wave's query block attends every key
  const int my_shift = __builtin_amdgcn_readfirstlane(2 * wave);
  if constexpr (SPARSE) {
    const int nmaps = fine ? NW : QB;
    const int nbits = fine ? (a.nk + 31) >> 5 : nkb;
    const int words = (nbits + 31) >> 5;  // the cursor reads no word past these
    for (int i = tid; i < (nmaps + 1) * words; i += 64 * NW)
      tile_bits[(i / words) * kBitmapWords + i % words] = 0u;
    __syncthreads();
    const int sinks = sink_waves;
    // marks routing block b (in units of the block size) in bitmap m
    auto mark = [&](int m, int b) __attribute__((always_inline)) {
      uint32_t* bm = tile_bits + m * kBitmapWords;
      if (a.bs == 128) {
        if (b >= 0 && b < (nkb + 1) / 2) {
          atomicOr(&bm[(2 * b) >> 5], 1u << ((2 * b) & 31));
          if (2 * b + 1 < nkb) atomicOr(&bm[(2 * b + 1) >> 5], 1u << ((2 * b + 1) & 31));
        }
      } else if (b >= 0 && b < nbits) {
        atomicOr(&bm[b >> 5], 1u << (b & 31));
      }
    };
    for (int i = tid; i < a.n_prot; i += 64 * NW) mark(0, a.prot[i]);
    for (int j = 0; j < nmaps; ++j) {
      const int row0 = qblk * BM + j * (fine ? 32 : 64);
      if (row0 >= a.nq) continue;
      map_valid |= 1 << j;
      // waves of this map's query block (a 128-row block spans two maps)
      const int wmask = fine ? (1 << j) : (a.bs == 128 ? 0xF << (4 * (j >> 1)) : 3 << (2 * j));
      const bool sink = (sinks & wmask) != 0;
      if (fine ? wave == j : (wave >> 1) == j) my_sink = sink;
      if (sink) {
        for (int i = tid; i < words; i += 64 * NW) tile_bits[(1 + j) * kBitmapWords + i] = ~0u;
        continue;
      }
      const int qb = row0 / a.bs;
      const int32_t* lst = a.tiles + ((int64_t)h * a.nqb + qb) * a.k_sel;
      for (int i = tid; i < a.k_sel; i += 64 * NW) mark(1 + j, lst[i]);
    }
    __syncthreads();
  }

  // ---- per-lane global byte offsets of this thread's wave loads (wave load i of a tile
  // belongs to wave i % 8)
  uint32_t koff[KDMA], voff[VDMA];
#pragma unroll
  for (int j = 0; j < KDMA; ++j) {
    const int slot = (wave + NW * j) * 64 + lane;
    if constexpr (Q8) {
      const int r = slot / L::KSL8, c = slot % L::KSL8;
      koff[j] = c == L::KSL8 - 1 ? kOutOfRange
                                 : (uint32_t)r * (uint32_t)(H * D) + (uint32_t)(c * 16);
    } else {
      const int r = slot / L::KSL, c = slot % L::KSL;
      koff[j] = c == L::KSL - 1 ? kOutOfRange
                                : (uint32_t)r * (uint32_t)(H * D * 2) + (uint32_t)(c * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < VDMA; ++j) {
    const int slot = (wave + NW * j) * 64 + lane;
    const int d = slot / L::VSL, c = slot % L::VSL;
    voff[j] = c == L::VSL - 1 ? kOutOfRange
                              : (uint32_t)d * (uint32_t)(a.nkp * 2) + (uint32_t)(c * 16);
  }
  auto dma_k = [&](int kb, uint16_t* kdst) __attribute__((always_inline)) {
    const int k0 = kb * 64;
    const int rows = min(64, a.nk - k0);
    if constexpr (Q8) {
      const void* kbase = a.k8 + ((int64_t)k0 * H + h) * D;
      const int kbytes = (rows - 1) * H * D + D;
#pragma unroll
      for (int j = 0; j < KDMA; ++j)
        if (wave + NW * j < L::KINS8)
          buffer_to_lds16(kbase, kbytes, (char*)kdst + (wave + NW * j) * 1024, koff[j]);
    } else {
      const void* kbase = kp + ((int64_t)k0 * H + h) * D;
      const int kbytes = (rows - 1) * H * D * 2 + D * 2;
#pragma unroll
      for (int j = 0; j < KDMA; ++j)
        if (wave + NW * j < L::KINS)
          buffer_to_lds16(kbase, kbytes, (char*)kdst + (wave + NW * j) * 1024, koff[j]);
    }
  };
  auto dma_v = [&](int kb, uint16_t* vdst) __attribute__((always_inline)) {
    const void* vbase = vtp + (int64_t)h * D * a.nkp + kb * 64;
    const int vbytes = (D - 1) * a.nkp * 2 + 128;
#pragma unroll
    for (int j = 0; j < VDMA; ++j)
      if (wave + NW * j < L::VINS)
        buffer_to_lds16(vbase, vbytes, (char*)vdst + (wave + NW * j) * 1024, voff[j]);
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
  // int8 QK: the key scales of a tile (every tile), staged like the key rows above
  float kscr = 0.f;
  auto scale_load = [&](int kb) __attribute__((always_inline)) {
    if (tid < 64) {
      const int key = kb * 64 + tid;
      kscr = key < a.nk ? a.ksc[(int64_t)key * H + h] : 0.f;
    }
  };
  auto scale_store = [&](float* sc) __attribute__((always_inline)) {
    if (tid < 64) sc[tid] = kscr;
  };

  // ---- tile classes: a tile is "fast" for this workgroup when all 64 keys are
  // present and its penalty is one scalar per query (no guide key, no query that takes
  // the penalty, or every key a guide row of one frame); every other tile is per-key.
  auto is_fast = [&](int flags) __attribute__((always_inline)) -> bool {
    return (flags & kTileFull) &&
           (!pen_wg || !(flags & kTileAnyGuide) || (flags & kTileUniformGuide));
  };
  // Walks the key tiles in ascending order, yielding those of one class that some
  // wave attends. Each wave examines 64 tiles at a time and keeps a ballot mask of
  // the matching ones; .qmask is the tile's attend mask (two bits per wave). Sparse
  // launches load the summaries of the next 64 tiles one refill ahead, so a refill does
  // not wait on memory. Every wave walks the same sequence.
  struct Cursor {
    int chunk; uint64_t mask; int flags_lane; float t_lane; float t2_lane; int qm_lane;
    TileInfo pre;
  };
  struct Tile { int kb; int flags; float t; int qmask; float t2; int split; };
  auto cursor_start = [&]() __attribute__((always_inline)) -> Cursor {
    TileInfo pre{64 << 8, 0.f, 0.f, 0};
    if (SPARSE && lane < nkb) pre = tinfo[lane];
    return Cursor{-1, 0ull, 0, 0.f, 0.f, 0, pre};
  };
  auto cursor_next = [&](Cursor& cu, bool want_fast) __attribute__((always_inline)) -> Tile {
    while (cu.mask == 0ull) {
      ++cu.chunk;
      if (cu.chunk * 64 >= ntiles) return Tile{ntiles, 0, 0.f, 0, 0.f, 64};
      const int kb = cu.chunk * 64 + lane;
      TileInfo ti{64 << 8, 0.f, 0.f, 0};
      if constexpr (SPARSE) {  // sparse passes scan many chunks per attended tile
        ti = cu.pre;
        if (kb + 64 < nkb) cu.pre = tinfo[kb + 64];
      } else if (kb < nkb) {
        ti = tinfo[kb];
      }
      int qm = 0;
      if (kb < nkb) {
        if constexpr (SPARSE) {
          if constexpr (fine) {  // two bits per map and tile
            const int w = kb >> 4, sh = 2 * (kb & 15);
            const uint32_t p2 = tile_bits[w] >> sh;
#pragma unroll
            for (int j = 0; j < NW; ++j)
              if ((map_valid >> j) & 1)
                qm |= (int)((p2 | (tile_bits[(1 + j) * kBitmapWords + w] >> sh)) & 3u) << (2 * j);
          } else {
            const int w = kb >> 5;
            const uint32_t b = 1u << (kb & 31);
            const bool pr = (tile_bits[w] & b) != 0u;
#pragma unroll
            for (int j = 0; j < QB; ++j)
              if (((map_valid >> j) & 1) && (pr || (tile_bits[(1 + j) * kBitmapWords + w] & b)))
                qm |= 0xF << (4 * j);
          }
        } else {
          qm = 0xFFFF;
        }
      }
      cu.mask = __ballot(qm != 0 && (is_fast(ti.flags) == want_fast));
      cu.flags_lane = ti.flags;
      cu.t_lane = ti.t;
      cu.t2_lane = ti.t2;
      cu.qm_lane = qm;
    }
    const int bit = __builtin_ctzll(cu.mask);
    cu.mask &= cu.mask - 1;
    const int fs = __builtin_amdgcn_readlane(cu.flags_lane, bit);
    return Tile{
        cu.chunk * 64 + bit,
        fs & kTileFlagMask,
        __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cu.t_lane), bit)),
        SPARSE ? __builtin_amdgcn_readlane(cu.qm_lane, bit) : 0xFFFF,
        want_fast ? 0.f
                  : __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cu.t2_lane), bit)),
        fs >> 8};
  };
  // does this wave compute tile tl?
  auto attends = [&](const Tile& tl) __attribute__((always_inline)) -> bool {
    return tl.kb < ntiles && (!SPARSE || ((tl.qmask >> my_shift) & 3));
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 sacc[NT];    // scores of the tile between its QK product and its softmax
  bf16x8 pb[NS];      // probabilities of the tile between its softmax and its PV product

  // ---- matrix-core slot: O^T += V^T P^T for the previous tile, then S^T = K Q^T.
  auto mfma_slot = [&](const uint16_t* kst, const uint16_t* vst, bool do_pv, bool do_qk)
      __attribute__((always_inline)) {
    if (do_pv) {
      const char* vsb = (const char*)vst + l32 * L::VRS + hh * 16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 va = *(const bf16x8*)(vsb + dt * 32 * L::VRS + s * 32);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], oacc[dt], 0, 0, 0);
        }
      }
      pipeline_lds_mfma<DT * NS, kLdsAhead>();
    }
    // keep the two products apart so their operand reads do not pile up in registers
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) {
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[c][r] = 0.f;
      if constexpr (Q8) {  // int32 sums in the score registers until the softmax slot
        const char* ksb = (const char*)kst + l32 * L::KRS8 + hh * 16;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
#pragma unroll
          for (int c = 0; c < NT; ++c) {
            const i32x4 ka = *(const i32x4*)(ksb + c * 32 * L::KRS8 + s * 32);
            sacc[c] = __builtin_bit_cast(
                f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            ka, q8reg[s], __builtin_bit_cast(i32x16, sacc[c]), 0, 0, 0));
          }
        }
        pipeline_lds_mfma<(D / 32) * NT, kLdsAhead>();
      } else {
      const char* ksb = (const char*)kst + l32 * L::KRS + hh * 16;
#pragma unroll
      for (int s = 0; s < DK; ++s) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const bf16x8 ka = *(const bf16x8*)(ksb + c * 32 * L::KRS + s * 32);
          sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], sacc[c], 0, 0, 0);
        }
      }
      pipeline_lds_mfma<DK * NT, kLdsAhead>();
      }
    }
  };

  // ---- softmax slot: scores with the penalty, online softmax, probabilities in bf16.
  // p = exp2(s * cc + mb) for the 32 scores of this lane, as bf16 into pb, with bias mb0
  // for keys 0-31 of the tile and mb1 for keys 32-63 (-inf drops a half); returns the
  // float32 sum of the 32 (four chains).
  auto exp_tile = [&](float cc, float mb0, float mb1) __attribute__((always_inline)) -> float {
    float r[4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      f32x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(
            fmaf(sacc[s >> 1][8 * (s & 1) + e], cc, (s >> 1) ? mb1 : mb0));
        r[e & 3] = (s == 0 && e < 4) ? pv[e] : r[e & 3] + pv[e];
      }
      pb[s] = __builtin_convertvector(pv, bf16x8);
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
  };
  // Raises the running maximum to cover this tile's scaled maximum `tmax` (log2 units,
  // equal in both lane halves), rescaling O and the running sum.
  auto raise_max = [&](float tmax) __attribute__((always_inline)) {
    const float m_new = __builtin_elementwise_maximum(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    l_run *= alpha;
    m_run = m_new;
  };
  // maximum of this lane's scores in the kept halves of the tile (a tree of three-input
  // maxima per half)
  auto score_max = [&](bool keep0, bool keep1) __attribute__((always_inline)) -> float {
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i >> 2, r = 4 * (i & 3);
      m[i] = __builtin_elementwise_maximum(
          __builtin_elementwise_maximum(sacc[c][r], sacc[c][r + 1]),
          __builtin_elementwise_maximum(sacc[c][r + 2], sacc[c][r + 3]));
    }
    const float m0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m[0], m[1]),
                                                   __builtin_elementwise_maximum(m[2], m[3]));
    const float m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m[4], m[5]),
                                                   __builtin_elementwise_maximum(m[6], m[7]));
    return __builtin_elementwise_maximum(keep0 ? m0 : -INFINITY, keep1 ? m1 : -INFINITY);
  };

  // ---- softmax slot: scores with the penalty, online softmax, probabilities in bf16.
  // Fast tiles are exponentiated against the running maximum straight away; only if a
  // lane's sum of the 32 exceeds 2^8 (so some probability might, or the maximum is still
  // -inf) does the tile take the maximum, rescale and exponentiate again. Probabilities
  // thus stay at most 2^8 while most tiles skip the maximum altogether.
  auto softmax_slot = [&](auto general_tag, const uint8_t* ksg, const float* ktt,
                          const float* kst8, const Tile& tl) __attribute__((always_inline)) {
    constexpr bool GENERAL = decltype(general_tag)::value;
    if constexpr (Q8) {  // int32 sums -> float scores times each key's scale
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        // whole-vector casts: the int32 sums live in the score registers
        f32x16 sf = __builtin_convertvector(__builtin_bit_cast(i32x16, sacc[c]), f32x16);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 sk = *(const f32x4*)(kst8 + 32 * c + 8 * g + 4 * hh);
#pragma unroll
          for (int i = 0; i < 4; ++i) sf[4 * g + i] *= sk[i];
        }
        sacc[c] = sf;
      }
    }
    // block size 32: this wave may attend only one half of the tile (keys 0-31 or 32-63);
    // the other half gets a -inf bias
    const int h2 = fine ? (tl.qmask >> my_shift) & 3 : 3;
    const bool keep0 = h2 & 1, keep1 = h2 & 2;
    if constexpr (!GENERAL) {
      float bb = 0.f;
      if (PEN && pen_wg && (tl.flags & kTileUniformGuide) && q_out)
        bb = -tara_pen(fabsf(qt - tl.t), a.window, a.inv_falloff, a.strength, a.cap) * kLog2e;
      float mb = bb - m_run;
      float rs = exp_tile(c_log2, keep0 ? mb : -INFINITY, keep1 ? mb : -INFINITY);
      if (__ballot(!(rs <= kRescaleSum)) != 0ull) {
        raise_max(pair_max_swap(score_max(keep0, keep1) * c_log2 + bb));
        mb = bb - m_run;
        rs = exp_tile(c_log2, keep0 ? mb : -INFINITY, keep1 ? mb : -INFINITY);
      }
      l_run += rs;
    } else {
      float mx = -INFINITY;
      if (tl.flags & kTileTwoRun) {
        // two runs, each with one per-query penalty: keys below the split take bA
        const float bA = (PEN && q_out && (tl.flags & kTileGuideA))
                             ? -tara_pen(fabsf(qt - tl.t), a.window, a.inv_falloff, a.strength,
                                         a.cap) * kLog2e
                             : 0.f;
        const float bB = (PEN && q_out && (tl.flags & kTileGuideB))
                             ? -tara_pen(fabsf(qt - tl.t2), a.window, a.inv_falloff, a.strength,
                                         a.cap) * kLog2e
                             : 0.f;
        const int thr = tl.split - 4 * hh;  // key offset 32c + 8(r/4) + r%4 below thr: run A
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const bool keep = c ? keep1 : keep0;
          const float cA = keep ? bA : -INFINITY, cB = keep ? bB : -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kofs = 32 * c + 8 * (r >> 2) + (r & 3);
            const float x = fmaf(sacc[c][r], c_log2, kofs < thr ? cA : cB);
            sacc[c][r] = x;
            mx = __builtin_elementwise_maximum(mx, x);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const float hb = (c ? keep1 : keep0) ? 0.f : -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);
            const uint32_t sg = ksg[kl];
            float x = fmaf(sacc[c][r], c_log2, hb);
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
      }
      const float tmax = pair_max_swap(mx);
      if (__ballot(tmax > m_run + kLazyRescale) != 0ull) raise_max(tmax);
      const float mb = m_run == -INFINITY ? 0.f : -m_run;
      l_run += exp_tile(1.f, mb, mb);
    }
  };

  // ---- one pass over the tiles of one class. Every wave runs the same sequence of
  // slots separated by workgroup barriers: matrix slot j (O += P_{j-1} V_{j-1}, then
  // S_j = Q K_j^T), softmax slot j (issue the loads of K_{j+2} and V_{j+1}, then the
  // softmax of S_j). Group 1 passes one extra barrier before its first slot and group 0
  // one after its last, so group 1 runs one slot behind group 0 and each SIMD overlaps
  // one wave's matrix products with the other wave's softmax. K_j sits in stage j % 3 and
  // V_j in stage j % 3: with the one-slot skew, a stage is refilled only after both groups
  // have finished reading it, and every load has two slots to land.
  auto run_pass = [&](auto general_tag) __attribute__((always_inline)) {
    constexpr bool GENERAL = decltype(general_tag)::value;
    Cursor cu = cursor_start();
    Tile tp{ntiles, 0, 0.f, 0, 0.f, 64}, tq{ntiles, 0, 0.f, 0, 0.f, 64}, tn{ntiles, 0, 0.f, 0, 0.f, 64};
    tq = cursor_next(cu, !GENERAL);
    if (tq.kb >= ntiles) return;
    tn = cursor_next(cu, !GENERAL);
    // prologue: K_0, K_1, V_0 (and the key rows of tiles 0 and 1)
    dma_k(tq.kb, ks0);
    dma_v(tq.kb, vs0);
    if (GENERAL) small_load(tq.kb);
    if (Q8) scale_load(tq.kb);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (GENERAL) small_store(kseg0, kt0);
    if (Q8) scale_store(ksc0);
    if (tn.kb < ntiles) {
      dma_k(tn.kb, ks1);
      if (GENERAL) small_load(tn.kb);
      if (Q8) scale_load(tn.kb);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if (GENERAL) small_store(kseg1, kt1);
      if (Q8) scale_store(ksc1);
    }
    slot_barrier<kWaitAll0>();
    if (grp_b) slot_barrier<kWaitAll0>();
    // One (matrix, softmax) slot pair; the stage arguments rotate with j % 3.
    auto step = [&](uint16_t* kcur, uint16_t* vprev, uint16_t* knn, uint16_t* vnext,
                    uint8_t* sgcur, float* ttcur, uint8_t* sgnext, float* ttnext,
                    float* sccur, float* scnext) __attribute__((always_inline)) {
      mfma_slot(kcur, vprev, attends(tp), attends(tq));
      // the key rows of tile j+1 were fetched during the previous softmax slot
      if (GENERAL && tn.kb < ntiles) small_store(sgnext, ttnext);
      if (Q8 && tn.kb < ntiles) scale_store(scnext);
      slot_barrier<kWaitAll0>();
      const Tile tnn = cursor_next(cu, !GENERAL);
      if (tnn.kb < ntiles) {
        dma_k(tnn.kb, knn);
        if (GENERAL) small_load(tnn.kb);
        if (Q8) scale_load(tnn.kb);
      }
      if (tn.kb < ntiles) dma_v(tn.kb, vnext);
      if (attends(tq)) softmax_slot(general_tag, sgcur, ttcur, sccur, tq);
      slot_barrier<kWaitLgkm0>();
      tp = tq;
      tq = tn;
      tn = tnn;
    };
    while (true) {
      step(ks0, vs2, ks2, vs1, kseg0, kt0, kseg1, kt1, ksc0, ksc1);
      if (tp.kb >= ntiles) break;
      step(ks1, vs0, ks0, vs2, kseg1, kt1, kseg2, kt2, ksc1, ksc2);
      if (tp.kb >= ntiles) break;
      step(ks2, vs1, ks1, vs0, kseg2, kt2, kseg0, kt0, ksc2, ksc0);
      if (tp.kb >= ntiles) break;
    }
    if (!grp_b) slot_barrier<kWaitAll0>();
  };
  run_pass(std::false_type{});
  run_pass(std::true_type{});

  // ---- combine lane halves, then normalise
  float l_tot = pair_sum_swap(l_run);
  // optional tail key of the query block: one more softmax term with logit tail_lse and
  // value tail_v, merged like any other key (log2 units here)
  float tail_w = 0.f;
  const float* tail_v = nullptr;
  if (SPARSE && a.tail_lse && qvalid && !my_sink) {
    const int64_t tb = (int64_t)h * a.nqb + qrow / a.bs;
    const float lt = a.tail_lse[tb] * kLog2e;
    if (lt != -INFINITY) {
      const float m_new = __builtin_elementwise_maximum(m_run, lt);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      tail_w = __builtin_amdgcn_exp2f(lt - m_new);
      l_tot = l_tot * alpha + tail_w;
      m_run = m_new;
      tail_v = a.tail_v + tb * D;
    }
  }
  if (qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t obase = ((int64_t)qrow * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ov;
        const int d = 32 * dt + 8 * g + 4 * hh;
        if (tail_v) {
          const f32x4 tv = *(const f32x4*)(tail_v + d);
#pragma unroll
          for (int j = 0; j < 4; ++j) oacc[dt][4 * g + j] += tail_w * tv[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = oacc[dt][4 * g + j] * inv;
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
  if constexpr (SPARSE) {
    if (a.q8) {  // int8 QK (block sizes 64 and 128)
      attn_bf16_kernel<D, true, PEN, false, true><<<grid, 512, 0, s>>>(a);
      return hipGetLastError();
    }
    if (a.bs == 32) {
      attn_bf16_kernel<D, true, PEN, true><<<grid, 512, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  attn_bf16_kernel<D, SPARSE, PEN, false><<<grid, 512, 0, s>>>(a);
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
