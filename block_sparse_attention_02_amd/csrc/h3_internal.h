// Internal declarations shared by the HIP translation units of libh3attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace h3 {

constexpr int kTile = 64;         // key tile of the attention kernels = 64 rows
constexpr int kSegText = 0, kSegGuide = 1, kSegAudio = 2, kSegOutput = 3;
constexpr int kSegInvalid = 255;  // marks key slots past the end of a tile
// Largest block count the router and the block-sparse kernels accept, at every block
// size, and at most this many 64-row tiles (896,000 rows): the per-workgroup bitmaps
// and the router's per-block scores live in LDS.
constexpr int kMaxBlocks = 14000;
constexpr int kBitmapWords = (kMaxBlocks + 31) / 32;

// Per 64-key tile summary (see tile_info_kernel).
constexpr int kTileAnyGuide = 1, kTileUniformGuide = 2, kTileFull = 4;
constexpr int kTileTwoRun = 8;     // full tile of two runs of equal (segment, time)
constexpr int kTileGuideA = 16;    // the first run is guide video
constexpr int kTileGuideB = 32;    // the second run is guide video
struct TileInfo {
  int flags;    // bits 0-7: the kTile* flags; bits 8-15: first key of the second run
                // (two-run tiles, else 64)
  float t;      // time of the first key
  float t2;     // time of the second run (two-run tiles)
  int pad;
};
constexpr int kTileFlagMask = 0xff;

// Arguments of one attention launch (dense or block-sparse).
struct AttnArgs {
  const void* q;            // [nq][H][D]  (bf16 bits or f32)
  const void* k;            // [nk][H][D]
  const void* v;            // [nk][H][D]  (f32 path)
  const uint16_t* vt;       // [H][D][nkp] bf16, keys permuted in 16-groups (bf16 path)
  const TileInfo* tinfo;    // [ceil(nk/64)] (bf16 path)
  const uint8_t* q_seg;
  const float* q_t;
  const uint8_t* k_seg;
  const float* k_t;
  void* o;                  // [nq][H][D]
  float* lse;               // [nq][H]
  int nq, nk, nkp, H;
  int o_f32;                // 1: o is float32, 0: bf16
  float scale;
  float strength, window, inv_falloff, cap;
  // block-sparse tile lists (unused by the dense launch)
  const int32_t* prot;
  int n_prot;
  const int32_t* tiles;     // [H][nqb][k_sel]
  int k_sel;
  int nqb;                  // query blocks of the lists: ceil(nq / bs)
  int bs;                   // rows per routing block: 32, 64 or 128
  uint32_t sink_mask;       // bit s: query blocks holding a row of segment s attend all keys
  // optional tail key per query block (block-sparse with tail term), else null
  const float* tail_lse;    // [H][nqb] natural log
  const float* tail_v;      // [H][nqb][D]
  // int8 QK product (block-sparse, bf16 path), else null: per-(row, head) int8 q and k
  // with their float32 scales
  const int8_t* q8;         // [nq][H][D]
  const float* qsc;         // [nq][H]
  const int8_t* k8;         // [nk][H][D]
  const float* ksc;         // [nk][H]
};

// Rounds a key count up to whole 64-key tiles.
inline int64_t pad_keys(int64_t nk) { return (nk + kTile - 1) / kTile * kTile; }

// bf16 path: transposes v into vt (see attn_bf16.hip), then runs attention.
hipError_t launch_vt_transpose(const uint16_t* v, uint16_t* vt, int nk, int H, int D,
                               hipStream_t s);
hipError_t launch_tile_info(const uint8_t* k_seg, const float* k_t, int nk, TileInfo* info,
                            hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, int D, bool sparse, bool penalty, hipStream_t s);
// Per-(row, head) int8 quantization (see quant.hip); pairs = rows * heads.
hipError_t launch_quant_int8(const void* x, bool bf16, int64_t pairs, int D, int8_t* x8,
                             float* sc, hipStream_t s);
// float32 path.
hipError_t launch_attn_f32(const AttnArgs& a, int D, bool sparse, bool penalty, hipStream_t s);

// Router.
struct RouterWs {
  float* qbar;     // [H][nb][D]
  float* kbar;     // [H][D][nbk] (d-major, row stride nbk = nb rounded up to 16)
  int32_t* video;  // [nb]
  int32_t* counts; // [2]: n_prot, n_video
  float* vbar;     // [H][nb][D] (tail term only, else null)
  float* wts;      // [H][nb][nbp] tail weights per (query block, video tile) (tail only)
  float* vbt;      // [H][D][nbp] V means of the video tiles, transposed (tail only)
  int nbp;         // nb rounded up to 32
  int nbk;         // row stride of kbar
};
// Tail term of the unrouted tiles (see router.hip); all pointers null when not wanted.
struct TailArgs {
  float scale;         // attention scale applied to the pooled scores
  int n;               // rows of the sequence (counts of the ragged last tile)
  int bs;              // rows per block
  const float* vbar;   // [H][nb][D] block means of v
  float* lse;          // [H][nb] natural-log logit of the tail key
  float* v;            // [H][nb][D] value of the tail key
  float* wts;          // [H][nb][nbp] normalised weights of the unrouted video tiles
  int nbp;
};
// Light reference protection (see router.hip): the ordinary routed count and, per
// reference range, its position in the video-tile list and its guaranteed count.
constexpr int kMaxRefRanges = 16;
struct RefQuota {
  int k_ord;                  // ordinary top-k over all video tiles
  int n;                      // reference ranges
  int lo[kMaxRefRanges];      // first position of the range in the video-tile list
  int hi[kMaxRefRanges];      // one past its last position
  int q[kMaxRefRanges];       // tiles of the range guaranteed to every query block
};
size_t router_ws_bytes(int n, int H, int D, int bs, bool tail);
RouterWs router_ws_carve(void* ws, int n, int H, int D, int bs, bool tail);
int router_max_blocks();
// guide_protected: Heavy reference protection (every block holding a guide row is
// protected); rq: Light reference quota, or null.
hipError_t launch_router(const void* q, const void* k, const void* v, bool bf16, int n, int H,
                         int D, int bs, const uint8_t* seg, int prefix, int k_sel,
                         int32_t* tiles, int32_t* prot, int prot_cap, const RouterWs& w,
                         float scale, float* tail_lse, float* tail_v, hipStream_t s,
                         bool guide_protected = false, const RefQuota* rq = nullptr);

// LSE merge and accumulator finalisation.
hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_i, const float* lse_i,
                            float log_w, const float* log_w_rows, int64_t pairs, int D,
                            hipStream_t s);
hipError_t launch_fill(float* o_acc, float* lse_acc, int64_t pairs, int D, hipStream_t s);
hipError_t launch_finalize(const float* o_acc, const float* lse_acc, void* o, int o_f32,
                           float* lse, int64_t pairs, int D, hipStream_t s);

}  // namespace h3
