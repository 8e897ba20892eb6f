// C entry points of libh3attn: argument checks, workspace layout, launch dispatch, and
// the host-side plan of the positive-partition ("via") path.
//
// Every check runs before the first HIP call, so a rejected call never touches the
// device. Kernels run on the caller's stream; nothing here synchronises.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/h3attn.h"
#include "h3_internal.h"

using namespace h3;

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool finite(float x) { return std::isfinite(x); }

int check_tara(float strength, float window, float falloff, float cap, float scale) {
  if (!finite(strength) || !finite(window) || !finite(falloff) || !finite(cap) || !finite(scale))
    return H3_EINVAL;
  if (strength < 0.f || window < 0.f || cap < 0.f || !(falloff > 0.f) || !(scale > 0.f))
    return H3_EINVAL;
  return H3_OK;
}

bool dtype_ok(int dt) { return dt == H3_DTYPE_F32 || dt == H3_DTYPE_BF16; }
// bf16 key sets: the transposed v copy is read through 32-bit buffer offsets
constexpr int kMaxBf16Keys = 1 << 23;
bool dim_ok(int d) { return d == 64 || d == 128; }
bool bs_ok(int bs) { return bs == 32 || bs == 64 || bs == 128; }
// Sequences the router and the block-sparse kernels take: at most kMaxBlocks blocks of
// the routing size and at most kMaxBlocks 64-row tiles.
bool blocks_ok(int n, int bs) {
  return (n + bs - 1) / bs <= kMaxBlocks && (n + kTile - 1) / kTile <= kMaxBlocks;
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Failure injection for the callers' dense fallback: H3ATTN_FORCE_FAIL holds a comma-
// separated list of call families ("dense", "router", "sparse"). Their entry points then
// return H3_EFORCED after the argument checks and before any HIP call. Read on every
// call, so a caller can switch it on and off at run time.
bool force_fail(const char* family) {
  const char* e = std::getenv("H3ATTN_FORCE_FAIL");
  if (!e) return false;
  const size_t n = std::strlen(family);
  for (const char* p = e;;) {
    const char* c = std::strchr(p, ',');
    const size_t len = c ? (size_t)(c - p) : std::strlen(p);
    if (len == n && std::strncmp(p, family, n) == 0) return true;
    if (!c) return false;
    p = c + 1;
  }
}

size_t vt_bytes(int nk, int heads, int head_dim) {
  return (size_t)pad_keys(nk) * (size_t)heads * (size_t)head_dim * sizeof(uint16_t);
}

// bf16 attention workspace: the transposed v copy, then the per-tile key summary.
size_t attn_ws_bytes(int nk, int heads, int head_dim) {
  return align256(vt_bytes(nk, heads, head_dim)) + align256((size_t)pad_keys(nk) / kTile * sizeof(TileInfo));
}

// int8 QK workspace after the attention workspace: q8, k8 [n][heads][head_dim] int8 and
// their scales [n][heads] float32, each 256-byte aligned.
size_t int8_ws_bytes(int n, int heads, int head_dim) {
  const size_t e = (size_t)n * heads * head_dim, p = (size_t)n * heads;
  return 2 * align256(e) + 2 * align256(p * sizeof(float));
}

AttnArgs make_args(const void* q, const void* k, const void* v, int nq, int nk, int heads,
                   const uint8_t* q_seg, const float* q_t, const uint8_t* k_seg,
                   const float* k_t, float strength, float window, float falloff, float cap,
                   float scale, void* o, int o_dtype, float* lse) {
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.vt = nullptr; a.tinfo = nullptr;
  a.q_seg = q_seg; a.q_t = q_t; a.k_seg = k_seg; a.k_t = k_t;
  a.o = o; a.lse = lse;
  a.nq = nq; a.nk = nk; a.nkp = (int)pad_keys(nk); a.H = heads;
  a.o_f32 = (o_dtype == H3_DTYPE_F32);
  a.scale = scale;
  a.strength = strength; a.window = window; a.inv_falloff = 1.f / falloff; a.cap = cap;
  a.prot = nullptr; a.n_prot = 0; a.tiles = nullptr; a.k_sel = 0; a.nqb = 0;
  a.bs = kTile; a.sink_mask = 0u;
  a.tail_lse = nullptr; a.tail_v = nullptr;
  a.q8 = nullptr; a.qsc = nullptr; a.k8 = nullptr; a.ksc = nullptr;
  return a;
}

// Fills a bf16 attention workspace for the keys of `a`: the transposed v copy and the
// per-tile key summary.
hipError_t prepare_keys(const AttnArgs& a, int head_dim, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  hipError_t e = launch_vt_transpose((const uint16_t*)a.v, (uint16_t*)w, a.nk, a.H, head_dim, s);
  if (e != hipSuccess) return e;
  return launch_tile_info(a.k_seg, a.k_t, a.nk,
                          (TileInfo*)(w + align256(vt_bytes(a.nk, a.H, head_dim))), s);
}

// One attention launch over (queries, keys); the bf16 path first prepares the key
// workspace unless `ready` says it already holds these keys.
hipError_t run_attention(AttnArgs a, int dtype, int head_dim, bool sparse, bool penalty,
                         void* ws, bool ready, hipStream_t s) {
  if (dtype == H3_DTYPE_BF16) {
    if (!ready) {
      hipError_t e = prepare_keys(a, head_dim, ws, s);
      if (e != hipSuccess) return e;
    }
    a.vt = (const uint16_t*)ws;
    a.tinfo = (const TileInfo*)((const char*)ws + align256(vt_bytes(a.nk, a.H, head_dim)));
    return launch_attn_bf16(a, head_dim, sparse, penalty, s);
  }
  return launch_attn_f32(a, head_dim, sparse, penalty, s);
}

// ------------------------------------------------------------- partition plan
struct Run { int a, b; };
struct Frame { int a, b; float t; };

std::vector<Run> runs_where(const uint8_t* seg, int n, bool (*pred)(uint8_t)) {
  std::vector<Run> out;
  int i = 0;
  while (i < n) {
    if (pred(seg[i])) {
      int j = i;
      while (j < n && pred(seg[j])) ++j;
      out.push_back({i, j});
      i = j;
    } else {
      ++i;
    }
  }
  return out;
}

bool is_output(uint8_t s) { return s == H3_SEG_OUTPUT; }
bool not_output(uint8_t s) { return s != H3_SEG_OUTPUT; }
bool is_guide(uint8_t s) { return s == H3_SEG_GUIDE; }
bool not_guide(uint8_t s) { return s != H3_SEG_GUIDE; }

// Frames: maximal runs of equal timestamp inside the runs of one segment kind.
std::vector<Frame> frames_of(const uint8_t* seg, const float* t, int n, bool (*pred)(uint8_t)) {
  std::vector<Frame> out;
  for (const Run& r : runs_where(seg, n, pred)) {
    int s = r.a;
    for (int i = r.a + 1; i <= r.b; ++i) {
      if (i == r.b || t[i] != t[s]) {
        out.push_back({s, i, t[s]});
        s = i;
      }
    }
  }
  return out;
}

struct ViaPlan {
  std::vector<Run> nonout_q, out_q, nonguide_k, guide_k;
  std::vector<Frame> guide_f, out_f;
  std::vector<Run> vt_ranges;       // key ranges with their own transposed v copy
  std::vector<size_t> vt_off;       // byte offsets in the workspace
  size_t acc_off = 0, acc_lse_off = 0, part_off = 0, part_lse_off = 0, total = 0;
  int max_out_rows = 0;
};

ViaPlan make_plan(const uint8_t* seg, const float* t, int n, int heads, int head_dim,
                  int dtype) {
  ViaPlan p;
  p.nonout_q = runs_where(seg, n, not_output);
  p.out_q = runs_where(seg, n, is_output);
  p.nonguide_k = runs_where(seg, n, not_guide);
  p.guide_k = runs_where(seg, n, is_guide);
  p.guide_f = frames_of(seg, t, n, is_guide);
  p.out_f = frames_of(seg, t, n, is_output);
  p.vt_ranges.push_back({0, n});
  for (const Run& r : p.nonguide_k) p.vt_ranges.push_back(r);
  for (const Run& r : p.guide_k) p.vt_ranges.push_back(r);
  for (const Frame& f : p.guide_f) p.vt_ranges.push_back({f.a, f.b});
  size_t off = 0;
  if (dtype == H3_DTYPE_BF16) {
    for (const Run& r : p.vt_ranges) {
      p.vt_off.push_back(off);
      off += attn_ws_bytes(r.b - r.a, heads, head_dim);
    }
  }
  for (const Run& r : p.out_q) p.max_out_rows = std::max(p.max_out_rows, r.b - r.a);
  const size_t pairs = (size_t)p.max_out_rows * heads;
  p.acc_off = off;
  off += align256(pairs * head_dim * sizeof(float));
  p.acc_lse_off = off;
  off += align256(pairs * sizeof(float));
  p.part_off = off;
  off += align256(pairs * head_dim * sizeof(float));
  p.part_lse_off = off;
  off += align256(pairs * sizeof(float));
  p.total = off;
  return p;
}

// make_plan without exceptions: false when host memory for the plan cannot be allocated
// (no exception may cross the C boundary).
bool plan_nothrow(const uint8_t* seg, const float* t, int n, int heads, int head_dim, int dtype,
                  ViaPlan& out) noexcept {
  try {
    out = make_plan(seg, t, n, heads, head_dim, dtype);
    return true;
  } catch (...) {
    return false;
  }
}

int vt_slot(const ViaPlan& p, int a, int b) {
  for (size_t i = 0; i < p.vt_ranges.size(); ++i)
    if (p.vt_ranges[i].a == a && p.vt_ranges[i].b == b) return (int)i;
  return -1;
}

double host_penalty(double dt, double strength, double window, double falloff, double cap) {
  const double x = std::max(dt - window, 0.0) / falloff;
  return std::min(strength * x * x, cap);
}

}  // namespace

extern "C" {

int h3attn_version(void) { return kVersion; }

const char* h3attn_status_string(int status) {
  switch (status) {
    case H3_OK: return "ok";
    case H3_EINVAL: return "invalid argument";
    case H3_EUNSUPPORTED: return "unsupported dtype, head_dim or block_size";
    case H3_ELAUNCH: return "kernel launch failed";
    case H3_EWORKSPACE: return "workspace missing or too small";
    case H3_ENOMEM: return "host memory for the call plan could not be allocated";
    case H3_EFORCED: return "failure forced by H3ATTN_FORCE_FAIL";
    case H3_ESCRATCH: return "problem larger than the static scratch of the call";
    default: return "unknown status";
  }
}

size_t attn_dense_tara_workspace(int nk, int heads, int head_dim, int dtype) {
  if (nk <= 0 || heads <= 0 || !dim_ok(head_dim) || dtype != H3_DTYPE_BF16) return 0;
  return attn_ws_bytes(nk, heads, head_dim);
}

int attn_dense_tara(const void* q, const void* k, const void* v, int dtype, int nq, int nk,
                    int heads, int head_dim, const uint8_t* q_seg, const float* q_t,
                    const uint8_t* k_seg, const float* k_t, float strength, float window,
                    float falloff, float cap, float scale, void* o, int o_dtype, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !q_seg || !q_t || !k_seg || !k_t || !o || !lse) return H3_EINVAL;
  if (nq <= 0 || nk <= 0 || heads <= 0) return H3_EINVAL;
  if (int st = check_tara(strength, window, falloff, cap, scale)) return st;
  if (!dtype_ok(dtype) || !dtype_ok(o_dtype) || !dim_ok(head_dim) || heads > 65535)
    return H3_EUNSUPPORTED;
  if (dtype == H3_DTYPE_BF16 && nk > kMaxBf16Keys) return H3_EUNSUPPORTED;
  const size_t need = attn_dense_tara_workspace(nk, heads, head_dim, dtype);
  if (need && (!ws || ws_bytes < need)) return H3_EWORKSPACE;
  if (force_fail("dense")) return H3_EFORCED;
  AttnArgs a = make_args(q, k, v, nq, nk, heads, q_seg, q_t, k_seg, k_t, strength, window,
                         falloff, cap, scale, o, o_dtype, lse);
  const bool pen = strength > 0.f && cap > 0.f;
  hipError_t e = run_attention(a, dtype, head_dim, false, pen, ws, false, (hipStream_t)stream);
  return e == hipSuccess ? H3_OK : H3_ELAUNCH;
}

int attn_router_plan(const uint8_t* seg_host, int n, int protected_prefix_len, int block_size,
                     double sparsity_ratio, int* nb, int* n_video, int* n_prot, int* k_sel) {
  if (!seg_host || n <= 0) return H3_EINVAL;
  if (protected_prefix_len < 0 || protected_prefix_len > n) return H3_EINVAL;
  if (!std::isfinite(sparsity_ratio) || sparsity_ratio < 0.0 || sparsity_ratio >= 1.0)
    return H3_EINVAL;
  if (!bs_ok(block_size)) return H3_EUNSUPPORTED;
  const int blocks = (n + block_size - 1) / block_size;
  int prot = 0;
  for (int b = 0; b < blocks; ++b) {
    const int lo = b * block_size, hi = std::min(n, lo + block_size);
    bool p = lo < protected_prefix_len;
    for (int r = lo; r < hi && !p; ++r)
      p = seg_host[r] == H3_SEG_TEXT || seg_host[r] == H3_SEG_AUDIO;
    prot += p ? 1 : 0;
  }
  const int video = blocks - prot;
  int k = 0;
  if (video > 0) {
    if (sparsity_ratio == 0.0) {
      k = video;
    } else {
      k = (int)std::ceil((1.0 - sparsity_ratio) * (double)video - 1e-9);
      k = std::min(video, std::max(1, k));
    }
  }
  if (nb) *nb = blocks;
  if (n_video) *n_video = video;
  if (n_prot) *n_prot = prot;
  if (k_sel) *k_sel = k;
  return H3_OK;
}

}  // extern "C"

namespace {

// Host plan of the routed lists under a reference-protection mode ("H3 SLA Attention",
// inputs table, reference_protection): the protected / candidate counts, the ordinary
// routed count, and for Light the reference ranges (maximal runs of video tiles with
// consecutive block indices holding a guide row) with their positions in the video-tile
// list and guaranteed counts at the fixed reference sparsity 0.85.
constexpr double kLightReferenceSparsity = 0.85;

int select_count(int m, double s) {
  if (m <= 0) return 0;
  if (s == 0.0) return m;
  const int k = (int)std::ceil((1.0 - s) * (double)m - 1e-9);
  return std::min(m, std::max(1, k));
}

struct RefPlan {
  int nb = 0, n_prot = 0, n_cand = 0, k_ord = 0, width = 0, n_ranges = 0;
  RefQuota rq{};
};

// Returns H3_OK, H3_EINVAL or H3_EUNSUPPORTED (block size, mode, or more than
// kMaxRefRanges reference ranges in Light mode).
int plan_ref(const uint8_t* seg, int n, int prefix, int bs, double s, int mode, RefPlan& p) {
  if (!seg || n <= 0 || prefix < 0 || prefix > n) return H3_EINVAL;
  if (!std::isfinite(s) || s < 0.0 || s >= 1.0) return H3_EINVAL;
  if (!bs_ok(bs)) return H3_EUNSUPPORTED;
  if (mode != H3_REF_OFF && mode != H3_REF_LIGHT && mode != H3_REF_HEAVY)
    return H3_EUNSUPPORTED;
  p = RefPlan{};
  p.nb = (n + bs - 1) / bs;
  int vpos = 0, prev_ref = -2;
  for (int b = 0; b < p.nb; ++b) {
    const int lo = b * bs, hi = std::min(n, lo + bs);
    bool text_audio = lo < prefix, guide = false;
    for (int r = lo; r < hi; ++r) {
      text_audio = text_audio || seg[r] == H3_SEG_TEXT || seg[r] == H3_SEG_AUDIO;
      guide = guide || seg[r] == H3_SEG_GUIDE;
    }
    const bool ref = !text_audio && guide;
    if (text_audio || (mode == H3_REF_HEAVY && ref)) {
      ++p.n_prot;
      continue;
    }
    if (mode == H3_REF_LIGHT && ref) {  // a reference range starts or goes on
      if (prev_ref != b - 1) {
        if (p.n_ranges == kMaxRefRanges) return H3_EUNSUPPORTED;
        p.rq.lo[p.n_ranges] = vpos;
        p.rq.hi[p.n_ranges] = vpos;
        ++p.n_ranges;
      }
      ++p.rq.hi[p.n_ranges - 1];
      prev_ref = b;
    }
    ++vpos;
  }
  p.n_cand = vpos;
  p.k_ord = select_count(p.n_cand, s);
  p.width = p.k_ord;
  p.rq.k_ord = p.k_ord;
  p.rq.n = p.n_ranges;
  for (int j = 0; j < p.n_ranges; ++j) {
    p.rq.q[j] = select_count(p.rq.hi[j] - p.rq.lo[j], kLightReferenceSparsity);
    p.width += p.rq.q[j];
  }
  p.width = std::min(p.width, p.n_cand);  // a union never exceeds the candidates
  return H3_OK;
}

}  // namespace

extern "C" {

int attn_router_plan_ref(const uint8_t* seg_host, int n, int protected_prefix_len,
                         int block_size, double sparsity_ratio, int reference_protection,
                         int* nb, int* n_video, int* n_prot, int* k_sel) {
  RefPlan p;
  if (int st = plan_ref(seg_host, n, protected_prefix_len, block_size, sparsity_ratio,
                        reference_protection, p))
    return st;
  if (nb) *nb = p.nb;
  if (n_video) *n_video = p.n_cand;
  if (n_prot) *n_prot = p.n_prot;
  if (k_sel) *k_sel = p.width;
  return H3_OK;
}

size_t attn_block_router_workspace(int n, int heads, int head_dim, int block_size) {
  if (n <= 0 || heads <= 0 || !dim_ok(head_dim) || !bs_ok(block_size)) return 0;
  return router_ws_bytes(n, heads, head_dim, block_size, false);
}

size_t attn_block_router_tail_workspace(int n, int heads, int head_dim, int block_size) {
  if (n <= 0 || heads <= 0 || !dim_ok(head_dim) || !bs_ok(block_size)) return 0;
  return router_ws_bytes(n, heads, head_dim, block_size, true);
}

}  // extern "C"

namespace {

// ------------------------------------------------------------- static scratch
// Scratch of attn_block_router_static: a file-scope device array; every GPU the library
// runs on holds its own copy until the process ends. In host code the array's name is
// only a host-side handle, so host code never passes it to a kernel or a copy: it takes
// each device's address of the array from hipGetSymbolAddress (once per device, on the
// entry point's first call there) and passes that address.
static __device__ __align__(256) unsigned char scratch[H3_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// This device's address of `scratch`, or null when the symbol lookup fails. Concurrent
// first calls on one device look it up twice and store the same address.
void* scratch_address() {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

int route(const void* q, const void* k, const void* v, int dtype, int n, int heads,
          int head_dim, const uint8_t* seg, int protected_prefix_len, int block_size, int k_sel,
          int32_t* tiles, int32_t* prot, int n_prot, bool tail, float scale, float* tail_lse,
          float* tail_v, void* ws, size_t ws_bytes, void* stream,
          bool guide_protected = false, const RefQuota* rq = nullptr,
          bool static_scratch = false) {
  if (!q || !k || !seg || n <= 0 || heads <= 0) return H3_EINVAL;
  if (tail && (!v || !tail_lse || !tail_v || !std::isfinite(scale) || !(scale > 0.f)))
    return H3_EINVAL;
  if (protected_prefix_len < 0 || protected_prefix_len > n) return H3_EINVAL;
  if (k_sel < 0 || n_prot < 0 || (k_sel > 0 && !tiles) || (n_prot > 0 && !prot))
    return H3_EINVAL;
  if (!dtype_ok(dtype) || !dim_ok(head_dim) || !bs_ok(block_size) || heads > 65535)
    return H3_EUNSUPPORTED;
  const int nb = (n + block_size - 1) / block_size;
  if (k_sel > nb) return H3_EINVAL;
  if (!blocks_ok(n, block_size) || nb > router_max_blocks()) return H3_EUNSUPPORTED;
  const size_t need = router_ws_bytes(n, heads, head_dim, block_size, tail);
  if (static_scratch) {
    if (need > (size_t)H3_STATIC_SCRATCH_BYTES) return H3_ESCRATCH;
  } else if (!ws || ws_bytes < need) {
    return H3_EWORKSPACE;
  }
  if (force_fail("router")) return H3_EFORCED;
  if (static_scratch) {  // every argument check has passed: the first HIP call
    ws = scratch_address();
    if (!ws) return H3_ELAUNCH;
    ws_bytes = H3_STATIC_SCRATCH_BYTES;
  }
  RouterWs w = router_ws_carve(ws, n, heads, head_dim, block_size, tail);
  hipError_t e = launch_router(q, k, v, dtype == H3_DTYPE_BF16, n, heads, head_dim, block_size,
                               seg, protected_prefix_len, k_sel, tiles, prot, n_prot, w, scale,
                               tail ? tail_lse : nullptr, tail ? tail_v : nullptr,
                               (hipStream_t)stream, guide_protected, rq);
  return e == hipSuccess ? H3_OK : H3_ELAUNCH;
}

int sparse(const void* q, const void* k, const void* v, int dtype, int n, int heads,
           int head_dim, const uint8_t* seg, const float* t, float strength, float window,
           float falloff, float cap, float scale, int block_size, const int32_t* tiles,
           int k_sel, const int32_t* prot, int n_prot, const float* tail_lse,
           const float* tail_v, uint32_t sink_mask, bool int8qk, void* o, int o_dtype,
           float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !seg || !t || !o || !lse) return H3_EINVAL;
  if (n <= 0 || heads <= 0) return H3_EINVAL;
  if (k_sel < 0 || n_prot < 0 || k_sel + n_prot == 0) return H3_EINVAL;
  if ((k_sel > 0 && !tiles) || (n_prot > 0 && !prot)) return H3_EINVAL;
  if (int st = check_tara(strength, window, falloff, cap, scale)) return st;
  if (sink_mask & ~0xFu) return H3_EINVAL;  // segment ids are 0..3
  if (!dtype_ok(dtype) || !dtype_ok(o_dtype) || !dim_ok(head_dim) || !bs_ok(block_size) ||
      heads > 65535)
    return H3_EUNSUPPORTED;
  if (!blocks_ok(n, block_size)) return H3_EUNSUPPORTED;
  if (int8qk && (dtype != H3_DTYPE_BF16 || block_size == 32)) return H3_EUNSUPPORTED;
  const size_t base = attn_dense_tara_workspace(n, heads, head_dim, dtype);
  const size_t need = base + (int8qk ? int8_ws_bytes(n, heads, head_dim) : 0);
  if (need && (!ws || ws_bytes < need)) return H3_EWORKSPACE;
  if (force_fail("sparse")) return H3_EFORCED;
  AttnArgs a = make_args(q, k, v, n, n, heads, seg, t, seg, t, strength, window, falloff, cap,
                         scale, o, o_dtype, lse);
  if (int8qk) {
    const size_t e = (size_t)n * heads * head_dim, p = (size_t)n * heads;
    char* w = (char*)ws + base;
    int8_t* q8 = (int8_t*)w;
    int8_t* k8 = (int8_t*)(w + align256(e));
    float* qsc = (float*)(w + 2 * align256(e));
    float* ksc = (float*)(w + 2 * align256(e) + align256(p * sizeof(float)));
    hipError_t e1 = launch_quant_int8(q, true, (int64_t)p, head_dim, q8, qsc, (hipStream_t)stream);
    if (e1 == hipSuccess)
      e1 = launch_quant_int8(k, true, (int64_t)p, head_dim, k8, ksc, (hipStream_t)stream);
    if (e1 != hipSuccess) return H3_ELAUNCH;
    a.q8 = q8; a.qsc = qsc; a.k8 = k8; a.ksc = ksc;
  }
  a.prot = prot;
  a.n_prot = n_prot;
  a.tiles = tiles;
  a.k_sel = k_sel;
  a.nqb = (n + block_size - 1) / block_size;
  a.bs = block_size;
  a.sink_mask = sink_mask;
  a.tail_lse = tail_lse;
  a.tail_v = tail_v;
  const bool pen = strength > 0.f && cap > 0.f;
  hipError_t e = run_attention(a, dtype, head_dim, true, pen, ws, false, (hipStream_t)stream);
  return e == hipSuccess ? H3_OK : H3_ELAUNCH;
}

}  // namespace

extern "C" {

int attn_block_router(const void* q, const void* k, int dtype, int n, int heads, int head_dim,
                      const uint8_t* seg, int protected_prefix_len, int block_size, int k_sel,
                      int32_t* tiles, int32_t* prot, int n_prot, void* ws, size_t ws_bytes,
                      void* stream) {
  return route(q, k, nullptr, dtype, n, heads, head_dim, seg, protected_prefix_len, block_size,
               k_sel, tiles, prot, n_prot, false, 0.f, nullptr, nullptr, ws, ws_bytes, stream);
}

int attn_block_router_static(const void* q, const void* k, int dtype, int n, int heads,
                             int head_dim, const uint8_t* seg, int protected_prefix_len,
                             int block_size, int k_sel, int32_t* tiles, int32_t* prot,
                             int n_prot, void* stream) {
  return route(q, k, nullptr, dtype, n, heads, head_dim, seg, protected_prefix_len, block_size,
               k_sel, tiles, prot, n_prot, false, 0.f, nullptr, nullptr, nullptr, 0, stream,
               false, nullptr, true);
}

int attn_block_router_tail(const void* q, const void* k, const void* v, int dtype, int n,
                           int heads, int head_dim, const uint8_t* seg, int protected_prefix_len,
                           int block_size, int k_sel, float scale, int32_t* tiles, int32_t* prot,
                           int n_prot, float* tail_lse, float* tail_v, void* ws, size_t ws_bytes,
                           void* stream) {
  return route(q, k, v, dtype, n, heads, head_dim, seg, protected_prefix_len, block_size, k_sel,
               tiles, prot, n_prot, true, scale, tail_lse, tail_v, ws, ws_bytes, stream);
}

int attn_block_router_ref(const void* q, const void* k, int dtype, int n, int heads,
                          int head_dim, const uint8_t* seg, const uint8_t* seg_host,
                          int protected_prefix_len, int block_size, double sparsity_ratio,
                          int reference_protection, int k_sel, int32_t* tiles, int32_t* prot,
                          int n_prot, void* ws, size_t ws_bytes, void* stream) {
  if (!seg_host) return H3_EINVAL;
  RefPlan p;
  if (int st = plan_ref(seg_host, n, protected_prefix_len, block_size, sparsity_ratio,
                        reference_protection, p))
    return st;
  if (k_sel != p.width) return H3_EINVAL;  // the list width of this plan, no truncation
  const bool light = reference_protection == H3_REF_LIGHT;
  return route(q, k, nullptr, dtype, n, heads, head_dim, seg, protected_prefix_len, block_size,
               k_sel, tiles, prot, n_prot, false, 0.f, nullptr, nullptr, ws, ws_bytes, stream,
               reference_protection == H3_REF_HEAVY, light ? &p.rq : nullptr);
}

size_t attn_block_sparse_workspace(int n, int heads, int head_dim, int dtype) {
  return attn_dense_tara_workspace(n, heads, head_dim, dtype);
}

int attn_block_sparse(const void* q, const void* k, const void* v, int dtype, int n, int heads,
                      int head_dim, const uint8_t* seg, const float* t, float strength,
                      float window, float falloff, float cap, float scale, int block_size,
                      const int32_t* tiles, int k_sel, const int32_t* prot, int n_prot, void* o,
                      int o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return sparse(q, k, v, dtype, n, heads, head_dim, seg, t, strength, window, falloff, cap,
                scale, block_size, tiles, k_sel, prot, n_prot, nullptr, nullptr, 0u, false, o,
                o_dtype, lse, ws, ws_bytes, stream);
}

int attn_block_sparse_tail(const void* q, const void* k, const void* v, int dtype, int n,
                           int heads, int head_dim, const uint8_t* seg, const float* t,
                           float strength, float window, float falloff, float cap, float scale,
                           int block_size, const int32_t* tiles, int k_sel, const int32_t* prot,
                           int n_prot, const float* tail_lse, const float* tail_v, void* o,
                           int o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!tail_lse || !tail_v) return H3_EINVAL;
  return sparse(q, k, v, dtype, n, heads, head_dim, seg, t, strength, window, falloff, cap,
                scale, block_size, tiles, k_sel, prot, n_prot, tail_lse, tail_v, 0u, false, o,
                o_dtype, lse, ws, ws_bytes, stream);
}

int attn_block_sparse_sinks(const void* q, const void* k, const void* v, int dtype, int n,
                            int heads, int head_dim, const uint8_t* seg, const float* t,
                            float strength, float window, float falloff, float cap, float scale,
                            int block_size, const int32_t* tiles, int k_sel,
                            const int32_t* prot, int n_prot, const float* tail_lse,
                            const float* tail_v, unsigned sink_segments, void* o, int o_dtype,
                            float* lse, void* ws, size_t ws_bytes, void* stream) {
  if ((tail_lse == nullptr) != (tail_v == nullptr)) return H3_EINVAL;
  return sparse(q, k, v, dtype, n, heads, head_dim, seg, t, strength, window, falloff, cap,
                scale, block_size, tiles, k_sel, prot, n_prot, tail_lse, tail_v,
                (uint32_t)sink_segments, false, o, o_dtype, lse, ws, ws_bytes, stream);
}

size_t attn_block_sparse_int8qk_workspace(int n, int heads, int head_dim) {
  if (n <= 0 || heads <= 0 || !dim_ok(head_dim)) return 0;
  return attn_ws_bytes(n, heads, head_dim) + int8_ws_bytes(n, heads, head_dim);
}

int attn_block_sparse_int8qk(const void* q, const void* k, const void* v, int dtype, int n,
                             int heads, int head_dim, const uint8_t* seg, const float* t,
                             float strength, float window, float falloff, float cap,
                             float scale, int block_size, const int32_t* tiles, int k_sel,
                             const int32_t* prot, int n_prot, const float* tail_lse,
                             const float* tail_v, unsigned sink_segments, void* o, int o_dtype,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
  if ((tail_lse == nullptr) != (tail_v == nullptr)) return H3_EINVAL;
  return sparse(q, k, v, dtype, n, heads, head_dim, seg, t, strength, window, falloff, cap,
                scale, block_size, tiles, k_sel, prot, n_prot, tail_lse, tail_v,
                (uint32_t)sink_segments, true, o, o_dtype, lse, ws, ws_bytes, stream);
}

int attn_quantize_int8(const void* x, int dtype, int rows, int heads, int head_dim, int8_t* x8,
                       float* scales, void* stream) {
  if (!x || !x8 || !scales || rows <= 0 || heads <= 0) return H3_EINVAL;
  if (!dtype_ok(dtype) || !dim_ok(head_dim)) return H3_EUNSUPPORTED;
  hipError_t e = launch_quant_int8(x, dtype == H3_DTYPE_BF16, (int64_t)rows * heads, head_dim,
                                   x8, scales, (hipStream_t)stream);
  return e == hipSuccess ? H3_OK : H3_ELAUNCH;
}

int partition_lse_merge(float* o_acc, float* lse_acc, const float* o_i, const float* lse_i,
                        float log_w, const float* log_w_rows, int rows, int heads, int head_dim,
                        void* stream) {
  if (!o_acc || !lse_acc || !o_i || !lse_i || rows <= 0 || heads <= 0) return H3_EINVAL;
  if (std::isnan(log_w) || log_w == INFINITY) return H3_EINVAL;
  if (!dim_ok(head_dim)) return H3_EUNSUPPORTED;
  if (log_w == -INFINITY) return H3_OK;
  hipError_t e = launch_lse_merge(o_acc, lse_acc, o_i, lse_i, log_w, log_w_rows,
                                  (int64_t)rows * heads, head_dim, (hipStream_t)stream);
  return e == hipSuccess ? H3_OK : H3_ELAUNCH;
}

size_t attn_dense_tara_via_workspace(const uint8_t* seg_host, const float* t_host, int n,
                                     int heads, int head_dim, int dtype) {
  if (!seg_host || !t_host || n <= 0 || heads <= 0 || !dim_ok(head_dim) || !dtype_ok(dtype))
    return 0;
  ViaPlan p;
  return plan_nothrow(seg_host, t_host, n, heads, head_dim, dtype, p) ? p.total : 0;
}

int attn_dense_tara_via(const void* q, const void* k, const void* v, int dtype, int n, int heads,
                        int head_dim, const uint8_t* seg, const float* t,
                        const uint8_t* seg_host, const float* t_host, float strength,
                        float window, float falloff, float cap, float scale, void* o,
                        int o_dtype, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !seg || !t || !seg_host || !t_host || !o || !lse) return H3_EINVAL;
  if (n <= 0 || heads <= 0) return H3_EINVAL;
  if (int st = check_tara(strength, window, falloff, cap, scale)) return st;
  if (!dtype_ok(dtype) || !dtype_ok(o_dtype) || !dim_ok(head_dim) || heads > 65535)
    return H3_EUNSUPPORTED;
  if (dtype == H3_DTYPE_BF16 && n > kMaxBf16Keys) return H3_EUNSUPPORTED;
  ViaPlan p;
  if (!plan_nothrow(seg_host, t_host, n, heads, head_dim, dtype, p)) return H3_ENOMEM;
  if (!ws || ws_bytes < p.total) return H3_EWORKSPACE;
  if (force_fail("dense")) return H3_EFORCED;

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  const int D = head_dim;
  const size_t esz = dtype == H3_DTYPE_BF16 ? 2 : 4;
  const size_t row_elems = (size_t)heads * D;
  auto qrow = [&](int r) { return (const char*)q + (size_t)r * row_elems * esz; };
  auto krow = [&](int r) { return (const char*)k + (size_t)r * row_elems * esz; };
  auto vrow = [&](int r) { return (const char*)v + (size_t)r * row_elems * esz; };
  float* acc = (float*)(w + p.acc_off);
  float* acc_lse = (float*)(w + p.acc_lse_off);
  float* part = (float*)(w + p.part_off);
  float* part_lse = (float*)(w + p.part_lse_off);

  // Key workspaces (transposed v copy + tile summary), one per key range used below.
  if (dtype == H3_DTYPE_BF16) {
    for (size_t i = 0; i < p.vt_ranges.size(); ++i) {
      const Run& r = p.vt_ranges[i];
      AttnArgs ka = make_args(qrow(r.a), krow(r.a), vrow(r.a), r.b - r.a, r.b - r.a, heads,
                              seg + r.a, t + r.a, seg + r.a, t + r.a, 0.f, window, falloff,
                              cap, scale, nullptr, H3_DTYPE_F32, nullptr);
      if (prepare_keys(ka, D, w + p.vt_off[i], s) != hipSuccess) return H3_ELAUNCH;
    }
  }
  // Ordinary attention of query rows [qa, qb) over key rows [ka, kb) into (out, out_lse).
  auto call = [&](int qa, int qb, int ka, int kb, void* out, int out_dtype,
                  float* out_lse) -> bool {
    AttnArgs a = make_args(qrow(qa), krow(ka), vrow(ka), qb - qa, kb - ka, heads, seg + qa,
                           t + qa, seg + ka, t + ka, 0.f, window, falloff, cap, scale, out,
                           out_dtype, out_lse);
    void* kws = nullptr;
    if (dtype == H3_DTYPE_BF16) {
      const int slot = vt_slot(p, ka, kb);
      if (slot < 0) return false;
      kws = w + p.vt_off[slot];
    }
    return run_attention(a, dtype, D, false, false, kws, true, s) == hipSuccess;
  };

  // Queries outside the output video: one ordinary call over every key.
  for (const Run& r : p.nonout_q) {
    float* l = lse + (size_t)r.a * heads;
    void* out = (char*)o + (size_t)r.a * row_elems * (o_dtype == H3_DTYPE_BF16 ? 2 : 4);
    if (!call(r.a, r.b, 0, n, out, o_dtype, l)) return H3_ELAUNCH;
  }
  const double base = -(double)cap;  // log of the uniform guide multiplier exp(-cap)
  for (const Run& r : p.out_q) {
    const int rows = r.b - r.a;
    const int64_t pairs = (int64_t)rows * heads;
    if (launch_fill(acc, acc_lse, pairs, D, s) != hipSuccess) return H3_ELAUNCH;
    auto merge = [&](int row0, int nrows, double log_w) -> bool {
      return launch_lse_merge(acc + (size_t)row0 * row_elems, acc_lse + (size_t)row0 * heads,
                              part, part_lse, (float)log_w, nullptr,
                              (int64_t)nrows * heads, D, s) == hipSuccess;
    };
    for (const Run& kr : p.nonguide_k) {
      if (!call(r.a, r.b, kr.a, kr.b, part, H3_DTYPE_F32, part_lse)) return H3_ELAUNCH;
      if (!merge(0, rows, 0.0)) return H3_ELAUNCH;
    }
    for (const Run& kr : p.guide_k) {
      if (!call(r.a, r.b, kr.a, kr.b, part, H3_DTYPE_F32, part_lse)) return H3_ELAUNCH;
      if (!merge(0, rows, base)) return H3_ELAUNCH;
    }
    for (const Frame& f : p.out_f) {
      if (f.a < r.a || f.b > r.b) continue;
      for (const Frame& g : p.guide_f) {
        const double pen = host_penalty(std::fabs((double)f.t - (double)g.t), strength, window,
                                        falloff, cap);
        const double corr = std::expm1((double)cap - pen);  // exp(-p) - exp(-cap), / exp(-cap)
        if (!(corr > 0.0)) continue;                        // zero-weight correction
        if (!call(f.a, f.b, g.a, g.b, part, H3_DTYPE_F32, part_lse)) return H3_ELAUNCH;
        if (!merge(f.a - r.a, f.b - f.a, base + std::log(corr))) return H3_ELAUNCH;
      }
    }
    void* out = (char*)o + (size_t)r.a * row_elems * (o_dtype == H3_DTYPE_BF16 ? 2 : 4);
    if (launch_finalize(acc, acc_lse, out, o_dtype == H3_DTYPE_F32,
                        lse + (size_t)r.a * heads, pairs, D, s) != hipSuccess)
      return H3_ELAUNCH;
  }
  return H3_OK;
}

}  // extern "C"
