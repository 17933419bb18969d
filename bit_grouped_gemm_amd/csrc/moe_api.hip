// moe_api.hip -- the C ABI declared in include/moe.h: argument checks, shape
// heuristics, workspace carve-up and the launch sequence.  Host code only;
// the kernels live in moe_kernels.hip.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <utility>

#include "../../include/moe.h"
#include "moe_launch.h"

namespace moe {

// Split-K targets about one workgroup per CU, keeping at least four K steps
// of 128 per workgroup.
constexpr long kSplitTargetWG = 256;
constexpr int kSplitMinKSteps = 4;
// average rows per touched group from which the many-row kernels take over
// (measured cold-cache crossovers, H=4096 E=64 top-8: e4m3 between 12 and 16
// rows, MXFP4 between 16 and 24)
constexpr double kBigMinAvgRowsFp8 = 14.0;
constexpr double kBigMinAvgRowsFp4 = 20.0;
// decode passes hold the mean row count of a touched group plus this many
// standard deviations of a Poisson count
constexpr double kNttSigmas = 3.0;

static int choose_split(long units, int nks, long target = kSplitTargetWG) {
  // Split K (a divisor of the K-step count) only until the launch has about
  // one workgroup per CU: small decode layers then reach every CU, while
  // larger ones avoid the partial-sum round trip through memory, which costs
  // more than the tail of a half-filled last round.  Each workgroup keeps at
  // least kSplitMinKSteps steps of 128 K.
  int best = 1;
  for (int d = 1; d <= nks; ++d) {
    if (nks % d) continue;
    if (nks / d < kSplitMinKSteps) break;
    best = d;
    if (units * d >= target) break;
  }
  return best;
}

static int choose_ntt(int T, int k, int E) {
  const double rows = double(T) * k;
  const double groups = std::fmin(double(E), rows);
  if (groups <= 0) return 1;
  const double avg = rows / groups;
  const double est = avg + kNttSigmas * std::sqrt(avg) + 1.0;
  return est <= 16 ? 1 : (est <= 32 ? 2 : 4);
}

// Upper bound on the decode GEMMs' work items, sum over non-empty groups of
// ceil(n_g / R): with N rows in at most Gn groups each group adds at most
// (n_g + R - 1) / R, and every item holds a row.
static int items_bound(long N, long Gn, int R) {
  if (N <= 0 || Gn <= 0) return 0;
  return int(std::min(N, (N + Gn * (R - 1)) / R));
}

Shape make_shape(int T, int H, int I, int E, int k, int wfmt, int wblk, int G, int shared, int af) {
  Shape s{};
  s.T = T; s.H = H; s.I = I; s.E = E; s.k = k; s.wfmt = wfmt; s.wblk = wblk; s.G = G; s.shared = shared;
  s.af = af;
  s.ngroups = E + shared;
  s.rows_cap = T * k + T * shared;
  s.slots_max = (T > 0) ? (std::min(E, T * k) + shared) : 0;
  s.g1_tiles = I / 128;
  s.g1_ntt = s.g2_ntt = choose_ntt(T, k, E);
  // four weight tiles per wave (256-row units) once a pass holds two or more
  // token tiles; with one token tile the smaller units keep more waves busy
  // (measured cold-cache: T = 64 layers 2-8 % faster, T <= 32 1-3 % slower)
  s.g2_nj = (H % 256 == 0 && s.g2_ntt >= 2) ? 4 : 2;
  // MXFP4 weights carry half the bytes per tile: twice the tiles per wave
  // keep as many bytes in flight, while the launch still has a unit per CU
  // (measured cold-cache, H=4096 E=64 top-8 I=1536: GEMM2 -1 to -4.5 us at
  // T = 8..128; at T = 1 the halved unit count costs 4 us, so not there)
  if (wfmt == 1 && H % (128 * s.g2_nj) == 0 &&
      long(s.slots_max) * (H / (128 * s.g2_nj)) >= kSplitTargetWG)
    s.g2_nj *= 2;
  s.g2_tiles = H / (64 * s.g2_nj);
  s.g1_items = items_bound(s.rows_cap, s.slots_max, 16 * s.g1_ntt);
  s.g2_items = items_bound(s.rows_cap, s.slots_max, 16 * s.g2_ntt);
  s.g1_split = choose_split(long(s.slots_max) * s.g1_tiles, H / 128);
  s.g2_split = choose_split(long(s.slots_max) * s.g2_tiles, I / 128);
  // partial sums are addressed with 32-bit byte offsets: keep them under 2 GiB
  auto fit = [&](int S, int nks, long row_floats) {
    while (S > 1 && 4L * S * s.rows_cap * row_floats >= (1L << 31)) {
      int d = S - 1;
      while (d > 1 && nks % d) --d;
      S = d;
    }
    return S;
  };
  s.g1_split = fit(s.g1_split, H / 128, 2L * I);
  s.g2_split = fit(s.g2_split, I / 128, H);
  // Big-tile kernels once experts hold enough rows that one pass of up to
  // 160 (or 64) token rows per 256 weight rows beats the decode kernel's
  // 16..64-row passes; they need 128-wide activation groups (one MFMA K step
  // per scale), 128x128 e4m3 blocks or MXFP4, and H a multiple of 256.
  const double groups = std::fmin(double(E), double(T) * k);
  const double avg_rows = groups > 0 ? double(T) * k / groups : 0.0;
  // the big-tile kernels keep a pass's token scales in LDS: K <= 8192 for both GEMMs
  const double min_rows = wfmt != 0 ? kBigMinAvgRowsFp4 : kBigMinAvgRowsFp8;
  s.big = (G == 128 && (wfmt != 0 || wblk == 128) && H % 256 == 0 && H <= 8192 && I <= 8192 &&
           avg_rows >= min_rows) ? 1 : 0;
  if (af == 1) s.big = 1;  // 4-bit activations run the many-row kernels at every T
  // 64 rows per pass while nearly every group fits (mean + 3 sd of a
  // Poisson count), which leaves LDS for a deeper ring; 160 beyond
  s.big_cap = avg_rows + 3.0 * std::sqrt(avg_rows) + 1.0 <= 64.0 ? 64 : 160;
  // NVFP4's fp16 operands leave registers for 96 token rows per pass
  if (wfmt == 2 && s.big_cap == 160) s.big_cap = 96;
  if (s.big) s.g1_split = s.g2_split = 1;
  // permute: one block places up to 4096 slots; beyond that the slots are
  // split into at most 64 chunks of at least 1024, each placed by its own
  // block after a counting pass
  const long n = long(T) * k;
  if (n <= 4096) {
    s.perm_chunk = int(std::max(n, 1L));
    s.perm_chunks = 1;
  } else {
    long chunk = std::max(1024L, (n + 63) / 64);
    chunk = (chunk + 63) / 64 * 64;
    s.perm_chunk = int(chunk);
    s.perm_chunks = int((n + chunk - 1) / chunk);
  }
  return s;
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

WsLayout make_ws_layout(const Shape& s) {
  WsLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + std::max<size_t>(bytes, 1));
    return at;
  };
  const size_t T = size_t(s.T), R = size_t(s.rows_cap);
  L.counts = take(4 * size_t(s.E + 1));
  L.offsets = take(4 * size_t(s.E + 2));
  L.expand_idx = take(4 * T * s.k);
  L.row_token = take(4 * R);
  L.xq = take(T * s.H);
  L.xs = take(4 * T * (s.H / s.G));
  L.hq = take(R * s.I);
  L.hs = take(4 * R * (s.I / s.G));
  L.y = take(4 * R * s.H);
  L.part1 = take(s.g1_split > 1 ? 4 * size_t(s.g1_split) * R * 2 * s.I : 0);
  L.part2 = take(s.g2_split > 1 ? 4 * size_t(s.g2_split) * R * s.H : 0);
  L.chunk_cnt = take(s.perm_chunks > 1 ? 4 * size_t(s.perm_chunks) * s.E : 0);
  // the counter arrays (split-K arrivals, then the persistent layer's
  // control block) are adjacent so one clear covers them all
  L.cnt1 = o;
  L.cnt2 = L.cnt1 + 4 * size_t(s.g1_items) * s.g1_tiles;
  L.pctl = align256(L.cnt2 + 4 * size_t(s.g2_items) * s.g2_tiles);
  o = align256(L.pctl + 4 * (size_t(kPersistCtlHead) + 2 * size_t(s.g1_items)));
  L.total = o;
  return L;
}

}  // namespace moe

using namespace moe;

namespace {

constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0, "scratch size");

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Shape and format checks of a (non-null) cfg.
int check_shape(const moe_cfg* c) {
  if (c->T < 0 || c->H < 1 || c->I < 1 || c->E < 1 || c->topk < 1 || c->topk > c->E) return MOE_ERR_BAD_SHAPE;
  if (c->topk > 32 || c->E > 1024) return MOE_ERR_BAD_SHAPE;
  if (c->H % 128 || c->I % 128) return MOE_ERR_BAD_SHAPE;
  if (int64_t(c->T) * c->topk >= (int64_t(1) << 24)) return MOE_ERR_BAD_SHAPE;
  // activation codes are addressed with 32-bit byte offsets inside the GEMMs
  const int64_t rows = int64_t(c->T) * (c->topk + (c->has_shared ? 1 : 0));
  if (int64_t(c->T) * c->H >= (int64_t(1) << 31) || rows * c->I >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
  if (c->has_shared != 0 && c->has_shared != 1) return MOE_ERR_BAD_SHAPE;
  if (c->wfmt == MOE_WFMT_FP8_BLOCK) {
    if (c->wblk != 32 && c->wblk != 128) return MOE_ERR_UNSUPPORTED;
    if (c->act_group != c->wblk) return MOE_ERR_BAD_SHAPE;
  } else if (c->wfmt == MOE_WFMT_MXFP4) {
    if (c->wblk != 32) return MOE_ERR_BAD_SHAPE;
    if (c->act_fmt == MOE_AFMT_FP8 && c->act_group != 128) return MOE_ERR_UNSUPPORTED;
  } else if (c->wfmt == MOE_WFMT_NVFP4) {
    if (c->wblk != 16) return MOE_ERR_BAD_SHAPE;
    if (c->act_fmt != MOE_AFMT_FP8 || c->act_group != 128) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  if (c->act_fmt == MOE_AFMT_MXFP4) {
    // 4-bit activations: MXFP4 weights, one e8m0 scale per 32 channels, and
    // the many-row kernels (their token-scale table holds K <= 8192)
    if (c->wfmt != MOE_WFMT_MXFP4) return MOE_ERR_UNSUPPORTED;
    if (c->act_group != 32) return MOE_ERR_BAD_SHAPE;
    if (c->H % 256 || c->H > 8192 || c->I > 8192) return MOE_ERR_UNSUPPORTED;
  } else if (c->act_fmt != MOE_AFMT_FP8) {
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

Shape shape_of(const moe_cfg* c) {
  return make_shape(c->T, c->H, c->I, c->E, c->topk, c->wfmt, c->wblk, c->act_group, c->has_shared, c->act_fmt);
}

// Argument checks of the layer entry points, in the order include/moe.h
// documents: NULL pointers first (the cfg, every required buffer -- NULL is
// accepted only for buffers of zero bytes, i.e. T == 0 -- and the weight
// tensors), then the shape, then alignment, then the weights' layout flag.
using PtrList = std::initializer_list<std::pair<const void*, bool>>;  // (pointer, required)

// The weight tensors a call reads: all four routed ones, plus the shared
// four when the cfg has a shared expert.
int weights_null(const moe_cfg* c, const moe_weights* w) {
  if (!w || !w->w1 || !w->w1s || !w->w2 || !w->w2s) return MOE_ERR_NULL_ARG;
  if (c->has_shared == 1 && (!w->sw1 || !w->sw1s || !w->sw2 || !w->sw2s)) return MOE_ERR_NULL_ARG;
  if (c->wfmt == MOE_WFMT_NVFP4) {  // the matrix scales
    if (!w->w1g || !w->w2g) return MOE_ERR_NULL_ARG;
    if (c->has_shared == 1 && (!w->sw1g || !w->sw2g)) return MOE_ERR_NULL_ARG;
  }
  return MOE_OK;
}

// Alignment of the weight tensors and their layout flag: `tiled` = 1 the
// layout the GEMMs read (prepacked), 0 canonical, -1 either.
int weights_layout(const moe_cfg* c, const moe_weights* w, int tiled) {
  const void* ps[8] = {w->w1, w->w1s, w->w2, w->w2s, w->sw1, w->sw1s, w->sw2, w->sw2s};
  for (int i = 0; i < (c->has_shared ? 8 : 4); ++i)
    if (misaligned(ps[i])) return MOE_ERR_MISALIGNED;
  if (c->wfmt == MOE_WFMT_NVFP4) {  // fp32 matrix scales: 4-byte aligned
    const float* gs[4] = {w->w1g, w->w2g, w->sw1g, w->sw2g};
    for (int i = 0; i < (c->has_shared ? 4 : 2); ++i)
      if (reinterpret_cast<uintptr_t>(gs[i]) & 3u) return MOE_ERR_MISALIGNED;
  }
  if (w->prepacked != 0 && w->prepacked != 1) return MOE_ERR_UNSUPPORTED;
  if (tiled >= 0 && w->prepacked != tiled) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// w == nullptr with needs_w false: the call takes no weights.
int check_args(const moe_cfg* c, PtrList ps, const moe_weights* w = nullptr, bool needs_w = false) {
  if (!c) return MOE_ERR_NULL_ARG;
  for (auto& pr : ps)
    if (pr.second && !pr.first) return MOE_ERR_NULL_ARG;
  int rc;
  if (needs_w && (rc = weights_null(c, w))) return rc;
  if ((rc = check_shape(c))) return rc;
  for (auto& pr : ps)
    if (pr.first && misaligned(pr.first)) return MOE_ERR_MISALIGNED;
  if (needs_w && (rc = weights_layout(c, w, 1))) return rc;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The GEMMs' view of the weights: GEMM1's gate|up tensors, GEMM2's down tensors.
WeightPtrs w1_ptrs(const moe_weights* w) {
  return WeightPtrs{static_cast<const uint8_t*>(w->w1), w->w1s, static_cast<const uint8_t*>(w->sw1), w->sw1s,
                    w->w1g, w->sw1g};
}
WeightPtrs w2_ptrs(const moe_weights* w) {
  return WeightPtrs{static_cast<const uint8_t*>(w->w2), w->w2s, static_cast<const uint8_t*>(w->sw2), w->sw2s,
                    w->w2g, w->sw2g};
}

// The layer's buffers inside a scratch region `b` of at least L.total bytes.
LayerBufs layer_bufs(const WsLayout& L, char* b) {
  LayerBufs r{};
  r.counts = reinterpret_cast<int32_t*>(b + L.counts);
  r.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  r.expand_idx = reinterpret_cast<int32_t*>(b + L.expand_idx);
  r.row_token = reinterpret_cast<int32_t*>(b + L.row_token);
  r.xq = reinterpret_cast<uint8_t*>(b + L.xq);
  r.xs = reinterpret_cast<float*>(b + L.xs);
  r.hq = reinterpret_cast<uint8_t*>(b + L.hq);
  r.hs = reinterpret_cast<float*>(b + L.hs);
  // GEMM2 rows stay inside the layer as bf16 (half the bytes of the fp32
  // rows the stage export returns); the combine accumulates them in fp32
  r.yb = reinterpret_cast<uint16_t*>(b + L.y);
  r.part1 = reinterpret_cast<float*>(b + L.part1);
  r.part2 = reinterpret_cast<float*>(b + L.part2);
  r.cnt1 = reinterpret_cast<int32_t*>(b + L.cnt1);
  r.cnt2 = reinterpret_cast<int32_t*>(b + L.cnt2);
  // the routing kernel zeroes every split-K arrival counter of the call
  r.clear = r.cnt1;
  r.nclear = int((L.total - L.cnt1) / 4);
  return r;
}

// The layer's launch sequence over a scratch region `b` of at least L.total
// bytes (a caller's workspace, or this GPU's static scratch array).
int enqueue_layer(const Shape& s, const WsLayout& L, const uint16_t* x, const int32_t* topk_ids,
                  const float* topk_weights, const moe_weights* w, uint16_t* out, char* b, hipStream_t st) {
  int rc;
  const LayerBufs B = layer_bufs(L, b);
  int32_t* chunk_cnt = reinterpret_cast<int32_t*>(b + L.chunk_cnt);
  if ((rc = hip_status(launch_route_quant(s, x, topk_ids, B.counts, B.offsets, B.expand_idx, B.row_token, B.xq,
                                          B.xs, B.clear, B.nclear, chunk_cnt, st))))
    return rc;
  if (s.T == 0) return MOE_OK;
  const WeightPtrs w1 = w1_ptrs(w), w2 = w2_ptrs(w);
  if (s.big) {
    if ((rc = hip_status(launch_gemm1_big(s, B.xq, B.xs, B.row_token, B.offsets, w1, B.hq, B.hs, 1, st)))) return rc;
    if ((rc = hip_status(launch_gemm2_big(s, B.hq, B.hs, B.offsets, w2, nullptr, B.yb, 1, st)))) return rc;
  } else {
    if ((rc = hip_status(launch_gemm1(s, B.xq, B.xs, B.row_token, B.offsets, w1, B.hq, B.hs, B.part1, B.cnt1, st))))
      return rc;
    if ((rc = hip_status(launch_gemm2(s, B.hq, B.hs, B.offsets, w2, nullptr, B.yb, B.part2, B.cnt2, st)))) return rc;
  }
  return hip_status(launch_combine(s, nullptr, B.yb, B.expand_idx, B.offsets, topk_weights, out, st));
}

// Scratch of moe_layer_static: one file-scope device array, which every GPU
// the library runs on holds (its own copy, at its own address) until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so it is never passed to a kernel or a copy: its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char* scratch_ptr[kMaxDevices] = {};

// This device's scratch array (the current device: the one the stream
// belongs to); the first call on a device resolves the address.
int static_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  if (!cfg || !bytes) return MOE_ERR_NULL_ARG;
  const int rc = check_shape(cfg);
  if (rc) return rc;
  *bytes = make_ws_layout(shape_of(cfg)).total;
  return MOE_OK;
}

int moe_permute(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, int32_t* counts,
                int32_t* offsets, int32_t* expand_idx, int32_t* row_token, uint8_t* xq, float* xs, void* ws,
                size_t ws_bytes, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  // more than 4096 slots are placed in chunks whose counts live in the workspace
  const bool chunked = cfg && int64_t(cfg->T) * cfg->topk > 4096;
  int rc = check_args(cfg, {{x, has_rows}, {topk_ids, has_rows}, {counts, true}, {offsets, true},
                            {expand_idx, has_rows}, {row_token, has_rows}, {xq, has_rows}, {xs, has_rows},
                            {ws, chunked}});
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  const WsLayout L = make_ws_layout(s);
  if (chunked && ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  int32_t* chunk_cnt = chunked ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.chunk_cnt) : nullptr;
  return hip_status(launch_route_quant(s, x, topk_ids, counts, offsets, expand_idx, row_token, xq, xs, nullptr,
                                       0, chunk_cnt, static_cast<hipStream_t>(stream)));
}

int moe_grouped_gemm1_swiglu(const moe_cfg* cfg, const uint8_t* xq, const float* xs, const int32_t* row_token,
                             const int32_t* offsets, const moe_weights* w, uint8_t* hq, float* hs, void* ws,
                             size_t ws_bytes, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  int rc = check_args(cfg, {{xq, has_rows}, {xs, has_rows}, {row_token, has_rows}, {offsets, true},
                            {hq, has_rows}, {hs, has_rows}, {ws, true}}, w, true);
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  const WsLayout L = make_ws_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!has_rows) return MOE_OK;
  char* base = static_cast<char*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.big)
    return hip_status(launch_gemm1_big(s, xq, xs, row_token, offsets,
                                       w1_ptrs(w),
                                       hq, hs, 1, st));
  int32_t* cnt = reinterpret_cast<int32_t*>(base + L.cnt1);
  if (s.g1_split > 1) {
    if ((rc = hip_status(launch_clear(cnt, s.g1_items * s.g1_tiles, st)))) return rc;
  }
  return hip_status(launch_gemm1(s, xq, xs, row_token, offsets,
                                 w1_ptrs(w),
                                 hq, hs, reinterpret_cast<float*>(base + L.part1), cnt, st));
}

int moe_grouped_gemm2(const moe_cfg* cfg, const uint8_t* hq, const float* hs, const int32_t* offsets,
                      const moe_weights* w, float* y, void* ws, size_t ws_bytes, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  int rc = check_args(cfg, {{hq, has_rows}, {hs, has_rows}, {offsets, true}, {y, has_rows}, {ws, true}}, w, true);
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  const WsLayout L = make_ws_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!has_rows) return MOE_OK;
  char* base = static_cast<char*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.big)
    return hip_status(launch_gemm2_big(s, hq, hs, offsets,
                                       w2_ptrs(w),
                                       y, nullptr, 1, st));
  int32_t* cnt = reinterpret_cast<int32_t*>(base + L.cnt2);
  if (s.g2_split > 1) {
    if ((rc = hip_status(launch_clear(cnt, s.g2_items * s.g2_tiles, st)))) return rc;
  }
  return hip_status(launch_gemm2(s, hq, hs, offsets,
                                 w2_ptrs(w),
                                 y, nullptr, reinterpret_cast<float*>(base + L.part2), cnt, st));
}

int moe_combine(const moe_cfg* cfg, const float* y, const int32_t* expand_idx, const int32_t* offsets,
                const float* topk_weights, uint16_t* out, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  const int rc = check_args(cfg, {{y, has_rows}, {expand_idx, has_rows}, {offsets, true}, {topk_weights, has_rows},
                                  {out, has_rows}});
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  return hip_status(
      launch_combine(s, y, nullptr, expand_idx, offsets, topk_weights, out, static_cast<hipStream_t>(stream)));
}

int moe_layer(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
              const moe_weights* w, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  int rc = check_args(cfg, {{x, has_rows}, {topk_ids, has_rows}, {topk_weights, has_rows}, {out, has_rows},
                            {ws, true}}, w, true);
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  const WsLayout L = make_ws_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return enqueue_layer(s, L, x, topk_ids, topk_weights, w, out, static_cast<char*>(ws),
                       static_cast<hipStream_t>(stream));
}

int moe_layer_static(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                     const moe_weights* w, uint16_t* out, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  int rc = check_args(cfg, {{x, has_rows}, {topk_ids, has_rows}, {topk_weights, has_rows}, {out, has_rows}}, w,
                      true);
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  const WsLayout L = make_ws_layout(s);
  if (L.total > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  char* base = nullptr;
  if ((rc = static_scratch(&base))) return rc;
  return enqueue_layer(s, L, x, topk_ids, topk_weights, w, out, base, static_cast<hipStream_t>(stream));
}

int moe_layer_persistent(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                         const moe_weights* w, uint16_t* out, void* ws, size_t ws_bytes, int32_t* status,
                         void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  int rc = check_args(cfg, {{x, has_rows}, {topk_ids, has_rows}, {topk_weights, has_rows}, {out, has_rows},
                            {ws, true}}, w, true);
  if (rc) return rc;
  const Shape s = shape_of(cfg);
  const WsLayout L = make_ws_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.T == 0) return MOE_OK;
  if (!persistent_supported(s)) return MOE_ERR_UNSUPPORTED;
  char* base = static_cast<char*>(ws);
  const LayerBufs b = layer_bufs(L, base);
  const WeightPtrs w1 = w1_ptrs(w), w2 = w2_ptrs(w);
  return hip_status(launch_layer_persistent(s, x, topk_ids, topk_weights, w1, w2, b,
                                            reinterpret_cast<int32_t*>(base + L.chunk_cnt), out,
                                            reinterpret_cast<int32_t*>(base + L.pctl), status,
                                            static_cast<hipStream_t>(stream)));
}

int moe_layer_persistent_spin_limit(int polls) {
  if (polls < 0) return MOE_ERR_BAD_SHAPE;
  set_persist_spin_limit(polls);
  return MOE_OK;
}

int moe_prepack_weights(const moe_cfg* cfg, const moe_weights* canonical, moe_weights* packed, void* stream) {
  if (!cfg || !canonical || !packed) return MOE_ERR_NULL_ARG;
  int rc;
  if ((rc = weights_null(cfg, canonical)) || (rc = weights_null(cfg, packed))) return rc;
  if ((rc = check_shape(cfg))) return rc;
  if ((rc = weights_layout(cfg, canonical, 0)) || (rc = weights_layout(cfg, packed, -1))) return rc;
  const moe_cfg& c = *cfg;
  const bool mx = c.wfmt != MOE_WFMT_FP8_BLOCK;  // scales re-laid out (MXFP4, NVFP4)
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // (codes, scales, matrices, rows N, reduction K) of each tensor pair
  struct Pair { const void *w, *s; void *wt, *stl; int mats, N, K; };
  Pair pairs[4] = {
      {canonical->w1, canonical->w1s, const_cast<void*>(packed->w1), const_cast<void*>(packed->w1s), c.E, 2 * c.I, c.H},
      {canonical->w2, canonical->w2s, const_cast<void*>(packed->w2), const_cast<void*>(packed->w2s), c.E, c.H, c.I},
      {canonical->sw1, canonical->sw1s, const_cast<void*>(packed->sw1), const_cast<void*>(packed->sw1s), 1, 2 * c.I, c.H},
      {canonical->sw2, canonical->sw2s, const_cast<void*>(packed->sw2), const_cast<void*>(packed->sw2s), 1, c.H, c.I}};
  const int np = c.has_shared ? 4 : 2;
  for (int i = 0; i < np; ++i)  // not in place
    if (pairs[i].w == pairs[i].wt || (mx && pairs[i].s == pairs[i].stl)) return MOE_ERR_UNSUPPORTED;
  for (int i = 0; i < np; ++i) {
    const Pair& q = pairs[i];
    if ((rc = hip_status(launch_tile_weights(c.wfmt, q.mats, q.N, q.K, static_cast<const uint8_t*>(q.w),
                                             static_cast<const uint8_t*>(q.s), static_cast<uint8_t*>(q.wt),
                                             static_cast<uint8_t*>(q.stl), st))))
      return rc;
    if (!mx && q.s != q.stl) {  // e4m3 block scales keep their layout
      const size_t sb = size_t(q.mats) * (q.N / c.wblk) * (q.K / c.wblk) * sizeof(float);
      if ((rc = hip_status(hipMemcpyAsync(q.stl, q.s, sb, hipMemcpyDeviceToDevice, st)))) return rc;
    }
  }
  if (c.wfmt == MOE_WFMT_NVFP4) {  // the matrix scales keep their layout
    const float* gsrc[4] = {canonical->w1g, canonical->w2g, canonical->sw1g, canonical->sw2g};
    const float* gdst[4] = {packed->w1g, packed->w2g, packed->sw1g, packed->sw2g};
    for (int i = 0; i < np; ++i) {
      const size_t gb = size_t(i < 2 ? c.E : 1) * sizeof(float);
      if (gsrc[i] != gdst[i] &&
          (rc = hip_status(hipMemcpyAsync(const_cast<float*>(gdst[i]), gsrc[i], gb, hipMemcpyDeviceToDevice, st))))
        return rc;
    }
  }
  packed->prepacked = 1;
  return MOE_OK;
}

int moe_stream_read(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (!buf || !sink) return MOE_ERR_NULL_ARG;
  if (misaligned(buf) || misaligned(sink)) return MOE_ERR_MISALIGNED;
  if (bytes % 16) return MOE_ERR_BAD_SHAPE;
  if (sink_bytes < 4 * size_t(stream_read_grid())) return MOE_ERR_WORKSPACE;
  return hip_status(launch_stream_read(buf, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)));
}

int moe_mfma_rate(int wfmt, int iters, void* sink, size_t sink_bytes, double* flops, void* stream) {
  if (!sink) return MOE_ERR_NULL_ARG;
  if (misaligned(sink)) return MOE_ERR_MISALIGNED;
  if (wfmt != MOE_WFMT_FP8_BLOCK && wfmt != MOE_WFMT_MXFP4 && wfmt != MOE_RATE_E2M1_E2M1) return MOE_ERR_UNSUPPORTED;
  if (iters < 1 || iters > 65536) return MOE_ERR_BAD_SHAPE;
  if (sink_bytes < 4 * size_t(mfma_rate_grid())) return MOE_ERR_WORKSPACE;
  return hip_status(launch_mfma_rate(wfmt, iters, static_cast<float*>(sink), flops, static_cast<hipStream_t>(stream)));
}

int moe_route_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  if (!cfg || !bytes) return MOE_ERR_NULL_ARG;
  const int rc = check_shape(cfg);
  if (rc) return rc;
  if (cfg->E > 256) return MOE_ERR_UNSUPPORTED;
  *bytes = route_workspace_bytes(cfg->T, cfg->H, cfg->E);
  return MOE_OK;
}

int moe_route(const moe_cfg* cfg, const uint16_t* x, const uint16_t* gate_w, int32_t* topk_ids, float* topk_weights,
              void* ws, size_t ws_bytes, void* stream) {
  const bool has_rows = cfg && cfg->T > 0;
  const size_t need = has_rows ? route_workspace_bytes(cfg->T, cfg->H, cfg->E) : 0;
  const int rc = check_args(cfg, {{x, has_rows}, {gate_w, true}, {topk_ids, has_rows}, {topk_weights, has_rows},
                                  {ws, need > 0}});
  if (rc) return rc;
  if (cfg->E > 256) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  return hip_status(launch_route_gemm(cfg->T, cfg->H, cfg->E, cfg->topk, x, gate_w, topk_ids, topk_weights,
                                      static_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

int moe_encode_e4m3(const float* v, size_t n, uint8_t* codes, void* stream) {
  if (n > 0 && (!v || !codes)) return MOE_ERR_NULL_ARG;
  if (misaligned(v) || misaligned(codes)) return MOE_ERR_MISALIGNED;
  if (n >= (size_t(1) << 40)) return MOE_ERR_BAD_SHAPE;
  return hip_status(launch_encode_e4m3(v, long(n), codes, static_cast<hipStream_t>(stream)));
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_ARG: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "invalid shape";
    case MOE_ERR_UNSUPPORTED: return "unsupported format / block / group combination";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
