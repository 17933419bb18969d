// moe_router.hip -- the router in front of the MoE layer: gate GEMM (bf16
// MFMA, fp32 accumulation), top-k selection and the softmax of the selected
// logits.  The DeepGEMM 26/09 news page describes this fusion for its Mega
// Gate (the routing GEMM and the routing operations -- matrix product,
// selection, data organisation -- in one kernel).  Here it is two launches
// at every T: the GEMM spreads the gate matrix over enough workgroups to
// fill the chip and writes fp32 partial logits per K split to the caller's
// workspace; a second kernel sums each token's splits in a fixed order and
// selects (one workgroup per token), so the result does not depend on
// timing.  The partials are the price of the split, 4 E bytes per token and
// split (16.8 MB at 4096 tokens, 256 experts, four splits); one kernel
// holding a token's whole K cannot fill the CUs below tens of thousands of
// tokens.
//
// Up to 512 tokens (decode) the GEMM is one wave per (16-token tile,
// 16-expert tile, K chunk), its operands loaded straight into registers.
// Above, one workgroup per (64-token tile, K split) stages its token rows
// and every expert's gate rows through LDS (k_route_tile), so each gate row
// is read once per 64 tokens.  The selection: k rounds of a wave-wide
// argmax (equal logits going to the lower expert id), then the softmax of
// the k selected logits.

#include <float.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRouteThreads = 256;
constexpr int kMaxExpertTiles = 16;   // E <= 256
constexpr int kStageK = 64;           // K per pipeline stage: two 16x16x32 MFMA steps

// Lane l's operand bytes of one stage: 16 rows (lane % 16) x 64 K, lane
// group g = l / 16 holding K [16 g, 16 g + 16) of the stage as two 8-element
// halves, one per MFMA step.  A and B use the same K assignment, so every
// product of the dot product is formed exactly once whatever order the MFMA
// sums them in.
template <int NTE, int NTT>
struct Stage {
  v4u a[NTE][2];  // expert tiles of this wave
  v4u b[NTT][2];  // token tiles
};

__device__ __forceinline__ v8bf as_bf(const v4u& u) { return __builtin_bit_cast(v8bf, u); }

// Wave-wide reductions through DPP moves (register to register, no LDS
// round trip): within each 16-lane row by the quad permutations (lane xor 1,
// xor 2), the half-row mirror (lane i and 7 - i) and the row mirror (i and
// 15 - i), then the four rows' results read out of lanes 0, 16, 32, 48 and
// combined in row order.  The result is the same in every lane.
__device__ __forceinline__ float lane_f32(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// The selection of one token by one wave: lane l holds the logits of experts
// l, l + 64, l + 128, l + 192 (entries past E ignored).  Each of k rounds
// takes the largest remaining logit (a wave-wide max) and, among the entries
// equal to it, the lowest expert id: ids run q-major (64 q + lane), so that is
// the lowest set lane of the first non-empty ballot in q order.  Lane j keeps
// the j-th pick; then the softmax of the k picks.  Writes ids[0..k) and
// weights[0..k).
__device__ __forceinline__ void select_topk(const float (&v)[4], int E, int k, int lane, int32_t* ids,
                                            float* weights) {
  int taken = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane + 64 * q >= E) taken |= 1 << q;
  float my_v = 0.0f;  // lane j keeps the j-th selected logit
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float lm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!(taken & (1 << q))) lm = fmaxf(lm, v[q]);
    const float top = wave_max_f32(lm);
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t b = __ballot(!(taken & (1 << q)) && v[q] == top);
      if (b) {
        bi = 64 * q + __ffsll((unsigned long long)b) - 1;
        break;
      }
    }
    if (bi != 0x7FFFFFFF && (bi & 63) == lane) taken |= 1 << (bi >> 6);
    if (lane == r) { my_v = top; my_i = bi; }
  }
  const float top = lane_f32(my_v, 0);
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  const float sum = wave_sum_f32(ex);
  if (lane < k) {
    ids[lane] = my_i;
    weights[lane] = ex / sum;
  }
}

// ---- many tokens: one workgroup per (64-token tile, K split) holds every
// expert.  Each 64-K stage of the tile's token rows and of all expert rows
// (128 bytes per row) is loaded as whole rows -- eight lanes per row, eight
// rows per wave and instruction -- into a ring of register stages, then
// stored to one of two LDS buffers, 16-byte chunk c of row r at chunk
// position c ^ (r & 7), so the fragment reads of eight consecutive rows at
// one chunk fall on eight different chunk positions (the layout the
// many-row GEMMs use for their token rows).  Of NW waves (4, or 8 from
// eight expert tiles on), wave w multiplies expert tiles w, w + NW, ... by
// the four token tiles (gate rows on the MFMA's 16-row side, tokens on its
// 16-column side), and the split's fp32 partial logits go to the workspace
// ([split][token][expert]), where k_route_select_wave sums them in split
// order and selects.
constexpr int kTileTok = 64;                                // tokens per workgroup
constexpr int kTileRows = kTileTok + kMaxExpertTiles * 16;  // LDS rows per stage (tokens, then experts)
constexpr int kTileRegStages = 4;                           // register stages of loads in flight (even)

struct RouteTileParams {
  const uint16_t* x;   // bf16 [T][H]
  const uint16_t* wg;  // bf16 [E][H]
  float* part;         // [S][T_pad][E]
  int T, H, E, steps;  // steps: 64-K stages per split
  int T_pad;           // tokens rounded up to the tile
  int splits;          // S
};

// NTE expert tiles per wave: the workgroup stages 64 token rows and 64 NTE
// expert rows, NP = 2 + 2 NTE 16-byte loads per thread and stage.  Every load,
// LDS store and MFMA is unconditional (rows past T or E repeat the last valid
// row, and their products are never stored), so the compiler counts the
// loads in flight exactly and waits only for the stage it stores.
template <int NTE, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_route_tile(RouteTileParams p) {
  constexpr int kThr = 64 * NW;
  constexpr int NP = (kTileTok + 16 * NW * NTE) * 8 / kThr;
  static_assert((kTileTok + 16 * NW * NTE) * 8 % kThr == 0 && kTileTok * 8 % kThr == 0, "whole loads per thread");
  __shared__ v4u lds[2][kTileRows * 8];  // two stages, up to 40 KB each
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  // work items w = tile + ntiles * split, split-major; workgroup L runs on
  // XCD L % 8 (the dispatcher deals workgroups to the eight XCDs in turn),
  // so with n a multiple of 8 XCD x takes the contiguous items [x n / 8,
  // (x + 1) n / 8): mostly one K split per XCD, whose gate slice then stays
  // in that XCD's L2
  const int ntiles = p.T_pad / kTileTok, n = ntiles * p.splits, L = blockIdx.x;
  const int wi = n % 8 == 0 ? (L % 8) * (n / 8) + L / 8 : L;
  const int tok0 = (wi % ntiles) * kTileTok, split = wi / ntiles;
  const int H = p.H, E = p.E, ET = (E + 15) / 16;
  // piece q of this thread is row (tid + 256 q) / 8, 16-byte chunk (tid + 256 q) % 8
  const uint16_t* src[NP];
  int dst[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int pc = tid + kThr * q, r = pc >> 3, c = pc & 7;
    src[q] = r < kTileTok ? p.x + long(min(tok0 + r, p.T - 1)) * H + 8 * c
                          : p.wg + long(min(r - kTileTok, E - 1)) * H + 8 * c;
    dst[q] = r * 8 + (c ^ (r & 7));
  }
  const long k_base = long(split) * p.steps * kStageK;
  // token rows are read once (non-temporal, so they do not push the gate
  // slice out of L2); gate rows are re-read by every token tile of the split
  auto gload = [&](v4u (&rg)[NP], int s) __attribute__((always_inline)) {
    const long k0 = k_base + long(s) * kStageK;
#pragma unroll
    for (int q = 0; q < NP; ++q)
      rg[q] = q < kTileTok * 8 / kThr ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src[q] + k0))
                    : *reinterpret_cast<const v4u*>(src[q] + k0);
  };
  auto swrite = [&](int b, const v4u (&rg)[NP]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NP; ++q) lds[b][dst[q]] = rg[q];
  };
  v4f acc[NTE][4];
#pragma unroll
  for (int j = 0; j < NTE; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // one stage from LDS buffer b: two 32-K MFMA steps; lane group g holds
  // K [32 h + 8 g, 32 h + 8 g + 8) of step h in chunk 4 h + g, for both
  // operands (rows 16 t + m and 64 + 16 tile + m both have r & 7 = m & 7)
  auto compute = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cpos = (4 * h + g) ^ (m & 7);
      v4u bt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bt[t] = lds[b][(16 * t + m) * 8 + cpos];
#pragma unroll
      for (int j = 0; j < NTE; ++j) {
        const v4u a = lds[b][(kTileTok + 16 * (w + NW * j) + m) * 8 + cpos];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a), as_bf(bt[t]), acc[j][t], 0, 0, 0);
      }
    }
  };
  // stage s sits in LDS buffer s % 2 while a ring of R register stages
  // holds stages s + 1 .. s + R (R - 1 stages of loads in flight while a
  // stage multiplies); one barrier per stage.  Past the last stage the loads
  // repeat it (cache hits, never multiplied), so every step issues and
  // stores the same loads and waits only for the oldest register stage.
  constexpr int R = kTileRegStages;
  static_assert(R % 2 == 0, "stage s + i sits in buffer i % 2 only when the ring's period is even");
  const int ns = p.steps;
  v4u rg[R][NP];
#pragma unroll
  for (int i = 0; i < R; ++i) gload(rg[i], min(i, ns - 1));
  swrite(0, rg[0]);
  __syncthreads();
  gload(rg[0], min(R, ns - 1));
  for (int s = 0; s < ns; s += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      // stage s + i: in buffer i % 2; rg[(i + 1) % R] holds stage s + i + 1
      if (s + i < ns) compute(i % 2);
      swrite((i + 1) % 2, rg[(i + 1) % R]);
      __syncthreads();
      gload(rg[(i + 1) % R], min(s + i + 1 + R, ns - 1));
    }
  }
  // lane l holds token 16 t + m, experts 16 tile + 4 g + (0..3)
#pragma unroll
  for (int j = 0; j < NTE; ++j) {
    const int tile = w + NW * j;
    if (tile >= ET) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = tok0 + 16 * t + m;
      if (tok >= p.T) continue;
      float* dstp = p.part + (long(split) * p.T_pad + tok) * E + 16 * tile + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * tile + 4 * g + i < E) dstp[i] = acc[j][t][i];
    }
  }
}

// ---- few tokens: the gate rows spread over many workgroups.  One wave per
// (16-token tile, 16-expert tile, K chunk) writes its fp32 partial logits to
// the workspace ([chunk][token][expert]); a second kernel sums a token's
// chunks in a fixed order and selects, one workgroup per token.
struct RoutePartParams {
  const uint16_t* x;
  const uint16_t* wg;
  float* part;
  int T, H, E, steps;  // steps: 64-K stages per chunk
  int T_pad;           // tokens rounded up to 16
};

constexpr int kPartStages = 4;  // register stages in flight per wave

__global__ __launch_bounds__(64) void k_route_part(RoutePartParams p) {
  const int tt = blockIdx.x, et = blockIdx.y, kc = blockIdx.z;
  const int lane = threadIdx.x, m = lane & 15, g = lane >> 4;
  const int H = p.H, E = p.E;
  const uint16_t* arow = p.wg + long(min(16 * et + m, E - 1)) * H + 16 * g;
  const uint16_t* brow = p.x + long(min(16 * tt + m, p.T - 1)) * H + 16 * g;
  const int s0 = kc * p.steps, ns = p.steps;
  Stage<1, 1> st[kPartStages];
  auto load = [&](Stage<1, 1>& s, int k0) __attribute__((always_inline)) {
    s.a[0][0] = *reinterpret_cast<const v4u*>(arow + k0);
    s.a[0][1] = *reinterpret_cast<const v4u*>(arow + k0 + 8);
    s.b[0][0] = *reinterpret_cast<const v4u*>(brow + k0);
    s.b[0][1] = *reinterpret_cast<const v4u*>(brow + k0 + 8);
  };
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < kPartStages - 1; ++r)
    if (r < ns) load(st[r], (s0 + r) * kStageK);
  for (int i = 0; i < ns; i += kPartStages) {
#pragma unroll
    for (int r = 0; r < kPartStages; ++r) {
      if (i + r < ns) {
        if (i + r + kPartStages - 1 < ns) load(st[(r + kPartStages - 1) % kPartStages], (s0 + i + r + kPartStages - 1) * kStageK);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(st[r].a[0][h]), as_bf(st[r].b[0][h]), acc, 0, 0, 0);
      }
    }
  }
  // lane l holds token 16 tt + m, experts 16 et + 4 g + (0..3)
  const int t = 16 * tt + m;
  float* dst = p.part + (long(kc) * p.T_pad + t) * E + 16 * et + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (16 * et + 4 * g + i < E) dst[i] = acc[i];
}

struct RouteSelParams {
  const float* part;
  int32_t* ids;
  float* weights;
  int T, E, k, nkc, T_pad;
};

template <int NB>
__global__ __launch_bounds__(256) void k_route_select(RouteSelParams p) {
  // one workgroup per token: wave w sums the chunks [w nkc / 4, (w + 1) nkc / 4)
  // in NB independent partial sums (NB loads in flight per lane: the
  // partials were written by other XCDs, so each round trip goes past L2),
  // folded pairwise in a fixed order;
  // the four waves' sums meet in LDS in wave order, wave 0 selects
  __shared__ float red[4][kMaxExpertTiles * 16];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int c0 = w * p.nkc / 4, c1 = (w + 1) * p.nkc / 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = min(lane + 64 * q, p.E - 1);
    float sp[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) sp[u] = 0.0f;
    // every load of a round of NB is issued (past c1 they re-read the last
    // chunk and are not added)
    for (int c = c0; c < c1; c += NB) {
      float x[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) x[u] = p.part[(long(min(c + u, c1 - 1)) * p.T_pad + t) * p.E + e];
#pragma unroll
      for (int u = 0; u < NB; ++u) sp[u] = c + u < c1 ? sp[u] + x[u] : sp[u];
    }
#pragma unroll
    for (int h = NB / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int u = 0; u < h; ++u) sp[u] += sp[u + h];
    if (lane + 64 * q < p.E) red[w][lane + 64 * q] = sp[0];
  }
  __syncthreads();
  if (w != 0) return;
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < p.E ? ((red[0][e] + red[1][e]) + (red[2][e] + red[3][e])) : 0.0f;
  }
  select_topk(v, p.E, p.k, lane, p.ids + long(t) * p.k, p.weights + long(t) * p.k);
}

// Many tokens: one wave per token, four tokens per workgroup.  Lane l sums
// its experts l, l + 64, l + 128, l + 192 over the splits in split order;
// every load is issued (up to NC splits; past the split count or E they
// re-read a valid entry and are not added), so a wave has its loads in
// flight at once.
constexpr int kSelMaxSplits = 32;

template <int NC>
__global__ __launch_bounds__(256) void k_route_select_wave(RouteSelParams p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;
  if (t >= p.T) return;
  const int nkc = p.nkc, E = p.E;
  const long pitch = long(p.T_pad) * E;
  const float* row = p.part + long(t) * E;
  float x[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float* r = row + min(c, nkc - 1) * pitch;
#pragma unroll
    for (int q = 0; q < 4; ++q) x[c][q] = r[min(lane + 64 * q, E - 1)];
  }
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float s = x[0][q];
#pragma unroll
    for (int c = 1; c < NC; ++c) s = c < nkc ? s + x[c][q] : s;
    v[q] = lane + 64 * q < E ? s : 0.0f;
  }
  select_topk(v, E, p.k, lane, p.ids + long(t) * p.k, p.weights + long(t) * p.k);
}

}  // namespace

// K chunks of the few-token path: the largest divisor of the H / 64 stages
// that keeps the launch within kRouteWaves waves (about two per CU), or half
// that up to 64 tokens (fewer partial logits for the reduction to gather:
// H=4096, E=64, T=64 12.5 -> 10.7 us; at T=256 the full count is faster)
constexpr int kRouteSmallMaxT = 512;
constexpr long kRouteWaves = 512;
constexpr int kRouteFewT = 64;
// K splits of the many-token path: the largest divisor of the H / 64 stages
// that keeps the launch within kRouteTileWGs workgroups (one per CU)
constexpr long kRouteTileWGs = 256;

static int largest_split(long units, int stages, long cap) {
  int best = 1;
  for (int d = 1; d <= stages; ++d)
    if (stages % d == 0 && units * d <= cap) best = d;
  return best;
}

static int route_chunks(int T, int H, int E) {
  if (T <= kRouteSmallMaxT)
    return largest_split(long((T + 15) / 16) * ((E + 15) / 16), H / kStageK, T <= kRouteFewT ? kRouteWaves / 2 : kRouteWaves);
  const long ntiles = (T + kTileTok - 1) / kTileTok;
  return largest_split(ntiles, H / kStageK, std::min(kRouteTileWGs, ntiles * kSelMaxSplits));
}

static long route_t_pad(int T) {
  const int tile = T <= kRouteSmallMaxT ? 16 : kTileTok;
  return long(T + tile - 1) / tile * tile;
}

size_t route_workspace_bytes(int T, int H, int E) {
  if (T == 0) return 0;
  return size_t(route_chunks(T, H, E)) * route_t_pad(T) * E * 4;
}

hipError_t launch_route_gemm(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wg, int32_t* ids,
                             float* weights, float* part, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nkc = route_chunks(T, H, E);
  const int T_pad = int(route_t_pad(T));
  const int steps = H / kStageK / nkc;
  if (T <= kRouteSmallMaxT) {
    RoutePartParams pp{x, wg, part, T, H, E, steps, T_pad};
    hipLaunchKernelGGL(k_route_part, dim3(unsigned(T_pad / 16), unsigned((E + 15) / 16), unsigned(nkc)), dim3(64), 0,
                       st, pp);
  } else {
    RouteTileParams tp{x, wg, part, T, H, E, steps, T_pad, nkc};
    const dim3 grid(unsigned(T_pad / kTileTok * nkc));
    // eight waves (two per SIMD, so one's LDS reads and barrier waits overlap
    // the other's MFMAs) once there are eight expert tiles, else four
    const int et = (E + 15) / 16;
    if (et > 8) hipLaunchKernelGGL((k_route_tile<2, 8>), grid, dim3(512), 0, st, tp);
    else if (et > 4) hipLaunchKernelGGL((k_route_tile<1, 8>), grid, dim3(512), 0, st, tp);
    else hipLaunchKernelGGL((k_route_tile<1, 4>), grid, dim3(256), 0, st, tp);
  }
  RouteSelParams sp{part, ids, weights, T, E, k, nkc, T_pad};
  if (T <= kRouteSmallMaxT) {
    // NB partial sums per lane: 4 when no wave has more than 4 chunks
    if ((nkc + 3) / 4 <= 4) hipLaunchKernelGGL(k_route_select<4>, dim3(unsigned(T)), dim3(256), 0, st, sp);
    else hipLaunchKernelGGL(k_route_select<16>, dim3(unsigned(T)), dim3(256), 0, st, sp);
  }
  else {
    const dim3 grid(unsigned((T + 3) / 4));
    if (nkc <= 4) hipLaunchKernelGGL(k_route_select_wave<4>, grid, dim3(256), 0, st, sp);
    else if (nkc <= 8) hipLaunchKernelGGL(k_route_select_wave<8>, grid, dim3(256), 0, st, sp);
    else if (nkc <= 16) hipLaunchKernelGGL(k_route_select_wave<16>, grid, dim3(256), 0, st, sp);
    else hipLaunchKernelGGL(k_route_select_wave<kSelMaxSplits>, grid, dim3(256), 0, st, sp);
  }
  return hipGetLastError();
}

}  // namespace moe
