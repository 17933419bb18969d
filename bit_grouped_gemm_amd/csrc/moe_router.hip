// moe_router.hip -- the router in front of the MoE layer, one kernel: gate
// GEMM (bf16 MFMA, fp32 accumulation), top-k selection and the softmax of
// the selected logits.  This is the fusion the DeepGEMM 26/09 news page
// describes for its Mega Gate (the routing GEMM and the routing operations
// -- matrix product, selection, data organisation -- in one kernel, so no
// logits go back to memory and no second launch is needed).
//
// Up to 512 tokens (decode) the gate matrix is spread over many workgroups:
// one wave per (16-token tile, 16-expert tile, K chunk) writes fp32 partial
// logits to the caller's workspace, and a second kernel sums each token's
// chunks in a fixed order and selects (one workgroup per token).  Above that one
// kernel: a workgroup owns NTT tiles of 16 tokens and every expert, its waves
// forming 4 expert slots x KG K groups (the wave of slot j and group g runs
// expert tiles j, j + 4, j + 8, j + 12 over its group's share of K, keeping
// RS register stages of 64 K in flight), with the gate rows on the MFMA's
// 16-row side and the tokens on its 16-column side; the K groups' partial
// logits meet in LDS and are summed in group order.  Either way the result
// does not depend on timing.  The selection: k rounds of a wave-wide argmax
// (equal logits going to the lower expert id), then the softmax of the k
// selected logits.

#include <float.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRouteThreads = 256;
constexpr int kMaxExpertTiles = 16;   // E <= 256
constexpr int kStageK = 64;           // K per pipeline stage: two 16x16x32 MFMA steps

struct RouteGemmParams {
  const uint16_t* x;   // bf16 [T][H]
  const uint16_t* wg;  // bf16 [E][H]
  int32_t* ids;        // [T][k]
  float* weights;      // [T][k]
  int T, H, E, k;
};

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

// (value, expert id) order of the selection: larger logit first, the lower
// id first among equal logits
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// The selection of one token by one wave: lane l holds the logits of experts
// l, l + 64, l + 128, l + 192 (entries past E ignored); k rounds of a
// wave-wide argmax over (logit, -id), lane j keeping the j-th pick, then the
// softmax of the k picks.  Writes ids[0..k) and weights[0..k).
__device__ __forceinline__ void select_topk(const float (&v)[4], int E, int k, int lane, int32_t* ids,
                                            float* weights) {
  int taken = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane + 64 * q >= E) taken |= 1 << q;
  float my_v = 0.0f;  // lane j keeps the j-th selected logit
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -FLT_MAX;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!(taken & (1 << q)) && beats(v[q], lane + 64 * q, bv, bi)) { bv = v[q]; bi = lane + 64 * q; }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (bi != 0x7FFFFFFF && (bi & 63) == lane) taken |= 1 << (bi >> 6);
    if (lane == r) { my_v = bv; my_i = bi; }
  }
  const float top = __shfl(my_v, 0, 64);
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
  if (lane < k) {
    ids[lane] = my_i;
    weights[lane] = ex / sum;
  }
}

template <int NTT, int KG, int RS, int NTE>
__global__ __launch_bounds__(256 * KG) void k_route(RouteGemmParams p) {
  constexpr int kTok = 16 * NTT;
  constexpr int kPitch = kMaxExpertTiles * 16 + 1;
  __shared__ float lg[KG][kTok][kPitch];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  const int slot = w & 3, kg = w >> 2;
  const int tok0 = blockIdx.x * kTok;
  const int H = p.H, E = p.E;
  const int ET = (E + 15) / 16;
  // this wave's expert tiles: slot, slot + 4, slot + 8, slot + 12 (those below
  // ET, at most NTE of them)
  int nte = 0;
  const uint16_t* arow[NTE];
#pragma unroll
  for (int j = 0; j < NTE; ++j) {
    const int tile = slot + 4 * j;
    if (tile < ET) nte = j + 1;
    const int e = min(16 * min(tile, ET - 1) + m, E - 1);
    arow[j] = p.wg + long(e) * H + 16 * g;
  }
  const uint16_t* brow[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) brow[t] = p.x + long(min(tok0 + 16 * t + m, p.T - 1)) * H + 16 * g;

  v4f acc[NTE][NTT];
#pragma unroll
  for (int j = 0; j < NTE; ++j)
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto load = [&](Stage<NTE, NTT>& s, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NTE; ++j)
      if (j < nte) {
        s.a[j][0] = *reinterpret_cast<const v4u*>(arow[j] + k0);
        s.a[j][1] = *reinterpret_cast<const v4u*>(arow[j] + k0 + 8);
      }
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      s.b[t][0] = *reinterpret_cast<const v4u*>(brow[t] + k0);
      s.b[t][1] = *reinterpret_cast<const v4u*>(brow[t] + k0 + 8);
    }
  };
  auto mma = [&](const Stage<NTE, NTT>& s) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < NTE; ++j)
        if (j < nte)
#pragma unroll
          for (int t = 0; t < NTT; ++t)
            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(s.a[j][h]), as_bf(s.b[t][h]), acc[j][t], 0, 0, 0);
  };
  // this group's stages [s0, s1) of the H / 64; RS register stages: the
  // loads of stages i + 1 .. i + RS - 1 are in flight while stage i multiplies
  const int nst = H / kStageK;
  const int s0 = kg * nst / KG, s1 = (kg + 1) * nst / KG, ns = s1 - s0;
  Stage<NTE, NTT> st[RS];
#pragma unroll
  for (int r = 0; r < RS - 1; ++r)
    if (r < ns) load(st[r], (s0 + r) * kStageK);
  for (int i = 0; i < ns; i += RS) {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      if (i + r < ns) {
        if (i + r + RS - 1 < ns) load(st[(r + RS - 1) % RS], (s0 + i + r + RS - 1) * kStageK);
        mma(st[r]);
      }
    }
  }
  // partial logits to LDS: lane l holds token 16 t + m, experts 16 tile + 4 g + (0..3)
#pragma unroll
  for (int j = 0; j < NTE; ++j)
    if (j < nte)
#pragma unroll
      for (int t = 0; t < NTT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lg[kg][16 * t + m][16 * (slot + 4 * j) + 4 * g + i] = acc[j][t][i];
  __syncthreads();
  if (KG > 1) {
    // the K groups' partial sums, in group order, into group 0's rows
    for (int idx = tid; idx < kTok * E; idx += 256 * KG) {
      const int tl = idx / E, e = idx - tl * E;
      float v = lg[0][tl][e];
#pragma unroll
      for (int q = 1; q < KG; ++q) v += lg[q][tl][e];
      lg[0][tl][e] = v;
    }
    __syncthreads();
  }

  // top-k per token: lane l holds experts l, l + 64, l + 128, l + 192
  for (int tl = w; tl < kTok; tl += 4 * KG) {
    const int t = tok0 + tl;
    if (t >= p.T) break;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? lg[0][tl][e] : 0.0f;
    }
    select_topk(v, E, p.k, lane, p.ids + long(t) * p.k, p.weights + long(t) * p.k);
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

__global__ __launch_bounds__(256) void k_route_select(RouteSelParams p) {
  // one workgroup per token: wave w sums the chunks [w nkc / 4, (w + 1) nkc / 4)
  // in sixteen independent partial sums (sixteen loads in flight per lane: the
  // partials were written by other XCDs, so each round trip goes past L2),
  // folded pairwise in a fixed order;
  // the four waves' sums meet in LDS in wave order, wave 0 selects
  __shared__ float red[4][kMaxExpertTiles * 16];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int c0 = w * p.nkc / 4, c1 = (w + 1) * p.nkc / 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e >= p.E) continue;
    float sp[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) sp[u] = 0.0f;
    for (int c = c0; c < c1; c += 16) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c + u < c1) sp[u] += p.part[(long(c + u) * p.T_pad + t) * p.E + e];
    }
#pragma unroll
    for (int h = 8; h >= 1; h >>= 1)
#pragma unroll
      for (int u = 0; u < h; ++u) sp[u] += sp[u + h];
    red[w][e] = sp[0];
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

}  // namespace

// K chunks of the few-token path: the largest divisor of the H / 64 stages
// that keeps the launch within kRouteWaves waves (about two per CU)
constexpr int kRouteSmallMaxT = 512;
constexpr long kRouteWaves = 512;

static int route_chunks(int T, int H, int E) {
  const long units = long((T + 15) / 16) * ((E + 15) / 16);
  const int stages = H / kStageK;
  int best = 1;
  for (int d = 1; d <= stages; ++d)
    if (stages % d == 0 && units * d <= kRouteWaves) best = d;
  return best;
}

size_t route_workspace_bytes(int T, int H, int E) {
  if (T == 0 || T > kRouteSmallMaxT) return 0;
  const long T_pad = (T + 15) / 16 * 16;
  return size_t(route_chunks(T, H, E)) * T_pad * E * 4;
}

hipError_t launch_route_gemm(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wg, int32_t* ids,
                             float* weights, float* part, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (T <= kRouteSmallMaxT) {
    const int nkc = route_chunks(T, H, E);
    const int T_pad = (T + 15) / 16 * 16;
    RoutePartParams pp{x, wg, part, T, H, E, H / kStageK / nkc, T_pad};
    hipLaunchKernelGGL(k_route_part, dim3(unsigned(T_pad / 16), unsigned((E + 15) / 16), unsigned(nkc)), dim3(64), 0,
                       st, pp);
    RouteSelParams sp{part, ids, weights, T, E, k, nkc, T_pad};
    hipLaunchKernelGGL(k_route_select, dim3(unsigned(T)), dim3(256), 0, st, sp);
    return hipGetLastError();
  }
  RouteGemmParams p{x, wg, ids, weights, T, H, E, k};
  // two token tiles per workgroup once there are enough tokens to fill the
  // CUs with them (half the gate-row reads per token); below that 16 waves
  // per 16-token tile, split four ways along K, with six register stages
  // when each wave holds one expert tile (E <= 64) and two otherwise
  if (T >= 4096) {
    hipLaunchKernelGGL((k_route<2, 1, 2, 4>), dim3(unsigned((T + 31) / 32)), dim3(kRouteThreads), 0, st, p);
  } else if (E <= 64) {
    hipLaunchKernelGGL((k_route<1, 4, 6, 1>), dim3(unsigned((T + 15) / 16)), dim3(4 * kRouteThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_route<1, 4, 2, 4>), dim3(unsigned((T + 15) / 16)), dim3(4 * kRouteThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace moe
