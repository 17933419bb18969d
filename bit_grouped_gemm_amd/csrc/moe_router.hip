// moe_router.hip -- the router in front of the MoE layer, one kernel: gate
// GEMM (bf16 MFMA, fp32 accumulation), top-k selection and the softmax of
// the selected logits.  This is the fusion the DeepGEMM 26/09 news page
// describes for its Mega Gate (the routing GEMM and the routing operations
// -- matrix product, selection, data organisation -- in one kernel, so no
// logits go back to memory and no second launch is needed).
//
// A workgroup owns NTT tiles of 16 tokens and every expert.  Its waves form
// 4 expert slots x KG K groups: the wave of slot j and group g runs the
// expert tiles j, j + 4, j + 8, j + 12 (those below E/16) over its group's
// share of the K range, with the gate rows on the MFMA's 16-row side and the
// tokens on its 16-column side, keeping RS register stages of 64 K in flight.
// The K groups' fp32 partial logits meet in LDS and are summed in group
// order (a fixed order: the result does not depend on timing); each wave then
// selects the top k of one token at a time (k rounds of a wave-wide argmax,
// equal logits going to the lower expert id) and turns the k selected logits
// into softmax weights.  Few tokens (decode) take 16 waves in 4 K groups, so
// that one workgroup streams the gate matrix with 16 waves' loads in flight.
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
    int taken = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? lg[0][tl][e] : -FLT_MAX;
      if (e >= E) taken |= 1 << q;
    }
    float my_v = 0.0f;  // lane j keeps the j-th selected logit
    int my_i = 0;
    for (int r = 0; r < p.k; ++r) {
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
    const float ex = lane < p.k ? expf(my_v - top) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (lane < p.k) {
      p.ids[long(t) * p.k + lane] = my_i;
      p.weights[long(t) * p.k + lane] = ex / sum;
    }
  }
}

}  // namespace

hipError_t launch_route_gemm(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wg, int32_t* ids,
                             float* weights, hipStream_t st) {
  if (T == 0) return hipSuccess;
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
