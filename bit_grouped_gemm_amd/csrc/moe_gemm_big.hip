// moe_gemm_big.hip -- grouped GEMMs for groups with many rows (prefill).
//
// When an expert holds ~100+ token rows (prefill: T = 4096, top-8 over 256
// experts gives ~128 rows per expert) a workgroup must cover all of them
// per pass, or each weight byte is read from HBM once per pass.  Here a
// workgroup of 8 waves owns 256 weight rows and up to 192 token rows:
//   * weights stream from HBM straight into registers in MFMA layout, one
//     128-K step ahead; the group's token rows of each step are staged
//     through LDS (two buffers, one barrier per step) and read by all waves;
//   * each of the 8 waves owns 32 of the 256 weight rows (two 16-row MFMA
//     tiles: in GEMM1 one gate and one up tile, so SwiGLU pairs meet in one
//     lane) across all 12 token tiles, which keeps 2 x 12 accumulator tiles
//     and a K step of weight operands in flight within 256 registers;
//   * LDS rows are XOR-swizzled by 16-byte chunk so the MFMA-layout reads
//     (16 lanes on 16 consecutive rows, same chunk) hit distinct banks;
//   * all tiles of one expert are dispatched to the same XCD (workgroup
//     ids are dealt round-robin over the 8 XCDs), so the expert's token rows
//     are fetched into that XCD's L2 once and re-read from there.
// GEMM1 mode: weight rows are 128 gate + 128 up rows (128 h columns = one
// requantisation group of 128), epilogue SwiGLU + FP8 requantisation.
// GEMM2 mode: 256 output rows, epilogue writes y.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kBigThreads = 512;
constexpr int kRows = 256;      // weight rows per workgroup
constexpr int kTokCap = 192;    // token rows per pass
constexpr int kTokTiles = kTokCap / 16;
constexpr int kBChunks = kTokCap * 8;      // 16-byte chunks of one staged token tile
constexpr int kBPT = kBChunks / kBigThreads;  // 3 token-row chunks per thread per step
static_assert(kBChunks % kBigThreads == 0, "every thread stages the same number of chunks");
constexpr int kBigStages = 2;  // weight register stages (ring positions 0, 1)

struct BigParams {
  const uint8_t* act;        // GEMM1: xq [T][H] by token; GEMM2: hq [rows][I] by row
  const float* act_s;
  const int32_t* row_token;  // GEMM1 only (null in GEMM2 mode)
  const int32_t* offsets;
  const uint8_t* w;
  const void* ws;
  const uint8_t* sw;
  const void* sws;
  uint8_t* hq;
  float* hs;
  float* y;
  int H, I, E, G, wblk, ngroups, ntiles, units, per_xcd, min_rows;
};

// byte offset of 16-byte chunk c (0..7) of token row r in LDS: rows of 128 B,
// chunk index XOR-ed with r & 7 so 8 lanes reading one chunk of 8
// consecutive rows hit 8 distinct 4-bank groups
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

struct Lds {
  uint8_t b[2][kTokCap * 128];   // token rows of one 128-K step, two buffers
  float xs[2][kBigThreads];      // their scales (one slot per thread; slots >= rows unused)
  float red[8][kTokCap];         // requantisation group maxima: [wave][token]
};

}  // namespace

template <int WF, int MODE>
__global__ __launch_bounds__(kBigThreads) void k_gemm_big(BigParams p) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  Lds& L = *reinterpret_cast<Lds*>(lds_raw);
  __shared__ int s_wsum[8], s_res;

  // ---- unit: XCD-aware order (blockIdx -> XCD is round-robin over 8)
  const int xcd = blockIdx.x & 7, k_in = blockIdx.x >> 3;
  const int u = xcd * p.per_xcd + k_in;
  if (k_in >= p.per_xcd || u >= p.units) return;
  const int slot = u / p.ntiles, tile = u % p.ntiles;
  const int tid = threadIdx.x;
  // slot-th group with at least min_rows rows
  {
    const int gpt = (p.ngroups + kBigThreads - 1) / kBigThreads;
    int local = 0;
    for (int q = 0; q < gpt; ++q) {
      const int gg = tid * gpt + q;
      if (gg < p.ngroups && p.offsets[gg + 1] - p.offsets[gg] >= p.min_rows) ++local;
    }
    int incl = local;
    const int ln = tid & 63, wv = tid >> 6;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (ln >= d) incl += v;
    }
    if (tid == 0) s_res = -1;
    if (ln == 63) s_wsum[wv] = incl;
    __syncthreads();
    int run = incl - local;
    for (int q = 0; q < wv; ++q) run += s_wsum[q];
    if (slot >= run && slot < run + local) {
      int c = run;
      for (int q = 0; q < gpt; ++q) {
        const int gg = tid * gpt + q;
        if (gg < p.ngroups && p.offsets[gg + 1] - p.offsets[gg] >= p.min_rows) {
          if (c == slot) s_res = gg;
          ++c;
        }
      }
    }
    __syncthreads();
  }
  const int e = s_res;
  if (e < 0) return;
  const int row0 = p.offsets[e], ne = p.offsets[e + 1] - row0;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, m = lane & 15, g = lane >> 4;
  const int H = p.H, I = p.I;
  const int K = MODE == 0 ? H : I;       // reduction length
  const int NR = MODE == 0 ? 2 * I : H;  // weight rows of the matrix
  const int n0 = tile * (MODE == 0 ? 128 : 256);
  const bool shared = e == p.E;
  const long ee = shared ? 0 : e;
  const long kb = WF == 0 ? K : K / 2;   // bytes per weight row
  const uint8_t* wmat = (shared ? p.sw : p.w) + ee * long(NR) * kb;
  const void* smat = shared ? p.sws : p.ws;
  const int nks = K / 128;

  // this wave's two 16-row weight tiles; GEMM1: gate rows n0+16w and up
  // rows I+n0+16w (h columns 16w..16w+15); GEMM2: output rows n0+32w+16j
  const uint8_t* wrow[2];
  const float* wsc[2];
  const uint8_t* wsb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = MODE == 0 ? (j == 0 ? n0 + 16 * w : I + n0 + 16 * w) : n0 + 32 * w + 16 * j;
    wrow[j] = wmat + long(rb + m) * kb;
    if (WF == 0) {
      const int b = p.wblk;
      wsc[j] = static_cast<const float*>(smat) + ee * long(NR / b) * (K / b) + long(rb / b) * (K / b);
      wsb[j] = nullptr;
    } else {
      wsb[j] = static_cast<const uint8_t*>(smat) + ee * long(NR) * (K / 32) + long(rb + m) * (K / 32);
      wsc[j] = nullptr;
    }
  }

  for (int pass0 = 0; pass0 < ne; pass0 += kTokCap) {
    const int npass = min(kTokCap, ne - pass0);
    const int ntt = (npass + 15) / 16;
    // staging assignment: chunk ch = tid + i*512 -> token ch>>3, 16-byte chunk ch&7
    int boff[kBPT];
#pragma unroll
    for (int i = 0; i < kBPT; ++i) {
      const int ch = tid + i * kBigThreads;
      const int tk = min(ch >> 3, npass - 1);
      const long arow = MODE == 0 ? long(p.row_token[row0 + pass0 + tk]) : long(row0 + pass0 + tk);
      boff[i] = int(arow * K) + (ch & 7) * 16;
    }
    const float* xs_src = p.act_s;
    if (tid < npass) {
      const long arow = MODE == 0 ? long(p.row_token[row0 + pass0 + tid]) : long(row0 + pass0 + tid);
      xs_src = p.act_s + arow * (K / p.G);
    }

    v4f acc[2][kTokTiles];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < kTokTiles; ++t) acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Weights travel through two register stages (loads for step ks + 1 are
    // issued while step ks is multiplied).  The
    // token rows of a step go through two register stages and two LDS
    // buffers: loaded two steps ahead, stored to LDS at the top of their
    // step, read after the barrier.  Each step issues its token-row loads
    // before its weight loads, so waiting for a token stage never waits for
    // younger weight stages.  Every load and LDS store is unconditional (rows
    // past the group repeat its last row, the step index is clamped at the
    // end): with no divergent branches around them the compiler counts
    // outstanding loads exactly instead of waiting for all of them.
    v8i af[kBigStages][2];
    int sa[kBigStages][2];
    float wsv[kBigStages][2];
    v4u bst[2][kBPT];
    float xst[2] = {0.0f, 0.0f};
    auto load_a = [&](int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (WF == 0) {
          af[slot][j] = load_e4m3_frag(wrow[j] + long(ks) * 128, g);
          wsv[slot][j] = wsc[j][ks];
          sa[slot][j] = kUnitScale;
        } else {
          af[slot][j] = load_e2m1_frag(wrow[j] + long(ks) * 64, g);
          sa[slot][j] = wsb[j][ks * 4 + g];
          wsv[slot][j] = 1.0f;
        }
      }
    };
    auto load_b = [&](int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kBPT; ++i) bst[slot][i] = ldg16(p.act + boff[i] + long(ks) * 128);
      xst[slot] = xs_src[tid < npass ? ks : 0];
    };
    load_b(0, 0);
    load_b(min(1, nks - 1), 1);
    load_a(0, 0);
    // one 128-K step at ring position SIDX (0 or 1, a compile-time constant
    // after unrolling): store the staged token rows, barrier, issue the loads
    // two steps (token rows) and one step (weights) ahead, multiply
#define MOE_BIG_STEP(KS, SIDX)                                                                              \
  {                                                                                                         \
    const int ks_ = (KS);                                                                                   \
    const int buf = (SIDX);                                                                                 \
    _Pragma("unroll") for (int i = 0; i < kBPT; ++i) {                                                      \
      const int ch = tid + i * kBigThreads;                                                                 \
      *reinterpret_cast<v4u*>(&L.b[buf][swz(ch >> 3, ch & 7)]) = bst[buf][i];                               \
    }                                                                                                       \
    L.xs[buf][tid] = xst[buf];                                                                              \
    __syncthreads();                                                                                        \
    load_b(min(ks_ + 2, nks - 1), buf);                                                                     \
    load_a(min(ks_ + 1, nks - 1), buf ^ 1);                                                                 \
    _Pragma("unroll") for (int t0 = 0; t0 < kTokTiles; t0 += 2) {                                          \
      if (t0 < ntt) {                                                                                       \
        v8i bf[2];                                                                                          \
        float xsv[2];                                                                                       \
        _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                                     \
          const int tk = (t0 + q) * 16 + m;                                                                 \
          const v4u lo = *reinterpret_cast<const v4u*>(&L.b[buf][swz(tk, g)]);                              \
          const v4u hi = *reinterpret_cast<const v4u*>(&L.b[buf][swz(tk, 4 + g)]);                          \
          bf[q] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])}; \
          xsv[q] = L.xs[buf][tk];                                                                           \
        }                                                                                                   \
        v4f d[2][2];                                                                                        \
        _Pragma("unroll") for (int q = 0; q < 2; ++q)                                                       \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                   \
            if (WF == 0) d[q][j] = mfma_scaled<kFmtE4M3, kFmtE4M3>(af[buf][j], bf[q], kUnitScale, kUnitScale); \
            else d[q][j] = mfma_scaled<kFmtE2M1, kFmtE4M3>(af[buf][j], bf[q], sa[buf][j], kUnitScale);     \
          }                                                                                                 \
        _Pragma("unroll") for (int q = 0; q < 2; ++q)                                                       \
          _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                     \
            acc[j][t0 + q] += d[q][j] * (WF == 0 ? wsv[buf][j] * xsv[q] : xsv[q]);                          \
      }                                                                                                     \
    }                                                                                                       \
  }
    // whole ring periods without per-step guards (no branch joins around
    // loads), then at most one guarded remainder step
    int ks0 = 0;
    for (; ks0 + 2 <= nks; ks0 += 2) {
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) MOE_BIG_STEP(ks0 + sidx, sidx)
    }
    if (ks0 < nks) MOE_BIG_STEP(ks0, 0)
#undef MOE_BIG_STEP

    // ---- epilogue
    if (MODE == 0) {
      // h = silu(gate) * up in place of the gate accumulator: h column
      // 16w + 4g + i, token column m of each tile
      float amax[kTokTiles];
#pragma unroll
      for (int t = 0; t < kTokTiles; ++t) {
        amax[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = acc[0][t][i], up = acc[1][t][i];
          const float v = gt / (1.0f + expf(-gt)) * up;
          acc[0][t][i] = v;
          amax[t] = fmaxf(amax[t], fabsf(v));
        }
        amax[t] = wave_max_xor(amax[t], 16);
        amax[t] = wave_max_xor(amax[t], 32);
      }
      __syncthreads();
      if (g == 0)
#pragma unroll
        for (int t = 0; t < kTokTiles; ++t) L.red[w][t * 16 + m] = amax[t];
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kTokTiles; ++t) {
        const int idx = t * 16 + m;
        if (t >= ntt || idx >= npass) continue;
        float am = L.red[0][idx];
#pragma unroll
        for (int q = 1; q < 8; ++q) am = fmaxf(am, L.red[q][idx]);
        const float mult = quant_mult(am);
        const long r = row0 + pass0 + idx;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) word |= enc_e4m3(acc[0][t][i] * mult) << (8 * i);
        *reinterpret_cast<uint32_t*>(p.hq + r * I + n0 + 16 * w + 4 * g) = word;
        if (g == 0 && w == 0) p.hs[r * (I / 128) + n0 / 128] = 1.0f / mult;
      }
    } else {
#pragma unroll
      for (int t = 0; t < kTokTiles; ++t) {
        const int idx = t * 16 + m;
        if (t >= ntt || idx >= npass) continue;
        const long r = row0 + pass0 + idx;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *reinterpret_cast<v4f*>(p.y + r * H + n0 + 32 * w + 16 * j + 4 * g) = acc[j][t];
      }
    }
    __syncthreads();  // LDS is reused by the next pass
  }
}

static hipError_t launch_big(const Shape& s, int mode, BigParams& p, hipStream_t st) {
  const int units = s.slots_max * p.ntiles;
  if (units == 0) return hipSuccess;
  p.units = units;
  p.per_xcd = (units + 7) / 8;
  const unsigned grid = unsigned(p.per_xcd) * 8;
  const size_t lds = sizeof(Lds);
  static_assert(sizeof(Lds) <= 64 * 1024, "within the default dynamic LDS limit");
  if (s.wfmt == 0) {
    if (mode == 0) hipLaunchKernelGGL((k_gemm_big<0, 0>), dim3(grid), dim3(kBigThreads), lds, st, p);
    else hipLaunchKernelGGL((k_gemm_big<0, 1>), dim3(grid), dim3(kBigThreads), lds, st, p);
  } else {
    if (mode == 0) hipLaunchKernelGGL((k_gemm_big<1, 0>), dim3(grid), dim3(kBigThreads), lds, st, p);
    else hipLaunchKernelGGL((k_gemm_big<1, 1>), dim3(grid), dim3(kBigThreads), lds, st, p);
  }
  return hipGetLastError();
}

size_t big_lds_bytes() { return sizeof(Lds); }

hipError_t launch_gemm1_big(const Shape& s, const uint8_t* xq, const float* xs, const int32_t* row_token,
                            const int32_t* offsets, WeightPtrs w1, uint8_t* hq, float* hs, int min_rows,
                            hipStream_t st) {
  BigParams p{};
  p.act = xq; p.act_s = xs; p.row_token = row_token; p.offsets = offsets;
  p.w = w1.w; p.ws = w1.ws; p.sw = w1.sw; p.sws = w1.sws;
  p.hq = hq; p.hs = hs;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.ntiles = s.I / 128; p.min_rows = min_rows;
  return launch_big(s, 0, p, st);
}

hipError_t launch_gemm2_big(const Shape& s, const uint8_t* hq, const float* hs, const int32_t* offsets,
                            WeightPtrs w2, float* y, int min_rows, hipStream_t st) {
  BigParams p{};
  p.act = hq; p.act_s = hs; p.offsets = offsets;
  p.w = w2.w; p.ws = w2.ws; p.sw = w2.sw; p.sws = w2.sws;
  p.y = y;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.ntiles = s.H / 256; p.min_rows = min_rows;
  return launch_big(s, 1, p, st);
}

}  // namespace moe
