// moe_gemm_big.hip -- grouped GEMMs for groups with many rows (prefill).
//
// When an expert holds ~100+ token rows (prefill: T = 4096, top-8 over 256
// experts gives ~128 rows per expert) a workgroup must cover all of them
// per pass, or each weight byte is read from HBM once per pass.  Here a
// workgroup of 8 waves owns 256 weight rows and up to 192 token rows, and
// walks K in steps of 128:
//   * both operands of a step travel HBM/L2 -> LDS by direct-to-LDS loads
//     (global_load_lds_dwordx4: 64 lanes x 16 B into 1 KB of LDS per
//     instruction, no registers held while in flight) through a ring of
//     stages (three for MXFP4 weights, two for e4m3 weights whose steps are
//     twice as large), so two steps of weights and token rows are in
//     flight while one is multiplied;
//   * weights come from the tiled layout (16-row x 128-K tiles in MFMA lane
//     order, see moe_tile.hip), one contiguous kilobyte per tile and step,
//     and land in LDS unchanged, so fragment reads are linear ds_read_b128;
//     token rows travel as whole 128-byte lines into a chunk-swizzled layout
//     whose fragment reads are conflict-free as well;
//   * the 8 waves form a 4 x 2 grid: a wave owns 4 weight tiles (64 rows;
//     in GEMM1 two gate and the two matching up tiles, so SwiGLU pairs meet
//     in one lane) and every second token tile, which keeps up to 4 x 6
//     fp32 accumulator tiles in registers and reads each token fragment
//     once per 4 MFMAs;
//   * one vmcnt wait and one barrier per step: each wave waits for its own
//     loads of the step, the barrier makes every wave's loads visible, and
//     the loads two steps ahead are issued after the barrier, into the
//     stage every wave has finished reading;
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
constexpr int kWTiles = 16;                  // 256 weight rows
constexpr int kAsBytes = 8 * 64 * 4;         // MXFP4 scales: one dword (4 x e8m0) per lane of 8 waves
constexpr int kMaxKSteps = 64;              // K <= 8192: the pass's token scales fit one LDS table
constexpr int kXsRow = kMaxKSteps + 1;       // floats per token row of the table (odd: no bank conflicts)
constexpr int kSinkBytes = 1024;             // target of token loads past the pass's tiles

// Geometry of one instantiation: weight format WF and token rows per pass
// CAP (160 for prefill-sized groups; 64 when groups are smaller, which
// leaves LDS for a three-stage ring with e4m3 weights too).
template <int WF, int CAP> struct BigGeo {
  static constexpr int kTokCap = CAP;
  static constexpr int kTokTiles = CAP / 16;
  static constexpr int kTokPerWave = kTokTiles / 2;       // token tiles of one wave column
  static constexpr int kTokLoads = (2 * kTokTiles + 7) / 8;  // token-row loads per wave per step
  static constexpr int kBBytes = kTokTiles * 2048;        // token tiles: 16 rows x 128 B, chunk-swizzled
  static constexpr int kStages = (WF == 1 || CAP <= 64) ? 3 : 2;
  static constexpr int kABytes = kWTiles * 1024 * (WF == 1 ? 1 : 2);
  static constexpr int kAOff = kBBytes;
  static constexpr int kAsOff = kAOff + kABytes;
  static constexpr int kSinkOff = kAsOff + (WF == 1 ? kAsBytes : 0);
  static constexpr int kStageBytes = kSinkOff + kSinkBytes;
  // direct-to-LDS loads per wave per stage: token rows, weight tiles 2
  // (MXFP4) or 4 (e4m3 halves), MXFP4 scales 1
  static constexpr int kLoadsPerStage = kTokLoads + (WF == 1 ? 2 + 1 : 4);
  static constexpr int kXsTabBytes = CAP * kXsRow * 4;    // [token][k step] fp32
  static constexpr int kLdsBytes = kStages * kStageBytes + kXsTabBytes;
  static_assert(kTokPerWave <= 6, "three pairs of token tiles, one load part after each");
  static_assert(kTokLoads <= 3, "token-row loads fit the three load parts");
  static_assert(4 * CAP * 4 <= kStageBytes, "epilogue maxima fit one stage");
  static_assert(kLdsBytes + 1024 <= 160 * 1024, "ring, scale table and small arrays fit the 160 KB LDS");
};

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
  uint16_t* yb;  // bf16 y instead when non-null (layer-internal)
  int H, I, E, G, wblk, ngroups, ntiles, units, per_xcd, min_rows;
};

// one 16-byte-per-lane direct load into LDS: lane l's bytes land at
// lds_base + 16 * l (lds_base wave-uniform)
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 4, 0, 0);
}

// wait until at most N vector-memory operations of this wave are pending
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, other counters at
// their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// byte offset of 16-byte chunk c (0..7) of row r (0..15) in a 2 KB token
// tile of 128-byte rows: the chunk index is XOR-ed with r & 7, so the MFMA
// fragment reads (16 lanes on 16 rows, one chunk each) hit distinct banks
// while a direct-to-LDS load still covers 8 whole rows (full cache lines)
__device__ __forceinline__ int tok_swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// instruction classes the scheduler may move across a load-issue point (the
// sched_barrier mask): ALU, VALU, SALU, MFMA, LDS reads, transcendentals --
// not the vector-memory loads themselves
constexpr int kSchedMayCross = 0x0001 | 0x0002 | 0x0004 | 0x0008 | 0x0100 | 0x0400;

// workgroup barrier that the compiler may not move memory operations across;
// the waits for the ring's direct-to-LDS loads are explicit (wait_vmcnt)
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int WF, int MODE, int CAP>
__global__ __launch_bounds__(kBigThreads) void k_gemm_big(BigParams p) {
  using Geo = BigGeo<WF, CAP>;
  constexpr int kTokCap = Geo::kTokCap, kTokPerWave = Geo::kTokPerWave, kTokLoads = Geo::kTokLoads;
  constexpr int S = Geo::kStages;
  // one array per ring stage: the compiler's alias analysis then tells the
  // stages apart and waits for a stage's own direct-to-LDS loads only
  __shared__ __align__(1024) uint8_t st0[Geo::kStageBytes];
  __shared__ __align__(1024) uint8_t st1[Geo::kStageBytes];
  __shared__ __align__(1024) uint8_t st2[S == 3 ? Geo::kStageBytes : 16];
  __shared__ __align__(16) float xs_tab[kTokCap * kXsRow];  // token scales of the pass
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
  const int wr = w & 3, wc = w >> 2;     // wave row (weight tiles), wave column (token tiles)
  const int H = p.H, I = p.I;
  const int K = MODE == 0 ? H : I;       // reduction length
  const int NR = MODE == 0 ? 2 * I : H;  // weight rows of the matrix
  const int n0 = tile * (MODE == 0 ? 128 : 256);
  const bool shared = e == p.E;
  const long ee = shared ? 0 : e;
  const int kb = WF == 0 ? K : K / 2;    // bytes per weight row
  const uint8_t* wmat = (shared ? p.sw : p.w) + ee * long(NR) * kb;
  const void* smat = shared ? p.sws : p.ws;
  const int nks = K / 128;
  // first matrix row of weight tile j (0..15): GEMM1 tiles 0..7 are gate
  // rows, 8..15 the up rows of the same h columns; GEMM2 rows in order
  auto wtile_row = [&](int j) { return MODE == 0 ? (j < 8 ? n0 + 16 * j : I + n0 + 16 * (j - 8)) : n0 + 16 * j; };

  // ---- loader side: this lane's sources in the tiled weights for the tiles
  // of wave w (tiles 2w, 2w+1: one contiguous kilobyte each, two for e4m3)
  // and their MXFP4 scales (the two tiles' 128 bytes are adjacent; lanes
  // 32..63 repeat lanes 0..31)
  const long wstep = long(NR / 16) * kTileBytes<WF>;       // bytes per K step
  const long sstep = long(NR / 16) * kTileScaleBytes;
  const uint8_t* a_src[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) a_src[q] = wmat + long(wtile_row(2 * w + q) / 16) * kTileBytes<WF> + lane * 16;
  const uint8_t* as_src = nullptr;
  if (WF == 1)
    as_src = static_cast<const uint8_t*>(smat) + ee * long(NR) * (K / 32) +
             long(wtile_row(2 * w) / 16) * kTileScaleBytes + (lane & 31) * 4;
  // ---- consumer side: this wave's weight tiles
  int ja[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ja[q] = MODE == 0 ? (q < 2 ? 2 * wr + q : 8 + 2 * wr + (q - 2)) : 4 * wr + q;
  const float* wsc[4];  // e4m3: scale row of each tile's 128 x 128 block (one scale per K step)
#pragma unroll
  for (int q = 0; q < 4; ++q)
    wsc[q] = WF == 0 ? static_cast<const float*>(smat) + ee * long(NR / 128) * (K / 128) +
                           long(wtile_row(ja[q]) / 128) * (K / 128)
                     : nullptr;

  for (int pass0 = 0; pass0 < ne; pass0 += kTokCap) {
    const int npass = min(kTokCap, ne - pass0);
    const int ntt = (npass + 15) / 16;
    const int ntw = (ntt + 1 - wc) / 2;  // token tiles of this wave: t = 2 * tt + wc
    // token-row sources: the pass's ntt tiles take 2 * ntt loads of 8 rows x
    // 128 B (load i: tile i / 2, rows 8 (i % 2) .. + 7), dealt round-robin to
    // the waves (load q of wave w is i = w + 8 q).  Lane l fills LDS chunk
    // l % 8 of row l / 8, i.e. global chunk (l % 8) ^ (row & 7).  Rows past
    // the group repeat its last row.  Every wave issues kTokLoads such loads
    // per step; the ones past the pass's tiles read one 16-byte chunk with
    // all lanes into the stage's sink, so every step has the same load count.
    const uint8_t* b_src[kTokLoads];
    int b_dst[kTokLoads];
#pragma unroll
    for (int q = 0; q < kTokLoads; ++q) {
      const int i = w + 8 * q;
      const int rl = (i & 1) * 8 + (lane >> 3);
      const bool real = i < 2 * ntt;
      const int tk = real ? min((i >> 1) * 16 + rl, npass - 1) : npass - 1;
      const long arow = MODE == 0 ? long(p.row_token[row0 + pass0 + tk]) : long(row0 + pass0 + tk);
      b_src[q] = p.act + arow * K + (real ? ((lane & 7) ^ (rl & 7)) << 4 : 0);
      b_dst[q] = real ? i * 1024 : Geo::kSinkOff;
    }
    // token scales of the whole pass, read once into a [token][k step]
    // table: one direct-to-LDS load per token (its K/128 scales are
    // contiguous; lanes past them repeat the last one), CAP / 8 per wave.  Being
    // direct loads into their own array, the table's reads wait only for
    // these loads, not for the ring's.
    for (int tk = w; tk < kTokCap; tk += 8) {
      const int c = min(tk, npass - 1);
      const long arow = MODE == 0 ? long(p.row_token[row0 + pass0 + c]) : long(row0 + pass0 + c);
      dma4(p.act_s + arow * nks + min(lane, nks - 1), reinterpret_cast<uint8_t*>(xs_tab + tk * kXsRow));
    }

    // the direct-to-LDS loads of step ks into stage buffer st, in three
    // parts (0: weight tiles, 1: weight scales and the first
    // token-row load, 2: the other two token-row loads)
    auto issue = [&](int ks, uint8_t* st, int part) __attribute__((always_inline)) {
      if (part == 0) {
        if (WF == 1) {
#pragma unroll
          for (int q = 0; q < 2; ++q) dma16(a_src[q] + ks * wstep, st + Geo::kAOff + (2 * w + q) * 1024);
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              dma16(a_src[q] + ks * wstep + 1024 * h, st + Geo::kAOff + (2 * (2 * w + q) + h) * 1024);
        }
      } else if (part == 1) {
        if (WF == 1) dma4(as_src + ks * sstep, st + Geo::kAsOff + w * 256);
        dma16(b_src[0] + long(ks) * 128, st + b_dst[0]);
      } else {
#pragma unroll
        for (int q = 1; q < kTokLoads; ++q) dma16(b_src[q] + long(ks) * 128, st + b_dst[q]);
      }
    };
    // pinned in place among the MFMAs: the load pipeline drains while the
    // matrix cores work instead of taking every wave's loads in one burst
    // (ALU, MFMA and LDS reads may still be scheduled across the point)
    auto issue_part = [&](int ks, uint8_t* st, int part) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(kSchedMayCross);
      issue(ks, st, part);
      __builtin_amdgcn_sched_barrier(kSchedMayCross);
    };

    // accumulators: e4m3 weights promote each step's MFMA result with a VALU
    // FMA (acc += d * ws * xs).  MXFP4 weights carry their scales inside
    // the MFMA, and the accumulator is kept in units of the current step's
    // token scale: before a step it is multiplied by xs_prev / xs_cur (a
    // multiply that depends only on the previous step), then the MFMA adds
    // the step's product in place; after the last step it is multiplied by
    // that step's xs.  Token scales are positive (at least 2^-64 / 448), so
    // the ratio is always defined.
    v4f acc[4][kTokPerWave];
    float xsp[kTokPerWave];  // MXFP4: the token scales of the previous step
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < kTokPerWave; ++t) acc[q][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < kTokPerWave; ++t) xsp[t] = 0.0f;

    // multiply one stage: A fragments of the wave's 4 weight tiles, then its
    // token tiles two at a time, with the next stage's loads issued in
    // between
    auto compute = [&](int ks, const uint8_t* st, int ksn, uint8_t* nxt) __attribute__((always_inline)) {
      v8i af[4];
      int sa[4];
      float wsv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (WF == 1) {
          const v4u a = *reinterpret_cast<const v4u*>(st + Geo::kAOff + ja[q] * 1024 + lane * 16);
          af[q] = v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
          sa[q] = st[Geo::kAsOff + (ja[q] >> 1) * 256 + (ja[q] & 1) * kTileScaleBytes + lane];
          wsv[q] = 1.0f;
        } else {
          const v4u lo = *reinterpret_cast<const v4u*>(st + Geo::kAOff + (2 * ja[q]) * 1024 + lane * 16);
          const v4u hi = *reinterpret_cast<const v4u*>(st + Geo::kAOff + (2 * ja[q] + 1) * 1024 + lane * 16);
          af[q] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
          sa[q] = kUnitScale;
          wsv[q] = wsc[q][ks];
        }
      }
      float xsv[kTokPerWave];
#pragma unroll
      for (int tt = 0; tt < kTokPerWave; ++tt)
        xsv[tt] = xs_tab[((2 * tt + wc) * 16 + m) * kXsRow + ks];
      if (WF == 1) {
        // rescale to this step's token scales
#pragma unroll
        for (int tt = 0; tt < kTokPerWave; ++tt) {
          if (tt < ntw) {
            const float r = xsp[tt] * __builtin_amdgcn_rcpf(xsv[tt]);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q][tt] *= r;
          }
          xsp[tt] = xsv[tt];
        }
      }
#pragma unroll
      for (int t0 = 0; t0 < 6; t0 += 2) {
        issue_part(ksn, nxt, t0 / 2);
        if (t0 < kTokPerWave && t0 < ntw) {
          // a pair of token tiles (the last one alone when the count is odd)
          v8i bf[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            if (t0 + r >= kTokPerWave) continue;
            const int t = 2 * (t0 + r) + wc;
            const v4u lo = *reinterpret_cast<const v4u*>(st + t * 2048 + tok_swz(m, g));
            const v4u hi = *reinterpret_cast<const v4u*>(st + t * 2048 + tok_swz(m, 4 + g));
            bf[r] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
          }
          if (WF == 1) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (t0 + r < kTokPerWave)
                  acc[q][t0 + r] = mfma_scaled_acc<kFmtE2M1, kFmtE4M3>(af[q], bf[r], acc[q][t0 + r], sa[q], kUnitScale);
          } else {
            v4f d[2][4];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (t0 + r < kTokPerWave) d[r][q] = mfma_scaled<kFmtE4M3, kFmtE4M3>(af[q], bf[r], kUnitScale, kUnitScale);
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (t0 + r < kTokPerWave) acc[q][t0 + r] += d[r][q] * (wsv[q] * xsv[t0 + r]);
          }
        }
      }
    };

    // ---- the K loop over the ring, unrolled by the ring depth so that each
    // step's stage buffers are fixed arrays.  Every step issues the loads of
    // the step S - 1 ahead, clamped to the last step (past the end they
    // re-load it into a stage that is not read again), so every step has
    // the same count of loads in flight and waits for the same count.
    auto step = [&](int ks, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
      wait_vmcnt<(S - 2) * Geo::kLoadsPerStage>();
      ring_barrier();
      compute(ks, cur, min(ks + S - 1, nks - 1), nxt);
    };
    for (int part = 0; part < 3; ++part) issue(0, st0, part);
    int ks = 0;
    if (S == 3) {
      for (int part = 0; part < 3; ++part) issue(min(1, nks - 1), st1, part);
      for (; ks + 3 <= nks; ks += 3) {
        step(ks, st0, st2);
        step(ks + 1, st1, st0);
        step(ks + 2, st2, st1);
      }
      if (ks < nks) step(ks, st0, st2);
      if (ks + 1 < nks) step(ks + 1, st1, st0);
    } else {
      for (; ks + 2 <= nks; ks += 2) {
        step(ks, st0, st1);
        step(ks + 1, st1, st0);
      }
      if (ks < nks) step(ks, st0, st1);
    }

    if (WF == 1)  // back from units of the last step's token scale
#pragma unroll
      for (int tt = 0; tt < kTokPerWave; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q][tt] *= xsp[tt];

    // ---- epilogue
    wait_vmcnt<0>();  // the clamped loads past the last step land in the ring too
    __syncthreads();  // all waves are done reading the ring
    if (MODE == 0) {
      // h = silu(gate) * up in place of the gate accumulators: h column
      // n0 + 32 wr + 16 q + 4 g + i, token 16 t + m with t = 2 tt + wc
      float* red = reinterpret_cast<float*>(st0);  // [4 wave rows][kTokCap]
      float amax[kTokPerWave];
#pragma unroll
      for (int tt = 0; tt < kTokPerWave; ++tt) {
        amax[tt] = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gt = acc[q][tt][i], up = acc[q + 2][tt][i];
            const float v = gt / (1.0f + expf(-gt)) * up;
            acc[q][tt][i] = v;
            amax[tt] = fmaxf(amax[tt], fabsf(v));
          }
        amax[tt] = wave_max_xor(amax[tt], 16);
        amax[tt] = wave_max_xor(amax[tt], 32);
      }
      if (g == 0)
#pragma unroll
        for (int tt = 0; tt < kTokPerWave; ++tt) red[wr * kTokCap + (2 * tt + wc) * 16 + m] = amax[tt];
      __syncthreads();
#pragma unroll
      for (int tt = 0; tt < kTokPerWave; ++tt) {
        const int idx = (2 * tt + wc) * 16 + m;
        if (tt >= ntw || idx >= npass) continue;
        float am = red[idx];
#pragma unroll
        for (int q = 1; q < 4; ++q) am = fmaxf(am, red[q * kTokCap + idx]);
        const float mult = quant_mult(am);
        const long r = row0 + pass0 + idx;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const v4f& hv = acc[q][tt];
          const uint32_t word = enc_e4m3x4(hv[0] * mult, hv[1] * mult, hv[2] * mult, hv[3] * mult);
          *reinterpret_cast<uint32_t*>(p.hq + r * I + n0 + 32 * wr + 16 * q + 4 * g) = word;
        }
        if (g == 0 && wr == 0) p.hs[r * (I / 128) + n0 / 128] = 1.0f / mult;
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < kTokPerWave; ++tt) {
        const int idx = (2 * tt + wc) * 16 + m;
        if (tt >= ntw || idx >= npass) continue;
        const long r = row0 + pass0 + idx;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (p.yb) store_bf16x4(p.yb + r * H + n0 + 64 * wr + 16 * q + 4 * g, acc[q][tt]);
          else *reinterpret_cast<v4f*>(p.y + r * H + n0 + 64 * wr + 16 * q + 4 * g) = acc[q][tt];
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
  const size_t lds = 0;  // static LDS
#define MOE_BIG_LAUNCH(WF, CAP)                                                                   \
  do {                                                                                            \
    if (mode == 0) hipLaunchKernelGGL((k_gemm_big<WF, 0, CAP>), dim3(grid), dim3(kBigThreads), lds, st, p); \
    else hipLaunchKernelGGL((k_gemm_big<WF, 1, CAP>), dim3(grid), dim3(kBigThreads), lds, st, p);           \
  } while (0)
  if (s.wfmt == 0) {
    if (s.big_cap == 64) MOE_BIG_LAUNCH(0, 64);
    else MOE_BIG_LAUNCH(0, 160);
  } else {
    if (s.big_cap == 64) MOE_BIG_LAUNCH(1, 64);
    else MOE_BIG_LAUNCH(1, 160);
  }
#undef MOE_BIG_LAUNCH
  return hipGetLastError();
}


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
                            WeightPtrs w2, float* y, uint16_t* yb, int min_rows, hipStream_t st) {
  BigParams p{};
  p.act = hq; p.act_s = hs; p.offsets = offsets;
  p.w = w2.w; p.ws = w2.ws; p.sw = w2.sw; p.sws = w2.sws;
  p.y = y;
  p.yb = yb;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.ntiles = s.H / 256; p.min_rows = min_rows;
  return launch_big(s, 1, p, st);
}

}  // namespace moe
