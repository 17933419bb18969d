// moe_gemm_big.hip -- grouped GEMMs for groups with many rows (prefill).
//
// When an expert holds ~100+ token rows (prefill: T = 4096, top-8 over 256
// experts gives ~128 rows per expert) a workgroup must cover all of them
// per pass, or each weight byte is read from HBM once per pass.  Here a
// workgroup of 8 waves owns 256 weight rows (a "unit") and up to CAP token
// rows (a "pass"), and walks K in steps of 128:
//   * both operands of a step travel HBM/L2 -> LDS by direct-to-LDS loads
//     (global_load_lds: 64 lanes x 16 B into 1 KB of LDS per instruction,
//     no registers held while in flight) through a ring of up to four
//     stages; a stage holds the step's token rows, weight tiles and MXFP4 or
//     NVFP4 weight scales, and the pass's token scales (and a unit's e4m3
//     block scales) sit in per-pass LDS tables, so nothing else is read from
//     memory in the K loop;
//   * weights come from the tiled layout (16-row x 128-K tiles in MFMA lane
//     order, see moe_tile.hip), one contiguous kilobyte per tile and step,
//     and land in LDS unchanged, so fragment reads are linear ds_read_b128;
//     token rows travel as whole 128-byte lines into a chunk-swizzled layout
//     whose fragment reads are conflict-free as well;
//   * the 8 waves form a 4 x 2 grid: a wave owns 4 weight tiles (64 rows;
//     in GEMM1 two gate and the two matching up tiles, so SwiGLU pairs meet
//     in one lane) and every second token tile, which keeps up to 4 x 5
//     fp32 accumulator tiles in registers;
//   * ping-pong: the two wave columns (one wave of each per SIMD) run half a
//     K step apart -- while column 0 reads step k's fragments out of LDS and
//     rescales its accumulators, column 1 multiplies step k - 1 from
//     registers, and the other way round in the second half -- so each
//     SIMD's matrix core is fed by one wave while the other waits on LDS,
//     instead of all eight waves waiting on the same read burst after each
//     barrier; one workgroup barrier per K step;
//   * the kernel is persistent (one workgroup per CU) and all tiles of one
//     expert run on one XCD (workgroup ids are dealt round-robin over the 8
//     XCDs), so the expert's token rows are fetched into that XCD's L2 once;
//     each workgroup finds its units' groups once (a table in LDS), loads
//     the next pass's token-row indices while the current pass runs, and
//     issues the next pass's first ring stages right after its epilogue.
// GEMM1 mode: weight rows are 128 gate + 128 up rows (128 h columns = one
// requantisation group of 128), epilogue SwiGLU + FP8 requantisation.
// GEMM2 mode: 256 output rows, epilogue writes y.
// NVFP4 weights (WF = 2: e2m1 codes, an e4m3 scale per 16 along K, an fp32
// scale per matrix): code tiles as MXFP4's, 2 KB of e4m3 scale tiles per
// unit and step; both operands are turned into fp16 in registers (exact) and
// multiplied on the fp16 MFMA (four 16x16x32 per 16x16x128 block), each
// step's products promoted with a VALU FMA like e4m3's; 96 token rows per
// pass at most (the fp16 operands and the step's products leave too few
// registers for more: 128 spilled inside the K loop and ran no faster).
// 4-bit activations (AF = 1, MXFP4 weights only): token rows are 64 bytes per
// K step (e2m1, two per byte) and their scales e8m0 per 32 channels, so the
// token operand's scale goes into the MFMA's B-operand scale like the
// weights' and the accumulators need no per-step rescale; GEMM1's epilogue
// requantises each wave row's 32 h columns (one MXFP4 group) to e2m1 + e8m0.
#include <algorithm>
#include <type_traits>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kBigThreads = 512;
constexpr int kWTiles = 16;           // 256 weight rows per unit
constexpr int kTabCap = 96;           // units of one workgroup described by one table build
constexpr int kLdsLimit = 160 * 1024;
constexpr int kMaxKSteps = 64;        // K <= 8192: a pass's token scales fit one table
constexpr int kXsRow = kMaxKSteps + 1;  // floats per table row (odd: conflict-free column reads)

// Geometry of one instantiation: weight format WF and token rows per pass
// CAP (160 for prefill-sized groups, 64 when groups are smaller).  Every
// wave issues the same kL direct-to-LDS loads of 16 bytes per lane per step
// (token rows, weight tiles, MXFP4 scales; spare slots load one hot line
// into the stage's sink).  A pass's token scales, [token][k step], and the
// unit's two e4m3 block-scale rows are read once per pass into tables.
template <int WF, int CAP, int AF> struct BigGeo {
  static constexpr int kTokTiles = CAP / 16;
  static constexpr int kTokPerWave = kTokTiles / 2;          // token tiles of one wave column
  static constexpr int kTokTileBytes = AF ? 1024 : 2048;     // 16 rows x 64 B (e2m1) or 128 B (e4m3)
  static constexpr int kTokLoads = AF ? kTokTiles : 2 * kTokTiles;  // 1 KB each: 16 x 64 B or 8 x 128 B
  static constexpr int kTokSlots = (kTokLoads + 7) / 8;      // token-row loads of one wave
  static constexpr int kWLoads = WF != 0 ? kWTiles : 2 * kWTiles;  // 1 KB each
  // 16 tiles x 64 B of e8m0 scales (MXFP4), or x 128 B of e4m3 scales (NVFP4)
  static constexpr int kScLoads = WF == 1 ? 1 : WF == 2 ? 2 : 0;
  static constexpr int kL = (kTokLoads + kWLoads + kScLoads + 7) / 8;
  static constexpr int kWOff = kTokTiles * kTokTileBytes;    // token tiles, chunk-swizzled
  static constexpr int kScOff = kWOff + kWLoads * 1024;
  static constexpr int kSinkOff = kScOff + kScLoads * 1024;
  static constexpr int kStageBytes = kSinkOff + 1024;
  static constexpr int kXsTabFloats = CAP * kXsRow;           // token scales of the pass
  static constexpr int kWsTabFloats = WF == 0 ? 2 * kXsRow : 1;  // e4m3 block scales of the unit
  static constexpr int kTabLoads = (CAP + 7) / 8;            // token-scale rows per wave
  static constexpr int kRedFloats = 4 * CAP;                 // epilogue maxima: per wave row, per token
  static constexpr int kFixedBytes = (kXsTabFloats + kWsTabFloats + kRedFloats) * 4 + kTabCap * 16 + 64;
  static constexpr int kStagesFit = (kLdsLimit - kFixedBytes) / kStageBytes;
  static constexpr int kStages = kStagesFit < 4 ? kStagesFit : 4;
  static_assert(kStageBytes % 256 == 0, "stage alignment");
  static_assert(kStages >= 2, "a ring of two stages at least");
  static_assert(kTabLoads <= 64, "token-scale rows of a wave fit one register");
  static_assert(kTokPerWave <= 5, "token tiles per wave");
  static_assert(kTokSlots <= 3, "token-row loads per wave");
  static_assert((kStages - 2) * kL < 64, "vmcnt range");
};

struct BigParams {
  const uint8_t* act;        // GEMM1: xq [T][H] by token; GEMM2: hq [rows][I] by row
  const float* act_s;        // its per-128 scales
  const int32_t* row_token;  // GEMM1 only (null in GEMM2 mode)
  const int32_t* offsets;
  const uint8_t* w;
  const void* ws;
  const uint8_t* sw;
  const void* sws;
  const float* wg;   // NVFP4: fp32 scale per routed matrix
  const float* swg;  // and the shared expert's
  uint8_t* hq;
  float* hs;
  float* y;
  uint16_t* yb;  // bf16 y instead when non-null (layer-internal)
  int H, I, E, G, wblk, ngroups, ntiles, units, per_xcd, min_rows;
};

// one 16-byte-per-lane direct load into LDS: lane l's bytes land at
// lds_base + 16 * l (lds_base wave-uniform).  Token rows are re-read by the
// group's other units and keep the default policy; weights and their scales
// are read once per pass and go non-temporal (cache-policy operand nt).
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma16nt(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 2);
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

// the same for a 1 KB tile of 64-byte rows (e2m1 tokens, chunks 0..3): the
// chunk index is XOR-ed with (r / 4) & 3, which puts the 16 rows' chunk-c
// reads on distinct banks; one direct-to-LDS load covers the whole tile
__device__ __forceinline__ int tok_swz4(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// instruction classes the scheduler may move across a load-issue point (the
// sched_barrier mask): ALU, VALU, SALU, MFMA, LDS reads, transcendentals --
// not the vector-memory loads themselves
constexpr int kSchedMayCross = 0x0001 | 0x0002 | 0x0004 | 0x0008 | 0x0100 | 0x0400;

// workgroup barrier after this wave's LDS reads and writes have completed;
// outstanding vector-memory loads stay in flight (unlike __syncthreads,
// whose release fence waits for them): the waits for the ring's
// direct-to-LDS loads are explicit (wait_vmcnt).  No instruction is
// scheduled across it (the compiler would otherwise sink MFMAs, which touch
// registers only, below the barrier into the next phase).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), other counters at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

template <int WF, int MODE, int CAP, int AF>
__global__ __launch_bounds__(kBigThreads) void k_gemm_big(BigParams p) {
  static_assert(AF == 0 || WF == 1, "4-bit activations run with MXFP4 weights");
  using Geo = BigGeo<WF, CAP, AF>;
  constexpr int S = Geo::kStages, L = Geo::kL, NTMAX = Geo::kTokPerWave;
  // one array per ring stage: the compiler's alias analysis then tells the
  // stages apart and waits for a stage's own direct-to-LDS loads only
  __shared__ __align__(256) uint8_t st0[Geo::kStageBytes];
  __shared__ __align__(256) uint8_t st1[Geo::kStageBytes];
  __shared__ __align__(256) uint8_t st2[S >= 3 ? Geo::kStageBytes : 256];
  __shared__ __align__(256) uint8_t st3[S >= 4 ? Geo::kStageBytes : 256];
  __shared__ __align__(16) float xs_tab[Geo::kXsTabFloats];
  __shared__ __align__(16) float ws_tab[Geo::kWsTabFloats];
  __shared__ __align__(16) float red[Geo::kRedFloats];
  __shared__ int4 tab[kTabCap];  // per unit of this workgroup: group, first row, rows, tile in group
  __shared__ int s_wsum[8];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, m = lane & 15, g = lane >> 4;
  const int wr = w & 3, wc = w >> 2;     // wave row (weight tiles), wave column (token tiles, ping-pong side)
  const int H = p.H, I = p.I;
  const int K = MODE == 0 ? H : I;       // reduction length
  const int NR = MODE == 0 ? 2 * I : H;  // weight rows of the matrix
  const int kb = WF == 0 ? K : K / 2;    // bytes per weight row
  const int ka = AF ? K / 2 : K;         // bytes per token row
  const int nks = K / 128;
  const long wstep = long(NR / 16) * kTileBytes<WF>;  // tiled weights: bytes per K step
  const long sstep = long(NR / 16) * (WF == 2 ? kTileScaleBytes16 : kTileScaleBytes);
  // this wave's weight tiles among the unit's 16 (GEMM1: tiles 0..7 are gate
  // rows, 8..15 the up rows of the same h columns; GEMM2 rows in order)
  int ja[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ja[q] = MODE == 0 ? (q < 2 ? 2 * wr + q : 8 + 2 * wr + (q - 2)) : 4 * wr + q;

  // ---- the units of this workgroup: workgroup ids are dealt round-robin
  // over the 8 XCDs, and XCD x works through units [x per_xcd, (x + 1)
  // per_xcd) with its nwx workgroups, unit i of this one being
  // x per_xcd + j0 + i nwx, so all tiles of one group run on one XCD and
  // share its L2
  const int xcd = blockIdx.x & 7, j0 = blockIdx.x >> 3, nwx = gridDim.x >> 3;
  const int ubase = xcd * p.per_xcd;
  const int kmax = min(p.per_xcd, p.units - ubase);
  const int nunits = kmax > j0 ? (kmax - j0 + nwx - 1) / nwx : 0;
  if (nunits <= 0) return;

  // table of units i0 .. i0 + kTabCap - 1: unit u belongs to slot u / ntiles,
  // slot r being the r-th group with at least min_rows rows; units past the
  // last such group keep group -1.  Every wave takes part (two barriers).
  int tab0 = 0;
  auto build_table = [&](int i0) __attribute__((always_inline)) {
    tab0 = i0;
    for (int idx = tid; idx < kTabCap; idx += kBigThreads) tab[idx] = make_int4(-1, 0, 0, 0);
    const int gpt = (p.ngroups + kBigThreads - 1) / kBigThreads;
    int local = 0;
    for (int q = 0; q < gpt; ++q) {
      const int gg = tid * gpt + q;
      if (gg < p.ngroups && p.offsets[gg + 1] - p.offsets[gg] >= p.min_rows) ++local;
    }
    int incl = local;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wsum[w] = incl;
    lds_barrier();
    int r = incl - local;
    for (int q = 0; q < w; ++q) r += s_wsum[q];
    for (int q = 0; q < gpt; ++q) {
      const int gg = tid * gpt + q;
      if (gg >= p.ngroups) break;
      const int o0 = p.offsets[gg], cnt = p.offsets[gg + 1] - o0;
      if (cnt < p.min_rows) continue;
      // this workgroup's units of slot r
      const int ulo = max(r * p.ntiles, ubase + j0), uhi = min((r + 1) * p.ntiles, ubase + kmax);
      for (int u = ulo + (nwx - (ulo - ubase - j0) % nwx) % nwx; u < uhi; u += nwx) {
        const int ii = (u - ubase - j0) / nwx - i0;
        if (ii >= 0 && ii < kTabCap) tab[ii] = make_int4(gg, o0, cnt, u - r * p.ntiles);
      }
      ++r;
    }
    lds_barrier();
  };

  // ---- per-lane token index of this wave's token-row load slot j (load
  // i = w + 8 j < kTokLoads: tile i / 2, rows 8 (i % 2) .. + 7, lane l on
  // row 8 (i % 2) + l / 8); the wave's token-scale table rows are tokens
  // w + 8 i (lane i holds the row of the i-th); rows past the pass repeat
  // its last row
  auto tok_of_slot = [&](int j) __attribute__((always_inline)) {
    const int i = w + 8 * j;
    return AF ? i * 16 + (lane >> 2) : (i >> 1) * 16 + (i & 1) * 8 + (lane >> 3);
  };
  int pf_row[Geo::kTokSlots], pf_tab = 0;  // rows of the next pass to load (GEMM1: token ids)
  bool pf_ok = false;
  auto prefetch = [&](int4 ent, int pass) __attribute__((always_inline)) {
    const int npass = min(CAP, ent.z - pass * CAP);
    const int base = ent.y + pass * CAP;
#pragma unroll
    for (int j = 0; j < Geo::kTokSlots; ++j) {
      pf_row[j] = 0;
      if (w + 8 * j < Geo::kTokLoads) {
        const int r = base + min(tok_of_slot(j), npass - 1);
        pf_row[j] = MODE == 0 ? p.row_token[r] : r;
      }
    }
    pf_tab = 0;
    if (lane < Geo::kTabLoads) {
      const int r = base + min(w + 8 * lane, npass - 1);
      pf_tab = MODE == 0 ? p.row_token[r] : r;
    }
    pf_ok = true;
  };

  // ---- loader state of the pass being loaded: per load slot the per-lane
  // source of the next step to issue (steps are issued in order, each slot
  // once per step, so the source just advances by the slot's stride), and
  // a destination offset in the stage
  const uint8_t* src16[L];
  long stride16[L];
  int dst16[L];
  int tab_row = 0;          // this wave's token-scale rows of the pass (lane i: token w + 8 i)
  const float* ws_src = nullptr;  // e4m3: the block-scale row this wave loads (waves 0, 1)
  int ld_row = 0, ld_npass = 0, ld_n0 = 0, ld_ntw = 0;  // first row of the pass, its rows, unit column, tiles
  float ld_gsc = 1.0f;      // NVFP4: the matrix scale of the pass's expert
  auto setup = [&](int4 ent, int pass) __attribute__((always_inline)) {
    if (!pf_ok) prefetch(ent, pass);
    pf_ok = false;
    const int e = ent.x;
    ld_n0 = ent.w * (MODE == 0 ? 128 : 256);
    ld_row = ent.y + pass * CAP;
    ld_npass = min(CAP, ent.z - pass * CAP);
    const int ntt = (ld_npass + 15) / 16;
    ld_ntw = (ntt + 1 - wc) / 2;  // token tiles of this wave: t = 2 tt + wc
    const bool shared = e == p.E;
    const long ee = shared ? 0 : e;
    const uint8_t* wmat = (shared ? p.sw : p.w) + ee * long(NR) * kb;
    const void* smat = shared ? p.sws : p.ws;
    if (WF == 2) ld_gsc = shared ? p.swg[0] : p.wg[ee];
    const int n0 = ld_n0;
    // first matrix row of unit weight tile t (0..15)
    auto wtile_row = [&](int t) __attribute__((always_inline)) { return MODE == 0 ? (t < 8 ? n0 + 16 * t : I + n0 + 16 * (t - 8)) : n0 + 16 * t; };
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int i = w + 8 * j;
      if (i < Geo::kTokLoads) {
        const long trow = pf_row[j < Geo::kTokSlots ? j : 0];
        if (AF) {
          // lane l fills LDS chunk l % 4 of tile row l / 4, i.e. global chunk (l % 4) ^ ((row / 4) & 3)
          const int rl = lane >> 2;
          src16[j] = p.act + trow * ka + (((lane & 3) ^ ((rl >> 2) & 3)) << 4);
          stride16[j] = 64;
        } else {
          // lane l fills LDS chunk l % 8 of its row, i.e. global chunk (l % 8) ^ (row & 7)
          const int rl = (i & 1) * 8 + (lane >> 3);
          src16[j] = p.act + trow * ka + (((lane & 7) ^ (rl & 7)) << 4);
          stride16[j] = 128;
        }
        dst16[j] = i * 1024;
      } else if (i < Geo::kTokLoads + Geo::kWLoads) {
        const int wi = i - Geo::kTokLoads;
        const int t = WF != 0 ? wi : wi >> 1, half = WF != 0 ? 0 : wi & 1;
        src16[j] = wmat + long(wtile_row(t) / 16) * kTileBytes<WF> + half * 1024 + lane * 16;
        stride16[j] = wstep;
        dst16[j] = Geo::kWOff + wi * 1024;
      } else if (i < Geo::kTokLoads + Geo::kWLoads + Geo::kScLoads) {
        if (WF == 2) {
          // NVFP4: load si = 0 the 8 tiles from unit tile 0 (1 KB adjacent),
          // si = 1 those from unit tile 8
          const int si = i - Geo::kTokLoads - Geo::kWLoads;
          const uint8_t* sb = static_cast<const uint8_t*>(smat) + ee * long(NR) * (K / 16);
          src16[j] = sb + long(wtile_row(8 * si) / 16) * kTileScaleBytes16 + lane * 16;
          dst16[j] = Geo::kScOff + si * 1024;
        } else {
          // the 16 tiles' e8m0 scales: lanes 0..31 the 8 tiles from unit tile 0
          // (512 adjacent bytes), lanes 32..63 those from unit tile 8
          const uint8_t* sb = static_cast<const uint8_t*>(smat) + ee * long(NR) * (K / 32);
          src16[j] = sb + long(wtile_row(lane < 32 ? 0 : 8) / 16) * kTileScaleBytes + (lane & 31) * 16;
          dst16[j] = Geo::kScOff;
        }
        stride16[j] = sstep;
      } else {  // spare slot: one hot line into the sink
        src16[j] = wmat;
        stride16[j] = 0;
        dst16[j] = Geo::kSinkOff;
      }
    }
    tab_row = pf_tab;
    if (WF == 0 && w < 2) {
      // e4m3 128 x 128 block scales of the unit's row block w (GEMM1: gate, up)
      const int brow = MODE == 0 ? (w ? I + n0 : n0) / 128 : n0 / 128 + w;
      ws_src = static_cast<const float*>(smat) + ee * long(NR / 128) * nks + long(brow) * nks;
    }
  };

  // this wave's direct-to-LDS loads [j0, j1) of its kL for the next step
  // (ks, the step they belong to, is implied by the order) into stage st
  auto issue_range = [&](int ks, uint8_t* st, int ja0, int ja1) __attribute__((always_inline)) {
    (void)ks;
#pragma unroll
    for (int j = 0; j < L; ++j)
      if (j >= ja0 && j < ja1) {
        // slot j is a token-row load in wave w when w + 8 j < kTokLoads
        if (8 * j + 7 < Geo::kTokLoads) dma16(src16[j], st + dst16[j]);
        else if (8 * j >= Geo::kTokLoads) dma16nt(src16[j], st + dst16[j]);
        else if (w + 8 * j < Geo::kTokLoads) dma16(src16[j], st + dst16[j]);
        else dma16nt(src16[j], st + dst16[j]);
        src16[j] += stride16[j];
      }
  };
  auto stage_ptr = [&](int s) __attribute__((always_inline)) -> uint8_t* { return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3; };
  // first loads of a pass: the token-scale table (one load per token: its
  // nks scales are contiguous; lanes past them repeat the last) and the
  // e4m3 block-scale rows, written to LDS by the waves themselves, then
  // steps 0 .. S - 2 into stages 0 .. S - 2.  The tables go through
  // registers, not direct-to-LDS loads: the compiler tracks a direct-to-LDS
  // load by its LDS target, and a K loop that reads a table so filled got a
  // wait for every load in flight (the ring's included) on each of its
  // iterations.  Filled this way, the tables cost one wait per pass, before
  // the first stage is issued; the first barrier of the K loop publishes
  // them.
  auto prologue = [&]() __attribute__((always_inline)) {
    float tv[Geo::kTabLoads];
#pragma unroll
    for (int i = 0; i < Geo::kTabLoads; ++i) {
      const int arow = __builtin_amdgcn_readlane(tab_row, i);
      tv[i] = p.act_s[long(arow) * nks + min(lane, nks - 1)];
    }
    float wv = 0.0f;
    if (WF == 0 && w < 2) wv = ws_src[min(lane, nks - 1)];
#pragma unroll
    for (int i = 0; i < Geo::kTabLoads; ++i) xs_tab[(w + 8 * i) * kXsRow + lane] = tv[i];
    if (WF == 0 && w < 2) ws_tab[w * kXsRow + lane] = wv;
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nks) issue_range(s, stage_ptr(s), 0, L);
  };
  // before step k's first read: this wave's loads of steps k + 1 ..
  // min(k + S - 2, nks - 1) may stay in flight (rem = nks - 1 - k)
  auto wait_ring = [&](int rem) __attribute__((always_inline)) {
    if (rem >= S - 2) wait_vmcnt<(S - 2) * L>();
    else if (rem == 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  };

  // ---- accumulators: e4m3 weights promote each step's MFMA result with a
  // VALU FMA (acc += d * ws * xs).  MXFP4 weights carry their e8m0 scales
  // inside the MFMA, and so does each token's scale xs = mt * 2^et (mt in
  // [1, 2)): its power of two 2^et is the MFMA's B-operand scale, exact
  // whatever the exponent.  The accumulator is kept in units of the current
  // step's mantissa mt: when a step's fragments are read it is multiplied by
  // mt_prev / mt_cur, a ratio in (1/2, 2) that cannot overflow or underflow
  // however far apart two steps' token scales are (an all-zero group next to
  // a huge one), then the MFMA adds the step's product in place; the epilogue
  // multiplies by the last step's mt.  Token scales are positive normal
  // floats (at least 2^-64 / 448), so the split is always defined.
  v4f acc[4][NTMAX];
  float xsp[NTMAX];  // MXFP4: the token-scale mantissas of the previous step
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < NTMAX; ++t) acc[q][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) xsp[t] = 0.0f;
  };
  zero_acc();

  // ---- epilogue of a finished pass (c_*: its first row, rows, unit column
  // and this wave's tile count).  GEMM1: part 1 forms h = silu(gate) * up in
  // place of the gate accumulators (h column n0 + 32 wr + 16 q + 4 g + i,
  // token 16 t + m with t = 2 tt + wc) and posts each token's partial
  // maximum to LDS; part 2, after a barrier, requantises with the maximum
  // over the four wave rows.  GEMM2: part 1 stores y.  Outputs go through
  // LDS so that the global stores write whole 128-byte lines: the last ring
  // stage holds them (the next pass's first loads go to stages 0 .. S - 2,
  // and stage S - 1 is not written before the next A(0) barrier, which every
  // wave reaches after its epilogue).
  constexpr int kEPitch = 144;  // bytes per buffered row: 128 of data + 16 (rows 36 banks apart)
  static_assert(CAP * kEPitch <= Geo::kStageBytes && 8 * 16 * kEPitch <= Geo::kStageBytes,
                "epilogue buffers fit one stage");
  uint8_t* const ebuf = stage_ptr(S - 1);
  int c_row = 0, c_npass = 0, c_n0 = 0, c_ntw = 0;
  float c_gsc = 1.0f;
  auto epi1 = [&]() __attribute__((always_inline)) {
    if (MODE == 0 && AF) {
      // 4-bit activations: the wave row's 32 h columns of a token are one
      // MXFP4 group, so its maximum is a reduction over the wave alone; codes
      // go to the buffer row of the token (64 bytes per unit), the e8m0 scale
      // straight to hs
      uint8_t* const hs8 = reinterpret_cast<uint8_t*>(p.hs);
#pragma unroll
      for (int tt = 0; tt < NTMAX; ++tt) {
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = swiglu(acc[q][tt][i], acc[q + 2][tt][i]);
            acc[q][tt][i] = v;
            amax = fmaxf(amax, fabsf(v));
          }
        amax = wave_max_xor(amax, 16);
        amax = wave_max_xor(amax, 32);
        if (tt >= c_ntw) continue;
        const int idx = (2 * tt + wc) * 16 + m;
        const uint32_t code = mx_scale_code(amax);
        const float inv = mx_inv_scale(code);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const v4f& hv = acc[q][tt];
          const uint32_t nib = enc_e2m1(hv[0] * inv) | (enc_e2m1(hv[1] * inv) << 4) |
                               (enc_e2m1(hv[2] * inv) << 8) | (enc_e2m1(hv[3] * inv) << 12);
          *reinterpret_cast<uint16_t*>(ebuf + idx * kEPitch + 16 * wr + 8 * q + 2 * g) = uint16_t(nib);
        }
        if (g == 0 && idx < c_npass) hs8[long(c_row + idx) * (I / 32) + c_n0 / 32 + wr] = uint8_t(code);
      }
    } else if (MODE == 0) {
#pragma unroll
      for (int tt = 0; tt < NTMAX; ++tt) {
        if (WF == 1)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q][tt] *= xsp[tt];
        if (WF == 2)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q][tt] *= c_gsc;
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = swiglu(acc[q][tt][i], acc[q + 2][tt][i]);
            acc[q][tt][i] = v;
            amax = fmaxf(amax, fabsf(v));
          }
        amax = wave_max_xor(amax, 16);
        amax = wave_max_xor(amax, 32);
        if (g == 0 && tt < c_ntw) red[wr * CAP + (2 * tt + wc) * 16 + m] = amax;
      }
    } else {
      // this wave's 16 x 64 block of a token tile, row by row through its
      // own slice of the buffer: 128 bytes per row (bf16: 64 columns; fp32:
      // 32 columns, two halves)
      uint8_t* const wb = ebuf + w * (16 * kEPitch);
      const int rr = lane >> 3, ch = lane & 7;  // read-back: rows rr, rr + 8, 16-byte chunk ch
#pragma unroll
      for (int tt = 0; tt < NTMAX; ++tt) {
        if (tt >= c_ntw) continue;
        const int t0 = (2 * tt + wc) * 16;
        v4f v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = (WF == 1 && !AF) ? acc[q][tt] * xsp[tt] : WF == 2 ? acc[q][tt] * c_gsc : acc[q][tt];
        if (p.yb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = f32_to_bf16(v[q][0]) | (f32_to_bf16(v[q][1]) << 16);
            o.y = f32_to_bf16(v[q][2]) | (f32_to_bf16(v[q][3]) << 16);
            *reinterpret_cast<uint2*>(wb + m * kEPitch + (16 * q + 4 * g) * 2) = o;
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 8 * h + rr;
            const v4u d = *reinterpret_cast<const v4u*>(wb + row * kEPitch + ch * 16);
            if (t0 + row < c_npass)
              *reinterpret_cast<v4u*>(p.yb + long(c_row + t0 + row) * H + c_n0 + 64 * wr + ch * 8) = d;
          }
        } else {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
              *reinterpret_cast<v4f*>(wb + m * kEPitch + (16 * q + 4 * g) * 4) = v[2 * half + q];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int row = 8 * h + rr;
              const v4u d = *reinterpret_cast<const v4u*>(wb + row * kEPitch + ch * 16);
              if (t0 + row < c_npass)
                *reinterpret_cast<v4u*>(p.y + long(c_row + t0 + row) * H + c_n0 + 64 * wr + 32 * half + ch * 4) = d;
            }
          }
        }
      }
    }
  };
  auto epi2 = [&]() __attribute__((always_inline)) {
    if (MODE != 0) return;
    if (AF) {  // the codes are in the buffer (epi1): 64 bytes per token
      for (int c = tid; c < c_npass * 4; c += kBigThreads) {
        const int row = c >> 2, part = c & 3;
        *reinterpret_cast<v4u*>(p.hq + long(c_row + row) * (I / 2) + c_n0 / 2 + part * 16) =
            *reinterpret_cast<const v4u*>(ebuf + row * kEPitch + part * 16);
      }
      return;
    }
    // codes of the pass's tokens: [token][128 h columns] in the buffer
#pragma unroll
    for (int tt = 0; tt < NTMAX; ++tt) {
      if (tt >= c_ntw) continue;
      const int idx = (2 * tt + wc) * 16 + m;
      float am = red[idx];
#pragma unroll
      for (int q = 1; q < 4; ++q) am = fmaxf(am, red[q * CAP + idx]);
      const float mult = quant_mult(am);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const v4f& hv = acc[q][tt];
        const uint32_t word = enc_e4m3x4(hv[0] * mult, hv[1] * mult, hv[2] * mult, hv[3] * mult);
        *reinterpret_cast<uint32_t*>(ebuf + idx * kEPitch + 32 * wr + 16 * q + 4 * g) = word;
      }
      if (g == 0 && wr == 0 && idx < c_npass) p.hs[long(c_row + idx) * (I / 128) + c_n0 / 128] = 1.0f / mult;
    }
    lds_barrier();
    for (int c = tid; c < c_npass * 8; c += kBigThreads) {
      const int row = c >> 3, part = c & 7;
      *reinterpret_cast<v4u*>(p.hq + long(c_row + row) * I + c_n0 + part * 16) =
          *reinterpret_cast<const v4u*>(ebuf + row * kEPitch + part * 16);
    }
  };

  // ---- work items: (unit i, pass) in order
  auto entry_of = [&](int i) __attribute__((always_inline)) -> int4 {
    if (i >= nunits) return make_int4(-1, 0, 0, 0);
    return tab[i - tab0];
  };
  auto next_of = [&](int i, int pass, int4 e, int& ni, int& np) __attribute__((always_inline)) {
    if ((pass + 1) * CAP < e.z) { ni = i; np = pass + 1; }
    else { ni = i + 1; np = 0; }
  };

  int ui = 0, upass = 0;
  build_table(0);
  int4 ent = entry_of(0);
  if (ent.x < 0) return;
  setup(ent, 0);
  {
    int ni, np;
    next_of(ui, upass, ent, ni, np);
    if (ni < nunits && ni < tab0 + kTabCap) {
      const int4 e2 = entry_of(ni);
      if (e2.x >= 0) prefetch(e2, np);
    }
  }
  prologue();

  // ---- one pass: half steps A(0), B(0), ..., A(nks), the same barriers in
  // every wave whatever its tile count NT
  auto run_pass = [&](auto ntc) __attribute__((always_inline)) {
    constexpr int NT = decltype(ntc)::value;
    constexpr int NA = NT > 0 ? NT : 1;  // array extent (no zero-length arrays)
    v8i af[4];
    int sa[4];
    float wsv[4];
    float xsv[NA];
    int sb[NA];  // MXFP4: e8m0 code of each token's scale exponent (B-operand scale)
    v8i bf[NA];
    // the fragments of step k in stage st; MXFP4: rescale to its token scales
    auto READ = [&](const uint8_t* st, int k) __attribute__((always_inline)) {
      // the step index passes through an empty asm statement, so the table
      // addresses are formed afresh at each step rather than carried in a
      // loop register (which the compiler may spill and reload before the
      // loop, and whose first use in the loop then waits for every load in
      // flight)
      asm volatile("" : "+s"(k));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (WF == 1) {
          const v4u a = *reinterpret_cast<const v4u*>(st + Geo::kWOff + ja[q] * 1024 + lane * 16);
          af[q] = v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
          sa[q] = st[Geo::kScOff + ja[q] * kTileScaleBytes + lane];
          wsv[q] = 1.0f;
        } else if (WF == 2) {
          // codes as MXFP4's; the lane's two e4m3 block scales (16-blocks 2g, 2g + 1 of row m)
          const v4u a = *reinterpret_cast<const v4u*>(st + Geo::kWOff + ja[q] * 1024 + lane * 16);
          af[q] = v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
          sa[q] = *reinterpret_cast<const uint16_t*>(st + Geo::kScOff + ja[q] * kTileScaleBytes16 + 8 * m + 2 * g);
          wsv[q] = 1.0f;
        } else {
          const v4u lo = *reinterpret_cast<const v4u*>(st + Geo::kWOff + (2 * ja[q]) * 1024 + lane * 16);
          const v4u hi = *reinterpret_cast<const v4u*>(st + Geo::kWOff + (2 * ja[q] + 1) * 1024 + lane * 16);
          af[q] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
          sa[q] = kUnitScale;
          // unit tiles 0..7 lie in the first 128-row block, 8..15 in the second
          wsv[q] = ws_tab[(ja[q] >> 3) * kXsRow + k];
        }
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int t = 2 * tt + wc;
        xsv[tt] = xs_tab[(t * 16 + m) * kXsRow + k];
        if (AF) {
          // e2m1 tokens: 16 bytes (32 K) per lane; the step's four e8m0 scales
          // of the token are one table word, byte g the scale of lane group g
          const v4u b = *reinterpret_cast<const v4u*>(st + t * 1024 + tok_swz4(m, g));
          bf[tt] = v8i{int(b[0]), int(b[1]), int(b[2]), int(b[3]), 0, 0, 0, 0};
          sb[tt] = int((__float_as_uint(xsv[tt]) >> (8 * g)) & 0xFFu);
        } else {
          // e4m3 operand order: chunks g and 4 + g of the row's 128 bytes;
          // NVFP4's fp16 path: the lane's 32 consecutive K, chunks 2g, 2g + 1
          const v4u lo = *reinterpret_cast<const v4u*>(st + t * 2048 + tok_swz(m, WF == 2 ? 2 * g : g));
          const v4u hi = *reinterpret_cast<const v4u*>(st + t * 2048 + tok_swz(m, WF == 2 ? 2 * g + 1 : 4 + g));
          bf[tt] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        }
      }
      if (WF == 1 && !AF) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          // xs = mantissa * 2^(e - 127): the biased exponent field is the
          // e8m0 code of that power of two; the mantissa keeps the low bits
          const uint32_t u = __float_as_uint(xsv[tt]);
          sb[tt] = int(u >> 23);
          const float mt = __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u);
          const float rr = xsp[tt] * __builtin_amdgcn_rcpf(mt);
          xsp[tt] = mt;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q][tt] *= rr;
        }
      }
    };
    // multiply the fragments in registers; the loads of step kn (when there
    // is one) go out into stage iss between the token tiles
    auto MMA = [&](int kn, uint8_t* iss) __attribute__((always_inline)) {
      const bool go = kn < nks;
      if (WF == 2) {
        // NVFP4: the step as four K quarters (lane group g: K 32 g + 8 i ..
        // + 7 of both operands in quarter i): per quarter the wave's four
        // weight tiles are turned into fp16 once (code times block scale,
        // exact) and multiplied with every token tile, whose e4m3 codes are
        // turned into fp16 likewise (exact); the step's products, one set
        // per token tile, are then promoted with the token scale.  The loads
        // of step kn go out between the quarters.
        v4f d[4][NA];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int tt = 0; tt < NA; ++tt) d[q][tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h8v a[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const h2v sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uint32_t(sa[q]), 1.0f, false);
            a[q] = cvt_e2m1x8_f16(uint32_t(af[q][i])) * (i < 2 ? sc[0] : sc[1]);
          }
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const h8v b = cvt_e4m3x8_f16(bf[tt][2 * i], bf[tt][2 * i + 1]);
#pragma unroll
            for (int q = 0; q < 4; ++q) d[q][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[q], b, d[q][tt], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(kSchedMayCross);
          if (go) issue_range(kn, iss, i * L / 4, (i + 1) * L / 4);
          __builtin_amdgcn_sched_barrier(kSchedMayCross);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q][tt] += d[q][tt] * xsv[tt];
        if (NT == 0 && go) issue_range(kn, iss, 0, L);
        return;
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        if (AF) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[q][tt] = mfma_scaled_acc<kFmtE2M1, kFmtE2M1>(af[q], bf[tt], acc[q][tt], sa[q], sb[tt]);
        } else if (WF == 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[q][tt] = mfma_scaled_acc<kFmtE2M1, kFmtE4M3>(af[q], bf[tt], acc[q][tt], sa[q], sb[tt]);
        } else {
          v4f d[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) d[q] = mfma_scaled<kFmtE4M3, kFmtE4M3>(af[q], bf[tt], kUnitScale, kUnitScale);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q][tt] += d[q] * (wsv[q] * xsv[tt]);
        }
        __builtin_amdgcn_sched_barrier(kSchedMayCross);
        if (go) issue_range(kn, iss, tt * L / NA, (tt + 1) * L / NA);
        __builtin_amdgcn_sched_barrier(kSchedMayCross);
      }
      if (NT == 0 && go) issue_range(kn, iss, 0, L);
    };
    // one barrier A(k) per step: after it column 0 reads step k's fragments
    // and multiplies them, while column 1 first multiplies step k - 1 from
    // registers and then reads step k, so the two columns of a SIMD stay half
    // a step apart and one's LDS reads overlap the other's MFMAs.  Each side
    // issues its loads of step k + S - 1 while it multiplies, into the stage
    // step k - 1 used: every wave finished reading that stage before A(k).
    // A(k) also publishes step k: every wave waits for its own loads of the
    // step before it.  The two columns run separate loops with the same
    // barriers (one straight-line order each).
    if (wc == 0) {
      wait_ring(nks - 1);
      lds_barrier();  // A(0)
      READ(st0, 0);
      MMA(S - 1, stage_ptr(S - 1));
      auto half_pair = [&](int k, const uint8_t* cur, uint8_t* iss) __attribute__((always_inline)) {
        wait_ring(nks - 1 - k);
        lds_barrier();  // A(k)
        READ(cur, k);
        MMA(k + S - 1, iss);
      };
      for (int k = 1; k < nks; k += S) {
        half_pair(k, stage_ptr(1 % S), stage_ptr(0));
        if (k + 1 < nks) half_pair(k + 1, stage_ptr(2 % S), stage_ptr(1 % S));
        if (S >= 3 && k + 2 < nks) half_pair(k + 2, stage_ptr(3 % S), stage_ptr(2 % S));
        if (S >= 4 && k + 3 < nks) half_pair(k + 3, stage_ptr(4 % S), stage_ptr(3 % S));
      }
      lds_barrier();  // A(nks)
    } else {
      wait_ring(nks - 1);
      lds_barrier();  // A(0)
      if (S - 1 < nks) issue_range(S - 1, stage_ptr(S - 1), 0, L);
      READ(st0, 0);
      auto half_pair = [&](int k, const uint8_t* cur, uint8_t* iss) __attribute__((always_inline)) {
        wait_ring(nks - 1 - k);
        lds_barrier();  // A(k)
        MMA(k + S - 1, iss);
        READ(cur, k);
      };
      for (int k = 1; k < nks; k += S) {
        half_pair(k, stage_ptr(1 % S), stage_ptr(0));
        if (k + 1 < nks) half_pair(k + 1, stage_ptr(2 % S), stage_ptr(1 % S));
        if (S >= 3 && k + 2 < nks) half_pair(k + 2, stage_ptr(3 % S), stage_ptr(2 % S));
        if (S >= 4 && k + 3 < nks) half_pair(k + 3, stage_ptr(4 % S), stage_ptr(3 % S));
      }
      lds_barrier();  // A(nks): multiply the last step
      MMA(nks, st0);
    }
  };
  // compiled tile counts: NTMAX and the two below it (at least 1); a wave
  // with fewer tiles runs the smallest and multiplies tiles the epilogue
  // ignores (their token rows repeat the pass's last row)
  constexpr int NT1 = NTMAX > 1 ? NTMAX - 1 : 1, NT2 = NTMAX > 2 ? NTMAX - 2 : 1;
  auto run_pass_any = [&](int nt) __attribute__((always_inline)) {
    if (nt >= NTMAX) run_pass(std::integral_constant<int, NTMAX>{});
    else if (NT1 < NTMAX && nt >= NT1) run_pass(std::integral_constant<int, NT1>{});
    else if (NT2 < NT1) run_pass(std::integral_constant<int, NT2>{});
    else run_pass(std::integral_constant<int, NT1>{});
  };

  while (true) {
    run_pass_any(ld_ntw);
    // nothing is in flight here (the last step waited for every load), and
    // saying so lets the compiler use the prefetched rows without a wait
    // behind the epilogue's stores
    wait_vmcnt<0>();
    // ---- the pass's epilogue first (the accumulators die with it, which
    // leaves the registers to the next pass's set-up), then the next pass's
    // first loads: every stage is free (the last reads were in B(nks - 1))
    c_row = ld_row; c_npass = ld_npass; c_n0 = ld_n0; c_ntw = ld_ntw; c_gsc = ld_gsc;
    epi1();
    lds_barrier();
    epi2();
    zero_acc();
    int ni, np;
    next_of(ui, upass, ent, ni, np);
    if (ni >= nunits) ni = -1;
    if (ni >= 0 && ni >= tab0 + kTabCap) {
      build_table(ni);
      pf_ok = false;
    }
    const int4 nent = ni >= 0 ? entry_of(ni) : make_int4(-1, 0, 0, 0);
    if (nent.x < 0) break;
    ui = ni; upass = np; ent = nent;
    setup(ent, upass);
    // the prefetch's own waits (and any reloads) come before the pass's
    // first loads are in flight, not behind them
    int ni2, np2;
    next_of(ui, upass, ent, ni2, np2);
    if (ni2 < nunits && ni2 < tab0 + kTabCap) {
      const int4 e2 = entry_of(ni2);
      if (e2.x >= 0) prefetch(e2, np2);
    }
    prologue();
  }
}

static hipError_t launch_big(const Shape& s, int mode, BigParams& p, hipStream_t st) {
  const int units = s.slots_max * p.ntiles;
  if (units == 0) return hipSuccess;
  p.units = units;
  p.per_xcd = (units + 7) / 8;
  // persistent: one workgroup per CU (the kernel's LDS allows one), the
  // same number on each of the 8 XCDs
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  const int nwx = std::max(1, std::min(ncu / 8, p.per_xcd));
  const unsigned grid = unsigned(nwx) * 8;
  const size_t lds = 0;  // static LDS
#define MOE_BIG_LAUNCH(WF, CAP, AF)                                                                   \
  do {                                                                                                \
    if (mode == 0) hipLaunchKernelGGL((k_gemm_big<WF, 0, CAP, AF>), dim3(grid), dim3(kBigThreads), lds, st, p); \
    else hipLaunchKernelGGL((k_gemm_big<WF, 1, CAP, AF>), dim3(grid), dim3(kBigThreads), lds, st, p);           \
  } while (0)
  if (s.af == 1) {
    if (s.big_cap == 64) MOE_BIG_LAUNCH(1, 64, 1);
    else MOE_BIG_LAUNCH(1, 160, 1);
  } else if (s.wfmt == 0) {
    if (s.big_cap == 64) MOE_BIG_LAUNCH(0, 64, 0);
    else MOE_BIG_LAUNCH(0, 160, 0);
  } else if (s.wfmt == 2) {
    if (s.big_cap == 64) MOE_BIG_LAUNCH(2, 64, 0);
    else MOE_BIG_LAUNCH(2, 96, 0);
  } else {
    if (s.big_cap == 64) MOE_BIG_LAUNCH(1, 64, 0);
    else MOE_BIG_LAUNCH(1, 160, 0);
  }
#undef MOE_BIG_LAUNCH
  return hipGetLastError();
}


hipError_t launch_gemm1_big(const Shape& s, const uint8_t* xq, const float* xs, const int32_t* row_token,
                            const int32_t* offsets, WeightPtrs w1, uint8_t* hq, float* hs, int min_rows,
                            hipStream_t st) {
  BigParams p{};
  p.act = xq; p.act_s = xs; p.row_token = row_token; p.offsets = offsets;
  p.w = w1.w; p.ws = w1.ws; p.sw = w1.sw; p.sws = w1.sws; p.wg = w1.g; p.swg = w1.sg;
  p.hq = hq; p.hs = hs;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.ntiles = s.I / 128; p.min_rows = min_rows;
  return launch_big(s, 0, p, st);
}

hipError_t launch_gemm2_big(const Shape& s, const uint8_t* hq, const float* hs, const int32_t* offsets,
                            WeightPtrs w2, float* y, uint16_t* yb, int min_rows, hipStream_t st) {
  BigParams p{};
  p.act = hq; p.act_s = hs; p.offsets = offsets;
  p.w = w2.w; p.ws = w2.ws; p.sw = w2.sw; p.sws = w2.sws; p.wg = w2.g; p.swg = w2.sg;
  p.y = y;
  p.yb = yb;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.ntiles = s.H / 256; p.min_rows = min_rows;
  return launch_big(s, 1, p, st);
}

}  // namespace moe
