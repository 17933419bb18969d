// moe_kernels.hip -- gfx950 kernels of the low-bit MoE expert layer.
//
//   k_route_quant  expert histogram, exclusive-scan offsets, stable expand
//                  index (block 0) and per-token FP8 activation
//                  quantisation (all other blocks), one launch; for many
//                  slots the first blocks only count their chunk of slots
//   k_permute_rank and one block per chunk then places that chunk's slots.
//   k_gemm1        grouped GEMM1 over gate|up weights (e4m3 with fp32
//                  block scales, or MXFP4 through the scaled MFMA), fp32
//                  accumulation, fused SwiGLU and FP8 requantisation;
//                  optional split-K whose last-arriving workgroup reduces
//                  the partial sums in a fixed order.
//   k_gemm2        grouped GEMM2 over the down weights, same machinery.
//   k_combine      top-k weighted gather-reduce back to token order, bf16.
//
// Dataflow follows the GMM1 -> SwiGLU -> GMM2 -> combine chain of the
// FusedDeepMoE family analysis (unified execution flow figure; OpDequant,
// OpSwiglu, OpBlockQuant) and the FP8/FP4 grouped GEMM with fused SwiGLU and
// requantisation of the GC-MoE abstract.  At decode the expert weights are
// most of the bytes moved (the GC-MoE abstract makes the same point for
// decode), so weight rows sit on the 16-row MFMA side and stream straight
// from HBM into registers, while the few tokens of an expert form the
// 16-column side.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kThreads = 256;  // 4 waves per workgroup everywhere
constexpr int kStages = 2;  // register stages of the K loop

// =====================================================================
// route + quant
// =====================================================================
struct RouteParams {
  const uint16_t* x;
  const int32_t* ids;
  int32_t* counts;
  int32_t* offsets;
  int32_t* expand_idx;
  int32_t* row_token;
  uint8_t* xq;
  float* xs;
  uint8_t* xq_scale8;  // MXFP4 activations: the e8m0 scales, [T][H/32] (aliases xs)
  int32_t* clear;
  int nclear;
  int32_t* chunk_cnt;  // chunked mode: per-chunk expert counts [nchunks][E]
  int chunk, nchunks;  // slots per chunk; nchunks == 1: one block places every slot
  int T, H, k, E, G, shared;
  int af;              // 1: MXFP4 activations (e2m1 codes, e8m0 per 32) instead of e4m3 per G
  int32_t* zero1;      // optional: one more word block 0 zeroes (the persistent layer's status)
};

// Place slots [c0, c1) (chunk b of nb): expert histogram of the chunk, the
// experts' row offsets (from this block's own counts when nb == 1, else
// from every chunk's counts in p.chunk_cnt), then stable ranks.  Block 0
// also writes counts, offsets and the layer's bookkeeping.
__device__ void permute_chunk(const RouteParams& p, int b, int nb, int c0, int c1) {
  __shared__ int cnt[4][1024];  // per-wave expert counts, then per-wave running row bases
  __shared__ int wsum[4];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int E = p.E, n = p.T * p.k;
  for (int i = tid; i < 4 * 1024; i += kThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  // each wave owns one contiguous, 64-aligned range of the chunk's slots
  const int per = ((c1 - c0 + 4 * 64 - 1) / (4 * 64)) * 64;
  const int i0 = min(c1, c0 + w * per), i1 = min(c1, i0 + per);
  // ids are read kBatch rounds of 64 at a time so the loads overlap
  constexpr int kBatch = 8;
  for (int base = i0; base < i1; base += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = base + q * 64 + lane;
      eb[q] = i < i1 ? p.ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (eb[q] >= 0 && eb[q] < E) atomicAdd(&cnt[w][eb[q]], 1);
  }
  __syncthreads();
  // totals per expert over all slots, their exclusive scan, and the rows
  // taken by earlier chunks (thread tid owns a contiguous run of at most 4
  // experts)
  const int ept = (E + kThreads - 1) / kThreads;
  int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
  int local = 0;
  for (int q = 0; q < ept; ++q) {
    const int e = tid * ept + q;
    if (e < E) {
      if (nb == 1) {
        tot[q] = cnt[0][e] + cnt[1][e] + cnt[2][e] + cnt[3][e];
      } else {
        // sixteen chunks' counts loaded at a time (past nb they re-read the
        // last chunk's and are not added), so their round trips overlap
        for (int bb0 = 0; bb0 < nb; bb0 += 16) {
          int cv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) cv[u] = p.chunk_cnt[min(bb0 + u, nb - 1) * E + e];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int bb = bb0 + u;
            tot[q] += bb < nb ? cv[u] : 0;
            pre[q] += bb < b ? cv[u] : 0;
          }
        }
      }
    }
    local += tot[q];
  }
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int run = incl - local;
  for (int q = 0; q < w; ++q) run += wsum[q];
  for (int q = 0; q < ept; ++q) {
    const int e = tid * ept + q;
    if (e < E) {
      if (b == 0) {
        p.counts[e] = tot[q];
        p.offsets[e] = run;
      }
      int bs = run + pre[q];
      for (int ww = 0; ww < 4; ++ww) {
        const int c = cnt[ww][e];
        cnt[ww][e] = bs;
        bs += c;
      }
      run += tot[q];
    }
  }
  const int R0 = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  if (b == 0 && tid == 0) {
    p.offsets[E] = R0;
    if (p.shared) {
      p.counts[E] = p.T;
      p.offsets[E + 1] = R0 + p.T;
    }
  }
  __syncthreads();
  // stable ranks: lanes with the same expert id are found with one ballot
  // per id bit; the rank is the number of such lanes below, and the lowest
  // of them advances the wave's running base for the next 64 slots.
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int base0 = i0; base0 < i1; base0 += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = base0 + q * 64 + lane;
      eb[q] = i < i1 ? p.ids[i] : -1;
    }
    for (int q = 0; q < kBatch; ++q) {
      const int base = base0 + q * 64;
      if (base >= i1) break;
      const int i = base + lane;
      const int e = eb[q];
      const bool valid = i < i1 && e >= 0 && e < E;
      uint64_t match = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool on = valid && ((e >> bit) & 1);
        const uint64_t bb = __ballot(on);
        match &= on ? bb : ~bb;
      }
      int row = -1;
      if (valid) row = cnt[w][e] + __popcll(match & below);
      __builtin_amdgcn_wave_barrier();
      if (valid && (match & below) == 0) cnt[w][e] = row + __popcll(match);
      __builtin_amdgcn_wave_barrier();
      if (i < i1) {
        p.expand_idx[i] = row;
        if (valid) p.row_token[row] = i / p.k;
      }
    }
  }
  if (b != 0) return;
  if (p.shared)
    for (int t = tid; t < p.T; t += kThreads) p.row_token[R0 + t] = t;
  const int R = R0 + (p.shared ? p.T : 0);
  const int cap = n + (p.shared ? p.T : 0);
  for (int r = R + tid; r < cap; r += kThreads) p.row_token[r] = -1;
  for (int q = tid; q < p.nclear; q += kThreads) p.clear[q] = 0;
  if (tid == 0 && p.zero1) *p.zero1 = 0;
}

// chunked mode, first pass: expert counts of chunk b into p.chunk_cnt[b][:]
__device__ void count_chunk(const RouteParams& p, int b) {
  __shared__ int c[1024];
  const int tid = threadIdx.x, E = p.E, n = p.T * p.k;
  for (int e = tid; e < E; e += kThreads) c[e] = 0;
  __syncthreads();
  const int c0 = b * p.chunk, c1 = min(n, c0 + p.chunk);
  for (int i = c0 + tid; i < c1; i += kThreads) {
    const int e = p.ids[i];
    if (e >= 0 && e < E) atomicAdd(&c[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) p.chunk_cnt[b * E + e] = c[e];
}

// one thread = 8 consecutive channels of one token; a group of G channels
// is G/8 consecutive lanes
__device__ void quant_block(const RouteParams& p, int blk) {
  const int tid = threadIdx.x;
  const long items = long(p.T) * (p.H / 8);
  const long item = long(blk) * kThreads + tid;
  float f[8];
  float amax = 0.0f;
  int t = 0, c0 = 0;
  if (item < items) {
    t = int(item / (p.H / 8));
    c0 = int(item % (p.H / 8)) * 8;
    const v4u v = *reinterpret_cast<const v4u*>(p.x + long(t) * p.H + c0);
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_to_f32(v[q] & 0xFFFFu);
      f[2 * q + 1] = bf16_to_f32(v[q] >> 16);
    }
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
  }
  const int lanes = p.G / 8;  // 4 or 16: the group's lanes, one aligned run
  amax = group_max_dpp(amax, lanes);
  if (p.af == 1) {
    // MXFP4: one e8m0 scale per 32 channels (4 lanes), 8 e2m1 codes per thread
    if (item < items) {
      const uint32_t code = mx_scale_code(amax);
      const float inv = mx_inv_scale(code);
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) word |= enc_e2m1(f[q] * inv) << (4 * q);
      *reinterpret_cast<uint32_t*>(p.xq + long(t) * (p.H / 2) + c0 / 2) = word;
      if ((tid & 3) == 0) p.xq_scale8[long(t) * (p.H / 32) + c0 / 32] = uint8_t(code);
    }
    return;
  }
  if (item < items) {
    const float mult = quant_mult(amax);
    const uint32_t lo = enc_e4m3x4(f[0] * mult, f[1] * mult, f[2] * mult, f[3] * mult);
    const uint32_t hi = enc_e4m3x4(f[4] * mult, f[5] * mult, f[6] * mult, f[7] * mult);
    uint2 o;
    o.x = lo;
    o.y = hi;
    *reinterpret_cast<uint2*>(p.xq + long(t) * p.H + c0) = o;
    if ((tid & (lanes - 1)) == 0) p.xs[long(t) * (p.H / p.G) + c0 / p.G] = 1.0f / mult;
  }
}

// units [0, nlead) route (the whole permute, or the chunk counts), the
// rest quantise
__device__ __forceinline__ void route_quant_unit(const RouteParams& p, int b) {
  const int nlead = p.nchunks == 1 ? 1 : p.nchunks;
  if (b >= nlead) quant_block(p, b - nlead);
  else if (p.nchunks == 1) permute_chunk(p, 0, 1, 0, p.T * p.k);
  else count_chunk(p, b);
}

__global__ __launch_bounds__(kThreads) void k_route_quant(RouteParams p) { route_quant_unit(p, blockIdx.x); }

// chunked mode, second pass: block b places chunk b's slots
__global__ __launch_bounds__(kThreads) void k_permute_rank(RouteParams p) {
  const int b = blockIdx.x, n = p.T * p.k;
  permute_chunk(p, b, p.nchunks, b * p.chunk, min(n, (b + 1) * p.chunk));
}

__global__ __launch_bounds__(kThreads) void k_clear(int32_t* p, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0;
}

// =====================================================================
// grouped GEMM machinery
// =====================================================================
// Work items of the decode GEMMs: a group with n rows holds ceil(n / R)
// items of R rows each (one pass of the kernel), so the passes of a heavy
// group run side by side on different workgroups rather than one after the
// other on one.  Returns the group of the item-th item (groups in order) and
// sets *pass to that item's index within its group, or returns -1 when there
// are fewer items.  Block-wide; every thread gets the same answer.
__device__ int nth_item(const int32_t* offsets, int ngroups, int item, int R, int* pass, int* s_wsum, int* s_res) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int gpt = (ngroups + kThreads - 1) / kThreads;  // <= 5
  int local = 0;
  for (int q = 0; q < gpt; ++q) {
    const int g = tid * gpt + q;
    if (g < ngroups) local += (offsets[g + 1] - offsets[g] + R - 1) / R;
  }
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (tid == 0) {
    s_res[0] = -1;
    s_res[1] = 0;
  }
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int run = incl - local;
  for (int q = 0; q < w; ++q) run += s_wsum[q];
  if (item >= run && item < run + local) {
    int c = run;
    for (int q = 0; q < gpt; ++q) {
      const int g = tid * gpt + q;
      if (g >= ngroups) break;
      const int n = (offsets[g + 1] - offsets[g] + R - 1) / R;
      if (item < c + n) {
        s_res[0] = g;
        s_res[1] = item - c;
        break;
      }
      c += n;
    }
  }
  __syncthreads();
  *pass = s_res[1];
  return s_res[0];
}

// Operands of one 128-K step for a wave: NJ weight tiles of 16 rows and NTT
// token tiles of 16 columns.
template <int WF, int NJ, int NTT>
struct Frag {
  v8i a[NJ];
  v8i b[NTT];
  float wsc[NJ];   // e4m3 weights, 128-blocks: wave-uniform weight scale
  int wsb[NJ];     // MXFP4: this lane's e8m0 byte (row m, 32-block g); NVFP4: its two e4m3 bytes
  float xsv[NTT];  // activation scale of this lane's token column
};

// Operand sources of the K loop: buffer resources over the group's weight
// matrix (tiled layout) and MXFP4 scale tiles, the activation codes and the
// activation scales, with this lane's byte offsets at K step 0.  A K step
// adds a wave-uniform stride through the scalar offset, so the per-lane
// offsets stay fixed over the loop and no 64-bit addresses are formed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// cache-policy operand of the buffer intrinsics for the weight and weight
// scale loads: nt (non-temporal: each weight byte is read once per layer, so
// its lines are not kept in the caches)
constexpr int kNt = 2;
constexpr int kSc1 = 16;  // cache-policy operand of the buffer intrinsics: sc1 (device-coherent)

// Results that one workgroup writes and another, possibly on another XCD
// (each XCD has its own L2), reads inside the same launch -- the persistent
// layer's h and y rows -- travel through device-coherent (sc1) stores and
// loads, which do not stop at a non-coherent L2; CO selects that form.
template <bool CO>
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  if (CO) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool CO>
__device__ __forceinline__ void st_f32(float* p, float v) {
  if (CO) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool CO>
__device__ __forceinline__ float ld_f32(const float* p) {
  if (CO) return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool CO>
__device__ __forceinline__ void st_bf16x4(uint16_t* dst, const v4f& v) {
  if (!CO) {
    store_bf16x4(dst, v);
    return;
  }
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  st_u32<true>(d, f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16));
  st_u32<true>(d + 1, f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16));
}

template <int NJ, int NTT>
struct KSrc {
  __amdgpu_buffer_rsrc_t wr, sr, ar, xr;
  int wo[NJ];   // weight tile j: the tile's offset + 16 lane
  int so[NJ];   // MXFP4: scale byte of tile j (the tile's 64 bytes + lane); NVFP4: row m's bytes 2g, 2g+1
  int bo[NTT];  // token column t: its code row + 16 g (NVFP4: + 32 g)
  int xo[NTT];  // token column t: its scale row, in bytes
  int wstep, sstep, astep;  // bytes per K step: weight tiles, scale tiles, activation scales
};

template <int WF, int NJ, int NTT, int B32, bool CO>
__device__ __forceinline__ void load_frag(Frag<WF, NJ, NTT>& f, const KSrc<NJ, NTT>& src,
                                          const float* const (&wsc)[NJ], int ks) {
  const int kw = ks * src.wstep, ksc = ks * src.sstep, ka = ks * 128, kx = ks * src.astep;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(src.wr, src.wo[j], kw, kNt);
    if (WF == 0) {
      const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(src.wr, src.wo[j] + 1024, kw, kNt);
      f.a[j] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      if (!B32) f.wsc[j] = wsc[j][ks];
    } else {
      f.a[j] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), 0, 0, 0, 0};
      if (WF == 1) f.wsb[j] = __builtin_amdgcn_raw_buffer_load_b8(src.sr, src.so[j], ksc, kNt);
      else f.wsb[j] = __builtin_amdgcn_raw_buffer_load_b16(src.sr, src.so[j], ksc, kNt);  // NVFP4: 16-blocks 2g, 2g+1
    }
  }
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    // e4m3 operand order: bytes 16 g .. and 64 + 16 g ..; NVFP4's f16 path:
    // the lane's 32 consecutive K, 32 g ..
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(src.ar, src.bo[t], ka, CO ? kSc1 : 0);
    const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(src.ar, src.bo[t] + (WF == 2 ? 16 : 64), ka, CO ? kSc1 : 0);
    f.b[t] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
    if (!B32) f.xsv[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(src.xr, src.xo[t], kx, CO ? kSc1 : 0));
  }
}

template <int WF, int NJ, int NTT, int B32, bool CO>
__device__ __forceinline__ void mma_frag(v4f (&acc)[NJ][NTT], const Frag<WF, NJ, NTT>& f,
                                         const float* const (&wsc)[NJ], const float* const (&bsc)[NTT],
                                         int ks, int g) {
  if (WF == 0 && B32) {
    // e4m3 weights with 32x32 scale blocks: one masked MFMA per 32-K block
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const v8i am = mask_e4m3_block(f.a[j], g, sb);
        const float ws = wsc[j][ks * 4 + sb];
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
          const v4f d = mfma_scaled<kFmtE4M3, kFmtE4M3>(am, f.b[t], kUnitScale, kUnitScale);
          acc[j][t] += d * (ws * ld_f32<CO>(&bsc[t][ks * 4 + sb]));
        }
      }
    }
  } else if (WF == 2) {
    // NVFP4 through the fp16 MFMA (16x16x32): lane (row or column 16-slot,
    // group g) holds K 32 g .. 32 g + 31 of the step for both operands, the
    // q-th instruction taking K 32 g + 8 q .. + 7, so the two operands agree
    // on every K.  Weights: e2m1 -> f16, times the e4m3 block scale as f16
    // (the product has at most 6 significant bits and stays in f16's normal
    // range, so it is exact); activations: e4m3 -> f16 (exact).  The
    // matrix scale is applied once after the K loop.
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      h8v bq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bq[q] = cvt_e4m3x8_f16(f.b[t][2 * q], f.b[t][2 * q + 1]);
      v4f d[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const h2v sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uint32_t(f.wsb[j]), 1.0f, false);
        d[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const h8v a = cvt_e2m1x8_f16(uint32_t(f.a[j][q])) * (q < 2 ? sc[0] : sc[1]);
          d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[q], d[j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j][t] += d[j] * f.xsv[t];
    }
  } else {
    // one token tile at a time: the NJ products land in separate registers
    // first, so the MFMAs issue back to back, then they are scaled into acc
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      v4f d[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (WF == 0) d[j] = mfma_scaled<kFmtE4M3, kFmtE4M3>(f.a[j], f.b[t], kUnitScale, kUnitScale);
        else d[j] = mfma_scaled<kFmtE2M1, kFmtE4M3>(f.a[j], f.b[t], f.wsb[j], kUnitScale);
      }
      __builtin_amdgcn_sched_barrier(0);  // all NJ products in flight before they are consumed
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (WF == 0) acc[j][t] += d[j] * (f.wsc[j] * f.xsv[t]);
        else acc[j][t] += d[j] * f.xsv[t];
      }
    }
  }
}

// acc += sum over K steps [ks0, ks1).  Operands travel through a ring of ST
// register stages: the loads for step ks + ST - 1 are issued before step ks
// is multiplied, so ST - 1 steps of weight bytes are in flight per wave.
// The loads are unconditional (past the end they repeat the last step and
// hit in cache) so the compiler can count outstanding loads exactly and
// wait only for the stage about to be used; only the MFMAs are predicated.
template <int WF, int NJ, int NTT, int B32, int ST, bool CO = false>
__device__ __forceinline__ void kloop(v4f (&acc)[NJ][NTT], const KSrc<NJ, NTT>& src, const float* const (&wsc)[NJ],
                                      const float* const (&bsc)[NTT], int ks0, int ks1, int g) {
  Frag<WF, NJ, NTT> f[ST];
#pragma unroll
  for (int s = 0; s < ST - 1; ++s) {
    load_frag<WF, NJ, NTT, B32, CO>(f[s], src, wsc, min(ks0 + s, ks1 - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep each stage's loads together, in stage order
  }
  for (int ks = ks0; ks < ks1; ks += ST) {
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      load_frag<WF, NJ, NTT, B32, CO>(f[(s + ST - 1) % ST], src, wsc, min(ks + s + ST - 1, ks1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (ks + s < ks1) mma_frag<WF, NJ, NTT, B32, CO>(acc, f[s], wsc, bsc, ks + s, g);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

struct GemmParams {
  const uint8_t* act;        // GEMM1: xq [T][H] by token; GEMM2: hq [rows][I] by row
  const float* act_s;        // matching scales
  const int32_t* row_token;  // GEMM1 only
  const int32_t* offsets;
  const uint8_t* w;
  const void* ws;
  const uint8_t* sw;
  const void* sws;
  const float* wg;           // NVFP4: fp32 scale per routed expert matrix [E]
  const float* swg;          // and the shared expert's [1]
  uint8_t* hq;               // GEMM1 outputs
  float* hs;
  float* y;                  // GEMM2 output (fp32), or
  uint16_t* yb;              // the same as bf16 when non-null (layer-internal)
  float* part;
  int32_t* cnt;
  int H, I, E, G, wblk, ngroups, S, ntiles, rows_cap;
};

// Split-K hand-off between workgroups that may sit on different XCDs (each
// XCD has its own L2).  Partial sums travel through device-coherent (sc1)
// stores and loads, which bypass the non-coherent L2 contents, so no L2
// writeback or invalidate is needed: a workgroup waits until its sc1 stores
// have completed, then counts itself in with a device-scope atomic; the
// workgroup that brings the count to S reads every partial back with sc1
// loads and finishes the unit.  Sums are taken in split order, so the result
// does not depend on which workgroup arrives last.
// Buffer resource over the partial-sum array; 16-byte accesses with the sc1
// cache policy bit are device-coherent.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ void st_coherent(__amdgpu_buffer_rsrc_t r, long elem, const v4f& v) {
  const v4u u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, int(elem * 4), 0, kSc1);
}

__device__ __forceinline__ v4f ld_coherent(__amdgpu_buffer_rsrc_t r, long elem) {
  const v4u u = __builtin_amdgcn_raw_buffer_load_b128(r, int(elem * 4), 0, kSc1);
  return v4f{__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3])};
}

// Every workgroup has issued its partial sums; returns true in exactly one
// workgroup of the unit (the last to arrive).
__device__ __forceinline__ bool arrive_last(int32_t* counter, int S, int* s_flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  return *s_flag;
}

// ---------------------------------------------------------------------
// GEMM1: unit = (work item, 128 h-columns, K split), a work item being one
// pass of 16 NTT rows of one group (nth_item).  Wave w owns h-columns
// [32w, 32w+32) of the unit: weight tiles j = 0,1 are gate rows
// n0+32w+16j+(0..15) and j = 2,3 the up rows I+n0+32w+16(j-2)+(0..15), so
// the gate and up values of one h element land in the same lane.
// ---------------------------------------------------------------------
template <int NTT, bool CO>
__device__ __forceinline__ void swiglu_requant_store(const v4f (&acc)[4][NTT], const GemmParams& p, int row0,
                                                     int ne, int pass, int n0, float (*s_red)[4][16]) {
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, m = lane & 15, g = lane >> 4;
  float h[NTT][8];
  float amax[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    amax[t] = 0.0f;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = swiglu(acc[jt][t][i], acc[2 + jt][t][i]);
        h[t][jt * 4 + i] = v;
        amax[t] = fmaxf(amax[t], fabsf(v));
      }
    amax[t] = wave_max_xor(amax[t], 16);
    amax[t] = wave_max_xor(amax[t], 32);
  }
  if (p.G == 128) {
    __syncthreads();
    if (g == 0)
#pragma unroll
      for (int t = 0; t < NTT; ++t) s_red[t][w][m] = amax[t];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTT; ++t)
      amax[t] = fmaxf(fmaxf(s_red[t][0][m], s_red[t][1][m]), fmaxf(s_red[t][2][m], s_red[t][3][m]));
  }
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    const int idx = pass * 16 * NTT + t * 16 + m;
    if (idx >= ne) continue;
    const long r = row0 + idx;
    const float mult = quant_mult(amax[t]);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const float* hv = h[t] + jt * 4;
      const uint32_t word = enc_e4m3x4(hv[0] * mult, hv[1] * mult, hv[2] * mult, hv[3] * mult);
      st_u32<CO>(reinterpret_cast<uint32_t*>(p.hq + r * p.I + n0 + 32 * w + 16 * jt + 4 * g), word);
    }
    if (g == 0) {
      if (p.G == 128) {
        if (w == 0) st_f32<CO>(p.hs + r * (p.I / 128) + n0 / 128, 1.0f / mult);
      } else {
        st_f32<CO>(p.hs + r * (p.I / 32) + (n0 + 32 * w) / 32, 1.0f / mult);
      }
    }
  }
}

// Occupancy with 128-blocks: two token tiles capped at 168 registers (three
// workgroups per CU, which runs a 64-expert T = 64 layer's 768 units in one
// round instead of one and a half), one token tile at 128 (four per CU); the
// compiler fits both without spills.
// (NVFP4's f16 operands take more registers: two workgroups per CU with
// two token tiles, where the K loop would otherwise spill)
template <int NTT>
constexpr int gemm1_occupancy(int b32, int wf = 0) {
  return b32 ? 1 : NTT == 2 ? (wf == 2 ? 2 : 3) : NTT == 1 ? 4 : 1;
}

// Unit u of GEMM1.  Returns true (in every thread) when this workgroup
// stored a finished 128-column slice of h: the only split (S == 1) or the
// last to arrive.
template <int WF, int NTT, int B32, bool CO = false>
__device__ __forceinline__ bool gemm1_unit(const GemmParams& p, int u) {
  __shared__ int s_wsum[4], s_res[2], s_flag;
  __shared__ float s_red[NTT][4][16];
  const int S = p.S, nt = p.ntiles;
  const int split = u % S, tile = (u / S) % nt, item = u / (S * nt);
  int pass0 = 0;
  const int e = nth_item(p.offsets, p.ngroups, item, 16 * NTT, &pass0, s_wsum, s_res);
  if (e < 0) return false;
  const int row0 = p.offsets[e], ne = p.offsets[e + 1] - row0;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, m = lane & 15, g = lane >> 4;
  const int H = p.H, I = p.I, n0 = tile * 128;
  const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(p.part);
  const bool shared = e == p.E;
  const long ee = shared ? 0 : e;
  const long kbytes = WF == 0 ? H : H / 2;
  KSrc<4, NTT> src;
  src.wr = buf_rsrc((shared ? p.sw : p.w) + ee * 2L * I * kbytes);
  src.sr = buf_rsrc(static_cast<const uint8_t*>(shared ? p.sws : p.ws) +
                    (WF == 1 ? ee * 2L * I * (H / 32) : WF == 2 ? ee * 2L * I * (H / 16) : 0));
  src.ar = buf_rsrc(p.act);
  src.xr = buf_rsrc(p.act_s);
  src.wstep = (2 * I / 16) * kTileBytes<WF>;
  src.sstep = (2 * I / 16) * (WF == 2 ? kTileScaleBytes16 : kTileScaleBytes);
  src.astep = 4;
  const float* wsc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rb = (j < 2) ? (n0 + 32 * w + 16 * j) : (I + n0 + 32 * w + 16 * (j - 2));
    src.wo[j] = (rb / 16) * kTileBytes<WF> + lane * 16;
    src.so[j] = WF == 2 ? (rb / 16) * kTileScaleBytes16 + 8 * m + 2 * g : (rb / 16) * kTileScaleBytes + lane;
    wsc[j] = nullptr;
    if (WF == 0) {
      const int b = p.wblk;
      const float* sb = static_cast<const float*>(shared ? p.sws : p.ws) + ee * long(2 * I / b) * (H / b);
      // 128-row blocks: a wave's two gate tiles (and its two up tiles) lie in
      // one block, so they share one scale pointer (and one load per step)
      const int brow = B32 ? rb / b : ((j < 2) ? n0 : I + n0) / 128;
      wsc[j] = sb + long(brow) * (H / b);
    }
  }
  const int nks = H / 128, kps = nks / S, ks0 = split * kps, ks1 = ks0 + kps;
  {  // this workgroup's one pass (work item) of the group's rows
    const int pass = pass0;
    const float* bsc[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int idx = min(pass * 16 * NTT + t * 16 + m, ne - 1);
      const int tok = p.row_token[row0 + idx];
      src.bo[t] = tok * H + (WF == 2 ? 32 : 16) * g;
      src.xo[t] = tok * (H / p.G) * 4;
      bsc[t] = p.act_s + long(tok) * (H / p.G);
    }
    v4f acc[4][NTT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < NTT; ++t) acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    kloop<WF, 4, NTT, B32, kStages>(acc, src, wsc, bsc, ks0, ks1, g);
    if (WF == 2) {  // NVFP4: the matrix scale
      const float gs = shared ? p.swg[0] : p.wg[ee];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < NTT; ++t) acc[j][t] *= gs;
    }
    if (S == 1) {
      swiglu_requant_store<NTT, CO>(acc, p, row0, ne, pass, n0, s_red);
      return true;
    } else {
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        const int idx = pass * 16 * NTT + t * 16 + m;
        if (idx >= ne) continue;
        const long dst = ((long(split) * nt + tile) * p.rows_cap + row0 + idx) * 256;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = (j >> 1) * 128 + 32 * w + 16 * (j & 1) + 4 * g;
          st_coherent(prs, dst + col, acc[j][t]);
        }
      }
    }
  }
  if (!arrive_last(p.cnt + item * nt + tile, S, &s_flag)) return false;
  {
    const int pass = pass0;
    v4f acc[4][NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int idx = min(pass * 16 * NTT + t * 16 + m, ne - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = (j >> 1) * 128 + 32 * w + 16 * (j & 1) + 4 * g;
        v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int sp = 0; sp < S; ++sp)
          s += ld_coherent(prs, ((long(sp) * nt + tile) * p.rows_cap + row0 + idx) * 256 + col);
        acc[j][t] = s;
      }
    }
    swiglu_requant_store<NTT, CO>(acc, p, row0, ne, pass, n0, s_red);
  }
  return true;
}

template <int WF, int NTT, int B32>
__global__ __launch_bounds__(kThreads, gemm1_occupancy<NTT>(B32, WF)) void k_gemm1(GemmParams p) {
  gemm1_unit<WF, NTT, B32>(p, blockIdx.x);
}

// ---------------------------------------------------------------------
// GEMM2: unit = (work item, 64 NJ output rows, K split); wave w owns output rows
// n0 + 16 NJ w + 16 j + (0..15), j < NJ (NJ = 4 when H allows 256-row
// units: twice the weight bytes in flight per wave; NJ = 8 for MXFP4, whose
// tiles carry half the bytes).
// ---------------------------------------------------------------------
// Unit u of GEMM2.  `ready(item)` is called (block-wide) once the unit's
// work item is known to hold rows; it returns when the item's h rows may be
// read, false if they never will be (the unit is then skipped).
struct Always {
  __device__ bool operator()(int) const { return true; }
};

// Returns the unit's work item, or -1 when the item holds no rows.
template <int WF, int NTT, int B32, int NJ, bool CO, class Ready>
__device__ __forceinline__ int gemm2_unit(const GemmParams& p, int u, const Ready& ready) {
  __shared__ int s_wsum[4], s_res[2], s_flag;
  const int S = p.S, nt = p.ntiles;
  const int split = u % S, tile = (u / S) % nt, item = u / (S * nt);
  int pass0 = 0;
  const int e = nth_item(p.offsets, p.ngroups, item, 16 * NTT, &pass0, s_wsum, s_res);
  if (e < 0) return -1;
  if (!ready(item)) return item;
  const int row0 = p.offsets[e], ne = p.offsets[e + 1] - row0;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, m = lane & 15, g = lane >> 4;
  constexpr int kRows = 64 * NJ;  // output rows of a unit
  const int H = p.H, I = p.I, n0 = tile * kRows;
  const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(p.part);
  const bool shared = e == p.E;
  const long ee = shared ? 0 : e;
  const long kbytes = WF == 0 ? I : I / 2;
  KSrc<NJ, NTT> src;
  src.wr = buf_rsrc((shared ? p.sw : p.w) + ee * long(H) * kbytes);
  src.sr = buf_rsrc(static_cast<const uint8_t*>(shared ? p.sws : p.ws) +
                    (WF == 1 ? ee * long(H) * (I / 32) : WF == 2 ? ee * long(H) * (I / 16) : 0));
  src.ar = buf_rsrc(p.act);
  src.xr = buf_rsrc(p.act_s);
  src.wstep = (H / 16) * kTileBytes<WF>;
  src.sstep = (H / 16) * (WF == 2 ? kTileScaleBytes16 : kTileScaleBytes);
  src.astep = 4;
  const float* wsc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int rb = n0 + 16 * NJ * w + 16 * j;
    src.wo[j] = (rb / 16) * kTileBytes<WF> + lane * 16;
    src.so[j] = WF == 2 ? (rb / 16) * kTileScaleBytes16 + 8 * m + 2 * g : (rb / 16) * kTileScaleBytes + lane;
    wsc[j] = nullptr;
    if (WF == 0) {
      const int b = p.wblk;
      const float* sb = static_cast<const float*>(shared ? p.sws : p.ws) + ee * long(H / b) * (I / b);
      // 128-row blocks: the wave's NJ tiles lie in one block and share its scale
      const int brow = B32 ? rb / b : (n0 + 16 * NJ * w) / 128;
      wsc[j] = sb + long(brow) * (I / b);
    }
  }
  const int nks = I / 128, kps = nks / S, ks0 = split * kps, ks1 = ks0 + kps;
  {  // this workgroup's one pass (work item) of the group's rows
    const int pass = pass0;
    const float* bsc[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int r = row0 + min(pass * 16 * NTT + t * 16 + m, ne - 1);
      src.bo[t] = r * I + (WF == 2 ? 32 : 16) * g;
      src.xo[t] = r * (I / p.G) * 4;
      bsc[t] = p.act_s + long(r) * (I / p.G);
    }
    v4f acc[NJ][NTT];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int t = 0; t < NTT; ++t) acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    kloop<WF, NJ, NTT, B32, kStages, CO>(acc, src, wsc, bsc, ks0, ks1, g);
    if (WF == 2) {  // NVFP4: the matrix scale
      const float gs = shared ? p.swg[0] : p.wg[ee];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int t = 0; t < NTT; ++t) acc[j][t] *= gs;
    }
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
      const int idx = pass * 16 * NTT + t * 16 + m;
      if (idx >= ne) continue;
      const long r = row0 + idx;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = 16 * NJ * w + 16 * j + 4 * g;
        if (S == 1) {
          if (p.yb) st_bf16x4<CO>(p.yb + r * H + n0 + col, acc[j][t]);
          else *reinterpret_cast<v4f*>(p.y + r * H + n0 + col) = acc[j][t];
        }
        else
          st_coherent(prs, ((long(split) * nt + tile) * p.rows_cap + r) * kRows + col, acc[j][t]);
      }
    }
  }
  if (S == 1) return item;
  if (!arrive_last(p.cnt + item * nt + tile, S, &s_flag)) return item;
  // reduce the S partial sums in split order: kRows columns x the pass's rows
  constexpr int kQ = kRows / 4;  // 4-column pieces per row
  const int r0 = pass0 * 16 * NTT, nr = min(ne - r0, 16 * NTT);
  for (int q = tid; q < nr * kQ; q += kThreads) {
    const long r = row0 + r0 + q / kQ;
    const int col = (q % kQ) * 4;
    v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int sp = 0; sp < S; ++sp)
      s += ld_coherent(prs, ((long(sp) * nt + tile) * p.rows_cap + r) * kRows + col);
    if (p.yb) st_bf16x4<CO>(p.yb + r * H + n0 + col, s);
    else *reinterpret_cast<v4f*>(p.y + r * H + n0 + col) = s;
  }
  return item;
}

template <int WF, int NTT, int B32, int NJ>
__global__ __launch_bounds__(kThreads) void k_gemm2(GemmParams p) {
  gemm2_unit<WF, NTT, B32, NJ, false>(p, blockIdx.x, Always{});
}

// =====================================================================
// combine: one workgroup per (token, channel chunk)
// =====================================================================
struct CombineParams {
  const float* y;            // fp32 rows, or
  const uint16_t* yb;        // bf16 rows when non-null
  const int32_t* expand_idx;
  const int32_t* offsets;
  const float* tw;
  uint16_t* out;
  int H, k, E, shared;
};

// One workgroup per (token, 256 NV channels), NV consecutive channels per
// thread: one 16-byte load per row (NV = 4 for fp32 rows, 8 for bf16 rows).
// The k slot rows are loaded in unrolled batches of 8 with no branch between
// the loads, so a thread has up to 8 loads in flight; masked slots read a
// valid row of the token with weight 0, whose product is an exact zero and
// leaves the ascending-order fp32 sum unchanged.
template <int NV> struct Row { v4f h[NV / 4]; };

// Each y row is read once, by the combine: the loads are non-temporal (their
// lines are not kept in the caches), which at 32768 rows keeps them from
// pushing out lines still to be read (prefill combine 108 -> 82 us).
template <int NV, bool CO>
__device__ __forceinline__ Row<NV> load_row(const CombineParams& p, long r, int c) {
  Row<NV> v;
  if (NV == 8) {
    const v4u u = CO ? __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(p.yb), int((r * p.H + c) * 2), 0, kSc1)
                     : __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p.yb + r * p.H + c));
#pragma unroll
    for (int h = 0; h < NV / 4; ++h)
      v.h[h] = v4f{bf16_to_f32(u[2 * h] & 0xFFFFu), bf16_to_f32(u[2 * h] >> 16), bf16_to_f32(u[2 * h + 1] & 0xFFFFu),
                   bf16_to_f32(u[2 * h + 1] >> 16)};
  } else {
    v.h[0] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p.y + r * p.H + c));
  }
  return v;
}

// unit b = (token b / nchunk, channel chunk b % nchunk)
template <int NV, bool CO = false>
__device__ __forceinline__ void combine_unit(const CombineParams& p, int b) {
  constexpr int kChunk = kThreads * NV;
  const int nchunk = (p.H + kChunk - 1) / kChunk;
  const long t = b / nchunk;
  const int c = (b % nchunk) * kChunk + threadIdx.x * NV;
  const int k = p.k;
  const int* ids = p.expand_idx + t * k;
  const float* tw = p.tw + t * k;
  const int srow = p.shared ? p.offsets[p.E] + int(t) : -1;
  int pad = srow;  // a valid row to stand in for masked slots
  for (int j = k - 1; j >= 0; --j)
    if (ids[j] >= 0) pad = ids[j];
  if (c >= p.H) return;
  Row<NV> acc;
#pragma unroll
  for (int h = 0; h < NV / 4; ++h) acc.h[h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if (pad >= 0) {
    for (int j0 = 0; j0 < k; j0 += 8) {
      Row<NV> v[8];
      float wj[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int r = j < k ? ids[j] : -1;
        wj[jj] = r >= 0 ? tw[j] : 0.0f;
        v[jj] = load_row<NV, CO>(p, r >= 0 ? r : pad, c);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int h = 0; h < NV / 4; ++h) acc.h[h] += wj[jj] * v[jj].h[h];
    }
    if (srow >= 0) {
      const Row<NV> v = load_row<NV, CO>(p, srow, c);
#pragma unroll
      for (int h = 0; h < NV / 4; ++h) acc.h[h] += v.h[h];
    }
  }
  uint32_t o[NV / 2];
#pragma unroll
  for (int h = 0; h < NV / 4; ++h) {
    o[2 * h] = f32_to_bf16(acc.h[h][0]) | (f32_to_bf16(acc.h[h][1]) << 16);
    o[2 * h + 1] = f32_to_bf16(acc.h[h][2]) | (f32_to_bf16(acc.h[h][3]) << 16);
  }
  if (NV == 8) *reinterpret_cast<v4u*>(p.out + t * p.H + c) = v4u{o[0], o[1], o[2], o[3]};
  else *reinterpret_cast<uint2*>(p.out + t * p.H + c) = uint2{o[0], o[1]};
}

template <int NV>
__global__ __launch_bounds__(kThreads) void k_combine(CombineParams p) { combine_unit<NV>(p, blockIdx.x); }

// =====================================================================
// persistent decode layer: GEMM1, GEMM2 and the combine in one launch
// =====================================================================
// After the routing and quantisation launch, a grid of as many workgroups
// as fit on the chip at once works through the units of GEMM1, then
// GEMM2, then the combine (each numbered as in its own launch; together
// the tickets 0, 1, ...): workgroup b takes tickets b, b + grid, b + 2 grid,
// ... in that order, so no shared counter is touched to hand out work.  A
// unit waits only for units of lower tickets: a GEMM2 unit for the GEMM1
// slices of its work item, a combine unit for the GEMM2 units of the work
// items holding its token's rows.  With every workgroup running at once
// (the grid is sized so), the lowest unfinished ticket always has its
// inputs ready, so the launch always finishes.  The waits are bounded all
// the same (a GPU shared with other work may not hold the whole grid): one
// that expires is counted in the control block and in the caller's status
// word, makes every later wait give up at once, and its unit is skipped.
// The h and y rows cross XCDs inside the launch, so they are written and
// read with device-coherent (sc1) accesses; a producing workgroup waits for
// its stores to complete before one device-scope increment of its work
// item's counter counts it in.  The control block lives in the workspace
// and is zeroed by the routing launch.
struct PersistParams {
  GemmParams g1, g2;
  CombineParams c;
  const int32_t* ids;  // topk ids [T][k] (the combine finds its rows' work items)
  int32_t* ctl;     // control block: kPersistCtlHead ints, then per work item the GEMM1 and the GEMM2 counters
  int32_t* status;  // optional: expired waits (zeroed by the routing launch)
  int n1, n2, nC;   // units of each step
  int items;        // work items of either GEMM (the same passes)
  int spin_limit;   // polls per wait before it expires
};

constexpr int kCtlExpired = 0;
static_assert(kCtlExpired < kPersistCtlHead, "control block head");

// The workgroup's stores have completed; then it counts itself in once.
__device__ __forceinline__ void count_in(int32_t* c) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *c >= target (block-wide answer): false if the wait expired
// or an earlier one did.
__device__ __forceinline__ bool wait_count(const int32_t* c, int target, int32_t* expired, int32_t* status,
                                           int limit) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int ok = 1;
    for (int n = 0; __hip_atomic_load(const_cast<int32_t*>(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target;
         ++n) {
      if (__hip_atomic_load(expired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        ok = 0;
        break;
      }
      if (n >= limit) {
        __hip_atomic_fetch_add(expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (status) __hip_atomic_fetch_add(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    s_ok = ok;
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  __syncthreads();  // s_ok is rewritten by the next wait
  return ok;
}

// The combine unit's wait: every work item holding one of token t's rows
// (its routed slots, and the shared expert's row) has all its GEMM2 units
// counted in.  An item is (group, pass of R rows); items are numbered group
// by group, so a row's item is the item count of the groups before its
// group plus its pass.
__device__ bool wait_token_rows(const CombineParams& c, const int32_t* ids, int t, int R, const int32_t* items2,
                                int per_item, int32_t* expired, int32_t* status, int limit) {
  __shared__ int s_base[1024 + 2];  // items of groups [0, g), g <= E + shared <= 1025
  __shared__ int s_wsum[4];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ngroups = c.E + c.shared;
  const int gpt = (ngroups + kThreads - 1) / kThreads;
  int local = 0;
  for (int q = 0; q < gpt; ++q) {
    const int g = tid * gpt + q;
    if (g < ngroups) local += (c.offsets[g + 1] - c.offsets[g] + R - 1) / R;
  }
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int run = incl - local;
  for (int q = 0; q < w; ++q) run += s_wsum[q];
  for (int q = 0; q < gpt; ++q) {
    const int g = tid * gpt + q;
    if (g < ngroups) {
      s_base[g] = run;
      run += (c.offsets[g + 1] - c.offsets[g] + R - 1) / R;
    }
  }
  __syncthreads();
  // wave 0 polls the (at most k + 1 <= 33) counters side by side, lane j
  // the item of slot j (the shared row in lane k)
  __shared__ int s_ok;
  if (w == 0) {
    int item = -1;
    if (lane < c.k) {
      const int r = c.expand_idx[long(t) * c.k + lane];
      if (r >= 0) {
        const int g = ids[long(t) * c.k + lane];
        item = s_base[g] + (r - c.offsets[g]) / R;
      }
    } else if (lane == c.k && c.shared) {
      item = s_base[c.E] + t / R;
    }
    int ok = 1;
    for (int n = 0;; ++n) {
      const bool wait = item >= 0 &&
                        __hip_atomic_load(const_cast<int32_t*>(items2) + item, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) < per_item;
      if (__ballot(wait) == 0) break;
      int stop = 0;
      if (lane == 0) {
        if (__hip_atomic_load(expired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          stop = 1;
        } else if (n >= limit) {
          __hip_atomic_fetch_add(expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (status) __hip_atomic_fetch_add(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          stop = 1;
        }
      }
      if (__shfl(stop, 0, 64)) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    if (lane == 0) s_ok = ok;
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  __syncthreads();
  return ok;
}

// The launch's arguments, read through a pointer the compiler cannot see
// through: each unit loads the part it needs when it starts, instead of
// every step's arguments staying live in scalar registers over the loop
// (which spills them).
typedef const PersistParams __attribute__((address_space(4)))* PersistArgs;
__device__ __forceinline__ const PersistParams* persist_args() {
  PersistArgs a = (PersistArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(a));
  return (const PersistParams*)a;
}

// Workgroups per CU the persistent kernel is compiled for: GEMM1's, or two
// (one with two token tiles) when GEMM2 takes eight weight tiles per wave.
template <int NTT, int B32, int NJ>
constexpr int persist_occupancy() {
  return NJ == 8 ? (NTT == 1 ? 2 : 1) : gemm1_occupancy<NTT>(B32);
}

template <int WF, int NTT, int B32, int NJ>
__global__ __launch_bounds__(kThreads, (persist_occupancy<NTT, B32, NJ>())) void k_layer_persistent(PersistParams p) {
  int32_t* const ctl = p.ctl;
  int32_t* const expired = ctl + kCtlExpired;
  int32_t* const items1 = ctl + kPersistCtlHead;
  int32_t* const items2 = items1 + p.items;
  int32_t* const status = p.status;
  const int lim = p.spin_limit;
  const int e2 = p.n1, e3 = e2 + p.n2, total = e3 + p.nC;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    __syncthreads();  // the previous unit is done with its LDS
    if (t < e2) {
      const GemmParams g1 = persist_args()->g1;
      if (gemm1_unit<WF, NTT, B32, true>(g1, t)) count_in(items1 + t / (g1.S * g1.ntiles));
    } else if (t < e3) {
      const int nt1 = persist_args()->g1.ntiles;
      const GemmParams g2 = persist_args()->g2;
      const int item = gemm2_unit<WF, NTT, B32, NJ, true>(
          g2, t - e2, [=](int it) { return wait_count(items1 + it, nt1, expired, status, lim); });
      if (item >= 0) count_in(items2 + item);
    } else {
      const CombineParams c = persist_args()->c;
      const GemmParams& g2 = persist_args()->g2;
      const int nchunk = (c.H + kThreads * 8 - 1) / (kThreads * 8);
      const int u = t - e3;
      if (wait_token_rows(c, persist_args()->ids, u / nchunk, 16 * NTT, items2, g2.S * g2.ntiles, expired, status,
                          lim))
        combine_unit<8, true>(c, u);
    }
  }
}

// =====================================================================
// host launchers
// =====================================================================
hipError_t launch_route_quant(const Shape& s, const uint16_t* x, const int32_t* ids, int32_t* counts,
                              int32_t* offsets, int32_t* expand_idx, int32_t* row_token, uint8_t* xq,
                              float* xs, int32_t* clear, int nclear, int32_t* chunk_cnt, hipStream_t st,
                              int32_t* zero1) {
  RouteParams p{x, ids, counts, offsets, expand_idx, row_token, xq, xs, reinterpret_cast<uint8_t*>(xs), clear, nclear,
                chunk_cnt, s.perm_chunk, s.perm_chunks, s.T, s.H, s.k, s.E, s.G, s.shared, s.af, zero1};
  const long items = long(s.T) * (s.H / 8);
  const long nq = (items + kThreads - 1) / kThreads;
  const int nlead = s.perm_chunks == 1 ? 1 : s.perm_chunks;
  hipLaunchKernelGGL(k_route_quant, dim3(unsigned(nlead + nq)), dim3(kThreads), 0, st, p);
  if (s.perm_chunks > 1) hipLaunchKernelGGL(k_permute_rank, dim3(unsigned(s.perm_chunks)), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_clear(int32_t* ptr, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_clear, dim3(unsigned((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, ptr, n);
  return hipGetLastError();
}

#define MOE_GEMM_DISPATCH(NAME)                                                              \
  static hipError_t dispatch_##NAME(const Shape& s, int ntt, unsigned grid, const GemmParams& p, \
                                    hipStream_t st) {                                        \
    const bool b32 = s.wfmt == 0 && s.wblk == 32;                                            \
    if (s.wfmt == 0 && !b32) {                                                               \
      if (ntt == 1) hipLaunchKernelGGL((NAME<0, 1, 0>), dim3(grid), dim3(kThreads), 0, st, p); \
      else if (ntt == 2) hipLaunchKernelGGL((NAME<0, 2, 0>), dim3(grid), dim3(kThreads), 0, st, p); \
      else hipLaunchKernelGGL((NAME<0, 4, 0>), dim3(grid), dim3(kThreads), 0, st, p);        \
    } else if (b32) {                                                                        \
      if (ntt == 1) hipLaunchKernelGGL((NAME<0, 1, 1>), dim3(grid), dim3(kThreads), 0, st, p); \
      else if (ntt == 2) hipLaunchKernelGGL((NAME<0, 2, 1>), dim3(grid), dim3(kThreads), 0, st, p); \
      else hipLaunchKernelGGL((NAME<0, 4, 1>), dim3(grid), dim3(kThreads), 0, st, p);        \
    } else if (s.wfmt == 2) {                                                                \
      if (ntt == 1) hipLaunchKernelGGL((NAME<2, 1, 0>), dim3(grid), dim3(kThreads), 0, st, p); \
      else if (ntt == 2) hipLaunchKernelGGL((NAME<2, 2, 0>), dim3(grid), dim3(kThreads), 0, st, p); \
      else hipLaunchKernelGGL((NAME<2, 4, 0>), dim3(grid), dim3(kThreads), 0, st, p);        \
    } else {                                                                                 \
      if (ntt == 1) hipLaunchKernelGGL((NAME<1, 1, 0>), dim3(grid), dim3(kThreads), 0, st, p); \
      else if (ntt == 2) hipLaunchKernelGGL((NAME<1, 2, 0>), dim3(grid), dim3(kThreads), 0, st, p); \
      else hipLaunchKernelGGL((NAME<1, 4, 0>), dim3(grid), dim3(kThreads), 0, st, p);        \
    }                                                                                        \
    return hipGetLastError();                                                                \
  }

MOE_GEMM_DISPATCH(k_gemm1)

// GEMM2 also picks its weight tiles per wave (NJ = 2, 4 or 8)
template <int NJ>
static hipError_t dispatch_gemm2_nj(const Shape& s, int ntt, unsigned grid, const GemmParams& p, hipStream_t st) {
  const bool b32 = s.wfmt == 0 && s.wblk == 32;
  const int wf = s.wfmt;
#define MOE_G2(WF, B32)                                                                                \
  do {                                                                                                 \
    if (ntt == 1) hipLaunchKernelGGL((k_gemm2<WF, 1, B32, NJ>), dim3(grid), dim3(kThreads), 0, st, p);  \
    else if (ntt == 2) hipLaunchKernelGGL((k_gemm2<WF, 2, B32, NJ>), dim3(grid), dim3(kThreads), 0, st, p); \
    else hipLaunchKernelGGL((k_gemm2<WF, 4, B32, NJ>), dim3(grid), dim3(kThreads), 0, st, p);          \
  } while (0)
  if (wf == 0 && !b32) MOE_G2(0, 0);
  else if (b32) MOE_G2(0, 1);
  else if (wf == 2) MOE_G2(2, 0);
  else MOE_G2(1, 0);
#undef MOE_G2
  return hipGetLastError();
}

hipError_t launch_gemm1(const Shape& s, const uint8_t* xq, const float* xs, const int32_t* row_token,
                        const int32_t* offsets, WeightPtrs w1, uint8_t* hq, float* hs, float* part,
                        int32_t* cnt, hipStream_t st) {
  GemmParams p{};
  p.act = xq; p.act_s = xs; p.row_token = row_token; p.offsets = offsets;
  p.w = w1.w; p.ws = w1.ws; p.sw = w1.sw; p.sws = w1.sws; p.wg = w1.g; p.swg = w1.sg;
  p.hq = hq; p.hs = hs; p.part = part; p.cnt = cnt;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.S = s.g1_split; p.ntiles = s.g1_tiles; p.rows_cap = s.rows_cap;
  const unsigned grid = unsigned(s.g1_items) * s.g1_tiles * s.g1_split;
  if (grid == 0) return hipSuccess;
  return dispatch_k_gemm1(s, s.g1_ntt, grid, p, st);
}

hipError_t launch_gemm2(const Shape& s, const uint8_t* hq, const float* hs, const int32_t* offsets,
                        WeightPtrs w2, float* y, uint16_t* yb, float* part, int32_t* cnt, hipStream_t st) {
  GemmParams p{};
  p.act = hq; p.act_s = hs; p.offsets = offsets;
  p.w = w2.w; p.ws = w2.ws; p.sw = w2.sw; p.sws = w2.sws; p.wg = w2.g; p.swg = w2.sg;
  p.y = y; p.yb = yb; p.part = part; p.cnt = cnt;
  p.H = s.H; p.I = s.I; p.E = s.E; p.G = s.G; p.wblk = s.wblk; p.ngroups = s.ngroups;
  p.S = s.g2_split; p.ntiles = s.g2_tiles; p.rows_cap = s.rows_cap;
  const unsigned grid = unsigned(s.g2_items) * s.g2_tiles * s.g2_split;
  if (grid == 0) return hipSuccess;
  if (s.g2_nj == 8) return dispatch_gemm2_nj<8>(s, s.g2_ntt, grid, p, st);
  return s.g2_nj == 4 ? dispatch_gemm2_nj<4>(s, s.g2_ntt, grid, p, st)
                      : dispatch_gemm2_nj<2>(s, s.g2_ntt, grid, p, st);
}

hipError_t launch_combine(const Shape& s, const float* y, const uint16_t* yb, const int32_t* expand_idx, const int32_t* offsets,
                          const float* topk_w, uint16_t* out, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  CombineParams p{y, yb, expand_idx, offsets, topk_w, out, s.H, s.k, s.E, s.shared};
  const int nv = yb ? 8 : 4;
  const long grid = long(s.T) * ((s.H + kThreads * nv - 1) / (kThreads * nv));
  if (yb) hipLaunchKernelGGL(k_combine<8>, dim3(unsigned(grid)), dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(k_combine<4>, dim3(unsigned(grid)), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

// Workgroups of one persistent launch: as many as fit on the device at once
// (the kernel's occupancy times the CU count), looked up once per device
// and kernel.
static int resident_grid(const void* fn) {
  struct Entry { int dev; const void* fn; int grid; };
  static Entry cache[256];
  static int n = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].dev == dev && cache[i].fn == fn) return cache[i].grid;
  int ncu = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess) return -1;
  const int grid = std::max(1, ncu * std::max(1, per_cu));
  if (n < 256) cache[n++] = Entry{dev, fn, grid};
  return grid;
}

// polls per wait of the persistent layer before the wait expires
static std::atomic<int> g_spin_limit{kPersistSpinLimit};
void set_persist_spin_limit(int polls) { g_spin_limit.store(polls); }

template <int WF, int NTT, int B32, int NJ>
static hipError_t launch_persistent_inst(const PersistParams& p, int total, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&k_layer_persistent<WF, NTT, B32, NJ>);
  const int grid = resident_grid(fn);
  if (grid < 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((k_layer_persistent<WF, NTT, B32, NJ>), dim3(unsigned(std::min(grid, total))), dim3(kThreads),
                     0, st, p);
  return hipGetLastError();
}

bool persistent_supported(const Shape& s) {
  return s.T > 0 && !s.big && s.af == 0 && s.wfmt != 2 && s.g1_ntt == s.g2_ntt &&
         s.g1_items <= kPersistMaxItems && (s.wfmt == 1 || s.g2_nj <= 4);
}

hipError_t launch_layer_persistent(const Shape& s, const uint16_t* x, const int32_t* ids, const float* tw,
                                   WeightPtrs w1, WeightPtrs w2, const LayerBufs& b, int32_t* chunk_cnt,
                                   uint16_t* out, int32_t* ctl, int32_t* status, hipStream_t st) {
  if (!persistent_supported(s)) return hipErrorInvalidValue;
  // routing and quantisation; also zeroes the control block (inside the
  // cleared counter range) and the status word
  const hipError_t e = launch_route_quant(s, x, ids, b.counts, b.offsets, b.expand_idx, b.row_token, b.xq, b.xs,
                                          b.clear, b.nclear, chunk_cnt, st, status);
  if (e != hipSuccess) return e;
  PersistParams p{};
  GemmParams& g1 = p.g1;
  g1.act = b.xq; g1.act_s = b.xs; g1.row_token = b.row_token; g1.offsets = b.offsets;
  g1.w = w1.w; g1.ws = w1.ws; g1.sw = w1.sw; g1.sws = w1.sws; g1.wg = w1.g; g1.swg = w1.sg;
  g1.hq = b.hq; g1.hs = b.hs; g1.part = b.part1; g1.cnt = b.cnt1;
  g1.H = s.H; g1.I = s.I; g1.E = s.E; g1.G = s.G; g1.wblk = s.wblk; g1.ngroups = s.ngroups;
  g1.S = s.g1_split; g1.ntiles = s.g1_tiles; g1.rows_cap = s.rows_cap;
  GemmParams& g2 = p.g2;
  g2.act = b.hq; g2.act_s = b.hs; g2.offsets = b.offsets;
  g2.w = w2.w; g2.ws = w2.ws; g2.sw = w2.sw; g2.sws = w2.sws; g2.wg = w2.g; g2.swg = w2.sg;
  g2.yb = b.yb; g2.part = b.part2; g2.cnt = b.cnt2;
  g2.H = s.H; g2.I = s.I; g2.E = s.E; g2.G = s.G; g2.wblk = s.wblk; g2.ngroups = s.ngroups;
  g2.S = s.g2_split; g2.ntiles = s.g2_tiles; g2.rows_cap = s.rows_cap;
  p.c = CombineParams{nullptr, b.yb, b.expand_idx, b.offsets, tw, out, s.H, s.k, s.E, s.shared};
  p.ids = ids;
  p.ctl = ctl;
  p.status = status;
  p.items = s.g1_items;
  p.n1 = s.g1_items * s.g1_tiles * s.g1_split;
  p.n2 = s.g2_items * s.g2_tiles * s.g2_split;
  p.nC = s.T * ((s.H + kThreads * 8 - 1) / (kThreads * 8));
  p.spin_limit = g_spin_limit.load();
  const int total = p.n1 + p.n2 + p.nC;
  const bool b32 = s.wfmt == 0 && s.wblk == 32;
#define MOE_P(WF, NTT, B32)                                                                       \
  do {                                                                                            \
    if (s.g2_nj == 2) return launch_persistent_inst<WF, NTT, B32, 2>(p, total, st);              \
    if (s.g2_nj == 4) return launch_persistent_inst<WF, NTT, B32, 4>(p, total, st);              \
    if (WF == 1) return launch_persistent_inst<1, NTT, 0, 8>(p, total, st);                      \
  } while (0)
  if (s.wfmt == 1) {
    if (s.g1_ntt == 1) MOE_P(1, 1, 0);
    else if (s.g1_ntt == 2) MOE_P(1, 2, 0);
    else MOE_P(1, 4, 0);
  } else if (b32) {
    if (s.g1_ntt == 1) MOE_P(0, 1, 1);
    else if (s.g1_ntt == 2) MOE_P(0, 2, 1);
    else MOE_P(0, 4, 1);
  } else {
    if (s.g1_ntt == 1) MOE_P(0, 1, 0);
    else if (s.g1_ntt == 2) MOE_P(0, 2, 0);
    else MOE_P(0, 4, 0);
  }
#undef MOE_P
  return hipErrorInvalidValue;
}

}  // namespace moe
