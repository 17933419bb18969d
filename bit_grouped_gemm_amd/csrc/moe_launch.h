// moe_launch.h -- internal interface between the C-ABI layer (moe_api.hip)
// and the kernels (moe_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Shape facts derived once on the host from a validated moe_cfg.
struct Shape {
  int T, H, I, E, k, wfmt, wblk, G, shared;
  int af;           // activation format: 0 e4m3 + fp32 scale per G, 1 MXFP4 (e2m1 + e8m0 per 32)
  int ngroups;      // E + shared
  int rows_cap;     // T*k + T*shared: upper bound on permuted rows
  int slots_max;    // upper bound on non-empty groups: min(E, T*k) + shared
  // GEMM1: unit = 128 h-columns (128 gate + 128 up weight rows) of one group
  int g1_tiles;     // I / 128
  int g1_split;     // K splits over H/128 steps
  int g1_ntt;       // 16-token tiles per pass (1, 2 or 4)
  int g1_items;     // upper bound on work items (one pass of 16 g1_ntt rows of one group)
  // GEMM2: unit = 64 g2_nj output rows of one group
  int g2_nj;        // weight tiles per wave: 2, 4 (256-row units, two or more token tiles), 8 (MXFP4 at one unit per CU)
  int g2_tiles;     // H / (64 g2_nj)
  int g2_split;     // K splits over I/128 steps
  int g2_ntt;
  int g2_items;     // as g1_items, passes of 16 g2_ntt rows
  // groups with many rows (prefill, larger decode batches) run the LDS-staged
  // kernels: 256 weight rows x big_cap token rows per pass
  int big;          // 1: both GEMMs use the big-tile kernels
  int big_cap;      // their token rows per pass: 64 or 160 (NVFP4: 64 or 96)
  // permute: slots per chunk and chunk count; one chunk = one block places
  // every slot, more = a counting pass then one placing block per chunk
  int perm_chunk, perm_chunks;
};

// Workspace carve (byte offsets from the caller's ws base; 256-aligned).
struct WsLayout {
  size_t counts, offsets, expand_idx, row_token;  // layer-internal permute outputs
  size_t xq, xs, hq, hs, y;                       // layer-internal activations
  size_t part1, part2;                            // split-K partial sums (fp32)
  size_t cnt1, cnt2;                              // split-K arrival counters (int32), per work item and tile
  size_t pctl;                                    // persistent layer's control block (int32)
  size_t chunk_cnt;                               // permute per-chunk expert counts (int32)
  size_t total;
};

Shape make_shape(int T, int H, int I, int E, int k, int wfmt, int wblk, int G, int shared, int af);
WsLayout make_ws_layout(const Shape& s);

struct WeightPtrs {
  const uint8_t* w;   // routed [E][N][Kbytes]
  const void* ws;     // routed scales
  const uint8_t* sw;  // shared expert (or null)
  const void* sws;
  const float* g = nullptr;   // NVFP4: fp32 scale per routed matrix [E]
  const float* sg = nullptr;  // and the shared expert's [1]
};

// clear: nclear ints zeroed by the routing block; zero1: one more int (or null)
hipError_t launch_route_quant(const Shape& s, const uint16_t* x, const int32_t* ids, int32_t* counts,
                              int32_t* offsets, int32_t* expand_idx, int32_t* row_token, uint8_t* xq,
                              float* xs, int32_t* clear, int nclear, int32_t* chunk_cnt, hipStream_t st,
                              int32_t* zero1 = nullptr);

hipError_t launch_clear(int32_t* p, int n, hipStream_t st);

hipError_t launch_gemm1(const Shape& s, const uint8_t* xq, const float* xs, const int32_t* row_token,
                        const int32_t* offsets, WeightPtrs w1, uint8_t* hq, float* hs, float* part,
                        int32_t* cnt, hipStream_t st);

hipError_t launch_gemm2(const Shape& s, const uint8_t* hq, const float* hs, const int32_t* offsets,
                        WeightPtrs w2, float* y, uint16_t* yb, float* part, int32_t* cnt, hipStream_t st);

hipError_t launch_gemm1_big(const Shape& s, const uint8_t* xq, const float* xs, const int32_t* row_token,
                            const int32_t* offsets, WeightPtrs w1, uint8_t* hq, float* hs, int min_rows,
                            hipStream_t st);

hipError_t launch_gemm2_big(const Shape& s, const uint8_t* hq, const float* hs, const int32_t* offsets,
                            WeightPtrs w2, float* y, uint16_t* yb, int min_rows, hipStream_t st);

// diagnostics (moe_diag.hip): plain read stream over a device buffer, and
// the issued rate of the scaled MFMA (flops: host, the FLOP count enqueued)
int stream_read_grid();
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
int mfma_rate_grid();
hipError_t launch_mfma_rate(int wfmt, int iters, float* sink, double* flops, hipStream_t st);
hipError_t launch_encode_e4m3(const float* v, long n, uint8_t* codes, hipStream_t st);

// router (moe_router.hip): gate GEMM + top-k + softmax of the selected logits,
// two kernels over `part`, a scratch of route_workspace_bytes(T, H, E) bytes
// (0 only for T = 0)
size_t route_workspace_bytes(int T, int H, int E);
hipError_t launch_route_gemm(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wg, int32_t* ids,
                             float* weights, float* part, hipStream_t st);

hipError_t launch_tile_weights(int wfmt, int mats, int N, int K, const uint8_t* w, const uint8_t* s, uint8_t* w_tiled,
                               uint8_t* s_tiled, hipStream_t st);

// The persistent decode layer (routing launch, then GEMM1, GEMM2 and the
// combine in one launch).  Its control block, in the workspace, holds
// kPersistCtlHead ints, then per work item a GEMM1 and a GEMM2 counter; the
// routing launch zeroes it.
constexpr int kPersistCtlHead = 128;
constexpr int kPersistMaxItems = 1 << 20;
constexpr int kPersistSpinLimit = 1 << 20;  // default polls per wait (about a second)
void set_persist_spin_limit(int polls);

// The layer's buffers inside a workspace (see WsLayout).
struct LayerBufs {
  int32_t *counts, *offsets, *expand_idx, *row_token;
  uint8_t* xq;
  float* xs;
  uint8_t* hq;
  float* hs;
  uint16_t* yb;
  float *part1, *part2;
  int32_t *cnt1, *cnt2;
  int32_t* clear;  // the split-K counters the routing unit zeroes (nclear ints)
  int nclear;
};

// Shapes the persistent layer runs: the decode kernels (not the many-row
// ones), FP8 activations, FP8 or MXFP4 weights.
bool persistent_supported(const Shape& s);
hipError_t launch_layer_persistent(const Shape& s, const uint16_t* x, const int32_t* ids, const float* tw,
                                   WeightPtrs w1, WeightPtrs w2, const LayerBufs& b, int32_t* chunk_cnt,
                                   uint16_t* out, int32_t* ctl, int32_t* status, hipStream_t st);

// y: GEMM2 output rows in fp32, or yb in bf16 (the layer's internal form; y unused then)
hipError_t launch_combine(const Shape& s, const float* y, const uint16_t* yb, const int32_t* expand_idx, const int32_t* offsets,
                          const float* topk_w, uint16_t* out, hipStream_t st);

}  // namespace moe
