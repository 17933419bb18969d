// moe_tile.hip -- reorder expert weights from the row-major layout into the
// tiled layout the grouped GEMMs read.
//
// Tile (k step ks, row tile rt) of a [N][K] matrix holds rows 16 rt .. +15
// and K 128 ks .. +127 in the lane order of the scaled-MFMA operand: lane l
// (row 16 rt + l % 16, K group l / 16) owns 16 bytes at l * 16, and e4m3
// tiles hold the second half of the step (K 64..127) in a second kilobyte.
// Tiles are stored k-step major, [mats][K/128][N/16][tile], so the tiles of
// consecutive rows for one k step are adjacent.  MXFP4 scales follow the
// same order with 64 bytes per tile, byte l being the e8m0 scale MFMA lane
// l consumes (row 16 rt + l % 16, 32-block 4 ks + l / 16).  NVFP4 codes
// tile as MXFP4's; its e4m3 scales take 128 bytes per tile, row m's eight
// 16-blocks of the step at 8 m.  The reorder is a permutation: sizes are
// those of the row-major tensors.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kTileThreads = 256;

// one thread per 16-byte chunk of the tiled tensor
template <int WF>
__global__ __launch_bounds__(kTileThreads) void k_tile_weights(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, long chunks, int N, int K) {
  constexpr int kChunksPerTile = kTileBytes<WF> / 16;
  const long kb = WF == 0 ? K : K / 2;  // bytes per row
  const int nrt = N / 16, nks = K / 128;
  for (long c = long(blockIdx.x) * kTileThreads + threadIdx.x; c < chunks; c += long(gridDim.x) * kTileThreads) {
    const long tile = c / kChunksPerTile;
    const int within = int(c % kChunksPerTile);
    const int half = within / 64, l = within % 64;
    const int rt = int(tile % nrt);
    const long rest = tile / nrt;
    const int ks = int(rest % nks);
    const long mat = rest / nks;
    const long row = long(rt) * 16 + (l & 15);
    const long byte = long(ks) * (WF == 0 ? 128 : 64) + half * 64 + (l >> 4) * 16;
    *reinterpret_cast<v4u*>(dst + c * 16) = ldg16(src + (mat * N + row) * kb + byte);
  }
}

// one thread per scale byte of the tiled MXFP4 scales
__global__ __launch_bounds__(kTileThreads) void k_tile_scales(const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst, long bytes, int N, int K) {
  const int nrt = N / 16, nks = K / 128, kg = K / 32;
  for (long i = long(blockIdx.x) * kTileThreads + threadIdx.x; i < bytes; i += long(gridDim.x) * kTileThreads) {
    const long tile = i / kTileScaleBytes;
    const int l = int(i % kTileScaleBytes);
    const int rt = int(tile % nrt);
    const long rest = tile / nrt;
    const int ks = int(rest % nks);
    const long mat = rest / nks;
    dst[i] = src[(mat * N + long(rt) * 16 + (l & 15)) * kg + ks * 4 + (l >> 4)];
  }
}

// one thread per scale byte of the tiled NVFP4 scales
__global__ __launch_bounds__(kTileThreads) void k_tile_scales16(const uint8_t* __restrict__ src,
                                                               uint8_t* __restrict__ dst, long bytes, int N, int K) {
  const int nrt = N / 16, nks = K / 128, kb = K / 16;
  for (long i = long(blockIdx.x) * kTileThreads + threadIdx.x; i < bytes; i += long(gridDim.x) * kTileThreads) {
    const long tile = i / kTileScaleBytes16;
    const int within = int(i % kTileScaleBytes16);
    const int rt = int(tile % nrt);
    const long rest = tile / nrt;
    const int ks = int(rest % nks);
    const long mat = rest / nks;
    dst[i] = src[(mat * N + long(rt) * 16 + within / 8) * kb + ks * 8 + within % 8];
  }
}

unsigned grid_for(long items) {
  const long blocks = (items + kTileThreads - 1) / kTileThreads;
  return unsigned(blocks < 8192 ? blocks : 8192);
}

}  // namespace

hipError_t launch_tile_weights(int wfmt, int mats, int N, int K, const uint8_t* w, const uint8_t* s, uint8_t* w_tiled,
                               uint8_t* s_tiled, hipStream_t st) {
  const long wbytes = long(mats) * N * (wfmt == 0 ? K : K / 2);
  const long chunks = wbytes / 16;
  if (chunks > 0) {
    if (wfmt == 0) hipLaunchKernelGGL(k_tile_weights<0>, dim3(grid_for(chunks)), dim3(kTileThreads), 0, st, w, w_tiled, chunks, N, K);
    else hipLaunchKernelGGL(k_tile_weights<1>, dim3(grid_for(chunks)), dim3(kTileThreads), 0, st, w, w_tiled, chunks, N, K);
  }
  if (wfmt == 1) {
    const long sbytes = long(mats) * N * (K / 32);
    if (sbytes > 0)
      hipLaunchKernelGGL(k_tile_scales, dim3(grid_for(sbytes)), dim3(kTileThreads), 0, st, s, s_tiled, sbytes, N, K);
  } else if (wfmt == 2) {
    const long sbytes = long(mats) * N * (K / 16);
    if (sbytes > 0)
      hipLaunchKernelGGL(k_tile_scales16, dim3(grid_for(sbytes)), dim3(kTileThreads), 0, st, s, s_tiled, sbytes, N, K);
  }
  return hipGetLastError();
}

}  // namespace moe
