// moe_diag.hip -- diagnostics the kernels are measured against: a plain HBM
// read stream (the achievable bandwidth), the issued rate of the scaled
// MFMA the GEMMs use (the achievable matrix-core rate), and the fp32 ->
// e4m3 conversion every quantiser uses, exposed on its own so it can be
// checked on every fp32 bit pattern.
//
// Read stream:
// The buffer is cut into one contiguous region per wave (a multiple of the
// 4 KiB a wave reads per step); a wave reads its region front to back with
// four 1 KiB non-temporal loads in flight (16 bytes a lane, consecutive
// lanes on consecutive chunks).  Four workgroups of four waves per CU.  Each
// workgroup folds what it read into one word of the sink, so the loads
// cannot be dropped.
#include <algorithm>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 4;                      // 1 KiB loads per wave per step
constexpr long kStreamStep = long(kWave) * kStreamLoads;  // 16-byte chunks per wave per step

__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const v4u* __restrict__ src, long n16, long per_wave,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_acc[kStreamThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const long wave = long(blockIdx.x) * (kStreamThreads / kWave) + threadIdx.x / kWave;
  const long beg = wave * per_wave;
  const long end = beg + per_wave < n16 ? beg + per_wave : n16;
  uint32_t acc = 0;
  long s = beg;
  for (; s + kStreamStep <= end; s += kStreamStep) {
    v4u v[kStreamLoads];
#pragma unroll
    for (int u = 0; u < kStreamLoads; ++u) v[u] = __builtin_nontemporal_load(src + s + u * kWave + lane);
#pragma unroll
    for (int u = 0; u < kStreamLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (long j = s + lane; j < end; j += kWave) {
    const v4u v = __builtin_nontemporal_load(src + j);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if (lane == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int w = 0; w < kStreamThreads / kWave; ++w) a ^= s_acc[w];
    sink[blockIdx.x] = a;
  }
}

// Issued-rate probe: every wave runs `iters` rounds of kRateAcc independent
// 16x16x128 scaled MFMAs (operand formats FA x FB, unit scales) on
// operands made of the codes a_word / b_word, so the matrix pipe never waits
// on a result; four workgroups of four waves per CU.  Lane 0 of wave 0
// stores the sum of its accumulators' elements: with both operands 1.0
// every MFMA adds exactly 128 to each element, so the stored value is
// 4 * 128 * kRateAcc * iters (exact in fp32 for iters <= 65536).
constexpr int kRateAcc = 8;

template <int FA, int FB>
__global__ __launch_bounds__(kStreamThreads) void k_mfma_rate(uint32_t a_word, uint32_t b_word, int iters,
                                                             float* __restrict__ sink) {
  const int aw = int(a_word), bw = int(b_word);
  const v8i a = {aw, aw, aw, aw, aw, aw, aw, aw};
  const v8i b = {bw, bw, bw, bw, bw, bw, bw, bw};
  v4f acc[kRateAcc];
#pragma unroll
  for (int j = 0; j < kRateAcc; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kRateAcc; ++j) acc[j] = mfma_scaled_acc<FA, FB>(a, b, acc[j], kUnitScale, kUnitScale);
  }
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < kRateAcc; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[blockIdx.x] = t;
  }
}

// The quantisers' fp32 -> e4m3 conversion (enc_e4m3x4: saturation at +-448,
// round to nearest even, sign kept) on n values, four per thread.
__global__ __launch_bounds__(kStreamThreads) void k_encode_e4m3(const float* __restrict__ v, long n,
                                                               uint8_t* __restrict__ codes) {
  const long n4 = n / 4;
  const long stride = long(gridDim.x) * kStreamThreads;
  for (long i = long(blockIdx.x) * kStreamThreads + threadIdx.x; i < n4; i += stride) {
    const v4f x = reinterpret_cast<const v4f*>(v)[i];
    reinterpret_cast<uint32_t*>(codes)[i] = enc_e4m3x4(x[0], x[1], x[2], x[3]);
  }
  const long t = n4 * 4 + threadIdx.x;  // the last n % 4 values, by block 0
  if (blockIdx.x == 0 && t < n) codes[t] = uint8_t(enc_e4m3x4(v[t], 0.0f, 0.0f, 0.0f) & 0xFFu);
}

}  // namespace

hipError_t launch_encode_e4m3(const float* v, long n, uint8_t* codes, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long blocks = std::min<long>(4096, (n / 4 + kStreamThreads - 1) / kStreamThreads + 1);
  hipLaunchKernelGGL(k_encode_e4m3, dim3(unsigned(blocks)), dim3(kStreamThreads), 0, st, v, n, codes);
  return hipGetLastError();
}

int mfma_rate_grid() { return stream_read_grid(); }

hipError_t launch_mfma_rate(int wfmt, int iters, float* sink, double* flops, hipStream_t st) {
  const int grid = mfma_rate_grid();
  if (flops) *flops = double(grid) * (kStreamThreads / kWave) * double(iters) * kRateAcc * (16.0 * 16.0 * 128.0 * 2.0);
  // operands of 1.0: e4m3 0x38 in every byte, e2m1 0x2 in every nibble
  if (wfmt == 0)
    hipLaunchKernelGGL((k_mfma_rate<kFmtE4M3, kFmtE4M3>), dim3(unsigned(grid)), dim3(kStreamThreads), 0, st,
                       0x38383838u, 0x38383838u, iters, sink);
  else if (wfmt == 1)
    hipLaunchKernelGGL((k_mfma_rate<kFmtE2M1, kFmtE4M3>), dim3(unsigned(grid)), dim3(kStreamThreads), 0, st,
                       0x22222222u, 0x38383838u, iters, sink);
  else  // e2m1 x e2m1 (MOE_RATE_E2M1_E2M1)
    hipLaunchKernelGGL((k_mfma_rate<kFmtE2M1, kFmtE2M1>), dim3(unsigned(grid)), dim3(kStreamThreads), 0, st,
                       0x22222222u, 0x22222222u, iters, sink);
  return hipGetLastError();
}

int stream_read_grid() {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  return 4 * ncu;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  const long n16 = long(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int grid = stream_read_grid();
  const long waves = long(grid) * (kStreamThreads / kWave);
  long per = (n16 + waves - 1) / waves;
  per = (per + kStreamStep - 1) / kStreamStep * kStreamStep;
  hipLaunchKernelGGL(k_stream_read, dim3(unsigned(grid)), dim3(kStreamThreads), 0, st, static_cast<const v4u*>(buf),
                     n16, per, sink);
  return hipGetLastError();
}

}  // namespace moe
