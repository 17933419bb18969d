// moe_bench_main.cpp -- a standalone C++ driver of the C ABI in include/moe.h.
//
// Runs one layer shape on synthetic inputs generated on the host (no
// PyTorch, no other GPU library in the process), so that a profiler's
// counter collection sees only this library's kernels and the runtime's
// host-to-device copies.  It is also the smallest complete example of
// calling the ABI from C++: canonical weights -> moe_prepack_weights ->
// moe_workspace_size -> moe_layer / the stage calls, all on one stream.
//
//   moe_bench copy MIB
//     three device-to-device copies of MIB MiB (the runtime's copy kernel):
//     a transfer of known size, to scale a profiler's byte counters by
//   moe_bench route WORKLOAD T REPS
//     the router (moe_route) on the workload's H, E and top-k: bf16 tokens
//     ~N(0,1) and gate rows ~N(0, 0.02), REPS timed calls after one untimed
//   moe_bench WORKLOAD T REPS [stages]
//     WORKLOAD  decode_fp8 | decode_mxfp4 | decode_fp8_zipf_shared | prefill_mxfp4 |
//               prefill_mxfp4_a4
//               (the shapes of the Python workloads of the same names)
//     T         tokens; REPS timed moe_layer calls (after one untimed call)
//     stages    also time REPS passes of the four stage calls
//
// Input values are synthetic and seeded (splitmix64): bf16 activations
// ~N(0,1), uniform (or Zipf) distinct top-k ids with softmax weights,
// random valid weight codes (no NaN codes) with scales near those of
// N(0, 0.02) weights.  Timings (hipEvent, median) go to stdout.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe.h"

namespace {

struct Shape {
  const char* name;
  int H, E, k, I, wfmt, wblk, G, shared, zipf, af;
};

const Shape kShapes[] = {
    {"decode_fp8", 4096, 64, 8, 1536, MOE_WFMT_FP8_BLOCK, 128, 128, 0, 0, MOE_AFMT_FP8},
    {"decode_mxfp4", 4096, 64, 8, 1536, MOE_WFMT_MXFP4, 32, 128, 0, 0, MOE_AFMT_FP8},
    {"decode_fp8_zipf_shared", 7168, 256, 8, 2048, MOE_WFMT_FP8_BLOCK, 128, 128, 1, 1, MOE_AFMT_FP8},
    {"prefill_mxfp4", 7168, 256, 8, 2048, MOE_WFMT_MXFP4, 32, 128, 0, 0, MOE_AFMT_FP8},
    {"prefill_mxfp4_a4", 7168, 256, 8, 2048, MOE_WFMT_MXFP4, 32, 32, 0, 0, MOE_AFMT_MXFP4},
};

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
double uniform(uint64_t& s) { return double(splitmix64(s) >> 11) * 0x1p-53; }
double normal(uint64_t& s) {  // Box-Muller
  const double u1 = std::max(uniform(s), 1e-300), u2 = uniform(s);
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
}
uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

#define HIP_CHECK(x)                                                                  \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
      std::exit(1);                                                                   \
    }                                                                                 \
  } while (0)
#define MOE_CHECK(x)                                                                  \
  do {                                                                                \
    int r_ = (x);                                                                     \
    if (r_ != MOE_OK) {                                                               \
      std::fprintf(stderr, "%s failed: %d (%s)\n", #x, r_, moe_status_str(r_));       \
      std::exit(1);                                                                   \
    }                                                                                 \
  } while (0)

void* upload(const void* host, size_t bytes) {
  void* d = nullptr;
  HIP_CHECK(hipMalloc(&d, std::max<size_t>(bytes, 16)));
  if (bytes) HIP_CHECK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

// One matrix set [mats][N][K] of weight codes and scales in the canonical layout.
void gen_matrix(const Shape& s, int mats, int N, int K, uint64_t seed, std::vector<uint8_t>& w,
                std::vector<uint8_t>& sc) {
  uint64_t st = seed;
  if (s.wfmt == MOE_WFMT_MXFP4) {
    w.resize(size_t(mats) * N * (K / 2));  // every nibble is a valid e2m1 code
    for (size_t i = 0; i < w.size(); i += 8) {
      const uint64_t r = splitmix64(st);
      std::memcpy(&w[i], &r, std::min<size_t>(8, w.size() - i));
    }
    sc.resize(size_t(mats) * N * (K / 32));
    for (auto& b : sc) b = uint8_t(119 + splitmix64(st) % 3);  // 2^-8 .. 2^-6
  } else {
    w.resize(size_t(mats) * N * K);
    for (size_t i = 0; i < w.size(); i += 8) {
      uint64_t r = splitmix64(st);
      for (size_t j = 0; j < 8 && i + j < w.size(); ++j, r >>= 8) {
        uint8_t c = uint8_t(r);
        if ((c & 0x7F) == 0x7F) c &= 0xFE;  // no NaN codes
        w[i + j] = c;
      }
    }
    const size_t ns = size_t(mats) * (N / s.wblk) * (K / s.wblk);
    sc.resize(ns * 4);
    for (size_t i = 0; i < ns; ++i) {
      const float v = float(0.08 / 448.0 * (0.9 + 0.2 * uniform(st)));
      std::memcpy(&sc[i * 4], &v, 4);
    }
  }
}

double median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v.empty() ? 0.0 : v[v.size() / 2];
}

}  // namespace

int main(int argc, char** argv) {
  if (argc == 3 && std::string(argv[1]) == "copy") {
    const size_t bytes = size_t(std::atol(argv[2])) << 20;
    void *src = nullptr, *dst = nullptr;
    HIP_CHECK(hipMalloc(&src, bytes));
    HIP_CHECK(hipMalloc(&dst, bytes));
    HIP_CHECK(hipMemset(src, 1, bytes));
    for (int i = 0; i < 3; ++i) HIP_CHECK(hipMemcpy(dst, src, bytes, hipMemcpyDeviceToDevice));
    HIP_CHECK(hipDeviceSynchronize());
    std::printf("copied %zu bytes 3 times\ndone\n", bytes);
    return 0;
  }
  if (argc < 4) {
    std::fprintf(stderr, "usage: %s WORKLOAD T REPS [stages] | %s route WORKLOAD T REPS | %s copy MIB\n", argv[0],
                 argv[0], argv[0]);
    return 2;
  }
  const bool route = std::string(argv[1]) == "route";
  if (route && argc < 5) return 2;
  const char* wname = route ? argv[2] : argv[1];
  const Shape* sp = nullptr;
  for (const auto& s : kShapes)
    if (std::string(wname) == s.name) sp = &s;
  if (!sp) {
    std::fprintf(stderr, "unknown workload %s\n", wname);
    return 2;
  }
  if (route) {
    const Shape& s = *sp;
    const int T = std::atoi(argv[3]), reps = std::atoi(argv[4]);
    if (T < 1 || reps < 1) return 2;
    moe_cfg cfg{T, s.H, s.I, s.E, s.k, s.wfmt, s.wblk, s.G, s.shared, s.af};
    uint64_t st = 0x5EED0001ull;
    std::vector<uint16_t> x(size_t(T) * s.H), g(size_t(s.E) * s.H);
    for (auto& v : x) v = to_bf16(float(normal(st)));
    for (auto& v : g) v = to_bf16(float(0.02 * normal(st)));
    void* dx = upload(x.data(), x.size() * 2);
    void* dg = upload(g.data(), g.size() * 2);
    void* ids = nullptr;
    void* tw = nullptr;
    HIP_CHECK(hipMalloc(&ids, size_t(T) * s.k * 4));
    HIP_CHECK(hipMalloc(&tw, size_t(T) * s.k * 4));
    size_t nws = 0;
    MOE_CHECK(moe_route_workspace_size(&cfg, &nws));
    void* ws = nullptr;
    HIP_CHECK(hipMalloc(&ws, std::max<size_t>(nws, 16)));
    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    auto call = [&] {
      MOE_CHECK(moe_route(&cfg, static_cast<const uint16_t*>(dx), static_cast<const uint16_t*>(dg),
                          static_cast<int32_t*>(ids), static_cast<float*>(tw), ws, nws, stream));
    };
    call();
    HIP_CHECK(hipStreamSynchronize(stream));
    hipEvent_t a, b;
    HIP_CHECK(hipEventCreate(&a));
    HIP_CHECK(hipEventCreate(&b));
    std::vector<double> us;
    for (int r = 0; r < reps; ++r) {
      HIP_CHECK(hipEventRecord(a, stream));
      call();
      HIP_CHECK(hipEventRecord(b, stream));
      HIP_CHECK(hipEventSynchronize(b));
      float ms = 0.0f;
      HIP_CHECK(hipEventElapsedTime(&ms, a, b));
      us.push_back(ms * 1e3);
    }
    std::printf("route %s T=%d: %.2f us median of %d (warm)\ndone\n", s.name, T, median(us), reps);
    return 0;
  }
  const Shape& s = *sp;
  const int T = std::atoi(argv[2]), reps = std::atoi(argv[3]);
  const bool stages = argc > 4 && std::string(argv[4]) == "stages";
  if (T < 0 || reps < 1) return 2;
  moe_cfg cfg{T, s.H, s.I, s.E, s.k, s.wfmt, s.wblk, s.G, s.shared, s.af};

  // ---- inputs on the host
  uint64_t st = 0x5EEDull + uint64_t(T);
  std::vector<uint16_t> x(size_t(T) * s.H);
  for (auto& v : x) v = to_bf16(float(normal(st)));
  std::vector<int32_t> ids(size_t(T) * s.k);
  std::vector<float> tw(size_t(T) * s.k);
  std::vector<double> zp(s.E);
  for (int e = 0; e < s.E; ++e) zp[e] = std::pow(double(e + 1), -1.2);
  for (int t = 0; t < T; ++t) {
    std::vector<char> used(s.E, 0);
    double tot = 0.0;
    for (int j = 0; j < s.k; ++j) {
      int e = 0;
      if (s.zipf) {  // draw, remove, renormalise
        double mass = 0.0;
        for (int q = 0; q < s.E; ++q) mass += used[q] ? 0.0 : zp[q];
        double u = uniform(st) * mass;
        for (e = 0; e < s.E - 1; ++e) {
          if (used[e]) continue;
          if ((u -= zp[e]) < 0.0) break;
        }
        while (used[e]) e = (e + 1) % s.E;
      } else {
        do e = int(splitmix64(st) % uint64_t(s.E)); while (used[e]);
      }
      used[e] = 1;
      ids[size_t(t) * s.k + j] = e;
      const double l = std::exp(normal(st));
      tw[size_t(t) * s.k + j] = float(l);
      tot += l;
    }
    for (int j = 0; j < s.k; ++j) tw[size_t(t) * s.k + j] = float(tw[size_t(t) * s.k + j] / tot);
  }
  std::vector<uint8_t> w1, w1s, w2, w2s, sw1, sw1s, sw2, sw2s;
  gen_matrix(s, s.E, 2 * s.I, s.H, 11, w1, w1s);
  gen_matrix(s, s.E, s.H, s.I, 12, w2, w2s);
  if (s.shared) {
    gen_matrix(s, 1, 2 * s.I, s.H, 13, sw1, sw1s);
    gen_matrix(s, 1, s.H, s.I, 14, sw2, sw2s);
  }

  // ---- device copies, re-layout, workspace
  moe_weights canon{upload(w1.data(), w1.size()), upload(w1s.data(), w1s.size()),
                    upload(w2.data(), w2.size()),  upload(w2s.data(), w2s.size()),
                    s.shared ? upload(sw1.data(), sw1.size()) : nullptr,
                    s.shared ? upload(sw1s.data(), sw1s.size()) : nullptr,
                    s.shared ? upload(sw2.data(), sw2.size()) : nullptr,
                    s.shared ? upload(sw2s.data(), sw2s.size()) : nullptr, 0};
  moe_weights tiled{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0};
  const size_t sizes[8] = {w1.size(), w1s.size(), w2.size(), w2s.size(), sw1.size(), sw1s.size(), sw2.size(),
                           sw2s.size()};
  const void** tp[8] = {&tiled.w1, &tiled.w1s, &tiled.w2, &tiled.w2s, &tiled.sw1, &tiled.sw1s, &tiled.sw2,
                        &tiled.sw2s};
  for (int i = 0; i < (s.shared ? 8 : 4); ++i) {
    void* d = nullptr;
    HIP_CHECK(hipMalloc(&d, sizes[i]));
    *tp[i] = d;
  }
  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));
  MOE_CHECK(moe_prepack_weights(&cfg, &canon, &tiled, stream));
  void* dx = upload(x.data(), x.size() * 2);
  void* dids = upload(ids.data(), ids.size() * 4);
  void* dtw = upload(tw.data(), tw.size() * 4);
  void* dout = nullptr;
  HIP_CHECK(hipMalloc(&dout, std::max<size_t>(size_t(T) * s.H * 2, 16)));
  size_t wsb = 0;
  MOE_CHECK(moe_workspace_size(&cfg, &wsb));
  void* ws = nullptr;
  HIP_CHECK(hipMalloc(&ws, wsb));
  const size_t R = size_t(T) * s.k + size_t(T) * s.shared;
  void *counts, *offsets, *eidx, *rtok, *xq, *xs, *hq, *hs, *y;
  HIP_CHECK(hipMalloc(&counts, 4 * size_t(s.E + 1)));
  HIP_CHECK(hipMalloc(&offsets, 4 * size_t(s.E + 2)));
  HIP_CHECK(hipMalloc(&eidx, 4 * std::max<size_t>(size_t(T) * s.k, 4)));
  HIP_CHECK(hipMalloc(&rtok, 4 * std::max<size_t>(R, 4)));
  HIP_CHECK(hipMalloc(&xq, std::max<size_t>(size_t(T) * s.H, 16)));
  HIP_CHECK(hipMalloc(&xs, 4 * std::max<size_t>(size_t(T) * (s.H / s.G), 4)));
  HIP_CHECK(hipMalloc(&hq, std::max<size_t>(R * s.I, 16)));
  HIP_CHECK(hipMalloc(&hs, 4 * std::max<size_t>(R * (s.I / s.G), 4)));
  HIP_CHECK(hipMalloc(&y, 4 * std::max<size_t>(R * s.H, 4)));
  HIP_CHECK(hipStreamSynchronize(stream));

  // ---- timed calls
  hipEvent_t a, b;
  HIP_CHECK(hipEventCreate(&a));
  HIP_CHECK(hipEventCreate(&b));
  auto layer = [&] {
    MOE_CHECK(moe_layer(&cfg, static_cast<const uint16_t*>(dx), static_cast<const int32_t*>(dids),
                        static_cast<const float*>(dtw), &tiled, static_cast<uint16_t*>(dout), ws, wsb, stream));
  };
  layer();
  std::vector<double> lat;
  for (int r = 0; r < reps; ++r) {
    HIP_CHECK(hipEventRecord(a, stream));
    layer();
    HIP_CHECK(hipEventRecord(b, stream));
    HIP_CHECK(hipEventSynchronize(b));
    float ms = 0.0f;
    HIP_CHECK(hipEventElapsedTime(&ms, a, b));
    lat.push_back(ms * 1e3);
  }
  std::printf("%s T=%d: moe_layer median %.1f us over %d calls (workspace %.1f MiB)\n", s.name, T, median(lat),
              reps, wsb / 1048576.0);
  if (stages) {
    std::vector<double> st_us[4];
    hipEvent_t e[5];
    for (auto& q : e) HIP_CHECK(hipEventCreate(&q));
    for (int r = 0; r < reps; ++r) {
      HIP_CHECK(hipEventRecord(e[0], stream));
      MOE_CHECK(moe_permute(&cfg, static_cast<const uint16_t*>(dx), static_cast<const int32_t*>(dids),
                            static_cast<int32_t*>(counts), static_cast<int32_t*>(offsets), static_cast<int32_t*>(eidx),
                            static_cast<int32_t*>(rtok), static_cast<uint8_t*>(xq), static_cast<float*>(xs), ws, wsb,
                            stream));
      HIP_CHECK(hipEventRecord(e[1], stream));
      MOE_CHECK(moe_grouped_gemm1_swiglu(&cfg, static_cast<uint8_t*>(xq), static_cast<float*>(xs),
                                         static_cast<int32_t*>(rtok), static_cast<int32_t*>(offsets), &tiled,
                                         static_cast<uint8_t*>(hq), static_cast<float*>(hs), ws, wsb, stream));
      HIP_CHECK(hipEventRecord(e[2], stream));
      MOE_CHECK(moe_grouped_gemm2(&cfg, static_cast<uint8_t*>(hq), static_cast<float*>(hs),
                                  static_cast<int32_t*>(offsets), &tiled, static_cast<float*>(y), ws, wsb, stream));
      HIP_CHECK(hipEventRecord(e[3], stream));
      MOE_CHECK(moe_combine(&cfg, static_cast<float*>(y), static_cast<int32_t*>(eidx), static_cast<int32_t*>(offsets),
                            static_cast<const float*>(dtw), static_cast<uint16_t*>(dout), stream));
      HIP_CHECK(hipEventRecord(e[4], stream));
      HIP_CHECK(hipEventSynchronize(e[4]));
      for (int q = 0; q < 4; ++q) {
        float ms = 0.0f;
        HIP_CHECK(hipEventElapsedTime(&ms, e[q], e[q + 1]));
        st_us[q].push_back(ms * 1e3);
      }
    }
    std::printf("  stages median us: permute %.1f  gemm1 %.1f  gemm2 %.1f  combine %.1f\n", median(st_us[0]),
                median(st_us[1]), median(st_us[2]), median(st_us[3]));
  }
  HIP_CHECK(hipStreamSynchronize(stream));
  std::printf("done\n");
  return 0;
}
