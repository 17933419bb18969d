// oracle.cpp -- plain, slow CPU reference of the low-bit MoE expert layer.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path loads, links or
// calls this file; only the tests, the smoke check and the bench's CPU
// baseline leg do.  It shares no code, header, table or constant generator
// with the HIP library.
//
// What it computes (the plain definition; grouping, tiling and fusion on the
// GPU only reorder floating-point sums):
//   1. per-token activation quantisation to FP8 e4m3, one fp32 scale per
//      group of G channels (FusedDeepMoE family analysis, QuantToken
//      snippet: multiplier = max-code / row max, code = round(x * multiplier),
//      stored scale = 1 / multiplier; here e4m3 with max 448, per group);
//   2. the local token permute: expert histogram, exclusive prefix-scan
//      offsets (the group list) and a stable expand index (same page,
//      gmGroupList / gmExpandIdx workspace objects and the
//      CalAndSendTokenCount step);
//   3. grouped GEMM1 over the gate|up weights with per-token / per-block
//      dequantisation (OpDequant: value = integer dot * weight scale *
//      per-token scale), SwiGLU (OpSwiglu: left half through SiLU times
//      right half) and requantisation (OpBlockQuant / BlockQuant), the
//      fusion the GC-MoE abstract describes for its grouped GEMM;
//   4. grouped GEMM2 with the same dequantisation;
//   5. the top-k weighted combine back to token order (ReducePermute:
//      accumulate each token's expert outputs), plus an always-on shared
//      expert with weight 1 (GC-MoE abstract: shared experts as an option;
//      FusedDeepMoE shared-expert path: all tokens, one group).
//
// Number formats (the pages name FP8, FP4 and MXFP4 but print no bit
// layouts; these are the OCP 8-bit float E4M3FN and Microscaling e2m1 /
// e8m0 definitions, rebuilt from sign / exponent / mantissa fields):
//   e4m3: bias 7, no infinities, S.1111.111 is NaN, max 448, subnormal step 2^-9
//   e2m1: bias 1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//   e8m0: 2^(c-127), c = 255 is NaN
//
// Precision: dot products, SwiGLU and the combine in fp64; the quantisers in
// fp32 (multiplier, product and reciprocal each rounded to fp32), which is
// the bit-exact contract for activation codes.  Built with -ffp-contract=off.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

int g_threads = 0;   // 0 = hardware concurrency
int g_mutation = 0;  // test-only planted mistakes, see oracle_set_mutation

// ---------------------------------------------------------------- formats
double dec_e4m3(uint8_t c) {
  const int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
  if (ex == 15 && m == 7) return NAN;
  const double mag = ex == 0 ? m * std::ldexp(1.0, -9) : (1.0 + m / 8.0) * std::ldexp(1.0, ex - 7);
  return s ? -mag : mag;
}

double dec_e2m1(uint8_t c) {
  c &= 15;
  const int s = c >> 3, ex = (c >> 1) & 3, m = c & 1;
  const double mag = ex == 0 ? m * 0.5 : (1.0 + m / 2.0) * std::ldexp(1.0, ex - 1);
  return s ? -mag : mag;
}

double dec_e8m0(uint8_t c) { return c == 255 ? NAN : std::ldexp(1.0, int(c) - 127); }

// Nearest finite e4m3 magnitude by exhaustive search; ties go to the even
// code; |v| >= 448 saturates to 448; the sign bit is copied from v (so -0
// and negative values that round to zero give 0x80).
uint8_t enc_e4m3(float v) {
  static const std::vector<double> mags = [] {
    std::vector<double> m(0x7F);
    for (int c = 0; c < 0x7F; ++c) m[c] = dec_e4m3(uint8_t(c));
    return m;
  }();
  const double a = std::fabs(double(v));
  int best = 0x7E;
  if (a < 448.0) {
    double bd = INFINITY;
    for (int c = 0; c < 0x7F; ++c) {
      const double d = std::fabs(mags[c] - a);
      if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
  }
  return uint8_t(best | (std::signbit(v) ? 0x80 : 0));
}

uint8_t enc_e2m1(float v) {
  const double a = std::fabs(double(v));
  int best = 7;
  if (a < 6.0) {
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
      const double d = std::fabs(dec_e2m1(uint8_t(c)) - a);
      if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
  }
  return uint8_t(best | (std::signbit(v) ? 8 : 0));
}

float bf16_to_f32(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ---------------------------------------------------------------- quantiser
// One group of G fp32 values -> G e4m3 codes and one fp32 dequant scale.
void quant_group(const float* v, int G, uint8_t* q, float* s) {
  float a = 0.0f;
  for (int i = 0; i < G; ++i) a = std::max(a, std::fabs(v[i]));
  const float ap = std::max(a, 0x1p-64f);
  const float mult = 448.0f / ap;
  for (int i = 0; i < G; ++i) {
    const float p = v[i] * mult;
    q[i] = enc_e4m3(p);
  }
  *s = 1.0f / mult;
}

// ---------------------------------------------------------------- threading
// Worker count: oracle_set_threads(n) if called, else OMP_NUM_THREADS, else
// the hardware concurrency capped at 16.
int default_threads() {
  if (g_threads > 0) return g_threads;
  if (const char* e = std::getenv("OMP_NUM_THREADS")) {
    const int v = std::atoi(e);
    if (v > 0) return v;
  }
  const int hw = int(std::thread::hardware_concurrency());
  return std::max(1, std::min(hw, 16));
}

template <class F>
void parallel_for(int64_t n, F f) {
  int nt = default_threads();
  if (n < nt) nt = int(n);
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([=, &f] {
      for (int64_t i = t; i < n; i += nt) f(i);
    });
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------- weights
struct Cfg {
  int T, H, I, E, k, wfmt, wblk, G, has_shared;
};

struct WSet {
  const uint8_t* w1;
  const void* w1s;
  const uint8_t* w2;
  const void* w2s;
  const uint8_t* sw1;
  const void* sw1s;
  const uint8_t* sw2;
  const void* sw2s;
};

// Dequantised weight value of matrix `which` (1: gate|up [2I,H], 2: down [H,I])
// of expert e (e == E: the shared expert), row n, column kk.
double wval(const Cfg& c, const WSet& w, int which, int e, int64_t n, int64_t kk) {
  const bool sh = e == c.E;
  const int64_t N = which == 1 ? 2LL * c.I : c.H;
  const int64_t K = which == 1 ? c.H : c.I;
  const uint8_t* codes = which == 1 ? (sh ? w.sw1 : w.w1) : (sh ? w.sw2 : w.w2);
  const void* sc = which == 1 ? (sh ? w.sw1s : w.w1s) : (sh ? w.sw2s : w.w2s);
  const int64_t ee = sh ? 0 : e;
  if (c.wfmt == 0) {  // FP8 e4m3 + fp32 scale per wblk x wblk block
    const int64_t b = c.wblk;
    const double code = dec_e4m3(codes[(ee * N + n) * K + kk]);
    const float* s = static_cast<const float*>(sc);
    int64_t kb = kk / b;
    if (g_mutation == 2 && kb == 0) return code;  // planted: drop the first K-block scale
    return code * double(s[(ee * (N / b) + n / b) * (K / b) + kb]);
  }
  // MXFP4: packed e2m1 (even K in the low nibble) + e8m0 per 32 along K
  const uint8_t byte = codes[(ee * N + n) * (K / 2) + kk / 2];
  const uint8_t nib = (kk & 1) ? (byte >> 4) : (byte & 15);
  const uint8_t* s = static_cast<const uint8_t*>(sc);
  return dec_e2m1(nib) * dec_e8m0(s[(ee * N + n) * (K / 32) + kk / 32]);
}

int expert_of_row(const int32_t* offsets, int ngroups, int64_t r) {
  for (int g = 0; g < ngroups; ++g)
    if (r >= offsets[g] && r < offsets[g + 1]) return g;
  return -1;
}

// GEMM1 + SwiGLU for one row: a = dequantised activation row (fp64, length H)
// -> h (fp32, length I).  gate = rows [0, I), up = rows [I, 2I).
void gemm1_swiglu_row(const Cfg& c, const WSet& w, int e, const double* a, float* h) {
  std::vector<double> g(2 * size_t(c.I));
  for (int64_t n = 0; n < 2LL * c.I; ++n) {
    double acc = 0.0;
    for (int64_t kk = 0; kk < c.H; ++kk) acc += a[kk] * wval(c, w, 1, e, n, kk);
    g[n] = acc;
  }
  for (int64_t n = 0; n < c.I; ++n) {
    double gate = g[n], up = g[c.I + n];
    if (g_mutation == 1) std::swap(gate, up);  // planted: gate and up swapped
    const double silu = gate / (1.0 + std::exp(-gate));
    h[n] = float(silu * up);
  }
}

// GEMM2 for one row: dequantised requantised h (fp64, length I) -> y (length H)
void gemm2_row(const Cfg& c, const WSet& w, int e, const double* hd, double* y) {
  for (int64_t n = 0; n < c.H; ++n) {
    double acc = 0.0;
    for (int64_t kk = 0; kk < c.I; ++kk) acc += hd[kk] * wval(c, w, 2, e, n, kk);
    y[n] = acc;
  }
}

void dequant_row(const uint8_t* q, const float* s, int64_t len, int G, double* out) {
  for (int64_t i = 0; i < len; ++i) out[i] = dec_e4m3(q[i]) * double(s[i / G]);
}

}  // namespace

extern "C" {

void oracle_set_threads(int n) { g_threads = n; }
int oracle_get_threads() { return default_threads(); }
// Test-only: plant a known mistake (0 = none, 1 = gate/up swapped,
// 2 = first K-block weight scale dropped, 3 = unstable row order inside an
// expert, 4 = offsets shifted by one) so tests can show their pins catch it.
void oracle_set_mutation(int m) { g_mutation = m; }

double oracle_dec_e4m3(int c) { return dec_e4m3(uint8_t(c)); }
double oracle_dec_e2m1(int c) { return dec_e2m1(uint8_t(c)); }
double oracle_dec_e8m0(int c) { return dec_e8m0(uint8_t(c)); }
int oracle_enc_e4m3(float v) { return enc_e4m3(v); }
int oracle_enc_e2m1(float v) { return enc_e2m1(v); }

void oracle_enc_e4m3_array(const float* v, int64_t n, uint8_t* q) {
  parallel_for((n + 4095) / 4096, [&](int64_t blk) {
    for (int64_t i = blk * 4096; i < std::min(n, (blk + 1) * 4096); ++i) q[i] = enc_e4m3(v[i]);
  });
}

// fp32 rows [rows, cols] -> codes [rows, cols], scales [rows, cols/G]
void oracle_quant_rows_f32(const float* v, int64_t rows, int64_t cols, int G, uint8_t* q, float* s) {
  parallel_for(rows, [&](int64_t r) {
    for (int64_t g = 0; g < cols / G; ++g)
      quant_group(v + r * cols + g * G, G, q + r * cols + g * G, s + r * (cols / G) + g);
  });
}

// bf16 activations [T, H] -> xq [T, H] e4m3, xs [T, H/G] fp32
void oracle_quant_act(const uint16_t* x, int64_t T, int64_t H, int G, uint8_t* xq, float* xs) {
  parallel_for(T, [&](int64_t t) {
    std::vector<float> row(H);
    for (int64_t i = 0; i < H; ++i) row[i] = bf16_to_f32(x[t * H + i]);
    for (int64_t g = 0; g < H / G; ++g) quant_group(row.data() + g * G, G, xq + t * H + g * G, xs + t * (H / G) + g);
  });
}

// Local permute.  ids [T*k] (values outside [0,E) are masked slots).
// counts [E + has_shared], offsets [E + 1 + has_shared] (exclusive scan),
// expand_idx [T*k] (-1 for masked slots), row_token [T*k + T*has_shared]
// (-1 past the last row).  Rows of expert e hold its slots in ascending flat
// index; shared rows follow the routed rows in token order.
void oracle_permute(const int32_t* ids, int T, int k, int E, int has_shared, int32_t* counts,
                    int32_t* offsets, int32_t* expand_idx, int32_t* row_token) {
  const int ng = E + (has_shared ? 1 : 0);
  const int64_t n = int64_t(T) * k;
  for (int g = 0; g < ng; ++g) counts[g] = 0;
  for (int64_t i = 0; i < n; ++i)
    if (ids[i] >= 0 && ids[i] < E) counts[ids[i]]++;
  if (has_shared) counts[E] = T;
  offsets[0] = 0;
  for (int g = 0; g < ng; ++g) offsets[g + 1] = offsets[g] + counts[g];
  std::vector<int32_t> cursor(offsets, offsets + E);
  for (int64_t i = 0; i < n; ++i) {
    const int e = ids[i];
    if (e < 0 || e >= E) { expand_idx[i] = -1; continue; }
    int32_t r = cursor[e]++;
    if (g_mutation == 3) r = offsets[e + 1] - 1 - (r - offsets[e]);  // planted: reversed order
    expand_idx[i] = r;
    row_token[r] = int32_t(i / k);
  }
  if (has_shared)
    for (int t = 0; t < T; ++t) row_token[offsets[E] + t] = t;
  const int64_t cap = n + (has_shared ? T : 0);
  for (int64_t r = offsets[ng]; r < cap; ++r) row_token[r] = -1;
  if (g_mutation == 4)  // planted: off-by-one group boundaries
    for (int g = 1; g < ng; ++g) offsets[g] += 1;
}

// Grouped GEMM1 + SwiGLU + requantisation for the listed rows.
// Inputs: xq [T,H], xs [T,H/G], row_token, offsets (group list).
// Outputs per listed row i: h [nrows, I] (fp32, before requant),
// hq [nrows, I] e4m3, hs [nrows, I/G].
void oracle_gemm1(const Cfg* c, const WSet* w, const uint8_t* xq, const float* xs,
                  const int32_t* row_token, const int32_t* offsets, int64_t nrows,
                  const int64_t* rows, float* h, uint8_t* hq, float* hs) {
  const int ng = c->E + (c->has_shared ? 1 : 0);
  parallel_for(nrows, [&](int64_t i) {
    const int64_t r = rows[i];
    const int e = expert_of_row(offsets, ng, r);
    const int t = row_token[r];
    std::vector<double> a(c->H);
    dequant_row(xq + int64_t(t) * c->H, xs + int64_t(t) * (c->H / c->G), c->H, c->G, a.data());
    float* hr = h + i * c->I;
    gemm1_swiglu_row(*c, *w, e, a.data(), hr);
    for (int64_t g = 0; g < c->I / c->G; ++g)
      quant_group(hr + g * c->G, c->G, hq + i * c->I + g * c->G, hs + i * (c->I / c->G) + g);
  });
}

// Grouped GEMM2 for the listed rows: hq [R, I], hs [R, I/G] (indexed by row id)
// -> y [nrows, H] in fp64.
void oracle_gemm2(const Cfg* c, const WSet* w, const uint8_t* hq, const float* hs,
                  const int32_t* offsets, int64_t nrows, const int64_t* rows, double* y) {
  const int ng = c->E + (c->has_shared ? 1 : 0);
  parallel_for(nrows, [&](int64_t i) {
    const int64_t r = rows[i];
    const int e = expert_of_row(offsets, ng, r);
    std::vector<double> hd(c->I);
    dequant_row(hq + r * c->I, hs + r * (c->I / c->G), c->I, c->G, hd.data());
    gemm2_row(*c, *w, e, hd.data(), y + i * c->H);
  });
}

// Top-k weighted combine for the listed tokens: y [R, H] fp32 indexed by row
// -> out [ntok, H] fp64.  Slots are summed in ascending j, then the shared row.
void oracle_combine(const Cfg* c, const float* y, const int32_t* expand_idx,
                    const int32_t* offsets, const float* topk_w, int64_t ntok,
                    const int64_t* toks, double* out) {
  parallel_for(ntok, [&](int64_t i) {
    const int64_t t = toks[i];
    double* o = out + i * c->H;
    for (int64_t n = 0; n < c->H; ++n) o[n] = 0.0;
    for (int j = 0; j < c->k; ++j) {
      const int32_t r = expand_idx[t * c->k + j];
      if (r < 0) continue;
      const double wt = topk_w[t * c->k + j];
      for (int64_t n = 0; n < c->H; ++n) o[n] += wt * double(y[int64_t(r) * c->H + n]);
    }
    if (c->has_shared) {
      const int64_t r = offsets[c->E] + t;
      for (int64_t n = 0; n < c->H; ++n) o[n] += double(y[r * c->H + n]);
    }
  });
}

// The whole layer for the listed tokens (tokens are independent once the
// permute is known): quantise x, permute, then per needed row GEMM1 + SwiGLU
// + requant and GEMM2 (fp64), then the combine in fp64.  out [ntok, H].
// Optional: xq/xs/counts/offsets/expand_idx/row_token outputs (may be NULL).
void oracle_layer(const Cfg* c, const WSet* w, const uint16_t* x, const int32_t* ids,
                  const float* topk_w, int64_t ntok, const int64_t* toks, double* out) {
  const int64_t T = c->T, H = c->H, k = c->k;
  std::vector<uint8_t> xq(T * H);
  std::vector<float> xs(T * (H / c->G));
  oracle_quant_act(x, T, H, c->G, xq.data(), xs.data());
  const int ng = c->E + (c->has_shared ? 1 : 0);
  std::vector<int32_t> counts(ng), offsets(ng + 1), eidx(T * k), rtok(T * k + (c->has_shared ? T : 0));
  oracle_permute(ids, c->T, c->k, c->E, c->has_shared, counts.data(), offsets.data(), eidx.data(),
                 rtok.data());
  // rows needed by the listed tokens, each once, ascending
  std::vector<int64_t> rows;
  for (int64_t i = 0; i < ntok; ++i) {
    for (int j = 0; j < k; ++j)
      if (eidx[toks[i] * k + j] >= 0) rows.push_back(eidx[toks[i] * k + j]);
    if (c->has_shared) rows.push_back(offsets[c->E] + toks[i]);
  }
  std::sort(rows.begin(), rows.end());
  rows.erase(std::unique(rows.begin(), rows.end()), rows.end());
  const int64_t nr = int64_t(rows.size());
  std::vector<float> h(nr * c->I), hs_l(nr * (c->I / c->G));
  std::vector<uint8_t> hq_l(nr * c->I);
  oracle_gemm1(c, w, xq.data(), xs.data(), rtok.data(), offsets.data(), nr, rows.data(), h.data(),
               hq_l.data(), hs_l.data());
  // scatter the listed rows' codes into row-indexed buffers for GEMM2
  const int64_t Rcap = int64_t(rtok.size());
  std::vector<uint8_t> hq(std::max<int64_t>(Rcap, 1) * c->I, 0);
  std::vector<float> hs(std::max<int64_t>(Rcap, 1) * (c->I / c->G), 0.0f);
  for (int64_t i = 0; i < nr; ++i) {
    std::memcpy(&hq[rows[i] * c->I], &hq_l[i * c->I], c->I);
    std::memcpy(&hs[rows[i] * (c->I / c->G)], &hs_l[i * (c->I / c->G)], sizeof(float) * (c->I / c->G));
  }
  std::vector<double> y_l(nr * H);
  oracle_gemm2(c, w, hq.data(), hs.data(), offsets.data(), nr, rows.data(), y_l.data());
  std::vector<int64_t> pos(Rcap, -1);
  for (int64_t i = 0; i < nr; ++i) pos[rows[i]] = i;
  // combine in fp64 directly from the fp64 GEMM2 rows
  parallel_for(ntok, [&](int64_t i) {
    const int64_t t = toks[i];
    double* o = out + i * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int32_t r = eidx[t * k + j];
      if (r < 0) continue;
      const double wt = topk_w[t * k + j];
      const double* yr = &y_l[pos[r] * H];
      for (int64_t n = 0; n < H; ++n) o[n] += wt * yr[n];
    }
    if (c->has_shared) {
      const double* yr = &y_l[pos[offsets[c->E] + t] * H];
      for (int64_t n = 0; n < H; ++n) o[n] += yr[n];
    }
  });
}

// Brute force (checks the oracle): no permute, no grouping.  For each listed
// token and each valid slot, run the token through that expert's dense
// dequantised MLP (weights dequantised into full fp64 matrices first), then
// requantise h with the same rule and add w * y; plus the shared expert.
void oracle_bruteforce(const Cfg* c, const WSet* w, const uint16_t* x, const int32_t* ids,
                       const float* topk_w, int64_t ntok, const int64_t* toks, double* out) {
  const int64_t H = c->H, I = c->I, G = c->G;
  const int nexp = c->E + (c->has_shared ? 1 : 0);
  // which experts are used by the listed tokens
  std::vector<char> used(nexp, 0);
  for (int64_t i = 0; i < ntok; ++i)
    for (int j = 0; j < c->k; ++j) {
      const int e = ids[toks[i] * c->k + j];
      if (e >= 0 && e < c->E) used[e] = 1;
    }
  if (c->has_shared) used[c->E] = 1;
  std::vector<std::vector<double>> W1d(nexp), W2d(nexp);
  parallel_for(nexp, [&](int64_t e) {
    if (!used[e]) return;
    W1d[e].resize(2 * I * H);
    W2d[e].resize(H * I);
    for (int64_t n = 0; n < 2 * I; ++n)
      for (int64_t kk = 0; kk < H; ++kk) W1d[e][n * H + kk] = wval(*c, *w, 1, int(e), n, kk);
    for (int64_t n = 0; n < H; ++n)
      for (int64_t kk = 0; kk < I; ++kk) W2d[e][n * I + kk] = wval(*c, *w, 2, int(e), n, kk);
  });
  parallel_for(ntok, [&](int64_t i) {
    const int64_t t = toks[i];
    // quantise this token (same rule as the activation quantiser)
    std::vector<float> xr(H);
    for (int64_t n = 0; n < H; ++n) xr[n] = bf16_to_f32(x[t * H + n]);
    std::vector<uint8_t> q(H);
    std::vector<float> s(H / G);
    for (int64_t g = 0; g < H / G; ++g) quant_group(&xr[g * G], int(G), &q[g * G], &s[g]);
    std::vector<double> xd(H);
    for (int64_t n = 0; n < H; ++n) xd[n] = dec_e4m3(q[n]) * double(s[n / G]);
    double* o = out + i * H;
    for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
    auto run_expert = [&](int e, double wt) {
      std::vector<double> gu(2 * I);
      for (int64_t n = 0; n < 2 * I; ++n) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < H; ++kk) acc += W1d[e][n * H + kk] * xd[kk];
        gu[n] = acc;
      }
      std::vector<float> h(I);
      for (int64_t n = 0; n < I; ++n) {
        const double gt = gu[n];
        h[n] = float(gt / (1.0 + std::exp(-gt)) * gu[I + n]);
      }
      std::vector<uint8_t> hq(I);
      std::vector<float> hs(I / G);
      for (int64_t g = 0; g < I / G; ++g) quant_group(&h[g * G], int(G), &hq[g * G], &hs[g]);
      std::vector<double> hd(I);
      for (int64_t n = 0; n < I; ++n) hd[n] = dec_e4m3(hq[n]) * double(hs[n / G]);
      for (int64_t n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < I; ++kk) acc += W2d[e][n * I + kk] * hd[kk];
        o[n] += wt * acc;
      }
    };
    for (int j = 0; j < c->k; ++j) {
      const int e = ids[t * c->k + j];
      if (e >= 0 && e < c->E) run_expert(e, double(topk_w[t * c->k + j]));
    }
    if (c->has_shared) run_expert(c->E, 1.0);
  });
}

}  // extern "C"
