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
//      FusedDeepMoE shared-expert path: all tokens, one group);
//   6. the router in front of the layer (the routing GEMM plus the routing
//      selection the DeepGEMM 26/09 news page's Mega Gate paragraph fuses
//      into one kernel): logits = x . Wg^T, the top-k experts by logit (ties
//      to the lower expert id), routing weights = the softmax of the k
//      selected logits (the full softmax renormalised over the top-k, as the
//      workload description states).
//
// Number formats (the pages name FP8, FP4 and MXFP4 but print no bit
// layouts; these are the OCP 8-bit float E4M3FN and Microscaling e2m1 /
// e8m0 definitions, rebuilt from sign / exponent / mantissa fields):
//   e4m3: bias 7, no infinities, S.1111.111 is NaN, max 448, subnormal step 2^-9
//   e2m1: bias 1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//   e8m0: 2^(c-127), c = 255 is NaN
//
// NVFP4 weights (wfmt 2; the pages name the format beside MXFP4 without
// defining it, so this is the published two-level definition): e2m1 codes
// packed two per byte (even K in the low nibble), one e4m3 scale per 16
// consecutive K of a row, and one fp32 scale per expert matrix; the weight
// is code * block scale * matrix scale.
//
// Activation formats (act_fmt): 0 = the FP8 rule above (e4m3 codes, one fp32
// scale per G channels); 1 = MXFP4 activations, the 4-bit-activation variant
// the FusedDeepMoE page describes for W4A8 (here e2m1 codes with one e8m0
// power-of-two scale per 32 channels, by the Microscaling rule: X =
// 2^(floor(log2 amax) - 2), the largest power of two with amax / X < 8,
// codes = e2m1(v / X) rounded to nearest even, saturating at 6).  The
// SwiGLU output is requantised with the same format.
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

// One group of 32 fp32 values -> 32 e2m1 codes (one per byte, sign in bit
// 3) and the e8m0 code of its scale X = 2^(floor(log2 amax) - 2), clamped to
// the e8m0 range (amax = 0, or below 2^-125, gives code 0, X = 2^-127).
// v / X is exact (X is a power of two and |v / X| < 8).
void quant_group_mx(const float* v, uint8_t* q, uint8_t* s) {
  float a = 0.0f;
  for (int i = 0; i < 32; ++i) a = std::max(a, std::fabs(v[i]));
  int code = 0;
  if (a > 0.0f) {
    int e = 0;
    std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1): floor(log2 a) = e - 1
    code = (e - 1) - 2 + 127;
    if (g_mutation == 9) code += 1;  // planted: scale exponent one too large
    code = std::min(std::max(code, 0), 254);
  }
  const double X = std::ldexp(1.0, code - 127);
  for (int i = 0; i < 32; ++i) q[i] = enc_e2m1(float(double(v[i]) / X));
  *s = uint8_t(code);
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
  int T, H, I, E, k, wfmt, wblk, G, has_shared, act_fmt;
};

// ---------------------------------------------------------------- activation codec
// Bytes of one quantised row of `len` channels: codes, then scales.
int64_t act_code_bytes(const Cfg& c, int64_t len) { return c.act_fmt == 1 ? len / 2 : len; }
int64_t act_scale_bytes(const Cfg& c, int64_t len) { return c.act_fmt == 1 ? len / 32 : 4 * (len / c.G); }

// Quantise one fp32 row with the cfg's activation format: FP8 per G with fp32
// scales, or MXFP4 per 32 (two codes per byte, even channel in the low nibble)
// with e8m0 scales.
void quant_act_row(const Cfg& c, const float* v, int64_t len, uint8_t* q, uint8_t* s) {
  if (c.act_fmt == 1) {
    uint8_t nib[32];
    for (int64_t g = 0; g < len / 32; ++g) {
      quant_group_mx(v + g * 32, nib, s + g);
      for (int i = 0; i < 32; i += 2) q[g * 16 + i / 2] = uint8_t(nib[i] | (nib[i + 1] << 4));
    }
    return;
  }
  float* sf = reinterpret_cast<float*>(s);
  for (int64_t g = 0; g < len / c.G; ++g) quant_group(v + g * c.G, c.G, q + g * c.G, sf + g);
}

// Dequantised row (fp64, exact) of a quantised row.
void dequant_act_row(const Cfg& c, const uint8_t* q, const uint8_t* s, int64_t len, double* out) {
  if (c.act_fmt == 1) {
    for (int64_t i = 0; i < len; ++i) {
      const uint8_t nib = (i & 1) ? (q[i / 2] >> 4) : (q[i / 2] & 15);
      out[i] = dec_e2m1(nib) * dec_e8m0(s[i / 32]);
    }
    return;
  }
  const float* sf = reinterpret_cast<const float*>(s);
  for (int64_t i = 0; i < len; ++i) out[i] = dec_e4m3(q[i]) * double(sf[i / c.G]);
}

struct WSet {
  const uint8_t* w1;
  const void* w1s;
  const uint8_t* w2;
  const void* w2s;
  const uint8_t* sw1;
  const void* sw1s;
  const uint8_t* sw2;
  const void* sw2s;
  const float* w1g;  // NVFP4: one fp32 scale per expert matrix ([E]; the shared expert's [1])
  const float* w2g;
  const float* sw1g;
  const float* sw2g;
};

// Decoded value of every code, filled once from the decoders above (the
// weight dequantisation below looks codes up instead of re-deriving them).
struct DecodeTables {
  double e4m3[256], e2m1[16], e8m0[256];
  DecodeTables() {
    for (int c = 0; c < 256; ++c) e4m3[c] = dec_e4m3(uint8_t(c));
    for (int c = 0; c < 16; ++c) e2m1[c] = dec_e2m1(uint8_t(c));
    for (int c = 0; c < 256; ++c) e8m0[c] = dec_e8m0(uint8_t(c));
  }
};
const DecodeTables& tables() {
  static const DecodeTables t;
  return t;
}

// Dequantised weight value of matrix `which` (1: gate|up [2I,H], 2: down [H,I])
// of expert e (e == E: the shared expert), row n, column kk.
double wval(const Cfg& c, const WSet& w, int which, int e, int64_t n, int64_t kk) {
  const DecodeTables& tab = tables();
  const bool sh = e == c.E;
  const int64_t N = which == 1 ? 2LL * c.I : c.H;
  const int64_t K = which == 1 ? c.H : c.I;
  const uint8_t* codes = which == 1 ? (sh ? w.sw1 : w.w1) : (sh ? w.sw2 : w.w2);
  const void* sc = which == 1 ? (sh ? w.sw1s : w.w1s) : (sh ? w.sw2s : w.w2s);
  // planted (10): every routed expert reads its neighbour's matrices
  const int64_t ee = sh ? 0 : (g_mutation == 10 ? (e + 1) % c.E : e);
  if (c.wfmt == 0) {  // FP8 e4m3 + fp32 scale per wblk x wblk block
    const int64_t b = c.wblk;
    const double code = tab.e4m3[codes[(ee * N + n) * K + kk]];
    const float* s = static_cast<const float*>(sc);
    int64_t kb = kk / b;
    if (g_mutation == 2 && kb == 0) return code;  // planted: drop the first K-block scale
    return code * double(s[(ee * (N / b) + n / b) * (K / b) + kb]);
  }
  // MXFP4 / NVFP4: packed e2m1 (even K in the low nibble)
  const uint8_t byte = codes[(ee * N + n) * (K / 2) + kk / 2];
  const uint8_t nib = (kk & 1) ? (byte >> 4) : (byte & 15);
  const uint8_t* s = static_cast<const uint8_t*>(sc);
  if (c.wfmt == 2) {  // NVFP4: e4m3 per 16 along K, times the matrix's fp32 scale
    const float* g = which == 1 ? (sh ? w.sw1g : w.w1g) : (sh ? w.sw2g : w.w2g);
    return tab.e2m1[nib] * tab.e4m3[s[(ee * N + n) * (K / 16) + kk / 16]] * double(g[ee]);
  }
  // MXFP4: e8m0 per 32 along K
  return tab.e2m1[nib] * tab.e8m0[s[(ee * N + n) * (K / 32) + kk / 32]];
}

int expert_of_row(const int32_t* offsets, int ngroups, int64_t r) {
  for (int g = 0; g < ngroups; ++g)
    if (r >= offsets[g] && r < offsets[g + 1]) return g;
  return -1;
}

// Weight rows [n0, n0 + nn) of matrix `which` (1: gate|up [2I,H], 2: down
// [H,I]) of group e, dequantised to fp64: each entry is wval(), the decoded
// code times its scale, which is exact in fp64.
void dequant_weight_rows(const Cfg& c, const WSet& w, int which, int e, int64_t n0, int64_t nn, double* out) {
  const int64_t K = which == 1 ? c.H : c.I;
  for (int64_t n = 0; n < nn; ++n)
    for (int64_t kk = 0; kk < K; ++kk) out[n * K + kk] = wval(c, w, which, e, n0 + n, kk);
}

// One dot product in fp64, summed in index order.
double dot(const double* a, const double* b, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

// SwiGLU of one output column: silu(gate) * up in fp64, rounded to fp32
// (left half through SiLU times the right half).
float swiglu(double gate, double up) {
  if (g_mutation == 1) std::swap(gate, up);  // planted: gate and up swapped
  const double silu = gate / (1.0 + std::exp(-gate));
  return float(silu * up);
}

// The listed rows (indices into `rows`) that belong to each group.
std::vector<std::vector<int64_t>> rows_by_group(const int32_t* offsets, int ng, int64_t nrows, const int64_t* rows) {
  std::vector<std::vector<int64_t>> m(ng);
  for (int64_t i = 0; i < nrows; ++i) {
    const int g = expert_of_row(offsets, ng, rows[i]);
    if (g >= 0) m[g].push_back(i);
  }
  return m;
}

}  // namespace

extern "C" {

void oracle_set_threads(int n) { g_threads = n; }
int oracle_get_threads() { return default_threads(); }
// Test-only: plant a known mistake (0 = none, 1 = gate/up swapped,
// 2 = first K-block weight scale dropped, 3 = unstable row order inside an
// expert, 4 = offsets shifted by one, 5 = the stage combine ignores routing
// weights, 6 = the stage combine reads token 0's shared row for every token,
// 7 = the router breaks logit ties towards the higher expert id, 8 = the
// router's softmax runs over all E logits, 9 = the MXFP4 activation scale
// exponent one too large) so tests can show their pins catch it.
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

// bf16 activations [T, H] -> the cfg's activation format: xq codes [T, code
// bytes of H], xs scales [T, scale bytes of H] (fp32 per G for FP8, e8m0 per
// 32 for MXFP4)
void oracle_quant_act_cfg(const Cfg* c, const uint16_t* x, int64_t T, uint8_t* xq, uint8_t* xs) {
  const int64_t H = c->H, cb = act_code_bytes(*c, H), sb = act_scale_bytes(*c, H);
  parallel_for(T, [&](int64_t t) {
    std::vector<float> row(H);
    for (int64_t i = 0; i < H; ++i) row[i] = bf16_to_f32(x[t * H + i]);
    quant_act_row(*c, row.data(), H, xq + t * cb, xs + t * sb);
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
// Inputs: xq / xs (the cfg's activation format, one row per token),
// row_token, offsets (group list).  Outputs per listed row i: h [nrows, I]
// (fp32, before requant), hq / hs the requantised row in the same format.
// For row i of group e and h column n: G_gate = sum over kk of a[kk] *
// W1[e][n][kk], G_up the same over row I + n, each one fp64 dot product in
// K order; h = swiglu(G_gate, G_up); then each G consecutive h values of
// the row are requantised together.  The work is split into independent
// tasks of (group, G consecutive h columns): a task dequantises the gate
// and up weight rows of its columns once and runs them against every
// listed row of its group (no sum is split or reordered by this).
void oracle_gemm1(const Cfg* c, const WSet* w, const uint8_t* xq, const uint8_t* xs,
                  const int32_t* row_token, const int32_t* offsets, int64_t nrows,
                  const int64_t* rows, float* h, uint8_t* hq, uint8_t* hs) {
  const int ng = c->E + (c->has_shared ? 1 : 0);
  const int64_t H = c->H, I = c->I, G = c->G;
  const int64_t xcb = act_code_bytes(*c, H), xsb = act_scale_bytes(*c, H);
  const int64_t hcb = act_code_bytes(*c, I), hsb = act_scale_bytes(*c, I);
  std::vector<double> a(std::max<int64_t>(nrows, 1) * H);  // dequantised activation of each listed row
  parallel_for(nrows, [&](int64_t i) {
    const int64_t t = row_token[rows[i]];
    dequant_act_row(*c, xq + t * xcb, xs + t * xsb, H, &a[i * H]);
  });
  const auto members = rows_by_group(offsets, ng, nrows, rows);
  const int64_t nch = I / G;
  parallel_for(int64_t(ng) * nch, [&](int64_t task) {
    const int e = int(task / nch);
    const int64_t n0 = (task % nch) * G;
    if (members[e].empty()) return;
    std::vector<double> wg(G * H), wu(G * H);
    dequant_weight_rows(*c, *w, 1, e, n0, G, wg.data());
    dequant_weight_rows(*c, *w, 1, e, I + n0, G, wu.data());
    for (const int64_t i : members[e]) {
      float* hr = h + i * I + n0;
      for (int64_t n = 0; n < G; ++n) hr[n] = swiglu(dot(&a[i * H], &wg[n * H], H), dot(&a[i * H], &wu[n * H], H));
      // this task's G columns are whole quantisation groups (G is the group size)
      quant_act_row(*c, hr, G, hq + i * hcb + act_code_bytes(*c, n0), hs + i * hsb + act_scale_bytes(*c, n0));
    }
  });
}

// Grouped GEMM2 for the listed rows: hq / hs quantised rows (indexed by row id)
// -> y [nrows, H] in fp64: y[i][n] = sum over kk of hd[kk] * W2[e][n][kk],
// one fp64 dot product in K order, hd the row's dequantised codes.  Tasks of
// (group, 128 output columns) dequantise their weight rows once.
void oracle_gemm2(const Cfg* c, const WSet* w, const uint8_t* hq, const uint8_t* hs,
                  const int32_t* offsets, int64_t nrows, const int64_t* rows, double* y) {
  const int ng = c->E + (c->has_shared ? 1 : 0);
  const int64_t H = c->H, I = c->I;
  const int64_t hcb = act_code_bytes(*c, I), hsb = act_scale_bytes(*c, I);
  std::vector<double> hd(std::max<int64_t>(nrows, 1) * I);
  parallel_for(nrows, [&](int64_t i) {
    const int64_t r = rows[i];
    dequant_act_row(*c, hq + r * hcb, hs + r * hsb, I, &hd[i * I]);
  });
  const auto members = rows_by_group(offsets, ng, nrows, rows);
  constexpr int64_t kCols = 128;  // H is a multiple of 128
  const int64_t nch = H / kCols;
  parallel_for(int64_t(ng) * nch, [&](int64_t task) {
    const int e = int(task / nch);
    const int64_t n0 = (task % nch) * kCols;
    if (members[e].empty()) return;
    std::vector<double> wd(kCols * I);
    dequant_weight_rows(*c, *w, 2, e, n0, kCols, wd.data());
    for (const int64_t i : members[e])
      for (int64_t n = 0; n < kCols; ++n) y[i * H + n0 + n] = dot(&hd[i * I], &wd[n * I], I);
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
      double wt = topk_w[t * c->k + j];
      if (g_mutation == 5) wt = 1.0;  // planted: routing weight ignored
      for (int64_t n = 0; n < c->H; ++n) o[n] += wt * double(y[int64_t(r) * c->H + n]);
    }
    if (c->has_shared) {
      int64_t r = offsets[c->E] + t;
      if (g_mutation == 6) r = offsets[c->E];  // planted: every token takes token 0's shared row
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
  const int64_t T = c->T, H = c->H, k = c->k, I = c->I;
  const int64_t xcb = act_code_bytes(*c, H), xsb = act_scale_bytes(*c, H);
  const int64_t hcb = act_code_bytes(*c, I), hsb = act_scale_bytes(*c, I);
  std::vector<uint8_t> xq(std::max<int64_t>(T, 1) * xcb), xs(std::max<int64_t>(T, 1) * xsb);
  oracle_quant_act_cfg(c, x, T, xq.data(), xs.data());
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
  std::vector<float> h(std::max<int64_t>(nr, 1) * I);
  std::vector<uint8_t> hq_l(std::max<int64_t>(nr, 1) * hcb), hs_l(std::max<int64_t>(nr, 1) * hsb);
  oracle_gemm1(c, w, xq.data(), xs.data(), rtok.data(), offsets.data(), nr, rows.data(), h.data(),
               hq_l.data(), hs_l.data());
  // scatter the listed rows' codes into row-indexed buffers for GEMM2
  const int64_t Rcap = int64_t(rtok.size());
  std::vector<uint8_t> hq(std::max<int64_t>(Rcap, 1) * hcb, 0), hs(std::max<int64_t>(Rcap, 1) * hsb, 0);
  for (int64_t i = 0; i < nr; ++i) {
    std::memcpy(&hq[rows[i] * hcb], &hq_l[i * hcb], hcb);
    std::memcpy(&hs[rows[i] * hsb], &hs_l[i * hsb], hsb);
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

// Router for T tokens: x bf16 [T][H], wg bf16 [E][H] (one gate row per
// expert).  logit[t][e] = sum over h of x[t][h] * wg[e][h] in fp64 (every
// product is exact), summed in h order; ids[t][0..k) = the k experts with
// the largest logits in descending order, equal logits going to the lower
// expert id (k rounds of: take the largest logit not yet taken, the lowest
// id among equal ones); weights[t][j] = exp(l_j - l_0) / sum over the k
// selected of exp(l_i - l_0), in fp64, rounded to fp32.  logits (optional,
// may be NULL): fp64 [T][E].
void oracle_router(const uint16_t* x, const uint16_t* wg, int64_t T, int64_t H, int E, int k, int32_t* ids,
                   float* weights, double* logits) {
  parallel_for(T, [&](int64_t t) {
    std::vector<double> l(E);
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h)
        acc += double(bf16_to_f32(x[t * H + h])) * double(bf16_to_f32(wg[int64_t(e) * H + h]));
      l[e] = acc;
      if (logits) logits[t * E + e] = acc;
    }
    std::vector<char> taken(E, 0);
    std::vector<double> sel(k);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        const bool better = best < 0 || l[e] > l[best] || (g_mutation == 7 && l[e] == l[best]);
        if (better) best = e;  // strict '>' keeps the lower id among equal logits
      }
      taken[best] = 1;
      ids[t * k + j] = best;
      sel[j] = l[best];
    }
    double sum = 0.0;
    if (g_mutation == 8) {  // planted: softmax over all E logits, not renormalised over the top-k
      for (int e = 0; e < E; ++e) sum += std::exp(l[e] - sel[0]);
    } else {
      for (int j = 0; j < k; ++j) sum += std::exp(sel[j] - sel[0]);
    }
    for (int j = 0; j < k; ++j) weights[t * k + j] = float(std::exp(sel[j] - sel[0]) / sum);
  });
}

// Brute force (checks the oracle): no permute, no grouping.  For each listed
// token and each valid slot, run the token through that expert's dense
// dequantised MLP (weights dequantised into full fp64 matrices first), then
// requantise h with the same rule and add w * y; plus the shared expert.
void oracle_bruteforce(const Cfg* c, const WSet* w, const uint16_t* x, const int32_t* ids,
                       const float* topk_w, int64_t ntok, const int64_t* toks, double* out) {
  const int64_t H = c->H, I = c->I;
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
    std::vector<uint8_t> q(act_code_bytes(*c, H)), s(act_scale_bytes(*c, H));
    quant_act_row(*c, xr.data(), H, q.data(), s.data());
    std::vector<double> xd(H);
    dequant_act_row(*c, q.data(), s.data(), H, xd.data());
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
      std::vector<uint8_t> hq(act_code_bytes(*c, I)), hs(act_scale_bytes(*c, I));
      quant_act_row(*c, h.data(), I, hq.data(), hs.data());
      std::vector<double> hd(I);
      dequant_act_row(*c, hq.data(), hs.data(), I, hd.data());
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
