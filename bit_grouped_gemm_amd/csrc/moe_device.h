// moe_device.h -- device-side building blocks shared by the gfx950 kernels:
// number-format codecs, wave reductions and the scaled-MFMA operand layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ codecs
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> e4m3 (OCP E4M3FN) code: round to nearest, ties to even, |v| >= 448
// saturates to 448, the sign bit is kept (values that round to zero keep
// their sign).  Integer formulation: subnormal codes are multiples of 2^-9
// (rint of v * 2^9, whose result 8 is the smallest normal code); normal
// codes keep the top three mantissa bits with the 20 dropped bits rounded
// to nearest-even, a carry stepping into the exponent field.
__device__ __forceinline__ uint32_t enc_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const float af = __uint_as_float(a);
  uint32_t code;
  if (!(af < 448.0f)) {
    code = 0x7Eu;
  } else if (af < 0x1p-6f) {
    code = uint32_t(__builtin_rintf(af * 512.0f));
  } else {
    code = ((((a >> 23) - 127u + 7u) << 3) | ((a >> 20) & 7u));
    const uint32_t rem = a & 0xFFFFFu;
    code += (rem > 0x80000u) | ((rem == 0x80000u) & (code & 1u));
  }
  return code | sign;
}

// Four fp32 -> four e4m3 codes (byte i = value i) with the same rounding as
// enc_e4m3, by the hardware conversion: the values are clamped to +-448 (the
// saturation) and converted two at a time with round-to-nearest-even.  The
// GPU test suite runs this conversion (exported as moe_encode_e4m3) on every
// finite fp32 bit pattern against PyTorch's conversion of the clamped value,
// and on the rounding boundaries against a brute-force CPU
// encoder: identical codes, signed zeros included.
__device__ __forceinline__ uint32_t enc_e4m3x4(float a, float b, float c, float d) {
  const auto sat = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return uint32_t(w);
}

// SwiGLU of one h element, left half through SiLU times the right half:
// silu(gate) * up with silu(z) = z / (1 + e^-z), IEEE division and the
// library exponential.  Every GEMM1 epilogue uses this one formula, so an
// h value does not depend on which kernel its group's row count selects.
__device__ __forceinline__ float swiglu(float gate, float up) { return gate / (1.0f + expf(-gate)) * up; }

// MXFP4 (Microscaling FP4): e8m0 code of the scale X = 2^(floor(log2 amax)
// - 2) of a group with absolute maximum amax, clamped to the e8m0 range.  For
// a normal amax floor(log2 amax) is its exponent field minus 127, so the
// code is that field minus 2; subnormal and zero maxima (field 0) and field
// 1 clamp to code 0 (X = 2^-127).
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const uint32_t ex = __float_as_uint(amax) >> 23;  // amax >= 0: the exponent field
  return ex >= 2u ? ex - 2u : 0u;
}

// 1 / X = 2^(127 - code) as an fp32 (biased exponent 254 - code, always
// normal for code <= 252); x * (1 / X) is exact.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// fp32 -> e2m1 code (sign in bit 3): round to nearest, ties to even, |v| >= 6
// saturates to 6.  The magnitude code counts the rounding boundaries below
// |v|; at a boundary that lies halfway, the comparison's strictness sends it
// to the even code (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0,
// 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0).
__device__ __forceinline__ uint32_t enc_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t m = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 8u);
}

// Quantisation multiplier and dequant scale of a group with absolute max a.
__device__ __forceinline__ float quant_mult(float amax) { return 448.0f / fmaxf(amax, 0x1p-64f); }

// ------------------------------------------------------------------ waves
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// Another lane's value within the lane's 16-lane row by a DPP move (CTRL:
// the DPP control word), register to register.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over each aligned group of `lanes` consecutive lanes (4 or 16), in
// every lane of the group: the quad permutations (lane xor 1, xor 2), then
// for 16 lanes the half-row mirror (lanes i, 7 - i) and the row mirror
// (i, 15 - i).  Every lane of the wave must be active.
__device__ __forceinline__ float group_max_dpp(float v, int lanes) {
  v = fmaxf(v, dpp_f32<0xB1>(v));  // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f32<0x4E>(v));  // quad_perm [2, 3, 0, 1]
  if (lanes > 4) {
    v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  }
  return v;
}

// ------------------------------------------------------------------ MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4, layout measured on gfx950:
//   operand lane l: row (A) / column (B) = l % 16, lane group g = l / 16.
//   e4m3 operand: bytes 0..15 hold K = 16g + j, bytes 16..31 hold
//     K = 64 + 16g + (j - 16).  For a K-contiguous row in memory the lane
//     loads 16 bytes at offset 16g and 16 bytes at offset 64 + 16g.
//   e2m1 operand (first four registers): nibble j (low nibble first) holds
//     K = 32g + j, i.e. 16 bytes at offset 16g of a packed row.
//   e8m0 scale operand: lane b*16 + m holds the scale of row/column m for
//     K block b (K = 32b .. 32b+31), byte 0 of the register.
//   result: lane l holds column l % 16, rows 4g .. 4g+3.
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_scaled(const v8i& a, const v8i& b, int sa, int sb) {
  v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, FA, FB, 0, sa, 0, sb);
}

// Same, accumulating into c (D = C + A.B in the matrix core).
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_scaled_acc(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

constexpr int kFmtE4M3 = 0;
constexpr int kFmtE2M1 = 4;
constexpr int kUnitScale = 127;  // e8m0 code of 1.0

__device__ __forceinline__ v4u ldg16(const uint8_t* p) { return *reinterpret_cast<const v4u*>(p); }

// Load one 16-row x 128-K e4m3 operand fragment for this lane from a
// K-contiguous row (row already selected by the caller).
__device__ __forceinline__ v8i load_e4m3_frag(const uint8_t* row_k0, int g) {
  const v4u lo = ldg16(row_k0 + 16 * g);
  const v4u hi = ldg16(row_k0 + 64 + 16 * g);
  v8i r;
  r[0] = int(lo[0]); r[1] = int(lo[1]); r[2] = int(lo[2]); r[3] = int(lo[3]);
  r[4] = int(hi[0]); r[5] = int(hi[1]); r[6] = int(hi[2]); r[7] = int(hi[3]);
  return r;
}

// e2m1 fragment: 16 bytes (32 nibbles) at offset 16g of the packed row's
// 64-byte K step.
__device__ __forceinline__ v8i load_e2m1_frag(const uint8_t* row_k0, int g) {
  const v4u lo = ldg16(row_k0 + 16 * g);
  v8i r;
  r[0] = int(lo[0]); r[1] = int(lo[1]); r[2] = int(lo[2]); r[3] = int(lo[3]);
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// four fp32 -> four bf16 (RNE), one 8-byte store
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, const v4f& v) {
  uint2 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = o;
}

// ------------------------------------------------------------ fp16 operands (NVFP4)
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Eight e2m1 codes (one word, low nibble first = lower K) as f16 (exact).
__device__ __forceinline__ h8v cvt_e2m1x8_f16(uint32_t w) {
  const h2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const h2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const h2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const h2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return h8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight e4m3 codes (two words, byte order = K order) as f16 (exact).
__device__ __forceinline__ h8v cvt_e4m3x8_f16(int w0, int w1) {
  const h2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uint32_t(w0), 1.0f, false);
  const h2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uint32_t(w0), 1.0f, true);
  const h2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uint32_t(w1), 1.0f, false);
  const h2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uint32_t(w1), 1.0f, true);
  return h8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ------------------------------------------------------------ tiled weights
// Expert weights are stored as tiles of 16 rows x 128 K in MFMA lane order,
// tile (k step, row tile) at ((ks * N/16) + rt) * kTileBytes<WF>: lane l's
// 16 bytes (row 16 rt + l % 16, K bytes 16 (l / 16) of the step's row chunk)
// at l * 16; e4m3 tiles carry the K bytes 64..127 of the step in a second
// kilobyte.  MXFP4 scales: 64 bytes per tile, byte l = e8m0 of row
// 16 rt + l % 16 and 32-block l / 16 of the step -- the scale operand of
// MFMA lane l.  NVFP4 (WF 2) codes tile as MXFP4's; its e4m3 scales take
// 128 bytes per tile, byte 8 m + j = row 16 rt + m, 16-block 8 ks + j.
template <int WF> constexpr int kTileBytes = WF == 0 ? 2048 : 1024;
constexpr int kTileScaleBytes = 64;
constexpr int kTileScaleBytes16 = 128;

// this lane's operand from a weight tile (tile_lane = tile base + 16 * lane)
template <int WF>
__device__ __forceinline__ v8i load_tile_frag(const uint8_t* tile_lane) {
  const v4u lo = ldg16(tile_lane);
  v8i r;
  r[0] = int(lo[0]); r[1] = int(lo[1]); r[2] = int(lo[2]); r[3] = int(lo[3]);
  if (WF == 0) {
    const v4u hi = ldg16(tile_lane + 1024);
    r[4] = int(hi[0]); r[5] = int(hi[1]); r[6] = int(hi[2]); r[7] = int(hi[3]);
  } else {
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  }
  return r;
}

// Keep only the bytes of 32-wide K block `blk` in an e4m3 fragment (used
// when the weight scales change every 32 along K): block blk lives in lane
// groups with (g >> 1) == (blk & 1), in byte half (blk >> 1).
__device__ __forceinline__ v8i mask_e4m3_block(const v8i& a, int g, int blk) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if ((g >> 1) == (blk & 1)) {
    if (blk >> 1) { r[4] = a[4]; r[5] = a[5]; r[6] = a[6]; r[7] = a[7]; }
    else { r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3]; }
  }
  return r;
}

}  // namespace moe
