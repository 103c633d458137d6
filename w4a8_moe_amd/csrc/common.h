// Device helpers shared by the libw4a8moe kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Saturate to the E4M3 range. The hardware conversion rounds to nearest even; values
// clamped to +-448 convert to the largest finite code, which is the saturating
// behaviour the method needs (without the clamp, out-of-range values give NaN).
__device__ __forceinline__ float sat_e4m3(float v) { return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f); }

// Four fp32 values -> four E4M3 codes in one word, byte i = value i.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), r, true);
  return (uint32_t)r;
}

// 16x16x128 fp8 x fp8 -> fp32 MFMA (gfx950). Both operands are E4M3 (format 0), no
// block scaling (scale operands 0 select the unscaled instruction).
// Operand layout, lane l: A holds 32 K-values of row (l % 16), B 32 K-values of column
// (l % 16); the K-values of a lane group (l / 16) sit at the same register/byte slots
// in A and B, so any assignment of K-values to (lane group, register, byte) that is
// the same for A and B gives the same dot products.
// Result: lane l holds D[4 * (l / 16) + v][l % 16], v = 0..3.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 MFMA: lane l holds 8 K-values of row/column (l % 16); same result layout.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- exact fp16 operands for the 16-bit matrix cores
// Which matrix core. gfx950's fp8 MFMA (16x16x128 f8f6f4, and the older 16x16x32 fp8)
// sums each instruction's products with about 14 bits of precision below the largest
// product of the instruction (measured on MI355X: 256 + 127 * 2^-9 comes out as
// 256.234375; random blocks up to 1.4e-4 of the sum of |products|), while its 16-bit
// MFMAs add these operands' exact products in fp32, with no error beyond fp32 rounding
// (probe on the same blocks). Against the oracle's exact sums, the fp8 instruction's
// error moves requantized codes and bf16 outputs across their rounding boundaries far
// more often than the method's output tolerance allows. An E4M3 value and an int4 code are
// both exact in fp16, so both grouped GEMMs multiply them on the fp16 MFMA (16x16x32),
// products exact and sums in fp32, as the method states.
//
// int4 -> fp16 in registers, 10 VALU ops per 8 weights, exact: flipping the top bit of a
// nibble turns q into c = q + 8 in [0, 15]; a byte permute places the low nibbles' c under
// the fp16 exponent of 1024 (bits 0x6400 | c = 1024 + c, two values per op) and one packed
// fp16 subtraction of 1032 leaves q. The high nibbles stay where they are (1024 + 16 c,
// minus 1152: 16 q), and the activations they meet are converted divided by 16, so no
// shift is needed. (Codes placed as fp16 subnormals would need no subtraction, but the
// fp16 MFMA loses precision on subnormal operands: measured on MI355X, a K = 14336 down
// projection erred by 5e-6 of its largest output instead of 1e-8.)
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// two E4M3 codes (bytes 0,1 or, with HIGH, bytes 2,3) -> two fp16 values, exact
template <bool HIGH>
__device__ __forceinline__ uint32_t cvt2_e4m3_f16(uint32_t codes, float scale = 1.0f) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, scale, HIGH));
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// bytes 0,1 (SEL 0x04010400) or 2,3 (SEL 0x04030402) of x placed under the fp16 exponent
// of 1024: the pair 1024 + x_byte (exact for any byte)
template <uint32_t SEL>
__device__ __forceinline__ v2h f16_1024_plus(uint32_t x) {
  return __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x, SEL));
}

// One packed word (8 int4 codes, reorder layout) -> 8 exact fp16 values in K order:
// q for elements 0..3 and 16 q for elements 4..7 (whose activations are staged / 16).
// c = q + 8 is the nibble with its top bit flipped; the low nibbles give 1024 + c, the
// high nibbles, left in place, 1024 + 16 c.
__device__ __forceinline__ v8h int4x8_to_f16(uint32_t w, uint32_t mlo, uint32_t mhi) {
  const uint32_t lo = (w ^ 0x88888888u) & mlo;                   // c of elements 0..3
  const uint32_t hi = (w ^ 0x88888888u) & mhi;                   // 16 c of elements 4..7
  const v2h off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};     // 1024 + 8
  const v2h off_hi = {(_Float16)1152.0f, (_Float16)1152.0f};     // 1024 + 16 * 8
  const v2h e01 = f16_1024_plus<0x04010400u>(lo) - off_lo, e23 = f16_1024_plus<0x04030402u>(lo) - off_lo;
  const v2h e45 = f16_1024_plus<0x04010400u>(hi) - off_hi, e67 = f16_1024_plus<0x04030402u>(hi) - off_hi;
  v8h r;
  r[0] = e01[0]; r[1] = e01[1]; r[2] = e23[0]; r[3] = e23[1];
  r[4] = e45[0]; r[5] = e45[1]; r[6] = e67[0]; r[7] = e67[1];
  return r;
}

__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 E4M3 codes (one 8-byte half of a 16-byte LDS slot) -> the fp16 B operand of one
// MFMA, exact; codes 4..7 face the weights' high nibbles (16 q) and are divided by 16
// (E4M3 keeps 3 mantissa bits, so the quotient is an exact fp16 normal).
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t lo4, uint32_t hi4) {
  return __builtin_bit_cast(v8h, make_uint4(cvt2_e4m3_f16<false>(lo4), cvt2_e4m3_f16<true>(lo4),
                                            cvt2_e4m3_f16<false>(hi4, 0.0625f), cvt2_e4m3_f16<true>(hi4, 0.0625f)));
}


__device__ __forceinline__ v8i operand_from(uint4 lo, uint4 hi) {
  v8i b;
  b[0] = (int)lo.x; b[1] = (int)lo.y; b[2] = (int)lo.z; b[3] = (int)lo.w;
  b[4] = (int)hi.x; b[5] = (int)hi.y; b[6] = (int)hi.z; b[7] = (int)hi.w;
  return b;
}

// Gated activations for the epilogues, fp32 and branch-free (lanes of a wave take
// different signs and ranges, so range-split library functions run every branch). Their
// relative error is about 1e-6 or less wherever the result is large enough to reach an
// E4M3 code; requant_value below takes the rounding decision from them only where that
// error cannot matter.
//   ACT 0, silu:      g * sigma(g),            sigma(y) = 1 / (1 + 2^(-y log2 e))
//   ACT 1, gelu_erf:  g * Phi(g), Phi from erfc(|g|/sqrt 2) = t 2^(Q(t) - g^2 log2(e) / 2),
//                     t = 1 / (1 + |g| / (2 sqrt 2)), Q a degree-9 polynomial: the form of
//                     the erfc approximation "erfcc" of Numerical Recipes, refitted by least
//                     squares in Chebyshev form on |g| in [0, 17] (max error 2.4e-7 in log2
//                     units; the coefficients are printed by w4a8_moe_amd/fit_erfc.py);
//                     g Phi(g) = max(g, 0) - |g| erfc/2 for either sign
//   ACT 2, gelu_tanh: g/2 (1 + tanh(y)) = g * sigma(2 y), y = sqrt(2/pi) (g + 0.044715 g^3)
__device__ __forceinline__ float sigmoid_fast(float y) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * 1.4426950408889634f));
}

template <int ACT>
__device__ __forceinline__ float act_fast(float g) {
  if (ACT == 0) return g * sigmoid_fast(g);
  if (ACT == 2) {
    const float y = 0.7978845608028654f * __builtin_fmaf(0.044715f * g * g, g, g);
    return g * sigmoid_fast(2.0f * y);
  }
  // th = t / 2 (the 1/2 of erfc/2 taken into the reciprocal, exactly); Q evaluated in th
  // with the coefficients of t^k scaled by 2^k, which gives the same fp32 values
  const float a = __builtin_fabsf(g);
  const float th = __builtin_amdgcn_rcpf(__builtin_fmaf(a, 0.70710678118654746f, 2.0f));
  float q = 116.59952545166016f;
  q = __builtin_fmaf(q, th, -277.265869140625f);
  q = __builtin_fmaf(q, th, 243.74142456054688f);
  q = __builtin_fmaf(q, th, -84.14982604980469f);
  q = __builtin_fmaf(q, th, 4.415352821350098f);
  q = __builtin_fmaf(q, th, -2.0990519523620605f);
  q = __builtin_fmaf(q, th, 0.7554525136947632f);
  q = __builtin_fmaf(q, th, 2.194683313369751f);
  q = __builtin_fmaf(q, th, 2.8835232257843018f);
  q = __builtin_fmaf(q, th, -1.8257052898406982f);
  const float half_erfc = th * __builtin_amdgcn_exp2f(__builtin_fmaf(-g * g, 0.7213475204444817f, q));
  // g * Phi(g) = max(g, 0) - |g| erfc(|g| / sqrt 2) / 2 for either sign
  return __builtin_fmaf(-a, half_erfc, __builtin_fmaxf(g, 0.0f));
}

__device__ __forceinline__ float act_fast_rt(float g, int act) {
  return act == 0 ? act_fast<0>(g) : act == 1 ? act_fast<1>(g) : act_fast<2>(g);
}

// x / s rounded to nearest, from r = the correctly rounded 1 / s (computed on the host):
// q = x r is within an ulp of the quotient, the fma gives its exact residual, and one
// correction step rounds correctly for quotients in the normal range.
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q = x * r;
  return __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
}

// ---- the requantization decision of the gated activation
// The oracle of the method forms a = act(g) u in double precision and rounds fp32(a) / s_a
// to E4M3. The fast fp32 activation differs from that by up to ~1e-6 relatively, which
// would move about one code in 10^5 across a rounding boundary: enough to change bf16
// outputs of whole tokens at the intermediate sizes of Grok-1 and Mixtral. So a value is
// taken from the fast path only when it lies farther than kBoundaryTau (relative) from every
// rounding boundary of E4M3; the few others (about 2.4e-4 of them) are recomputed in double
// precision from the same gate and up values, with the oracle's formulas.
constexpr float kBoundaryTau = 1e-5f;

// E4M3 rounding boundaries (midpoints of adjacent codes): odd multiples of 2^(e-4) for
// |v| in [2^e, 2^(e+1)), e >= -6 (3 mantissa bits), and odd multiples of 2^-10 below 2^-6
// (subnormals, spacing 2^-9). t = |v| scaled so that the boundaries are the odd integers
// (t < 32, exact); r = its distance to the nearest one. Saturated values (>= 464) hit
// spurious "boundaries", which only send them through the exact path.
__device__ __forceinline__ bool near_e4m3_boundary(float v) {
  const float a = __builtin_fabsf(v);
  const int e = __builtin_amdgcn_frexp_expf(a);               // a = f 2^e, f in [0.5, 1)
  const int sh = (e - 1 > -6 ? e - 1 : -6) - 4;
  const float t = __builtin_ldexpf(a, -sh);
  const float r = t - __builtin_fmaf(2.0f, __builtin_floorf(0.5f * t), 1.0f);
  return __builtin_fabsf(r) < kBoundaryTau * t;
}

// The activation in double precision, the oracle's formulas.
__device__ __forceinline__ double act_f64(double g, int act) {
  if (act == 0) return g / (1.0 + exp(-g));
  if (act == 1) return 0.5 * g * (1.0 + erf(g / 1.4142135623730951));
  return 0.5 * g * (1.0 + tanh(0.7978845608028654 * (g + 0.044715 * (g * g * g))));
}

// fp32(act(g) u) / s_a, correctly rounded at each of the two steps (IEEE division).
__device__ __attribute__((noinline)) float requant_value_exact(float g, float u, float s_a, int act) {
  const float a = (float)(act_f64((double)g, act) * (double)u);
  return a / s_a;
}

// The value whose E4M3 code (nearest, saturated) is the requantized activation.
template <int ACT>
__device__ __forceinline__ float requant_value(float g, float u, float s_a, float inv_s_a) {
  const float v = div_rn(act_fast<ACT>(g) * u, s_a, inv_s_a);
  if (__builtin_expect(near_e4m3_boundary(v), 0)) return requant_value_exact(g, u, s_a, ACT);
  return v;
}

__device__ __forceinline__ float requant_value_rt(float g, float u, float s_a, float inv_s_a, int act) {
  const float v = div_rn(act_fast_rt(g, act) * u, s_a, inv_s_a);
  if (__builtin_expect(near_e4m3_boundary(v), 0)) return requant_value_exact(g, u, s_a, act);
  return v;
}

// Barrier for LDS hand-off only: waits for this wave's LDS operations, not for its
// outstanding global loads (a prefetch stays in flight across it; __syncthreads would
// wait for every load first).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }
__device__ __forceinline__ int lane_id() { return threadIdx.x % kWave; }

// fp8_quant_static's arithmetic: e4m3(fp32(x / s)) (correctly rounded quotient, nearest
// even, saturated) over n bf16 elements, 8 per thread and round: groups [8 i, 8 i + 8) for
// i = first, first + stride, ... < n / 8, then the n % 8 tail by threads first < 8. Every
// caller runs this same code, so the codes are the same bytes wherever x is quantized.
__device__ __forceinline__ uint32_t quant4_e4m3(uint32_t lo, uint32_t hi, float s) {
  return pack4_e4m3(bf16_bits_to_f32(lo & 0xFFFFu) / s, bf16_bits_to_f32(lo >> 16) / s,
                    bf16_bits_to_f32(hi & 0xFFFFu) / s, bf16_bits_to_f32(hi >> 16) / s);
}

__device__ __forceinline__ void fp8_quant_span(const uint16_t* __restrict__ x, int64_t n, float s,
                                               uint8_t* __restrict__ out, int64_t first, int64_t stride) {
  const int64_t n8 = n >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x);
  uint2* dst = reinterpret_cast<uint2*>(out);
  for (int64_t i = first; i < n8; i += stride) {
    const uint4 v = src[i];
    dst[i] = make_uint2(quant4_e4m3(v.x, v.y, s), quant4_e4m3(v.z, v.w, s));
  }
  const int64_t t = n8 * 8 + first;                         // the tail: one element per thread
  if (t < n && first < 8) {
    const uint32_t c = pack4_e4m3(bf16_bits_to_f32(x[t]) / s, 0.f, 0.f, 0.f);
    out[t] = (uint8_t)(c & 0xFFu);
  }
}

}  // namespace w4a8
