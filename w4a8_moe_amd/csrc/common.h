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

__device__ __forceinline__ v8i operand_from(uint4 lo, uint4 hi) {
  v8i b;
  b[0] = (int)lo.x; b[1] = (int)lo.y; b[2] = (int)lo.z; b[3] = (int)lo.w;
  b[4] = (int)hi.x; b[5] = (int)hi.y; b[6] = (int)hi.z; b[7] = (int)hi.w;
  return b;
}

// Gated activations for the epilogues, fp32 and branch-free (lanes of a wave take
// different signs and ranges, so range-split library functions run every branch). The
// relative error is about 1e-6 or less wherever the result is large enough to reach an
// E4M3 code, so an exact-arithmetic activation rounds to a different code only when the
// value sits within that distance of a rounding boundary.
//   ACT 0, silu:      g * sigma(g),            sigma(y) = 1 / (1 + 2^(-y log2 e))
//   ACT 1, gelu_erf:  g * Phi(g), Phi from erfc(|g|/sqrt 2) = t 2^(Q(t) - g^2 log2(e) / 2),
//                     t = 1 / (1 + |g| / (2 sqrt 2)), Q a degree-9 polynomial fitted here
//                     (least squares in Chebyshev form on |g| in [0, 17], max error 8e-8
//                     in log2 units); g Phi(g) = max(g, 0) - |g| erfc/2 for either sign
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
  float q = 113.79635620117188f;
  q = __builtin_fmaf(q, th, -269.8727722167969f);
  q = __builtin_fmaf(q, th, 235.36532592773438f);
  q = __builtin_fmaf(q, th, -78.82111358642578f);
  q = __builtin_fmaf(q, th, 2.327209711074829f);
  q = __builtin_fmaf(q, th, -1.5790550708770752f);
  q = __builtin_fmaf(q, th, 0.673623263835907f);
  q = __builtin_fmaf(q, th, 2.2024853229522705f);
  q = __builtin_fmaf(q, th, 2.8831162452697754f);
  q = __builtin_fmaf(q, th, -1.8256964683532715f);
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
