// Device helpers shared by the libw4a8moe kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
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

// int4 -> E4M3 in registers, "offset" form used by the streaming (decode) kernels.
// In the reorder packing, byte b of a word holds elements b (low nibble) and 4+b (high
// nibble). XOR with 0x8 turns a two's-complement nibble q into q + 8 in [0, 15], and the
// E4M3 code c in [0, 15] has the value c * 2^-9 (subnormals then the first binade), so the
// two words below are exact E4M3 codes of (q + 8) * 2^-9 for elements 0..3 and 4..7.
// The MFMA then yields 2^-9 * sum x (q + 8); a second MFMA of the same B operand against
// the constant code 0x88 (= -8 * 2^-9) removes the offset.
__device__ __forceinline__ void int4x8_to_e4m3_offset(uint32_t w, uint32_t& lo, uint32_t& hi) {
  uint32_t y = w ^ 0x88888888u;
  lo = y & 0x0F0F0F0Fu;
  hi = (y >> 4) & 0x0F0F0F0Fu;
}

constexpr uint32_t kOffsetCorrCode = 0x88888888u;   // four E4M3 codes of -2^-6 = -8 * 2^-9

// 16 bytes of packed int4 (32 K-values, natural K order after unpacking) -> the 8
// registers of an MFMA operand in offset form.
__device__ __forceinline__ v8i int4x32_to_operand_offset(uint4 q) {
  v8i a;
  uint32_t lo, hi;
  int4x8_to_e4m3_offset(q.x, lo, hi); a[0] = (int)lo; a[1] = (int)hi;
  int4x8_to_e4m3_offset(q.y, lo, hi); a[2] = (int)lo; a[3] = (int)hi;
  int4x8_to_e4m3_offset(q.z, lo, hi); a[4] = (int)lo; a[5] = (int)hi;
  int4x8_to_e4m3_offset(q.w, lo, hi); a[6] = (int)lo; a[7] = (int)hi;
  return a;
}

__device__ __forceinline__ v8i operand_from(uint4 lo, uint4 hi) {
  v8i b;
  b[0] = (int)lo.x; b[1] = (int)lo.y; b[2] = (int)lo.z; b[3] = (int)lo.w;
  b[4] = (int)hi.x; b[5] = (int)hi.y; b[6] = (int)hi.z; b[7] = (int)hi.w;
  return b;
}

__device__ __forceinline__ float act_fn(float g, int act) {
  if (act == 0) return g / (1.0f + expf(-g));                        // silu
  if (act == 1) return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f));  // gelu (erf)
  const float c = 0.7978845608028654f;                                // sqrt(2/pi)
  return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g))); // gelu (tanh)
}

__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }
__device__ __forceinline__ int lane_id() { return threadIdx.x % kWave; }

}  // namespace w4a8
