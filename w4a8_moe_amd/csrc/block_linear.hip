// Block-FP8 weight-only decode GEMV / small-M GEMM (the FP8_PB_WO projections of the
// page "qwen4_exp: serve the block-FP8 dense projections natively (+25% decode)":
// e4m3 weight [N,K] and one fp32 scale per 128x128 block; the activation stays bf16).
//
//   y[m][n] = bf16( sum_kb S[n/128][kb] * sum_{k in kb} x[m][k] * dec(W[n][k]) )
//
// The contraction runs on the bf16 MFMA: an E4M3 value is exact in bf16 (3 mantissa
// bits, exponents 2^-9..2^8), so each weight byte is widened in registers
// (v_cvt_pk_f32_fp8, then the upper halves of two fp32 are packed into one dword) and
// multiplied against the bf16 activations with fp32 accumulation. Each 128-column block
// is accumulated on its own and added to the running sum with its scale.
//
// Mapping: a 16-row block is owned by kBlSplit (4) waves, each streaming one contiguous
// quarter of K; their partial sums meet in LDS and are added in wave order
// (deterministic). A workgroup holds RB such row blocks (2 for M <= 2, 4 above: the M
// activation rows are staged once per workgroup in LDS, compactly, so a larger M wants
// more rows to share them). A GEMV has no other parallelism to hide HBM latency with:
// splitting K gives 4 N/16 waves. Weight loads are 2 x 16 B per lane per 128-K block,
// kBlDepth blocks ahead (one: the many waves in flight hide the latency; measured best).
//
// Tuning knobs (defaults chosen by measurement on MI355X): W4A8_BL_SPLIT waves per row
// block, W4A8_BL_DEPTH blocks in flight, W4A8_BL_RB_SMALL_M / W4A8_BL_RB_LARGE_M row
// blocks per workgroup for M <= 2 / M > 2.
//
// The per-tensor FP8 linear (the dense projections of the W4A8 model: quant_method "fp8"
// with static activations on the page "ROCm: enable trillion-parameter MoE models with
// INT4-FP8 single node") has the same mapping; its activations are quantized with their
// static scale, both operands are widened to bf16 in registers (exact), and the one scale
// s_x * s_w multiplies the sum. Up to 2 rows fp8_linear_kernel quantizes the activations
// itself and stages their codes in LDS (one launch); above, fp8_linear_wide_kernel reads
// the codes, quantized once into the workspace, straight from L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

#ifndef W4A8_GEMV_NT
#define W4A8_GEMV_NT 0
#endif
// 16 bytes of weights (nontemporal hint behind the knob)
__device__ __forceinline__ uint4 ld_w16(const uint8_t* p) {
  typedef unsigned u4v __attribute__((ext_vector_type(4)));
  if (W4A8_GEMV_NT) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p)));
  return *reinterpret_cast<const uint4*>(p);
}

#ifndef W4A8_BL_SPLIT
#define W4A8_BL_SPLIT 4
#endif
constexpr int kBlSplit = W4A8_BL_SPLIT;   // waves per 16-row block, each on a part of K
#ifndef W4A8_BL_DEPTH
#define W4A8_BL_DEPTH 1
#endif
constexpr int kBlDepth = W4A8_BL_DEPTH;   // 128-K blocks of weights in flight per wave

// 4 E4M3 codes -> 4 bf16 values in two dwords (exact).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t c, uint32_t& lo, uint32_t& hi) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
  const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
  lo = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
}

__device__ __forceinline__ v8bf bf16_operand(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
  v4i t = {(int)d0, (int)d1, (int)d2, (int)d3};
  return __builtin_bit_cast(v8bf, t);
}

template <int RB>   // 16-row blocks per workgroup
__global__ __launch_bounds__(RB * kBlSplit * kWave) void fp8_block_linear_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w, const float* __restrict__ S,
    int M, int N, int K, uint16_t* __restrict__ y) {
  constexpr int kWaves = RB * kBlSplit;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int KB = K >> 7;
  const int rb = min(blockIdx.x * RB + wave / kBlSplit, N / 16 - 1);   // 16-row block
  const bool rb_ok = blockIdx.x * RB + wave / kBlSplit < N / 16;      // else: no K blocks, no store
  const int part_k = wave % kBlSplit;
  const int i = lane & 15, g = lane >> 4;
  const uint8_t* wp = w + (size_t)(rb * 16 + i) * K + g * 32;
  const float* srow = S + (size_t)((rb * 16) >> 7) * KB;
  const bool col_ok = i < M;
  // this wave's 128-K blocks [kb_begin, kb_end)
  const int per = (KB + kBlSplit - 1) / kBlSplit;
  const int kb_begin = min(KB, part_k * per), kb_end = rb_ok ? min(KB, kb_begin + per) : kb_begin;
  // the first weight blocks are requested before x is staged (they do not depend on it)
  uint4 q0[kBlDepth], q1[kBlDepth];
#pragma unroll
  for (int d = 0; d < kBlDepth; ++d)
    if (kb_begin + d < kb_end) {
      q0[d] = ld_w16(wp + (kb_begin + d) * 128);
      q1[d] = ld_w16(wp + (kb_begin + d) * 128 + 16);
    }
  // ---- stage x: unit (kb, j, g, m) = 8 bf16 = x[m][kb*128 + g*32 + j*8 .. +8], stored at
  //      ((kb*4 + j)*4 + g)*M + m, so lane (m, g) of MFMA j reads 16 contiguous bytes.
  const int units = M * (K >> 3);
  for (int u = tid; u < units; u += kWaves * kWave) {
    const int m = u / (K >> 3), c8 = u - m * (K >> 3);       // 8-element chunk of row m
    const int kb = c8 >> 4, within = c8 & 15;                // 16 chunks per 128-K block
    const int gg = within >> 2, j = within & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + c8 * 8);
    *reinterpret_cast<uint4*>(lds + ((((kb * 4 + j) * 4 + gg) * M + m) << 4)) = v;
  }
  __syncthreads();

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = kb_begin; kb0 < kb_end; kb0 += kBlDepth) {
#pragma unroll
    for (int d = 0; d < kBlDepth; ++d) {
      const int kb = kb0 + d;
      if (kb < kb_end) {
        const uint4 a0 = q0[d], a1 = q1[d];
        if (kb + kBlDepth < kb_end) {
          q0[d] = ld_w16(wp + (kb + kBlDepth) * 128);
          q1[d] = ld_w16(wp + (kb + kBlDepth) * 128 + 16);
        }
        const uint32_t c[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        v4f blk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {                        // MFMA j: bytes 8j..8j+7 of the lane's 32
          uint32_t d0, d1, d2, d3;
          e4m3x4_to_bf16x4(c[2 * j], d0, d1);
          e4m3x4_to_bf16x4(c[2 * j + 1], d2, d3);
          const v8bf a = bf16_operand(d0, d1, d2, d3);
          uint4 bv = make_uint4(0, 0, 0, 0);
          if (col_ok) bv = *reinterpret_cast<const uint4*>(lds + ((((kb * 4 + j) * 4 + g) * M + i) << 4));
          const v8bf b = bf16_operand(bv.x, bv.y, bv.z, bv.w);
          blk = mfma_bf16_16x16x32(a, b, blk);
        }
        const float sc = srow[kb];
        acc[0] += sc * blk[0]; acc[1] += sc * blk[1]; acc[2] += sc * blk[2]; acc[3] += sc * blk[3];
      }
    }
  }
  // ---- the partial sums of a row block's waves meet in LDS over the staged x (once every
  //      wave is done with it): its K-part 0 wave adds parts 1, 2, 3 in order
  v4f* part = reinterpret_cast<v4f*>(lds);
  __syncthreads();
  if (part_k > 0) part[(wave - 1) * kWave + lane] = acc;     // slot of wave w: w - 1
  __syncthreads();
  if (part_k > 0 || !col_ok || !rb_ok) return;
#pragma unroll
  for (int v = 1; v < kBlSplit; ++v) {
    const v4f o = part[(wave + v - 1) * kWave + lane];
    acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
  }
  // lane holds rows rb*16 + 4g + v of column (token) i
  const int n = rb * 16 + 4 * g;
  uint2 o;
  o.x = f32_to_bf16_bits(acc[0]) | f32_to_bf16_bits(acc[1]) << 16;
  o.y = f32_to_bf16_bits(acc[2]) | f32_to_bf16_bits(acc[3]) << 16;
  *reinterpret_cast<uint2*>(y + (size_t)i * N + n) = o;
}

// Block-FP8 GEMV past 16 rows or past 64 KB of activations: the mapping of the whole-x
// kernel with NT 16-column tiles of rows per weight block, the bf16 activations staged in
// LDS chunk by chunk: all waves walk their K-quarters in step, CK = 4 / NT 128-K blocks at
// a time, and a chunk holds those blocks of all four quarters for all rows (64 KB), a
// barrier per chunk; the per-128-block scales applied per block. (Reading the activations
// straight from L2 instead, as the per-tensor FP8 linear does with its 1-byte codes,
// measured slower here: 27.7 vs 18.0 us at 32 rows of [16384, 2560], twice the bytes; with
// two or three 128-K blocks in flight per lane, 28.0-28.6 vs 17.8 us. Loading the next
// chunk into registers while the current one is computed: 18.9 vs 17.9 us.)
// Unit (q, cb, j, g, m) = 8 bf16 of row m at K = (q*per + c*CK + cb)*128 + g*32 + j*8, at
// byte (((((q*CK + cb)*4 + j)*4 + g)*Mp + m) << 4), Mp = 16 * NT.
template <int RB, int NT>
__global__ __launch_bounds__(RB * kBlSplit * kWave) void fp8_block_linear_wide_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w, const float* __restrict__ S, int M, int N, int K,
    uint16_t* __restrict__ y) {
  constexpr int kWaves = RB * kBlSplit, Mp = 16 * NT, CK = 4 / NT;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int KB = K >> 7;
  const int per = (KB + kBlSplit - 1) / kBlSplit;
  const int chunks = (per + CK - 1) / CK;
  const int rb = min(blockIdx.x * RB + wave / kBlSplit, N / 16 - 1);
  const bool rb_ok = blockIdx.x * RB + wave / kBlSplit < N / 16;
  const int part_k = wave % kBlSplit;
  const int i = lane & 15, g = lane >> 4;
  const uint8_t* wp = w + (size_t)(rb * 16 + i) * K + g * 32;
  const float* srow = S + (size_t)((rb * 16) >> 7) * KB;
  const int kb_begin = min(KB, part_k * per), kb_end = rb_ok ? min(KB, kb_begin + per) : kb_begin;

  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 q0 = make_uint4(0u, 0u, 0u, 0u), q1 = q0;
  if (kb_begin < kb_end) {
    q0 = ld_w16(wp + kb_begin * 128);
    q1 = ld_w16(wp + kb_begin * 128 + 16);
  }
  const int units = kBlSplit * CK * 16 * M;
  for (int c = 0; c < chunks; ++c) {
    if (c > 0) lds_barrier();
    for (int u = tid; u < units; u += kWaves * kWave) {
      const int m = u % M, r = u / M;
      const int jg = r & 15, qcb = r >> 4;
      const int gg = jg >> 2, jj = jg & 3, cb = qcb % CK, q = qcb / CK;
      const int kb = q * per + c * CK + cb;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (kb < min(KB, (q + 1) * per) && c * CK + cb < per)
        v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + kb * 128 + gg * 32 + jj * 8);
      *reinterpret_cast<uint4*>(lds + (((((q * CK + cb) * 4 + jj) * 4 + gg) * Mp + m) << 4)) = v;
    }
    lds_barrier();
#pragma unroll
    for (int cb = 0; cb < CK; ++cb) {
      const int kb = kb_begin + c * CK + cb;
      if (kb < kb_end) {
        const uint4 a0 = q0, a1 = q1;
        if (kb + 1 < kb_end) {
          q0 = ld_w16(wp + (kb + 1) * 128);
          q1 = ld_w16(wp + (kb + 1) * 128 + 16);
        }
        const uint32_t cw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        v4f blk[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) blk[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t d0, d1, d2, d3;
          e4m3x4_to_bf16x4(cw[2 * j], d0, d1);
          e4m3x4_to_bf16x4(cw[2 * j + 1], d2, d3);
          const v8bf a = bf16_operand(d0, d1, d2, d3);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int m = t * 16 + i;
            uint4 bv = make_uint4(0u, 0u, 0u, 0u);
            if (m < M)
              bv = *reinterpret_cast<const uint4*>(lds + (((((part_k * CK + cb) * 4 + j) * 4 + g) * Mp + m) << 4));
            blk[t] = mfma_bf16_16x16x32(a, bf16_operand(bv.x, bv.y, bv.z, bv.w), blk[t]);
          }
        }
        const float sc = srow[kb];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[t][0] += sc * blk[t][0]; acc[t][1] += sc * blk[t][1];
          acc[t][2] += sc * blk[t][2]; acc[t][3] += sc * blk[t][3];
        }
      }
    }
  }
  v4f* part = reinterpret_cast<v4f*>(lds);
  __syncthreads();
  if (part_k > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) part[((wave - 1) * NT + t) * kWave + lane] = acc[t];
  }
  __syncthreads();
  if (part_k > 0 || !rb_ok) return;
  const int n = rb * 16 + 4 * g;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = t * 16 + i;
    v4f a = acc[t];
#pragma unroll
    for (int v = 1; v < kBlSplit; ++v) {
      const v4f o = part[((wave + v - 1) * NT + t) * kWave + lane];
      a[0] += o[0]; a[1] += o[1]; a[2] += o[2]; a[3] += o[3];
    }
    if (m < M) {
      uint2 o;
      o.x = f32_to_bf16_bits(a[0]) | f32_to_bf16_bits(a[1]) << 16;
      o.y = f32_to_bf16_bits(a[2]) | f32_to_bf16_bits(a[3]) << 16;
      *reinterpret_cast<uint2*>(y + (size_t)m * N + n) = o;
    }
  }
}

template <int NT>
static void launch_blw(const uint16_t* x, const uint8_t* w, const float* s, int M, int N, int K, uint16_t* y,
                       hipStream_t st) {
  constexpr int RB = 4;   // four row blocks share one staging of x (2 measured 15-25% slower)
  const unsigned grid = (unsigned)((N / 16 + RB - 1) / RB);
  const size_t lds = std::max((size_t)kBlSplit * (4 / NT) * 128 * 16 * NT * 2,
                              (size_t)(RB * kBlSplit - 1) * NT * kWave * sizeof(v4f));
  hipLaunchKernelGGL((fp8_block_linear_wide_kernel<RB, NT>), dim3(grid), dim3(RB * kBlSplit * kWave), lds, st, x, w,
                     s, M, N, K, y);
}

template <int RB>
static void launch_bl(const uint16_t* x, const uint8_t* w, const float* s, int M, int N, int K, uint16_t* y,
                      hipStream_t st) {
  const unsigned grid = (unsigned)((N / 16 + RB - 1) / RB);   // N % 16 == 0 is checked by the caller
  // staged x, later reused for the partial sums
  const size_t lds =
      std::max((size_t)M * K * sizeof(uint16_t), (size_t)(RB * kBlSplit - 1) * kWave * sizeof(v4f));
  hipLaunchKernelGGL(fp8_block_linear_kernel<RB>, dim3(grid), dim3(RB * kBlSplit * kWave), lds, st, x, w, s, M, N,
                     K, y);
}

void launch_fp8_block_linear(const uint16_t* x, const uint8_t* w, const float* s, int M, int N, int K,
                             uint16_t* y, hipStream_t st) {
#ifndef W4A8_BL_RB_SMALL_M
#define W4A8_BL_RB_SMALL_M 2
#endif
#ifndef W4A8_BL_RB_LARGE_M
#define W4A8_BL_RB_LARGE_M 4
#endif
  // fewer row blocks per workgroup while staging x costs little, more as M grows; past 16
  // rows or 64 KB of bf16 activations, the chunked kernel
  if (M > 16 || (int64_t)M * K * 2 > 65536) {
    if (M <= 16) launch_blw<1>(x, w, s, M, N, K, y, st);
    else if (M <= 32) launch_blw<2>(x, w, s, M, N, K, y, st);
    else launch_blw<4>(x, w, s, M, N, K, y, st);
  } else if (M <= 2) {
    launch_bl<W4A8_BL_RB_SMALL_M>(x, w, s, M, N, K, y, st);
  } else {
    launch_bl<W4A8_BL_RB_LARGE_M>(x, w, s, M, N, K, y, st);
  }
}

// ---------------------------------------------------------------- per-tensor FP8 linear
// y[m][n] = bf16( scale * sum_k dec(xq[m][k]) * dec(W[n][k]) ), scale = s_x * s_w.
// Staged unit (kb, j, g, m) = 8 codes of x[m][kb*128 + g*32 + j*8 .. +8] at byte
// ((((kb*4 + j)*4 + g)*M + m) << 3): lane (m, g) of MFMA j reads 8 contiguous bytes.
// Every workgroup quantizes the M x K activations itself while staging them (the
// arithmetic of fp8_quant_static: correctly rounded x / s_x, nearest even, saturated), and
// the call is one launch: the path for M <= 2 (a few KB of activations).
template <int RB>   // 16-row blocks per workgroup
__global__ __launch_bounds__(RB * kBlSplit * kWave) void fp8_linear_kernel(
    const uint16_t* __restrict__ x, float s_x, const uint8_t* __restrict__ w, float scale, int M, int N, int K,
    uint16_t* __restrict__ y) {
  constexpr int kWaves = RB * kBlSplit;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int KB = K >> 7;
  const int units = M * (K >> 3);
  for (int u = tid; u < units; u += kWaves * kWave) {
    const int m = u / (K >> 3), c8 = u - m * (K >> 3);
    const int kb = c8 >> 4, within = c8 & 15;
    const int g = within >> 2, j = within & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + c8 * 8);
    *reinterpret_cast<uint2*>(lds + ((((kb * 4 + j) * 4 + g) * M + m) << 3)) =
        make_uint2(quant4_e4m3(v.x, v.y, s_x), quant4_e4m3(v.z, v.w, s_x));
  }
  __syncthreads();
  const int rb = min(blockIdx.x * RB + wave / kBlSplit, N / 16 - 1);
  const bool rb_ok = blockIdx.x * RB + wave / kBlSplit < N / 16;
  const int part_k = wave % kBlSplit;
  const int i = lane & 15, g = lane >> 4;
  const uint8_t* wp = w + (size_t)(rb * 16 + i) * K + g * 32;
  const bool col_ok = i < M;
  const int per = (KB + kBlSplit - 1) / kBlSplit;
  const int kb_begin = min(KB, part_k * per), kb_end = rb_ok ? min(KB, kb_begin + per) : kb_begin;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  uint4 q0[kBlDepth], q1[kBlDepth];
#pragma unroll
  for (int d = 0; d < kBlDepth; ++d)
    if (kb_begin + d < kb_end) {
      q0[d] = ld_w16(wp + (kb_begin + d) * 128);
      q1[d] = ld_w16(wp + (kb_begin + d) * 128 + 16);
    }
  for (int kb0 = kb_begin; kb0 < kb_end; kb0 += kBlDepth) {
#pragma unroll
    for (int d = 0; d < kBlDepth; ++d) {
      const int kb = kb0 + d;
      if (kb < kb_end) {
        const uint4 a0 = q0[d], a1 = q1[d];
        if (kb + kBlDepth < kb_end) {
          q0[d] = ld_w16(wp + (kb + kBlDepth) * 128);
          q1[d] = ld_w16(wp + (kb + kBlDepth) * 128 + 16);
        }
        const uint32_t c[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {                        // MFMA j: bytes 8j..8j+7 of the lane's 32
          uint32_t d0, d1, d2, d3;
          e4m3x4_to_bf16x4(c[2 * j], d0, d1);
          e4m3x4_to_bf16x4(c[2 * j + 1], d2, d3);
          const v8bf a = bf16_operand(d0, d1, d2, d3);
          uint2 bx = make_uint2(0u, 0u);
          if (col_ok) bx = *reinterpret_cast<const uint2*>(lds + ((((kb * 4 + j) * 4 + g) * M + i) << 3));
          uint32_t e0, e1, e2, e3;
          e4m3x4_to_bf16x4(bx.x, e0, e1);
          e4m3x4_to_bf16x4(bx.y, e2, e3);
          acc = mfma_bf16_16x16x32(a, bf16_operand(e0, e1, e2, e3), acc);
        }
      }
    }
  }
  // the partial sums of a row block's waves meet in LDS (over the staged codes, once every
  // wave is done with them): its K-part 0 wave adds parts 1, 2, 3 in order
  v4f* part = reinterpret_cast<v4f*>(lds);
  __syncthreads();
  if (part_k > 0) part[(wave - 1) * kWave + lane] = acc;
  __syncthreads();
  if (part_k > 0 || !col_ok || !rb_ok) return;
#pragma unroll
  for (int v = 1; v < kBlSplit; ++v) {
    const v4f o = part[(wave + v - 1) * kWave + lane];
    acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
  }
  const int n = rb * 16 + 4 * g;
  uint2 o;
  o.x = f32_to_bf16_bits(scale * acc[0]) | f32_to_bf16_bits(scale * acc[1]) << 16;
  o.y = f32_to_bf16_bits(scale * acc[2]) | f32_to_bf16_bits(scale * acc[3]) << 16;
  *reinterpret_cast<uint2*>(y + (size_t)i * N + n) = o;
}

// Up to 64 rows, any K: the same mapping (four waves per 16-row block, one K-quarter each),
// with NT 16-column tiles of rows per weight block, and the B operands (the activation
// codes, M x K bytes, resident in L2) read by each lane straight from global memory, D
// 128-K blocks ahead together with its weights, with no LDS staging and no barrier in the
// k-loop. Staging them in LDS chunk by chunk instead (every workgroup restaging all of x
// behind a barrier per chunk) measured 31.4 us against 21.9 us at 32 rows of the Grok-1
// q|k|v projection. Two blocks ahead measured faster at 8 rows (q|k|v 15.8 -> 15.0 us, o
// 15.0 -> 14.4 us) and slower at 32 (22.2 -> 23.5 us); three, slower at both.
// A tile row past M reads row 0 instead: its products reach only output rows not stored.
template <int RB, int NT, int D>
__global__ __launch_bounds__(RB * kBlSplit * kWave) void fp8_linear_wide_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ w, float scale, int M, int N, int K,
    uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = lane_id(), wave = wave_id();
  const int KB = K >> 7;
  const int per = (KB + kBlSplit - 1) / kBlSplit;
  const int rb = min(blockIdx.x * RB + wave / kBlSplit, N / 16 - 1);
  const bool rb_ok = blockIdx.x * RB + wave / kBlSplit < N / 16;
  const int part_k = wave % kBlSplit;
  const int i = lane & 15, g = lane >> 4;
  const uint8_t* wp = w + (size_t)(rb * 16 + i) * K + g * 32;
  const int kb_begin = min(KB, part_k * per), kb_end = rb_ok ? min(KB, kb_begin + per) : kb_begin;
  const uint8_t* xp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = t * 16 + i;
    xp[t] = xq + (size_t)(m < M ? m : 0) * K + g * 32;
  }
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 q0[D], q1[D], b0[D][NT], b1[D][NT];     // ring: block kb sits in slot (kb - kb_begin) % D
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int kb = kb_begin + d;
    if (kb < kb_end) {
      q0[d] = ld_w16(wp + kb * 128);
      q1[d] = ld_w16(wp + kb * 128 + 16);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        b0[d][t] = *reinterpret_cast<const uint4*>(xp[t] + kb * 128);
        b1[d][t] = *reinterpret_cast<const uint4*>(xp[t] + kb * 128 + 16);
      }
    }
  }
  for (int kb0 = kb_begin; kb0 < kb_end; kb0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kb = kb0 + d;
      if (kb < kb_end) {
        const uint4 a0 = q0[d], a1 = q1[d];
        uint4 c0[NT], c1[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) { c0[t] = b0[d][t]; c1[t] = b1[d][t]; }
        if (kb + D < kb_end) {
          q0[d] = ld_w16(wp + (kb + D) * 128);
          q1[d] = ld_w16(wp + (kb + D) * 128 + 16);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            b0[d][t] = *reinterpret_cast<const uint4*>(xp[t] + (kb + D) * 128);
            b1[d][t] = *reinterpret_cast<const uint4*>(xp[t] + (kb + D) * 128 + 16);
          }
        }
        const uint32_t cw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t d0, d1, d2, d3;
          e4m3x4_to_bf16x4(cw[2 * j], d0, d1);
          e4m3x4_to_bf16x4(cw[2 * j + 1], d2, d3);
          const v8bf a = bf16_operand(d0, d1, d2, d3);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint32_t bw[8] = {c0[t].x, c0[t].y, c0[t].z, c0[t].w, c1[t].x, c1[t].y, c1[t].z, c1[t].w};
            uint32_t e0, e1, e2, e3;
            e4m3x4_to_bf16x4(bw[2 * j], e0, e1);
            e4m3x4_to_bf16x4(bw[2 * j + 1], e2, e3);
            acc[t] = mfma_bf16_16x16x32(a, bf16_operand(e0, e1, e2, e3), acc[t]);
          }
        }
      }
    }
  }
  v4f* part = reinterpret_cast<v4f*>(lds);
  if (part_k > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) part[((wave - 1) * NT + t) * kWave + lane] = acc[t];
  }
  __syncthreads();
  if (part_k > 0 || !rb_ok) return;
  const int n = rb * 16 + 4 * g;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = t * 16 + i;
    v4f a = acc[t];
#pragma unroll
    for (int v = 1; v < kBlSplit; ++v) {
      const v4f o = part[((wave + v - 1) * NT + t) * kWave + lane];
      a[0] += o[0]; a[1] += o[1]; a[2] += o[2]; a[3] += o[3];
    }
    if (m < M) {
      uint2 o;
      o.x = f32_to_bf16_bits(scale * a[0]) | f32_to_bf16_bits(scale * a[1]) << 16;
      o.y = f32_to_bf16_bits(scale * a[2]) | f32_to_bf16_bits(scale * a[3]) << 16;
      *reinterpret_cast<uint2*>(y + (size_t)m * N + n) = o;
    }
  }
}

template <int NT, int D>
static void launch_flw(const uint8_t* xq, const uint8_t* w, float scale, int M, int N, int K, uint16_t* y,
                       hipStream_t st) {
  constexpr int RB = 1;   // one row block per workgroup (2 measured the same, 4 slower)
  const unsigned grid = (unsigned)((N / 16 + RB - 1) / RB);
  const size_t lds = (size_t)(RB * kBlSplit - 1) * NT * kWave * sizeof(v4f);   // the partial sums
  hipLaunchKernelGGL((fp8_linear_wide_kernel<RB, NT, D>), dim3(grid), dim3(RB * kBlSplit * kWave), lds, st, xq, w,
                     scale, M, N, K, y);
}

template <int RB>
static void launch_fl(const uint16_t* x, float s_x, const uint8_t* w, float scale, int M, int N, int K, uint16_t* y,
                      hipStream_t st) {
  const unsigned grid = (unsigned)((N / 16 + RB - 1) / RB);
  const size_t lds = std::max((size_t)M * K, (size_t)(RB * kBlSplit - 1) * kWave * sizeof(v4f));
  hipLaunchKernelGGL((fp8_linear_kernel<RB>), dim3(grid), dim3(RB * kBlSplit * kWave), lds, st, x, s_x, w, scale, M,
                     N, K, y);
}

bool fp8_linear_quant_inside(int M) { return M <= 2; }

// the whole activation in LDS (M <= 16, M * K <= 65536), else the chunked kernel
static bool fp8_linear_whole_x(int M, int K) { return M <= 16 && (int64_t)M * K <= 65536; }

void launch_fp8_linear(const uint16_t* x, float s_x, uint8_t* xq, const uint8_t* w, float scale, int M, int N,
                       int K, uint16_t* y, hipStream_t st) {
  if (fp8_linear_quant_inside(M) && fp8_linear_whole_x(M, K)) {
    launch_fl<W4A8_BL_RB_SMALL_M>(x, s_x, w, scale, M, N, K, y, st);
    return;
  }
  // the codes quantized once into the workspace, then B read from L2 by every lane (for
  // 3..16 rows this measured faster than staging the codes in LDS: 8 rows of q|k|v 19.2 ->
  // 15.7 us, of o 18.3 -> 14.6 us)
  launch_fp8_quant(x, (int64_t)M * K, s_x, xq, st);
  if (M <= 16) launch_flw<1, 2>(xq, w, scale, M, N, K, y, st);
  else if (M <= 32) launch_flw<2, 1>(xq, w, scale, M, N, K, y, st);
  else launch_flw<4, 1>(xq, w, scale, M, N, K, y, st);
}

}  // namespace w4a8
