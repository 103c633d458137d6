// Streaming (decode-shaped) grouped GEMM of the routed experts: few tokens per expert,
// every int4 weight read from HBM exactly once.
//
// The method ("INT4 MoE weights, FP8 compute", page "ROCm: enable trillion-parameter
// MoE models with INT4-FP8 single node"; int4 MoE weights upcast to float8 for fp8
// math, page "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm"): every
// product is an E4M3 activation times an int4 weight code, summed in fp32. The
// per-channel weight scale and the static activation scale are constant along K, so
// they are applied once, in the epilogue.
//
// Which matrix core. gfx950's fp8 MFMA (16x16x128 f8f6f4, and the older 16x16x32 fp8)
// sums each instruction's products with about 14 bits of precision below the largest
// product of the instruction (measured on MI355X: 256 + 127 * 2^-9 comes out as
// 256.234375), while its 16-bit MFMAs return exact fp32 sums for these operands. An
// E4M3 value and an int4 code are both exact in fp16, so this kernel, which is bound
// by HBM and leaves the matrix cores mostly idle, multiplies them on the fp16 MFMA
// (16x16x32) and accumulates exactly as the method states. The tiled prefill kernel,
// bound by the matrix cores, uses the fp8 MFMA.
//
// int4 -> fp16 in registers, 1 VALU op per weight: XOR with 0x8 turns a nibble q into
// q + 8 in [0, 15]; the E4M3 code c in [0, 15] has the value c * 2^-9 (subnormals then
// the first binade), so masking the nibbles into bytes gives exact E4M3 codes of
// (q + 8) * 2^-9, and v_cvt_scalef32_pk_f16_fp8 widens two of them per op to normal
// fp16 values. A third MFMA per 32-K step multiplies the same activations by the
// constant -8 * 2^-9 and removes the offset; the sums are exact in fp32 before that
// subtraction, so only fp32 rounding is left.
//
// Mapping. A workgroup = 8 waves on one expert and one K-slice. The activation rows of
// the expert (at most 64: four 16-column tiles) for a K-chunk are staged in LDS as
// fp16, in the order the MFMA B operand is read (one ds_read_b128 per lane covers 1 KB
// per wave without bank conflicts). Each wave owns two blocks of 16 weight rows (gate
// rows n..n+15 and up rows I+n..I+n+15, or two blocks of down rows) and streams them
// with 16-byte loads, prefetched kDepth k-steps (of 128) ahead; one load instruction of
// a wave covers 64 contiguous bytes of 16 rows.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

constexpr int kDepth = 4;          // k-steps of weights in flight per wave
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// two E4M3 codes (bytes 0,1 or, with HIGH, bytes 2,3) -> two fp16 values, exact
template <bool HIGH>
__device__ __forceinline__ uint32_t cvt2_e4m3_f16(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.0f, HIGH));
}

// One packed word (8 int4 codes, reorder layout) -> 8 fp16 values (q + 8) * 2^-9 in K order.
__device__ __forceinline__ v8h int4x8_to_f16_offset(uint32_t w) {
  const uint32_t y = w ^ 0x88888888u;
  const uint32_t lo = y & 0x0F0F0F0Fu;            // codes of elements 0..3
  const uint32_t hi = (y >> 4) & 0x0F0F0F0Fu;     // codes of elements 4..7
  v4i r = {(int)cvt2_e4m3_f16<false>(lo), (int)cvt2_e4m3_f16<true>(lo),
           (int)cvt2_e4m3_f16<false>(hi), (int)cvt2_e4m3_f16<true>(hi)};
  return __builtin_bit_cast(v8h, r);
}

__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int m) {
  return m == 0 ? q.x : (m == 1 ? q.y : (m == 2 ? q.z : q.w));
}

template <bool GATEUP, int MAXT>
__global__ __launch_bounds__(kDecodeWaves * kWave) void moe_decode_kernel(MoeGemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  int bid = blockIdx.x;
  const int group = bid % p.groups; bid /= p.groups;
  const int slice = bid % p.ksplit;
  const int e = bid / p.ksplit;
  const int seg0 = p.offsets[e];
  const int cnt = p.offsets[e + 1] - seg0;
  if (cnt <= 0) return;                                     // untouched expert: no weight traffic
  const int nt = min((cnt + 15) >> 4, MAXT);
  const int k_begin = slice * p.kslice;
  const int k_end = min(p.K, k_begin + p.kslice);
  const int kc_max = ((p.lds_bytes / (32 * nt)) / 128) * 128;   // fp16 rows of 16*nt tokens

  // weight row blocks of this wave: gate|up -> (cb, n_out/16 + cb); down -> (2cb, 2cb + 1)
  const int cb = group * kDecodeWaves + wave;
  const int blk0 = GATEUP ? cb : 2 * cb;
  const int blk1 = GATEUP ? (p.n_out / 16 + cb) : 2 * cb + 1;
  const bool has_work = blk0 * 16 < (GATEUP ? p.n_out : p.Nw);
  const bool has1 = GATEUP || blk1 * 16 < p.Nw;
  const int i = lane & 15, g = lane >> 4;
  const size_t row_bytes = (size_t)p.K / 2;
  const uint8_t* wbase = reinterpret_cast<const uint8_t*>(p.w) + (size_t)e * p.Nw * row_bytes + g * 16;
  const uint8_t* w0_ptr = wbase + (size_t)(blk0 * 16 + i) * row_bytes;
  const uint8_t* w1_ptr = wbase + (size_t)((has1 ? blk1 : blk0) * 16 + i) * row_bytes;

  v4f acc0[MAXT], acc1[MAXT], corr[MAXT];
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    acc0[j] = v4f{0.f, 0.f, 0.f, 0.f}; acc1[j] = acc0[j]; corr[j] = acc0[j];
  }
  v8h corr_op;
#pragma unroll
  for (int r = 0; r < 8; ++r) corr_op[r] = (_Float16)(-8.0f / 512.0f);

  for (int kc0 = k_begin; kc0 < k_end; kc0 += kc_max) {
    const int klen = min(kc_max, k_end - kc0);
    const int S = klen >> 7;                                // k-steps of 128 in this chunk
    if (kc0 != k_begin) __syncthreads();                    // LDS reuse
    // ---- stage the activation rows of this chunk as fp16. Unit = 8 codes of one row:
    //      (tile j, k-step s, sub-step m, lane c + 16 g) -> 16 bytes at
    //      ((j*S + s)*4 + m)*1024 + lane*16, so MFMA m of k-step s reads one b128 per lane.
    {
      const int R = klen >> 3;                              // 8-code units per row
      const int units = nt * 16 * R;
      for (int u = tid; u < units; u += kDecodeWaves * kWave) {
        const int col = u / R, kk = u - col * R;
        const int j = col >> 4, c = col & 15;
        const int s = kk >> 4, gg = (kk >> 2) & 3, m = kk & 3;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (col < cnt) {
          const int src_row = GATEUP ? (p.sorted_pair[seg0 + col] >> 1) : (seg0 + col);
          const uint2 q = *reinterpret_cast<const uint2*>(p.act + (size_t)src_row * p.K + kc0 + kk * 8);
          v = make_uint4(cvt2_e4m3_f16<false>(q.x), cvt2_e4m3_f16<true>(q.x),
                         cvt2_e4m3_f16<false>(q.y), cvt2_e4m3_f16<true>(q.y));
        }
        *reinterpret_cast<uint4*>(lds + ((j * S + s) * 4 + m) * 1024 + (c + 16 * gg) * 16) = v;
      }
    }
    __syncthreads();
    if (!has_work) continue;
    // ---- stream the weights of this chunk
    const uint8_t* p0 = w0_ptr + kc0 / 2;
    const uint8_t* p1 = w1_ptr + kc0 / 2;
    uint4 q0[kDepth], q1[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (d < S) {
        q0[d] = ld16(p0 + d * 64);
        if (has1) q1[d] = ld16(p1 + d * 64);
      }
    }
    for (int s0 = 0; s0 < S; s0 += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int s = s0 + d;
        if (s < S) {
          const uint4 a0 = q0[d];
          const uint4 a1 = has1 ? q1[d] : a0;
          if (s + kDepth < S) {
            q0[d] = ld16(p0 + (s + kDepth) * 64);
            if (has1) q1[d] = ld16(p1 + (s + kDepth) * 64);
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {                     // 4 MFMAs of K = 32
            const v8h A0 = int4x8_to_f16_offset(word_of(a0, m));
            const v8h A1 = int4x8_to_f16_offset(word_of(a1, m));
#pragma unroll
            for (int j = 0; j < MAXT; ++j) {
              if (j < nt) {
                const v8h b = __builtin_bit_cast(
                    v8h, *reinterpret_cast<const uint4*>(lds + ((j * S + s) * 4 + m) * 1024 + lane * 16));
                acc0[j] = mfma_f16(A0, b, acc0[j]);
                acc1[j] = mfma_f16(A1, b, acc1[j]);
                corr[j] = mfma_f16(corr_op, b, corr[j]);
              }
            }
          }
        }
      }
    }
  }
  if (!has_work) return;

  // ---- epilogue: lane holds rows 4g..4g+3 of each block, column (token row) j*16 + i
  const float* ws = p.w_scale + (size_t)e * p.Nw;
  const float k0 = 512.0f * p.s_act;                        // undo the 2^-9 of the offset codes
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    const int col = j * 16 + i;
    if (j >= nt || col >= cnt) continue;
    const int r = seg0 + col;
    if (GATEUP) {
      const int nb = cb * 16 + 4 * g;
      const float4 sg = *reinterpret_cast<const float4*>(ws + nb);
      const float4 su = *reinterpret_cast<const float4*>(ws + p.n_out + nb);
      float gv[4], uv[4], av[4];
      const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        gv[v] = (acc0[j][v] + corr[j][v]) * k0 * sgv[v];
        uv[v] = (acc1[j][v] + corr[j][v]) * k0 * suv[v];
        av[v] = act_fn(gv[v], p.act_fn) * uv[v] / p.s_a;
      }
      *reinterpret_cast<uint32_t*>(p.a_out + (size_t)r * p.n_out + nb) = pack4_e4m3(av[0], av[1], av[2], av[3]);
      if (p.dbg) {
        float* d = p.dbg + (size_t)r * 2 * p.n_out;
        *reinterpret_cast<float4*>(d + nb) = make_float4(gv[0], gv[1], gv[2], gv[3]);
        *reinterpret_cast<float4*>(d + p.n_out + nb) = make_float4(uv[0], uv[1], uv[2], uv[3]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (b == 1 && !has1) break;
        const int nb = (b == 0 ? blk0 : blk1) * 16 + 4 * g;
        const v4f acc = b == 0 ? acc0[j] : acc1[j];
        const float4 sw = *reinterpret_cast<const float4*>(ws + nb);
        float4 o;
        o.x = (acc[0] + corr[j][0]) * k0 * sw.x;
        o.y = (acc[1] + corr[j][1]) * k0 * sw.y;
        o.z = (acc[2] + corr[j][2]) * k0 * sw.z;
        o.w = (acc[3] + corr[j][3]) * k0 * sw.w;
        *reinterpret_cast<float4*>(p.partial + ((size_t)slice * p.P + r) * p.n_out + nb) = o;
      }
    }
  }
}

bool decode_fits(int T) { return T <= 16 * kDecodeMaxTiles; }

void plan_decode(MoeGemmParams& p, bool gateup) {
  // an expert never holds more rows than there are tokens (its two slots differ)
  const int T = p.P / 2;
  p.max_tiles = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  p.lds_bytes = kDecodeLds;
  const int chans_per_wg = kDecodeWaves * (gateup ? 16 : 32);
  p.groups = (p.n_out + chans_per_wg - 1) / chans_per_wg;
  if (gateup) {
    p.kslice = p.K;                  // the fused epilogue needs the whole reduction
    p.ksplit = 1;
  } else {
    // two LDS chunks per slice when an expert holds up to 16 rows
    p.kslice = std::min(p.K, 2 * ((kDecodeLds / 32) / 128) * 128);
    p.ksplit = (p.K + p.kslice - 1) / p.kslice;
  }
}

template <bool GATEUP>
static void launch_decode_t(const MoeGemmParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)(p.groups * p.ksplit * p.E);
  const dim3 block(kDecodeWaves * kWave);
  if (p.max_tiles <= 1)
    hipLaunchKernelGGL((moe_decode_kernel<GATEUP, 1>), dim3(grid), block, p.lds_bytes, st, p);
  else if (p.max_tiles == 2)
    hipLaunchKernelGGL((moe_decode_kernel<GATEUP, 2>), dim3(grid), block, p.lds_bytes, st, p);
  else
    hipLaunchKernelGGL((moe_decode_kernel<GATEUP, 4>), dim3(grid), block, p.lds_bytes, st, p);
}

void launch_moe_decode(const MoeGemmParams& p, bool gateup, hipStream_t st) {
  if (gateup) launch_decode_t<true>(p, st);
  else launch_decode_t<false>(p, st);
}

// ---------------------------------------------------------------------------- combine
// out[t][n] = w0 * Y0 + w1 * Y1, Y = sum over split-K slices in slice order; fp32, then
// bf16 (nearest even) or fp32. 4 channels per thread; a 1-D grid over (token, chunk).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial, int ksplit, int P, int H,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int chunks,
                                                      int out_bf16, void* __restrict__ out) {
  const int t = blockIdx.x / chunks;
  const int n = ((blockIdx.x % chunks) * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  const int r0 = pair_pos[2 * t], r1 = pair_pos[2 * t + 1];
  const float w0 = topk_w[2 * t], w1 = topk_w[2 * t + 1];
  float4 y0 = make_float4(0.f, 0.f, 0.f, 0.f), y1 = y0;
  for (int s = 0; s < ksplit; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(partial + ((size_t)s * P + r0) * H + n);
    const float4 b = *reinterpret_cast<const float4*>(partial + ((size_t)s * P + r1) * H + n);
    y0.x += a.x; y0.y += a.y; y0.z += a.z; y0.w += a.w;
    y1.x += b.x; y1.y += b.y; y1.z += b.z; y1.w += b.w;
  }
  float4 o;
  o.x = w0 * y0.x + w1 * y1.x;
  o.y = w0 * y0.y + w1 * y1.y;
  o.z = w0 * y0.z + w1 * y1.z;
  o.w = w0 * y0.w + w1 * y1.w;
  if (out_bf16) {
    uint2 v;
    v.x = f32_to_bf16_bits(o.x) | f32_to_bf16_bits(o.y) << 16;
    v.y = f32_to_bf16_bits(o.z) | f32_to_bf16_bits(o.w) << 16;
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + n) = v;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H + n) = o;
  }
}

void launch_combine(const float* partial, int ksplit, int P, int H, const int32_t* pair_pos,
                    const float* topk_w, int T, bool out_bf16, void* out, hipStream_t st) {
  const int chunks = (H / 4 + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((size_t)T * chunks)), dim3(256), 0, st, partial, ksplit, P, H,
                     pair_pos, topk_w, chunks, out_bf16 ? 1 : 0, out);
}

}  // namespace w4a8
