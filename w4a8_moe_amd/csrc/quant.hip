// Load-time and elementwise quantization kernels:
//  * w4_pack: column-wise symmetric int4 quantization + reorder packing into int32
//    (int4_experts {bits 4, sym, group column} and pack_method reorder in the
//    quantization_config of the page "ROCm: enable trillion-parameter MoE models with
//    INT4-FP8 single node"; column-wise INT4 quantization and INT4-into-INT32 packing
//    in the Highlights of "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm").
//  * fp8_quant_static: tensor-wise static E4M3 quantization (same Highlights;
//    activation_scheme static).
//  * fp8_block_quant: 128x128 block-scaled E4M3 weights (FP8_PB_WO layout of the page
//    "qwen4_exp: serve the block-FP8 dense projections natively (+25% decode)").
//  * fp8_kv_cache_store: key and value rows to E4M3 with their static group scales, into
//    cache slots (kv_cache_scheme static, kv_cache_group k_proj / v_proj of the first page).
//  * fp8_tensor_quant: tensor-wise E4M3 weights, one scale max|w| / 448 for the tensor
//    (the dense projections of the first page's quant_method "fp8"; tensor-wise FP8
//    quantization in the Highlights of the second).
// All quotients are formed with the correctly rounded fp32 division (the library is
// built without fast-math), then rounded to nearest even.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

// ---------------------------------------------------------------------------- w4_pack
// One 256-thread workgroup per weight row. Pass 1 reduces max|w| (bf16 magnitudes
// compare as integers), pass 2 re-reads the row (an L2 hit) and writes one int32 per
// 8 elements. Loads are 16 B per lane, stores 4 B per lane, both contiguous per wave.
constexpr int kPackThreads = 256;

__device__ __forceinline__ uint32_t quant_nibble(uint32_t bits, float s) {
  float q = __builtin_rintf(bf16_bits_to_f32(bits) / s);
  q = __builtin_fminf(__builtin_fmaxf(q, -8.0f), 7.0f);
  return (uint32_t)((int)q) & 0xFu;
}

__global__ __launch_bounds__(kPackThreads) void w4_pack_kernel(
    const uint16_t* __restrict__ w, int K, int32_t* __restrict__ packed, float* __restrict__ scale) {
  const size_t row = blockIdx.x;
  const int G = K >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(w + row * (size_t)K);
  uint32_t amax = 0;
  for (int j = threadIdx.x; j < G; j += kPackThreads) {
    uint4 v = src[j];
    uint32_t m = max(max(max(v.x & 0x7FFFu, v.x >> 16 & 0x7FFFu), max(v.y & 0x7FFFu, v.y >> 16 & 0x7FFFu)),
                     max(max(v.z & 0x7FFFu, v.z >> 16 & 0x7FFFu), max(v.w & 0x7FFFu, v.w >> 16 & 0x7FFFu)));
    amax = max(amax, m);
  }
  // workgroup max: wave reduction, then across the 4 waves through LDS
  for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  __shared__ uint32_t red[kPackThreads / kWave];
  if (lane_id() == 0) red[wave_id()] = amax;
  __syncthreads();
  amax = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = bf16_bits_to_f32(amax) / 7.0f;
  if (threadIdx.x == 0) scale[row] = s;
  int32_t* dst = packed + row * (size_t)G;
  for (int j = threadIdx.x; j < G; j += kPackThreads) {
    uint32_t word = 0;
    if (s != 0.0f) {
      uint4 v = src[j];
      // element e of the group: e = 0..7 at bf16 slot e of the 16-byte load
      const uint32_t e0 = v.x & 0xFFFFu, e1 = v.x >> 16, e2 = v.y & 0xFFFFu, e3 = v.y >> 16;
      const uint32_t e4 = v.z & 0xFFFFu, e5 = v.z >> 16, e6 = v.w & 0xFFFFu, e7 = v.w >> 16;
      // reorder layout: byte b = element b (low nibble) | element 4+b (high nibble)
      word = quant_nibble(e0, s) | quant_nibble(e4, s) << 4 |
             quant_nibble(e1, s) << 8 | quant_nibble(e5, s) << 12 |
             quant_nibble(e2, s) << 16 | quant_nibble(e6, s) << 20 |
             quant_nibble(e3, s) << 24 | quant_nibble(e7, s) << 28;
    }
    dst[j] = (int32_t)word;
  }
}

void launch_w4_pack(const uint16_t* w, int64_t rows, int K, int32_t* packed, float* scale, hipStream_t st) {
  // rows <= E * N < 2^31 is checked by the caller
  hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)rows), dim3(kPackThreads), 0, st, w, K, packed, scale);
}

// -------------------------------------------------------------------- w4_tile
// One thread per 16 output bytes: writes are contiguous, each read is 16 bytes of a row.
__global__ __launch_bounds__(256) void w4_tile_kernel(const uint4* __restrict__ src, int64_t units, int N, int K,
                                                      uint4* __restrict__ dst) {
  const int64_t kt = K / kTileK, nb_per_e = N / kTileRows, row_units = K / 32;   // 16-byte units of a row
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < units; u += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(u & 63);
    const int64_t tile = u >> 6;
    const int64_t ks = tile % kt, blk = tile / kt;               // blk = e * N/16 + nb
    const int64_t e = blk / nb_per_e, nb = blk - e * nb_per_e;
    const int64_t row = e * N + nb * kTileRows + (lane & 15);
    dst[u] = src[row * row_units + ks * 4 + (lane >> 4)];
  }
}

void launch_w4_tile(const int32_t* packed, int64_t E, int N, int K, int32_t* tiled, hipStream_t st) {
  const int64_t units = E * N * (int64_t)(K / 32);
  const unsigned grid = (unsigned)std::min<int64_t>((units + 255) / 256, 65536);
  hipLaunchKernelGGL(w4_tile_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<const uint4*>(packed), units, N,
                     K, reinterpret_cast<uint4*>(tiled));
}

// -------------------------------------------------------------------- fp8_quant_static
// 8 elements per thread per iteration (16 B in, 8 B out); a grid-stride loop
// (fp8_quant_span, shared with the routing launch that quantizes x alongside).
__global__ __launch_bounds__(256) void fp8_quant_kernel(const uint16_t* __restrict__ x, int64_t n, float s,
                                                        uint8_t* __restrict__ out) {
  fp8_quant_span(x, n, s, out, blockIdx.x * (int64_t)blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
}

int fp8_quant_blocks(int64_t n) {
  const int64_t blocks = ((n >> 3) + 255) / 256;
  return (int)std::min<int64_t>(std::max<int64_t>(blocks, 1), 8192);
}

void launch_fp8_quant(const uint16_t* x, int64_t n, float s, uint8_t* out, hipStream_t st) {
  hipLaunchKernelGGL(fp8_quant_kernel, dim3((unsigned)fp8_quant_blocks(n)), dim3(256), 0, st, x, n, s, out);
}

// ---------------------------------------------------------------- fp8_block_quant
// One 256-thread workgroup per 128x128 block: thread -> (row = tid / 2, 64-column half).
__global__ __launch_bounds__(256) void fp8_block_quant_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                              uint8_t* __restrict__ q, float* __restrict__ S) {
  const int nb = blockIdx.y, kb = blockIdx.x, KB = gridDim.x;
  const int r = nb * 128 + (threadIdx.x >> 1);
  const int c0 = kb * 128 + (threadIdx.x & 1) * 64;
  const bool row_ok = r < N;
  uint4 v[8];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c0 + 8 * i;
    if (row_ok && c < K) {
      v[i] = *reinterpret_cast<const uint4*>(w + (size_t)r * K + c);
      amax = max(amax, max(max(max(v[i].x & 0x7FFFu, v[i].x >> 16 & 0x7FFFu), max(v[i].y & 0x7FFFu, v[i].y >> 16 & 0x7FFFu)),
                           max(max(v[i].z & 0x7FFFu, v[i].z >> 16 & 0x7FFFu), max(v[i].w & 0x7FFFu, v[i].w >> 16 & 0x7FFFu))));
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  __shared__ uint32_t red[4];
  if (lane_id() == 0) red[wave_id()] = amax;
  __syncthreads();
  amax = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = bf16_bits_to_f32(amax) / 448.0f;
  if (threadIdx.x == 0) S[(size_t)nb * KB + kb] = s;
  if (!row_ok) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c0 + 8 * i;
    if (c >= K) break;
    uint2 o = make_uint2(0, 0);
    if (s != 0.0f) o = make_uint2(quant4_e4m3(v[i].x, v[i].y, s), quant4_e4m3(v[i].z, v[i].w, s));
    *reinterpret_cast<uint2*>(q + (size_t)r * K + c) = o;
  }
}

void launch_fp8_block_quant(const uint16_t* w, int N, int K, uint8_t* q, float* S, hipStream_t st) {
  dim3 grid((K + 127) / 128, (N + 127) / 128);
  hipLaunchKernelGGL(fp8_block_quant_kernel, grid, dim3(256), 0, st, w, N, K, q, S);
}

// ---------------------------------------------------------------- fp8_tensor_quant
// Pass 1: each workgroup reduces max|w| over a grid-stride share of the tensor (bf16
// magnitudes compare as integers) into partial[block]. Pass 2: every workgroup reduces
// the partial maxima (order-independent, so deterministic), forms s = fp32(amax / 448)
// and quantizes its share with fp8_quant_span; workgroup 0 stores s. amax = 0 gives s = 0
// and all-zero codes.
constexpr int kTqThreads = 256;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[kTqThreads / kWave];
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < kTqThreads / kWave; ++w) r = max(r, red[w]);
  return r;
}

__global__ __launch_bounds__(kTqThreads) void tensor_amax_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                                 uint32_t* __restrict__ partial) {
  const int64_t first = blockIdx.x * (int64_t)kTqThreads + threadIdx.x, stride = (int64_t)gridDim.x * kTqThreads;
  const uint4* src = reinterpret_cast<const uint4*>(w);
  uint32_t m = 0;
  for (int64_t i = first; i < (n >> 3); i += stride) {
    const uint4 v = src[i];
    m = max(m, max(max(v.x & 0x7FFFu, v.x >> 16 & 0x7FFFu), max(v.y & 0x7FFFu, v.y >> 16 & 0x7FFFu)));
    m = max(m, max(max(v.z & 0x7FFFu, v.z >> 16 & 0x7FFFu), max(v.w & 0x7FFFu, v.w >> 16 & 0x7FFFu)));
  }
  const int64_t t = (n >> 3) * 8 + first;                   // the n % 8 tail
  if (t < n && first < 8) m = max(m, (uint32_t)w[t] & 0x7FFFu);
  m = block_max_u32(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kTqThreads) void tensor_quant_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                                  const uint32_t* __restrict__ partial, int parts,
                                                                  uint8_t* __restrict__ q, float* __restrict__ s_out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < parts; i += kTqThreads) m = max(m, partial[i]);
  m = block_max_u32(m);
  const float s = bf16_bits_to_f32(m) / 448.0f;             // correctly rounded
  if (blockIdx.x == 0 && threadIdx.x == 0) *s_out = s;
  const int64_t first = blockIdx.x * (int64_t)kTqThreads + threadIdx.x, stride = (int64_t)gridDim.x * kTqThreads;
  if (s > 0.0f) {
    fp8_quant_span(w, n, s, q, first, stride);
  } else {
    for (int64_t i = first; i < (n >> 3); i += stride) reinterpret_cast<uint2*>(q)[i] = make_uint2(0u, 0u);
    const int64_t t = (n >> 3) * 8 + first;
    if (t < n && first < 8) q[t] = 0;
  }
}

int tensor_quant_parts(int64_t n) {
  return (int)std::min<int64_t>(std::max<int64_t>(((n >> 3) + kTqThreads - 1) / kTqThreads, 1), kTensorQuantParts);
}

void launch_fp8_tensor_quant(const uint16_t* w, int64_t n, uint8_t* q, float* s, uint32_t* partial,
                             hipStream_t st) {
  const int parts = tensor_quant_parts(n);
  hipLaunchKernelGGL(tensor_amax_kernel, dim3((unsigned)parts), dim3(kTqThreads), 0, st, w, n, partial);
  hipLaunchKernelGGL(tensor_quant_kernel, dim3((unsigned)parts), dim3(kTqThreads), 0, st, w, n, partial, parts, q,
                     s);
}

// ---------------------------------------------------------------- fp8_kv_cache_store
// Workgroup (token t, group k or v): 8 elements per thread and round, quantized with the
// group's scale (correctly rounded quotient, nearest even, saturated) and written to row
// slots[t] of the group's cache. A slot outside [0, num_slots) stores nothing.
__global__ __launch_bounds__(256) void kv_cache_store_kernel(const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const int32_t* __restrict__ slots, int D, float s_k,
                                                             float s_v, uint8_t* __restrict__ k_cache,
                                                             uint8_t* __restrict__ v_cache, int num_slots) {
  const int t = blockIdx.x;
  const int slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const bool is_v = blockIdx.y == 1;
  const uint4* src = reinterpret_cast<const uint4*>((is_v ? v : k) + (size_t)t * D);
  uint2* dst = reinterpret_cast<uint2*>((is_v ? v_cache : k_cache) + (size_t)slot * D);
  const float s = is_v ? s_v : s_k;
  for (int i = threadIdx.x; i < D / 8; i += blockDim.x) {
    const uint4 q = src[i];
    dst[i] = make_uint2(quant4_e4m3(q.x, q.y, s), quant4_e4m3(q.z, q.w, s));
  }
}

void launch_kv_cache_store(const uint16_t* k, const uint16_t* v, const int32_t* slots, int T, int D, float s_k,
                           float s_v, uint8_t* k_cache, uint8_t* v_cache, int num_slots, hipStream_t st) {
  hipLaunchKernelGGL(kv_cache_store_kernel, dim3((unsigned)T, 2), dim3(std::min(256, std::max(64, D / 8))), 0, st, k,
                     v, slots, D, s_k, s_v, k_cache, v_cache, num_slots);
}

}  // namespace w4a8
