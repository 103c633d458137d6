// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a8 {
// Tiled int4 weight layout read by the MoE GEMMs: per expert, [N/16][K/128] tiles of
// 1 KB, k-steps of one 16-row block consecutive; in tile (nb, ks) the 16 bytes at
// 16 * (i + 16 g) are bytes 64 ks + 16 g .. +16 of row 16 nb + i of the packed matrix.
// One 16-byte load per lane fetches a whole tile, and lane (i, g) then holds
// K = 128 ks + 32 g .. +32 of row i, the order the matrix instructions take.
constexpr int kTileRows = 16, kTileK = 128;
constexpr uint32_t kTileBytes = 1024;

// ---- quant.hip
void launch_w4_pack(const uint16_t* w, int64_t rows, int K, int32_t* packed, float* scale, hipStream_t st);
void launch_w4_tile(const int32_t* packed, int64_t E, int N, int K, int32_t* tiled, hipStream_t st);
void launch_fp8_quant(const uint16_t* x, int64_t n, float s, uint8_t* out, hipStream_t st);
int fp8_quant_blocks(int64_t n);      // 256-thread workgroups of one quantization launch
void launch_fp8_block_quant(const uint16_t* w, int N, int K, uint8_t* q, float* S, hipStream_t st);
// KV cache store: rows of k and v [T][D] to E4M3 with their scales, into rows slots[t]
void launch_kv_cache_store(const uint16_t* k, const uint16_t* v, const int32_t* slots, int T, int D, float s_k,
                           float s_v, uint8_t* k_cache, uint8_t* v_cache, int num_slots, hipStream_t st);
constexpr int kTensorQuantParts = 1024;   // most partial maxima of one fp8_tensor_quant
// two launches: partial maxima into partial[kTensorQuantParts], then scale + codes
void launch_fp8_tensor_quant(const uint16_t* w, int64_t n, uint8_t* q, float* s, uint32_t* partial,
                             hipStream_t st);

// ---- route.hip
size_t route_workspace_bytes(int T, int E);
// with x (T*H bf16, xn elements): also xq = fp8_quant_static(x, s_x), in the same launch
// when the routing is one workgroup
void launch_route_sort(const float* logits, int T, int E, int32_t* ids, float* tw, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws, hipStream_t st,
                       const uint16_t* x = nullptr, int64_t xn = 0, float s_x = 1.0f, uint8_t* xq = nullptr);

// ---- moe_decode.hip / moe_prefill.hip: grouped GEMM of the routed experts
// One description serves both GEMMs:
//   gate|up (gemm1): rows of the activation are tokens gathered through sorted_pair,
//     K = H, weight rows Nw = 2I, output channels n_out = I (gate row n pairs with up
//     row I + n), fused activation + fp8 requant into a_out, optional fp32 dbg.
//   down (gemm2):    rows are the sorted rows themselves, K = I, Nw = n_out = H,
//     fp32 output Y (scaled) into partial[slice][P][H].
struct MoeGemmParams {
  const uint8_t* act;          // E4M3 activation rows, [rows][K]
  const int32_t* w;            // packed int4 [E][Nw][K/8]
  const float* w_scale;        // [E][Nw]
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted_pair;  // [P] (gate|up only)
  int E, K, Nw, n_out, P;
  float s_act;                 // static scale of the activation rows
  // gate|up epilogue
  int act_fn;
  float s_a, inv_s_a;          // inv_s_a = 1 / s_a correctly rounded (host division)
  uint8_t* a_out;              // [P][I]
  float* dbg;                  // [P][2I] or nullptr
  // down epilogue
  float* partial;              // [ksplit][P][H]
  // decode launch shape (set by plan_decode)
  int kslice, ksplit, groups, lds_bytes, max_tiles, waves;
};

#ifndef W4A8_DECODE_WAVES
#define W4A8_DECODE_WAVES 8
#endif
#ifndef W4A8_DECODE_LDS_KB
#define W4A8_DECODE_LDS_KB 64
#endif
constexpr int kDecodeWaves = W4A8_DECODE_WAVES;   // most waves per workgroup of the streaming kernel
constexpr int kDecodeMaxTiles = 2;                // 16-row column tiles per pass (32 rows)
constexpr int kDecodeLds = W4A8_DECODE_LDS_KB * 1024;

bool decode_fits(int T);             // the streaming kernel handles T tokens
int device_cus();                    // CUs of the current device (cached per device, thread-safe)
void plan_decode(MoeGemmParams& p, bool gateup);
void launch_moe_decode(const MoeGemmParams& p, bool gateup, hipStream_t st);

bool prefill_available();
int prefill_token_blocks(int P, int E, bool gateup);   // 16-row token blocks per tile of the tiled kernel
void plan_prefill(MoeGemmParams& p, bool gateup);   // split-K of the tiled down projection
void launch_moe_prefill(const MoeGemmParams& p, bool gateup, hipStream_t st);

// combine: out[t] = w0 * sum_s partial[s][pair_pos[2t]] + w1 * sum_s partial[s][pair_pos[2t+1]]
void launch_combine(const float* partial, int ksplit, int P, int H, const int32_t* pair_pos,
                    const float* topk_w, int T, bool out_bf16, void* out, hipStream_t st);

// ---- block_linear.hip
void launch_fp8_block_linear(const uint16_t* x, const uint8_t* w, const float* s, int M, int N, int K,
                             uint16_t* y, hipStream_t st);
// per-tensor FP8 linear: xq = e4m3(x / s_x), y = bf16(scale * sum_k xq * wq); xq (M * K
// bytes of workspace) is used unless fp8_linear_quant_inside(M), where the kernel quantizes
bool fp8_linear_quant_inside(int M);
void launch_fp8_linear(const uint16_t* x, float s_x, uint8_t* xq, const uint8_t* w, float scale, int M, int N,
                       int K, uint16_t* y, hipStream_t st);

}  // namespace w4a8
