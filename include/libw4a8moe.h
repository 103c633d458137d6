/*
 * libw4a8moe -- W4A8 mixture-of-experts layer and block-FP8 dense linear for AMD
 * MI355X (gfx950), hand-written HIP.
 *
 * The method, as the source pages state it:
 *  - page "ROCm: enable trillion-parameter MoE models with INT4-FP8 single node"
 *    (sglang pull request 4152): "INT4 MoE weights, FP8 compute"; the Grok-1
 *    W4A8KV8 config.json quantization_config: quant_method fp8, int4_experts {bits 4,
 *    sym true, group column}, activation_scheme static, kv_cache_scheme static, export
 *    pack_method reorder, kv_cache_group and min_kv_scale; routing
 *    num_local_experts 8, num_experts_per_tok 2, the router gate left unquantized
 *    (ignored_layers).
 *  - page "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm" (sglang
 *    pull request 7392): experts quantized online to int4; int4 weights upcast to
 *    float8 for fp8 math; "Core Quantization Utilities": tensor-wise FP8
 *    quantization, column-wise INT4 quantization, packing INT4 values into INT32.
 *  - page "qwen4_exp: serve the block-FP8 dense projections natively (+25% decode)"
 *    (FreeToken pull request 392): block-FP8 weight-only projections (FP8_PB_WO),
 *    e4m3 weight [N,K] with one fp32 scale per 128x128 block (weight_scale_inv),
 *    e.g. [16384,2560] with scales [128,20].
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers, 16-byte aligned, row-major, owned by
 *    the caller. The library never allocates, frees or synchronizes, and keeps no
 *    pointer after a call returns. Outputs must not alias inputs.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is
 *    enqueued on it; the call returns without waiting.
 *  - bf16 tensors are uint16_t bit patterns. fp8 tensors are OCP E4M3 ("e4m3fn":
 *    bias 7, subnormals, max 448, no infinities) codes in uint8_t.
 *  - Status: W4A8_OK (0) or a negative code. Argument, shape, alignment and
 *    workspace errors are detected on the host before any HIP call; nothing is
 *    enqueued then. W4A8_ERR_HIP reports a failed launch (hipGetLastError).
 *  - Data preconditions that are NOT checked (the result is undefined if broken):
 *    finite inputs; router logits without NaN; offsets / sorted_pair / pair_pos as
 *    produced by moe_route_sort for the same T and E.
 *  - Workspace: `ws` is caller-owned device scratch of at least
 *    w4a8_workspace_bytes(op, ...) bytes (NULL allowed when that is 0). Its contents
 *    are undefined between calls. Calls that share one workspace must not overlap.
 *  - The sorted order: pair p = 2*t + slot (slot 0 = the higher-weighted expert).
 *    moe_route_sort lists the 2T pairs expert by expert; "sorted row r" is the pair
 *    sorted_pair[r]. Intermediate MoE tensors are indexed by sorted row.
 *  - Calls are deterministic: the same inputs give byte-identical outputs (no
 *    floating-point atomics; all reductions have a fixed order).
 */
#ifndef LIBW4A8MOE_H
#define LIBW4A8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define W4A8_OK               0
#define W4A8_ERR_NULL        -1  /* a required pointer is NULL */
#define W4A8_ERR_SHAPE       -2  /* a size is out of range or breaks a divisibility rule */
#define W4A8_ERR_ALIGN       -3  /* a pointer is not 16-byte aligned */
#define W4A8_ERR_WORKSPACE   -4  /* ws_bytes smaller than w4a8_workspace_bytes(...) */
#define W4A8_ERR_UNSUPPORTED -5  /* a valid but unsupported configuration */
#define W4A8_ERR_ARG         -6  /* a bad enum value or a non-positive / non-finite scale */
#define W4A8_ERR_HIP         -7  /* the HIP runtime reported an error at launch */

/* gated activations of moe_gemm1_w4a8 */
#define W4A8_ACT_SILU       0   /* g / (1 + exp(-g)) (SwiGLU, Mixtral) */
#define W4A8_ACT_GELU_ERF   1   /* g/2 (1 + erf(g / sqrt 2)) (GELU-gated, Grok-1) */
#define W4A8_ACT_GELU_TANH  2   /* g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) */

/* element types */
#define W4A8_DT_F32   0
#define W4A8_DT_BF16  1
#define W4A8_DT_E4M3  2

/* ops of w4a8_workspace_bytes */
#define W4A8_OP_ROUTE_SORT    1   /* args: T, -, -, E */
#define W4A8_OP_GEMM1         2   /* args: T, H, I, E; plus x_dtype via W4A8_OP_GEMM1_BF16 */
#define W4A8_OP_GEMM1_BF16    3   /* gemm1 with a bf16 x (holds the quantized x) */
#define W4A8_OP_GEMM2         4   /* args: T, H, I, E */
#define W4A8_OP_BLOCK_LINEAR  5   /* args: M, N, K, - */
#define W4A8_OP_TENSOR_QUANT  6   /* args: -, -, -, - */
#define W4A8_OP_FP8_LINEAR    7   /* args: M, N, K, - */
#define W4A8_OP_LAYER         8   /* moe_layer_w4a8; args: T, H, I, E */

/* Size limits checked by every MoE call. */
#define W4A8_MAX_EXPERTS 256

/*
 * w4_pack -- column-wise symmetric int4 quantization of expert weights, packed
 * into int32 ("column-wise INT4 quantization" and "packing of INT4 values into
 * INT32", page "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm",
 * Highlights; int4_experts {bits 4, sym, group column}, page "ROCm: enable
 * trillion-parameter MoE models with INT4-FP8 single node", config.json).
 *
 *   w_bf16  [E][N][K] bf16   weights in torch Linear layout [out, in] per expert
 *   packed  [E][N][K/8] int32 (output)
 *   scale   [E][N] fp32       (output)
 * Per row (e, n): s = fp32(max_k |w| / 7) (correctly rounded); q = clamp(
 * round-half-even(fp32(w / s)), -8, 7) (quotient correctly rounded); an all-zero
 * row gives s = 0, q = 0. Packing ("reorder"): in word j of a row, byte b holds
 * element 8j+b in its low nibble and element 8j+4+b in its high nibble, two's
 * complement. Requires E >= 1, N >= 1, K >= 8, K % 8 == 0.
 */
int32_t w4_pack(const uint16_t* w_bf16, int32_t E, int32_t N, int32_t K,
                int32_t* packed, float* scale, void* stream);

/*
 * w4_tile -- the tiled layout the MoE GEMMs read their int4 weights in, made once at load
 * time from w4_pack's output (a byte permutation: values and nibble order unchanged).
 *
 *   packed  [E][N][K/8] int32 from w4_pack (rows of K/2 bytes)
 *   tiled   [E][N/16][K/128][256] int32 (output, the same byte count): per expert, tiles
 *           of 16 rows x 128 K (1 KB), the k-steps of one 16-row block consecutive; in
 *           tile (nb, ks) the 16 bytes at offset 16 * (i + 16 g), 0 <= i < 16, 0 <= g < 4,
 *           are bytes 64 ks + 16 g .. 64 ks + 16 g + 15 of row 16 nb + i of `packed`.
 * One 16-byte load per lane of a 64-lane wave then fetches a whole contiguous tile in the
 * order the matrix instructions take it (row i, K = 128 ks + 32 g .. +32).
 * Requires E >= 1, N % 16 == 0, K % 128 == 0 (N >= 16, K >= 128), E*N < 2^31, both
 * pointers 16-byte aligned, and the two buffers not overlapping (W4A8_ERR_ARG).
 */
int32_t w4_tile(const int32_t* packed, int32_t E, int32_t N, int32_t K, int32_t* tiled, void* stream);

/*
 * fp8_quant_static -- tensor-wise static FP8 quantization ("tensor-wise FP8
 * quantization", Highlights of the page "[AMD][Quantization] Add int4fp8_moe online
 * quantization on ROCm"; activation_scheme static, page "ROCm: enable ...").
 *   x_bf16 [n] bf16; out [n] e4m3 = e4m3(fp32(x / s)) rounded to nearest even,
 *   saturated to +-448. s: the static scale, finite and > 0. n >= 0.
 * Gives exactly the codes moe_gemm1_w4a8 uses for a bf16 x.
 */
int32_t fp8_quant_static(const uint16_t* x_bf16, int64_t n, float s, uint8_t* out, void* stream);

/*
 * moe_route_sort -- top-2 routing on unquantized router logits and the
 * expert-contiguous order of the (token, slot) pairs (num_local_experts /
 * num_experts_per_tok and the unquantized router gate, config.json of the page
 * "ROCm: enable trillion-parameter MoE models with INT4-FP8 single node").
 *
 *   logits      [T][E] fp32
 *   topk_ids    [T][2] int32 (out) slot 0 = the higher logit; equal logits -> lower id
 *   topk_w      [T][2] fp32  (out) softmax over E, top 2, renormalised:
 *                              w0 = 1 / (1 + exp(l1 - l0)), w1 = 1 - w0
 *   counts      [E]    int32 (out) pairs per expert
 *   offsets     [E+1]  int32 (out) exclusive prefix sum of counts, offsets[E] = 2T
 *   sorted_pair [2T]   int32 (out) pair ids expert by expert, increasing within an expert
 *   pair_pos    [2T]   int32 (out) inverse: sorted_pair[pair_pos[p]] == p
 * Requires 2 <= E <= 256, 0 <= T <= 2^22. T == 0 writes offsets (all 0) and counts.
 */
int32_t moe_route_sort(const float* logits, int32_t T, int32_t E,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_pair, int32_t* pair_pos,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_sort_quant -- moe_route_sort and fp8_quant_static of the layer's input in one
 * call: the per-token work that precedes the grouped GEMMs (same passages). Up to 256
 * tokens both run in a single launch (the quantization in extra workgroups beside the
 * routing one); above, the routing kernels and then the quantization.
 *
 *   logits .. pair_pos, ws, ws_bytes  exactly as moe_route_sort
 *   x_bf16  [T][H] bf16;  s_x its static scale (finite, > 0)
 *   x_e4m3  [T][H] (out) the same bytes fp8_quant_static(x_bf16, T*H, s_x) writes
 * Requires what moe_route_sort requires, H >= 1, T*H < 2^31; x_bf16 and x_e4m3 16-byte
 * aligned when T > 0.
 */
int32_t moe_route_sort_quant(const float* logits, int32_t T, int32_t E,
                             int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos,
                             const uint16_t* x_bf16, int32_t H, float s_x, uint8_t* x_e4m3,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gemm1_w4a8 -- gate|up grouped GEMM of the routed experts with int4 weights
 * upcast in registers, products of E4M3 activations and int4 codes with fp32
 * accumulation, fused gated activation and static fp8 requantization ("INT4 MoE weights, FP8 compute",
 * page "ROCm: enable ..."; int4 weights upcast to float8 for fp8 math, page
 * "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm").
 *
 *   x        [T][H]  x_dtype W4A8_DT_BF16 (quantized here with s_x exactly as
 *                    fp8_quant_static does) or W4A8_DT_E4M3 (already quantized codes)
 *   s_x      static scale of x (finite, > 0)
 *   w13      [E][2I/16][H/128][256] int32 from w4_tile (of w4_pack's [E][2I][H/8]):
 *            rows [0,I) gate, rows [I,2I) up
 *   s_w13    [E][2I] fp32 from w4_pack
 *   offsets, sorted_pair from moe_route_sort
 *   act      W4A8_ACT_*;  s_a  static scale of the intermediate (finite, > 0)
 *   a_fp8    [2T][I] e4m3 (out), row r = sorted row r:
 *              h = s_x * s_w13[e][n] * sum_k x_hat[t][k] * q13[e][n][k]   (t = sorted_pair[r]/2)
 *              a_fp8[r][n] = e4m3(fp32(act(h[n]) * h[I+n]) / s_a)
 *   gateup_dbg [2T][2I] fp32 (out, optional, NULL to skip): h per sorted row
 * Accuracy (both kernels of w4a8_moe_kernel): every product x_hat * q is exact (both are
 * exact in fp16; the 16-bit matrix instruction forms them) and the sums are fp32, so h
 * differs from the exact sum by fp32 rounding only (about 1e-7 of its row's largest value).
 * The requantization decision is taken in double precision, from the same h and with the
 * activation's textbook formula, for every value within a relative 1e-5 of an E4M3
 * rounding boundary, and from a fast fp32 activation (relative error about 1e-6) for the
 * others: a code of a_fp8 is then the one that fp32(act(h[n]) * h[I+n]) / s_a, computed
 * exactly from the kernel's h, rounds to.
 * Requires H % 128 == 0, I % 128 == 0, 2 <= E <= 256, 0 <= T <= 2^22, 2T*H < 2^31, I*H < 2^31.
 * Workspace: w4a8_workspace_bytes(x_dtype == BF16 ? W4A8_OP_GEMM1_BF16 : W4A8_OP_GEMM1, T, H, I, E).
 */
int32_t moe_gemm1_w4a8(const void* x, int32_t x_dtype, float s_x,
                       const int32_t* w13, const float* s_w13,
                       const int32_t* offsets, const int32_t* sorted_pair,
                       int32_t T, int32_t H, int32_t I, int32_t E, int32_t act, float s_a,
                       uint8_t* a_fp8, float* gateup_dbg,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gemm2_w4a8 -- down projection of the routed experts (int4 weights upcast in
 * registers, exact products of E4M3 codes and int4 codes, fp32 accumulation) and the
 * deterministic top-2 combine (same passages as moe_gemm1_w4a8).
 *
 *   a_fp8   [2T][I] e4m3 from moe_gemm1_w4a8 (sorted rows);  s_a its static scale
 *   w2      [E][H/16][I/128][256] int32 from w4_tile (of w4_pack's [E][H][I/8]);
 *           s_w2 [E][H] fp32 from w4_pack
 *   offsets, pair_pos from moe_route_sort;  topk_w [T][2] from moe_route_sort
 *   out     [T][H] (out) out_dtype W4A8_DT_BF16 (round to nearest even) or W4A8_DT_F32:
 *             Y[r][n]  = s_a * s_w2[e][n] * sum_j a_hat[r][j] * q2[e][n][j]
 *             out[t][n] = topk_w[t][0] * Y[pair_pos[2t]][n] + topk_w[t][1] * Y[pair_pos[2t+1]][n]
 *           (fp32, slot 0 first; split-K partial sums are added in a fixed order)
 * Requires H % 128 == 0, I % 128 == 0, 2 <= E <= 256, 0 <= T <= 2^22, 2T*H < 2^31, I*H < 2^31.
 * Workspace: w4a8_workspace_bytes(W4A8_OP_GEMM2, T, H, I, E).
 */
int32_t moe_gemm2_w4a8(const uint8_t* a_fp8, float s_a,
                       const int32_t* w2, const float* s_w2,
                       const int32_t* offsets, const int32_t* pair_pos, const float* topk_w,
                       int32_t T, int32_t H, int32_t I, int32_t E,
                       int32_t out_dtype, void* out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gemm2_w4a8_noalloc -- moe_gemm2_w4a8 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without ws / ws_bytes. The split-K partials live in a
 * library-owned device array of moe_gemm2_w4a8_noalloc_max_workspace() bytes (32 MiB), one
 * per GPU, held until the process ends; the call allocates and frees nothing. Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (other streams, other
 * threads) race: serialize them. Its contents are left from the last call; this call
 * writes every value it reads.
 * Returns W4A8_ERR_WORKSPACE when w4a8_workspace_bytes(W4A8_OP_GEMM2, T, H, I, E) exceeds
 * the array (decode batches fit: Grok-1-shaped T = 32 needs 12.6 MB; prefill-sized T does
 * not), W4A8_ERR_HIP if the array's address cannot be obtained, else as moe_gemm2_w4a8.
 */
int32_t moe_gemm2_w4a8_noalloc(const uint8_t* a_fp8, float s_a,
                               const int32_t* w2, const float* s_w2,
                               const int32_t* offsets, const int32_t* pair_pos, const float* topk_w,
                               int32_t T, int32_t H, int32_t I, int32_t E,
                               int32_t out_dtype, void* out, void* stream);
size_t moe_gemm2_w4a8_noalloc_max_workspace(void);

/*
 * moe_layer_w4a8 -- the whole routed-expert layer in one call: moe_route_sort_quant,
 * moe_gemm1_w4a8 and moe_gemm2_w4a8 on the same arguments, with every intermediate in the
 * workspace (the computation of pages "ROCm: enable trillion-parameter MoE models with
 * INT4-FP8 single node", INT4 MoE weights with FP8 compute and top-2 of 8 routing on the
 * unquantized router, and "[AMD][Quantization] Add int4fp8_moe online quantization on
 * ROCm", int4 weights upcast to FP8).
 *
 *   logits [T][E] fp32, x_bf16 [T][H] bf16, s_x, w13 / s_w13, w2 / s_w2, act, s_a,
 *   out_dtype and out as in the three calls; out = the output of moe_gemm2_w4a8 after
 *   those calls, byte for byte (the same launches, in the same order, on the stream).
 * Requires what the three calls require. Workspace: w4a8_workspace_bytes(W4A8_OP_LAYER,
 * T, H, I, E) (routing outputs, x codes, intermediate codes, partial sums).
 */
int32_t moe_layer_w4a8(const float* logits, const uint16_t* x_bf16, float s_x,
                       const int32_t* w13, const float* s_w13,
                       const int32_t* w2, const float* s_w2,
                       int32_t T, int32_t H, int32_t I, int32_t E, int32_t act, float s_a,
                       int32_t out_dtype, void* out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_block_quant -- block-FP8 quantization of a dense bf16 weight (the FP8_PB_WO
 * layout of the page "qwen4_exp: serve the block-FP8 dense projections natively
 * (+25% decode)": e4m3 weight plus one fp32 scale per 128x128 block).
 *   w_bf16 [N][K]; w_e4m3 [N][K] (out); scales [ceil(N/128)][ceil(K/128)] fp32 (out):
 *   S = fp32(max|w in block| / 448), W = e4m3(fp32(w / S)); a zero block: S = 0, W = 0.
 * Requires N >= 1, K >= 1, K % 16 == 0.
 */
int32_t fp8_block_quant(const uint16_t* w_bf16, int32_t N, int32_t K,
                        uint8_t* w_e4m3, float* scales, void* stream);

/*
 * fp8_block_linear -- block-FP8 weight-only decode GEMV/GEMM (same page): x stays bf16,
 *   y[m][n] = bf16( sum_kb S[n/128][kb] * sum_{k in block kb} x[m][k] * W[n][k] )
 *   x_bf16 [M][K], w_e4m3 [N][K], s [ceil(N/128)][K/128] fp32, y_bf16 [M][N] (out).
 * Requires 1 <= M <= 64, N % 16 == 0, K % 128 == 0. Up to 16 rows with M * K * 2 <=
 * 65536 the activations are staged whole in LDS; otherwise in chunks of K.
 * Workspace: w4a8_workspace_bytes(W4A8_OP_BLOCK_LINEAR, M, N, K, 0) (currently 0).
 */
int32_t fp8_block_linear(const uint16_t* x_bf16, const uint8_t* w_e4m3, const float* s,
                         int32_t M, int32_t N, int32_t K, uint16_t* y_bf16,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_tensor_quant -- tensor-wise FP8 quantization of a dense bf16 weight (page "ROCm:
 *   enable trillion-parameter MoE models with INT4-FP8 single node": quant_method "fp8"
 *   for every linear but the router gates and lm_head; page "[AMD][Quantization] Add
 *   int4fp8_moe online quantization on ROCm": tensor-wise FP8 quantization):
 *     s_w = fp32(max|w| / 448) (correctly rounded), w_e4m3 = e4m3(fp32(w / s_w)) (nearest
 *     even, saturating); an all-zero tensor gives s_w = 0 and zero codes.
 *   w_bf16 [n] (n >= 1), w_e4m3 [n] (out), s_w (out, one float in device memory; it is
 *   written by the second of the call's two launches). Deterministic.
 *   Workspace: w4a8_workspace_bytes(W4A8_OP_TENSOR_QUANT, 0, 0, 0, 0) bytes (partial maxima).
 *   Non-finite weights give undefined output.
 */
int32_t fp8_tensor_quant(const uint16_t* w_bf16, int64_t n, uint8_t* w_e4m3, float* s_w,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_linear_w8a8 -- per-tensor static FP8 dense linear for decode rows (the same two
 *   pages; activation_scheme static):
 *   xq = e4m3(fp32(x / s_x)) (the arithmetic of fp8_quant_static; in the linear's own
 *   kernel for M <= 2 with M * K <= 65536, else in a launch of its own into the
 *   workspace), then
 *   y[m][n] = bf16( fp32(s_x * s_w) * sum_k dec(xq[m][k]) * dec(w[n][k]) ), nearest even;
 *   the products are exact and summed in fp32.
 *   x_bf16 [M][K], s_x > 0 (static activation scale, host value), w_e4m3 [N][K] with its
 *   tensor scale s_w >= 0 (host value), y_bf16 [M][N] (out).
 *   Requires 1 <= M <= 64, N % 16 == 0, K % 128 == 0. Up to 2 rows with M * K <= 65536
 *   the kernel quantizes x itself and stages the codes in LDS (one launch); otherwise the
 *   codes are quantized into the workspace first and read from there by the GEMV.
 *   Workspace: w4a8_workspace_bytes(W4A8_OP_FP8_LINEAR, M, N, K, 0) bytes: 0 for M <= 2
 *   with M * K <= 65536 (ws may be NULL), else M * K rounded up to 256 (holds xq).
 */
int32_t fp8_linear_w8a8(const uint16_t* x_bf16, float s_x, const uint8_t* w_e4m3, float s_w,
                        int32_t M, int32_t N, int32_t K, uint16_t* y_bf16,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_kv_cache_store -- the FP8 KV cache with static scales (page "ROCm: enable
 *   trillion-parameter MoE models with INT4-FP8 single node": kv_cache_scheme static,
 *   export kv_cache_group ["*k_proj", "*v_proj"], min_kv_scale 1.0): each token's key and
 *   value rows quantized with their group's static scale, e4m3(fp32(v / s)) (nearest even,
 *   saturating), written to row slots[t] of the group's cache.
 *   k_bf16, v_bf16 [T][D] (D = key/value heads x head dim, D % 8 == 0), slots [T] int32
 *   (a slot outside [0, num_slots) marks a token that is not stored), s_k, s_v > 0 (the
 *   caller applies the min_kv_scale floor), k_cache, v_cache [num_slots][D] E4M3 (in/out:
 *   rows not written keep their bytes). Slots of one call must be distinct.
 *   Workspace: none.
 */
int32_t fp8_kv_cache_store(const uint16_t* k_bf16, const uint16_t* v_bf16, const int32_t* slots,
                           int32_t T, int32_t D, float s_k, float s_v,
                           uint8_t* k_cache, uint8_t* v_cache, int32_t num_slots, void* stream);

/* Workspace size in bytes of one call (0 when none is needed); 0 also for bad args. */
size_t w4a8_workspace_bytes(int32_t op, int32_t T_or_M, int32_t H_or_N, int32_t I_or_K, int32_t E);

/* A static, human-readable description of a status code. */
const char* w4a8_status_str(int32_t status);

/* Which kernel the MoE GEMM calls use for T tokens (T >= 0): W4A8_KERNEL_STREAM, the
 * weight-streaming kernel for few tokens per expert (bound by HBM), or
 * W4A8_KERNEL_TILED, the tiled kernel for many tokens per expert (32-, 64- or 256-row
 * tiles x 256 weight rows, bound by the 16-bit matrix cores). Both take the same exact
 * products, so results of either meet the same accuracy contract. */
#define W4A8_KERNEL_STREAM 0
#define W4A8_KERNEL_TILED  1
int32_t w4a8_moe_kernel(int32_t T);

#ifdef __cplusplus
}
#endif

#endif /* LIBW4A8MOE_H */
