// C-ABI host layer of libw4a8moe: argument validation (before any HIP call), workspace
// sizing, launch planning, and the launches on the caller's stream. See
// include/libw4a8moe.h for the contract of every entry point.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/libw4a8moe.h"
#include "kernels.h"

using namespace w4a8;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int32_t launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

constexpr int64_t kMaxRouteTokens = int64_t(1) << 22;

// Shapes shared by the MoE GEMM calls.
int32_t check_moe_shape(int32_t T, int32_t H, int32_t I, int32_t E) {
  if (T < 0 || T > kMaxRouteTokens) return W4A8_ERR_SHAPE;
  if (E < 2 || E > W4A8_MAX_EXPERTS) return W4A8_ERR_SHAPE;
  if (H <= 0 || I <= 0 || H % 128 != 0 || I % 128 != 0) return W4A8_ERR_SHAPE;
  if ((int64_t)2 * T * H >= (int64_t(1) << 31)) return W4A8_ERR_SHAPE;   // x, partials: 32-bit offsets
  if ((int64_t)E * 2 * I * (H / 8) >= (int64_t(1) << 40)) return W4A8_ERR_SHAPE;
  if ((int64_t)I * H >= (int64_t(1) << 31)) return W4A8_ERR_SHAPE;   // one expert's packed matrix < 2 GiB
  return W4A8_OK;
}

// gemm1 workspace: the quantized x (bf16 input only)
size_t gemm1_ws(int32_t T, int32_t H, bool bf16_x) { return bf16_x ? round_up((size_t)T * H, 256) : 0; }

// gemm2's split-K partials: the same plan the launch uses.
int gemm2_ksplit(int32_t T, int32_t H, int32_t I, int32_t E) {
  MoeGemmParams p{};
  p.E = E; p.K = I; p.Nw = H; p.n_out = H; p.P = 2 * T;
  if (decode_fits(T)) plan_decode(p, false);
  else plan_prefill(p, false);
  return p.ksplit;
}

// gemm2 workspace: the split-K partials of the down projection
size_t gemm2_ws(int32_t T, int32_t H, int32_t I, int32_t E) {
  return round_up((size_t)gemm2_ksplit(T, H, I, E) * 2 * T * H * sizeof(float), 256);
}

// moe_layer_w4a8's workspace: the routing outputs, x codes, intermediate codes and the down
// projection's partial sums, each at a 256-byte boundary.
struct LayerWs {
  size_t ids, tw, counts, offsets, sorted_pair, pair_pos, route, xq, a, partial, total;
};

LayerWs layer_ws(int32_t T, int32_t H, int32_t I, int32_t E) {
  LayerWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes, 256); return at; };
  w.ids = take((size_t)2 * T * sizeof(int32_t));
  w.tw = take((size_t)2 * T * sizeof(float));
  w.counts = take((size_t)E * sizeof(int32_t));
  w.offsets = take((size_t)(E + 1) * sizeof(int32_t));
  w.sorted_pair = take((size_t)2 * T * sizeof(int32_t));
  w.pair_pos = take((size_t)2 * T * sizeof(int32_t));
  w.route = take(route_workspace_bytes(T, E));
  w.xq = take((size_t)T * H);
  w.a = take((size_t)2 * T * I);
  w.partial = take(gemm2_ws(T, H, I, E));
  w.total = o;
  return w;
}

// ---- the allocation-free variant's scratch: the down projection's split-K partials in a
// file-scope device array, one copy per GPU for the life of the process. Its address on
// each device comes from hipGetSymbolAddress, taken once per device with that device
// current; host code uses only that address (the array's own name is a host-side stand-in).
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The scratch array's device address on the current device, or nullptr on a HIP error.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* w4a8_status_str(int32_t status) {
  switch (status) {
    case W4A8_OK: return "ok";
    case W4A8_ERR_NULL: return "a required pointer is NULL";
    case W4A8_ERR_SHAPE: return "a size is out of range or breaks a divisibility rule";
    case W4A8_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case W4A8_ERR_WORKSPACE: return "workspace too small";
    case W4A8_ERR_UNSUPPORTED: return "unsupported configuration";
    case W4A8_ERR_ARG: return "bad enum value or scale";
    case W4A8_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int32_t w4a8_moe_kernel(int32_t T) { return decode_fits(T) ? W4A8_KERNEL_STREAM : W4A8_KERNEL_TILED; }

size_t w4a8_workspace_bytes(int32_t op, int32_t T_or_M, int32_t H_or_N, int32_t I_or_K, int32_t E) {
  switch (op) {
    case W4A8_OP_ROUTE_SORT:
      if (T_or_M < 0 || T_or_M > kMaxRouteTokens || E < 2 || E > W4A8_MAX_EXPERTS) return 0;
      return round_up(route_workspace_bytes(T_or_M, E), 256);
    case W4A8_OP_GEMM1:
    case W4A8_OP_GEMM1_BF16:
      if (check_moe_shape(T_or_M, H_or_N, I_or_K, E) != W4A8_OK) return 0;
      return gemm1_ws(T_or_M, H_or_N, op == W4A8_OP_GEMM1_BF16);
    case W4A8_OP_GEMM2:
      if (check_moe_shape(T_or_M, H_or_N, I_or_K, E) != W4A8_OK) return 0;
      return gemm2_ws(T_or_M, H_or_N, I_or_K, E);
    case W4A8_OP_LAYER:
      if (check_moe_shape(T_or_M, H_or_N, I_or_K, E) != W4A8_OK) return 0;
      return T_or_M == 0 ? 0 : layer_ws(T_or_M, H_or_N, I_or_K, E).total;
    case W4A8_OP_BLOCK_LINEAR:
      return 0;
    case W4A8_OP_TENSOR_QUANT:
      return (size_t)kTensorQuantParts * sizeof(uint32_t);
    case W4A8_OP_FP8_LINEAR:
      if (T_or_M < 1 || I_or_K < 1) return 0;
      if (fp8_linear_quant_inside(T_or_M) && (int64_t)T_or_M * I_or_K <= 65536) return 0;
      return round_up((size_t)T_or_M * (size_t)I_or_K, 256);   // the activation codes
    default:
      return 0;
  }
}

int32_t w4_pack(const uint16_t* w_bf16, int32_t E, int32_t N, int32_t K, int32_t* packed, float* scale,
                void* stream) {
  if (!w_bf16 || !packed || !scale) return W4A8_ERR_NULL;
  if (E < 1 || N < 1 || K < 8 || K % 8 != 0) return W4A8_ERR_SHAPE;
  if ((int64_t)E * N >= (int64_t(1) << 31)) return W4A8_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(packed) || !aligned16(scale)) return W4A8_ERR_ALIGN;
  launch_w4_pack(w_bf16, (int64_t)E * N, K, packed, scale, as_stream(stream));
  return launch_status();
}

int32_t w4_tile(const int32_t* packed, int32_t E, int32_t N, int32_t K, int32_t* tiled, void* stream) {
  if (!packed || !tiled) return W4A8_ERR_NULL;
  if (E < 1 || N < kTileRows || K < kTileK || N % kTileRows != 0 || K % kTileK != 0) return W4A8_ERR_SHAPE;
  if ((int64_t)E * N >= (int64_t(1) << 31)) return W4A8_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(tiled)) return W4A8_ERR_ALIGN;
  const uint64_t bytes = (uint64_t)E * N * (uint64_t)(K / 2);
  const uint64_t a = reinterpret_cast<uint64_t>(packed), b = reinterpret_cast<uint64_t>(tiled);
  if (a < b + bytes && b < a + bytes) return W4A8_ERR_ARG;         // the two must not overlap
  launch_w4_tile(packed, E, N, K, tiled, as_stream(stream));
  return launch_status();
}

int32_t fp8_quant_static(const uint16_t* x_bf16, int64_t n, float s, uint8_t* out, void* stream) {
  if (n < 0) return W4A8_ERR_SHAPE;
  if (!good_scale(s)) return W4A8_ERR_ARG;
  if (n == 0) return W4A8_OK;
  if (!x_bf16 || !out) return W4A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(out)) return W4A8_ERR_ALIGN;
  launch_fp8_quant(x_bf16, n, s, out, as_stream(stream));
  return launch_status();
}

int32_t moe_route_sort(const float* logits, int32_t T, int32_t E, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws,
                       size_t ws_bytes, void* stream) {
  if (T < 0 || T > kMaxRouteTokens || E < 2 || E > W4A8_MAX_EXPERTS) return W4A8_ERR_SHAPE;
  if (!counts || !offsets) return W4A8_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_pair || !pair_pos)) return W4A8_ERR_NULL;
  if (!aligned16(counts) || !aligned16(offsets)) return W4A8_ERR_ALIGN;
  if (T > 0 && (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(sorted_pair) ||
                !aligned16(pair_pos)))
    return W4A8_ERR_ALIGN;
  const size_t need = w4a8_workspace_bytes(W4A8_OP_ROUTE_SORT, T, 0, 0, E);
  if (ws_bytes < need) return W4A8_ERR_WORKSPACE;
  if (need > 0 && !ws) return W4A8_ERR_NULL;
  if (need > 0 && !aligned16(ws)) return W4A8_ERR_ALIGN;
  launch_route_sort(logits, T, E, topk_ids, topk_w, counts, offsets, sorted_pair, pair_pos, ws,
                    as_stream(stream));
  return launch_status();
}

int32_t moe_route_sort_quant(const float* logits, int32_t T, int32_t E, int32_t* topk_ids, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                             const uint16_t* x_bf16, int32_t H, float s_x, uint8_t* x_e4m3, void* ws,
                             size_t ws_bytes, void* stream) {
  if (T < 0 || T > kMaxRouteTokens || E < 2 || E > W4A8_MAX_EXPERTS || H < 1) return W4A8_ERR_SHAPE;
  if ((int64_t)T * H >= (int64_t(1) << 31)) return W4A8_ERR_SHAPE;
  if (!good_scale(s_x)) return W4A8_ERR_ARG;
  if (!counts || !offsets) return W4A8_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_pair || !pair_pos || !x_bf16 || !x_e4m3))
    return W4A8_ERR_NULL;
  if (!aligned16(counts) || !aligned16(offsets)) return W4A8_ERR_ALIGN;
  if (T > 0 && (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(sorted_pair) ||
                !aligned16(pair_pos) || !aligned16(x_bf16) || !aligned16(x_e4m3)))
    return W4A8_ERR_ALIGN;
  const size_t need = w4a8_workspace_bytes(W4A8_OP_ROUTE_SORT, T, 0, 0, E);
  if (ws_bytes < need) return W4A8_ERR_WORKSPACE;
  if (need > 0 && !ws) return W4A8_ERR_NULL;
  if (need > 0 && !aligned16(ws)) return W4A8_ERR_ALIGN;
  launch_route_sort(logits, T, E, topk_ids, topk_w, counts, offsets, sorted_pair, pair_pos, ws, as_stream(stream),
                    T > 0 ? x_bf16 : nullptr, (int64_t)T * H, s_x, x_e4m3);
  return launch_status();
}

int32_t moe_gemm1_w4a8(const void* x, int32_t x_dtype, float s_x, const int32_t* w13, const float* s_w13,
                       const int32_t* offsets, const int32_t* sorted_pair, int32_t T, int32_t H, int32_t I,
                       int32_t E, int32_t act, float s_a, uint8_t* a_fp8, float* gateup_dbg, void* ws,
                       size_t ws_bytes, void* stream) {
  int32_t st = check_moe_shape(T, H, I, E);
  if (st != W4A8_OK) return st;
  if (x_dtype != W4A8_DT_BF16 && x_dtype != W4A8_DT_E4M3) return W4A8_ERR_ARG;
  if (act != W4A8_ACT_SILU && act != W4A8_ACT_GELU_ERF && act != W4A8_ACT_GELU_TANH) return W4A8_ERR_ARG;
  if (!good_scale(s_x) || !good_scale(s_a)) return W4A8_ERR_ARG;
  if (T == 0) return W4A8_OK;
  if (!x || !w13 || !s_w13 || !offsets || !sorted_pair || !a_fp8) return W4A8_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(s_w13) || !aligned16(offsets) || !aligned16(sorted_pair) ||
      !aligned16(a_fp8) || (gateup_dbg && !aligned16(gateup_dbg)))
    return W4A8_ERR_ALIGN;
  const bool bf16_x = x_dtype == W4A8_DT_BF16;
  const size_t need = gemm1_ws(T, H, bf16_x);
  if (ws_bytes < need) return W4A8_ERR_WORKSPACE;
  if (need > 0 && !ws) return W4A8_ERR_NULL;
  if (need > 0 && !aligned16(ws)) return W4A8_ERR_ALIGN;
  const bool decode = decode_fits(T);
  if (!decode && !prefill_available()) return W4A8_ERR_UNSUPPORTED;

  hipStream_t s = as_stream(stream);
  const uint8_t* xq = static_cast<const uint8_t*>(x);
  if (bf16_x) {
    launch_fp8_quant(static_cast<const uint16_t*>(x), (int64_t)T * H, s_x, static_cast<uint8_t*>(ws), s);
    xq = static_cast<const uint8_t*>(ws);
  }
  MoeGemmParams p{};
  p.act = xq; p.w = w13; p.w_scale = s_w13; p.offsets = offsets; p.sorted_pair = sorted_pair;
  p.E = E; p.K = H; p.Nw = 2 * I; p.n_out = I; p.P = 2 * T;
  p.s_act = s_x; p.act_fn = act; p.s_a = s_a; p.inv_s_a = 1.0f / s_a; p.a_out = a_fp8; p.dbg = gateup_dbg;
  if (decode) {
    plan_decode(p, true);
    launch_moe_decode(p, true, s);
  } else {
    plan_prefill(p, true);
    launch_moe_prefill(p, true, s);
  }
  return launch_status();
}

int32_t moe_gemm2_w4a8(const uint8_t* a_fp8, float s_a, const int32_t* w2, const float* s_w2,
                       const int32_t* offsets, const int32_t* pair_pos, const float* topk_w, int32_t T,
                       int32_t H, int32_t I, int32_t E, int32_t out_dtype, void* out, void* ws, size_t ws_bytes,
                       void* stream) {
  int32_t st = check_moe_shape(T, H, I, E);
  if (st != W4A8_OK) return st;
  if (out_dtype != W4A8_DT_BF16 && out_dtype != W4A8_DT_F32) return W4A8_ERR_ARG;
  if (!good_scale(s_a)) return W4A8_ERR_ARG;
  if (T == 0) return W4A8_OK;
  if (!a_fp8 || !w2 || !s_w2 || !offsets || !pair_pos || !topk_w || !out) return W4A8_ERR_NULL;
  if (!aligned16(a_fp8) || !aligned16(w2) || !aligned16(s_w2) || !aligned16(offsets) || !aligned16(pair_pos) ||
      !aligned16(topk_w) || !aligned16(out))
    return W4A8_ERR_ALIGN;
  const size_t need = gemm2_ws(T, H, I, E);
  if (ws_bytes < need) return W4A8_ERR_WORKSPACE;
  if (!ws) return W4A8_ERR_NULL;
  if (!aligned16(ws)) return W4A8_ERR_ALIGN;
  const bool decode = decode_fits(T);
  if (!decode && !prefill_available()) return W4A8_ERR_UNSUPPORTED;

  hipStream_t s = as_stream(stream);
  MoeGemmParams p{};
  p.act = a_fp8; p.w = w2; p.w_scale = s_w2; p.offsets = offsets; p.sorted_pair = nullptr;
  p.E = E; p.K = I; p.Nw = H; p.n_out = H; p.P = 2 * T;
  p.s_act = s_a; p.partial = static_cast<float*>(ws);
  int ksplit = 1;
  if (decode) {
    plan_decode(p, false);
    ksplit = p.ksplit;
    launch_moe_decode(p, false, s);
  } else {
    plan_prefill(p, false);
    ksplit = p.ksplit;
    launch_moe_prefill(p, false, s);
  }
  if (launch_status() != W4A8_OK) return W4A8_ERR_HIP;
  launch_combine(p.partial, ksplit, 2 * T, H, pair_pos, topk_w, T, out_dtype == W4A8_DT_BF16, out, s);
  return launch_status();
}

int32_t moe_gemm2_w4a8_noalloc(const uint8_t* a_fp8, float s_a, const int32_t* w2, const float* s_w2,
                               const int32_t* offsets, const int32_t* pair_pos, const float* topk_w, int32_t T,
                               int32_t H, int32_t I, int32_t E, int32_t out_dtype, void* out, void* stream) {
  int32_t st = check_moe_shape(T, H, I, E);
  if (st != W4A8_OK) return st;
  if (out_dtype != W4A8_DT_BF16 && out_dtype != W4A8_DT_F32) return W4A8_ERR_ARG;
  if (!good_scale(s_a)) return W4A8_ERR_ARG;
  if (T == 0) return W4A8_OK;
  if (!a_fp8 || !w2 || !s_w2 || !offsets || !pair_pos || !topk_w || !out) return W4A8_ERR_NULL;
  if (!aligned16(a_fp8) || !aligned16(w2) || !aligned16(s_w2) || !aligned16(offsets) || !aligned16(pair_pos) ||
      !aligned16(topk_w) || !aligned16(out))
    return W4A8_ERR_ALIGN;
  if (gemm2_ws(T, H, I, E) > kScratchBytes) return W4A8_ERR_WORKSPACE;
  void* ws = scratch_address();                            // the first HIP call
  if (ws == nullptr) return W4A8_ERR_HIP;
  return moe_gemm2_w4a8(a_fp8, s_a, w2, s_w2, offsets, pair_pos, topk_w, T, H, I, E, out_dtype, out, ws,
                        kScratchBytes, stream);
}

size_t moe_gemm2_w4a8_noalloc_max_workspace(void) { return kScratchBytes; }

int32_t moe_layer_w4a8(const float* logits, const uint16_t* x_bf16, float s_x, const int32_t* w13,
                       const float* s_w13, const int32_t* w2, const float* s_w2, int32_t T, int32_t H, int32_t I,
                       int32_t E, int32_t act, float s_a, int32_t out_dtype, void* out, void* ws, size_t ws_bytes,
                       void* stream) {
  int32_t st = check_moe_shape(T, H, I, E);
  if (st != W4A8_OK) return st;
  if (act != W4A8_ACT_SILU && act != W4A8_ACT_GELU_ERF && act != W4A8_ACT_GELU_TANH) return W4A8_ERR_ARG;
  if (out_dtype != W4A8_DT_BF16 && out_dtype != W4A8_DT_F32) return W4A8_ERR_ARG;
  if (!good_scale(s_x) || !good_scale(s_a)) return W4A8_ERR_ARG;
  if (T == 0) return W4A8_OK;
  if (!logits || !x_bf16 || !w13 || !s_w13 || !w2 || !s_w2 || !out || !ws) return W4A8_ERR_NULL;
  if (!aligned16(logits) || !aligned16(x_bf16) || !aligned16(w13) || !aligned16(s_w13) || !aligned16(w2) ||
      !aligned16(s_w2) || !aligned16(out) || !aligned16(ws))
    return W4A8_ERR_ALIGN;
  const LayerWs w = layer_ws(T, H, I, E);
  if (ws_bytes < w.total) return W4A8_ERR_WORKSPACE;
  const bool decode = decode_fits(T);
  if (!decode && !prefill_available()) return W4A8_ERR_UNSUPPORTED;

  hipStream_t s = as_stream(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* ids = reinterpret_cast<int32_t*>(base + w.ids);
  float* tw = reinterpret_cast<float*>(base + w.tw);
  int32_t* counts = reinterpret_cast<int32_t*>(base + w.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + w.offsets);
  int32_t* sorted_pair = reinterpret_cast<int32_t*>(base + w.sorted_pair);
  int32_t* pair_pos = reinterpret_cast<int32_t*>(base + w.pair_pos);
  uint8_t* xq = base + w.xq;
  uint8_t* a = base + w.a;
  float* partial = reinterpret_cast<float*>(base + w.partial);
  launch_route_sort(logits, T, E, ids, tw, counts, offsets, sorted_pair, pair_pos, base + w.route, s, x_bf16,
                    (int64_t)T * H, s_x, xq);
  if (launch_status() != W4A8_OK) return W4A8_ERR_HIP;

  MoeGemmParams g{};
  g.act = xq; g.w = w13; g.w_scale = s_w13; g.offsets = offsets; g.sorted_pair = sorted_pair;
  g.E = E; g.K = H; g.Nw = 2 * I; g.n_out = I; g.P = 2 * T;
  g.s_act = s_x; g.act_fn = act; g.s_a = s_a; g.inv_s_a = 1.0f / s_a; g.a_out = a; g.dbg = nullptr;
  MoeGemmParams d{};
  d.act = a; d.w = w2; d.w_scale = s_w2; d.offsets = offsets; d.sorted_pair = nullptr;
  d.E = E; d.K = I; d.Nw = H; d.n_out = H; d.P = 2 * T;
  d.s_act = s_a; d.partial = partial;
  if (decode) {
    plan_decode(g, true);
    launch_moe_decode(g, true, s);
    if (launch_status() != W4A8_OK) return W4A8_ERR_HIP;
    plan_decode(d, false);
    launch_moe_decode(d, false, s);
  } else {
    plan_prefill(g, true);
    launch_moe_prefill(g, true, s);
    if (launch_status() != W4A8_OK) return W4A8_ERR_HIP;
    plan_prefill(d, false);
    launch_moe_prefill(d, false, s);
  }
  if (launch_status() != W4A8_OK) return W4A8_ERR_HIP;
  launch_combine(partial, d.ksplit, 2 * T, H, pair_pos, tw, T, out_dtype == W4A8_DT_BF16, out, s);
  return launch_status();
}

int32_t fp8_block_quant(const uint16_t* w_bf16, int32_t N, int32_t K, uint8_t* w_e4m3, float* scales,
                        void* stream) {
  if (!w_bf16 || !w_e4m3 || !scales) return W4A8_ERR_NULL;
  if (N < 1 || K < 16 || K % 16 != 0 || (int64_t)N * K >= (int64_t(1) << 40)) return W4A8_ERR_SHAPE;
  if ((N + 127) / 128 > 65535) return W4A8_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(w_e4m3) || !aligned16(scales)) return W4A8_ERR_ALIGN;
  launch_fp8_block_quant(w_bf16, N, K, w_e4m3, scales, as_stream(stream));
  return launch_status();
}

int32_t fp8_block_linear(const uint16_t* x_bf16, const uint8_t* w_e4m3, const float* s, int32_t M, int32_t N,
                         int32_t K, uint16_t* y_bf16, void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  if (!x_bf16 || !w_e4m3 || !s || !y_bf16) return W4A8_ERR_NULL;
  if (M < 1 || M > 64 || N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0) return W4A8_ERR_SHAPE;
  if ((int64_t)N * K >= (int64_t(1) << 40) || (int64_t)M * K >= (int64_t(1) << 30)) return W4A8_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(w_e4m3) || !aligned16(s) || !aligned16(y_bf16)) return W4A8_ERR_ALIGN;
  launch_fp8_block_linear(x_bf16, w_e4m3, s, M, N, K, y_bf16, as_stream(stream));
  return launch_status();
}

int32_t fp8_tensor_quant(const uint16_t* w_bf16, int64_t n, uint8_t* w_e4m3, float* s_w, void* ws, size_t ws_bytes,
                         void* stream) {
  if (n < 1 || n >= (int64_t(1) << 40)) return W4A8_ERR_SHAPE;
  if (!w_bf16 || !w_e4m3 || !s_w || !ws) return W4A8_ERR_NULL;
  if (!aligned16(w_bf16) || !aligned16(w_e4m3) || !aligned16(ws)) return W4A8_ERR_ALIGN;
  if (ws_bytes < w4a8_workspace_bytes(W4A8_OP_TENSOR_QUANT, 0, 0, 0, 0)) return W4A8_ERR_WORKSPACE;
  launch_fp8_tensor_quant(w_bf16, n, w_e4m3, s_w, static_cast<uint32_t*>(ws), as_stream(stream));
  return launch_status();
}

int32_t fp8_linear_w8a8(const uint16_t* x_bf16, float s_x, const uint8_t* w_e4m3, float s_w, int32_t M, int32_t N,
                        int32_t K, uint16_t* y_bf16, void* ws, size_t ws_bytes, void* stream) {
  if (!x_bf16 || !w_e4m3 || !y_bf16) return W4A8_ERR_NULL;
  if (M < 1 || M > 64 || N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0) return W4A8_ERR_SHAPE;
  if ((int64_t)N * K >= (int64_t(1) << 40) || (int64_t)M * K >= (int64_t(1) << 31)) return W4A8_ERR_SHAPE;
  if (!good_scale(s_x) || !std::isfinite(s_w) || s_w < 0.0f) return W4A8_ERR_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_e4m3) || !aligned16(y_bf16)) return W4A8_ERR_ALIGN;
  const size_t need = w4a8_workspace_bytes(W4A8_OP_FP8_LINEAR, M, N, K, 0);
  if (need > 0) {
    if (!ws) return W4A8_ERR_NULL;
    if (!aligned16(ws)) return W4A8_ERR_ALIGN;
    if (ws_bytes < need) return W4A8_ERR_WORKSPACE;
  }
  launch_fp8_linear(x_bf16, s_x, static_cast<uint8_t*>(ws), w_e4m3, s_x * s_w, M, N, K, y_bf16, as_stream(stream));
  return launch_status();
}

int32_t fp8_kv_cache_store(const uint16_t* k_bf16, const uint16_t* v_bf16, const int32_t* slots, int32_t T,
                           int32_t D, float s_k, float s_v, uint8_t* k_cache, uint8_t* v_cache, int32_t num_slots,
                           void* stream) {
  if (T < 0 || D < 8 || D % 8 != 0 || num_slots < 1 || (int64_t)num_slots * D >= (int64_t(1) << 40))
    return W4A8_ERR_SHAPE;
  if ((int64_t)T * D >= (int64_t(1) << 40)) return W4A8_ERR_SHAPE;
  if (!good_scale(s_k) || !good_scale(s_v)) return W4A8_ERR_ARG;
  if (T == 0) return W4A8_OK;
  if (!k_bf16 || !v_bf16 || !slots || !k_cache || !v_cache) return W4A8_ERR_NULL;
  if (!aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(slots) || !aligned16(k_cache) || !aligned16(v_cache))
    return W4A8_ERR_ALIGN;
  launch_kv_cache_store(k_bf16, v_bf16, slots, T, D, s_k, s_v, k_cache, v_cache, num_slots, as_stream(stream));
  return launch_status();
}

}  // extern "C"
