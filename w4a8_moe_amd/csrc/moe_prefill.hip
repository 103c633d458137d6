// Tiled (prefill-shaped) grouped GEMM of the routed experts: many tokens per expert,
// bound by the matrix cores.
//
// The method ("INT4 MoE weights, FP8 compute", page "ROCm: enable trillion-parameter
// MoE models with INT4-FP8 single node"; int4 weights upcast to float8 for fp8 math,
// page "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm"): int4 codes are
// turned into exact E4M3 codes and multiplied against the E4M3 activations on the fp8
// MFMA (16x16x128), accumulating in fp32; the per-channel and static scales are applied
// in the epilogue.
//
// Tile. A workgroup computes 256 sorted rows (tokens of one expert) x 256 weight rows,
// K in steps of 128, with 4 waves of 128 x 128 each. For gate|up the 256 weight rows are
// 128 gate channels and the 128 matching up channels, and each wave holds 64 of each, so
// act(gate) * up is formed in registers. Per k-step the workgroup
//  * loads the token tile (256 x 128 E4M3 codes, gathered through sorted_pair for
//    gate|up) and the weight tile (256 x 64 bytes of int4),
//  * converts every weight code once to E4M3 (v_perm table lookup, exact for all 16
//    two's-complement codes) and stores both tiles in LDS in MFMA operand order
//    (lane l reads 16 contiguous bytes, 1 KB per wave instruction),
//  * and runs 64 MFMAs per wave.
// The next k-step's global loads are issued before the MFMAs of the current one.
// Accumulation note: gfx950's fp8 MFMA keeps about 14 bits below the largest product of
// an instruction, so results differ from exact fp32 sums by about 1e-5 of the row scale.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

constexpr int kPM = 256;          // sorted rows per tile
constexpr int kPN = 256;          // weight rows per tile
constexpr int kPThreads = 256;    // 4 waves, 2 x 2 of 128 x 128
constexpr int kPTileBytes = 16 * 2048;                    // 16 blocks of 16 rows x 128 codes
constexpr int kPLds = 2 * kPTileBytes;                     // tokens, then weights
constexpr int kGroupM = 8;        // M-tiles per band of the tile order
constexpr uint32_t kPOutOfRange = 0x80000000u;   // past every buffer (all are < 2^31 bytes)

__device__ __forceinline__ uint4 pf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Four two's-complement nibbles (bits 0..3 of each byte, other bits zero) -> four exact
// E4M3 codes: 0..7 -> 00 38 40 44 48 4A 4C 4E, -8..-1 -> D0 CE CC CA C8 C4 C0 B8.
__device__ __forceinline__ uint32_t nib4_to_e4m3(uint32_t x) {
  const uint32_t sel = x & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, sel);
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, sel);
  // selector 12 reads as 0x00, 13 as 0xFF: a byte mask of the sign bits
  const uint32_t msk = __builtin_amdgcn_perm(0u, 0u, ((x >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  return (msk & neg) | (~msk & pos);
}

struct TileOrigin {
  int e, seg0, cnt, m0;   // expert, its first sorted row, its row count, tile's first row in it
};

// Linear M-tile index -> (expert, first row). Returns false past the last tile.
__device__ __forceinline__ bool locate_mtile(const int32_t* __restrict__ offsets, int E, int mt, TileOrigin& o) {
  int before = 0;
  for (int e = 0; e < E; ++e) {
    const int s0 = offsets[e], c = offsets[e + 1] - s0;
    const int nt = (c + kPM - 1) / kPM;
    if (mt < before + nt) {
      o.e = e; o.seg0 = s0; o.cnt = c; o.m0 = (mt - before) * kPM;
      return true;
    }
    before += nt;
  }
  return false;
}

template <bool GATEUP>
__global__ __launch_bounds__(kPThreads, 1) void moe_prefill_kernel(MoeGemmParams p, int mtiles_upper, int ntiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* ldsT = lds;
  uint8_t* ldsW = lds + kPTileBytes;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int wm = wave & 1, wn = wave >> 1;
  // Tile order. Workgroups are dispatched round-robin over the 8 XCDs, so workgroup b runs
  // on XCD b % 8; each XCD gets a contiguous run of the tile order, and the order walks
  // bands of kGroupM M-tiles, all N-tiles of a band before the next band. The workgroups
  // resident on one XCD then share a few token tiles and a few weight tiles in its L2.
  const int nblk = gridDim.x, b = blockIdx.x;
  const int q = nblk / 8, rr = nblk % 8, xcd = b % 8;
  const int t = (xcd < rr ? xcd * (q + 1) : rr * (q + 1) + (xcd - rr) * q) + b / 8;
  const int span = kGroupM * ntiles, band = t / span, rem = t % span;
  const int gm = min(kGroupM, mtiles_upper - band * kGroupM);
  const int mt = band * kGroupM + rem % gm, ntile = rem / gm;
  TileOrigin o;
  if (!locate_mtile(p.offsets, p.E, mt, o)) return;
  const int rows = min(kPM, o.cnt - o.m0);                  // valid sorted rows in this tile
  // weight rows of the tile: gate|up -> 128 gate channels + the 128 matching up channels
  const int n0 = GATEUP ? ntile * (kPN / 2) : ntile * kPN;

  // ---- per-thread load assignment (fixed for the whole K loop). Raw buffer loads: rows
  // outside the tile get an offset past the buffer's end and read as zeros.
  // weights: 1024 chunks of 16 bytes per k-step, chunk c = tid + 256 j: tile row c/4, part c%4
  const uint32_t row_bytes = (uint32_t)p.K / 2;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const uint8_t*>(p.w) + (size_t)o.e * p.Nw * row_bytes), (short)0,
      (int)(p.Nw * row_bytes), 0x00020000);
  uint32_t woff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + kPThreads * j, rho = c >> 2, part = c & 3;
    const int half = GATEUP && rho >= kPN / 2;
    const int chan = n0 + rho - half * (kPN / 2);
    const int grow = chan + half * p.n_out;
    woff[j] = chan < (GATEUP ? p.n_out : p.Nw) ? (uint32_t)grow * row_bytes + part * 16 : kPOutOfRange;
  }
  // tokens: 2048 chunks of 16 bytes per k-step, chunk c = tid + 256 j: tile row c/8, part c%8
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.act, (short)0, (int)((GATEUP ? p.P / 2 : p.P) * p.K), 0x00020000);
  uint32_t toff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = tid + kPThreads * j, r = c >> 3, part = c & 7;
    uint32_t off = kPOutOfRange;
    if (r < rows) {
      const int srow = GATEUP ? (p.sorted_pair[o.seg0 + o.m0 + r] >> 1) : (o.seg0 + o.m0 + r);
      off = (uint32_t)srow * p.K + part * 16;
    }
    toff[j] = off;
  }

  v4f acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 wq[4], tq[8];
  // an out-of-range offset stays out of range after adding k (offsets < 2^31, k < 2^30)
  auto load_step = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) wq[j] = pf_ld16(wr, woff[j] + (uint32_t)(k0 / 2));
#pragma unroll
    for (int j = 0; j < 8; ++j) tq[j] = pf_ld16(tr, toff[j] + (uint32_t)k0);
  };

  const int steps = p.K / 128;
  load_step(0);
  for (int s = 0; s < steps; ++s) {
    // convert this step's weights (exact E4M3 codes)
    uint4 wc[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {wq[j].x, wq[j].y, wq[j].z, wq[j].w};
      uint32_t cd[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        cd[2 * t] = nib4_to_e4m3(w[t] & 0x0F0F0F0Fu);
        cd[2 * t + 1] = nib4_to_e4m3((w[t] >> 4) & 0x0F0F0F0Fu);
      }
      wc[j][0] = make_uint4(cd[0], cd[1], cd[2], cd[3]);
      wc[j][1] = make_uint4(cd[4], cd[5], cd[6], cd[7]);
    }
    __syncthreads();                                        // previous step's reads are done
    // store both tiles in MFMA operand order: block b (16 rows) = [h][lane][16 B]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + kPThreads * j, rho = c >> 2, part = c & 3;
      uint8_t* d = ldsW + (rho >> 4) * 2048 + ((rho & 15) + 16 * part) * 16;
      *reinterpret_cast<uint4*>(d) = wc[j][0];
      *reinterpret_cast<uint4*>(d + 1024) = wc[j][1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + kPThreads * j, r = c >> 3, part = c & 7;
      const int g = part >> 1, h = part & 1;
      *reinterpret_cast<uint4*>(ldsT + (r >> 4) * 2048 + h * 1024 + ((r & 15) + 16 * g) * 16) = tq[j];
    }
    __syncthreads();
    if (s + 1 < steps) load_step((s + 1) * 128);            // in flight during the MFMAs
    // ---- MFMAs: token blocks 8wm.., weight blocks of this wave
    v8i bt[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint8_t* q = ldsT + (8 * wm + b) * 2048 + lane * 16;
      bt[b] = operand_from(*reinterpret_cast<const uint4*>(q), *reinterpret_cast<const uint4*>(q + 1024));
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int wb = GATEUP ? (a < 4 ? 4 * wn + a : 8 + 4 * wn + (a - 4)) : 8 * wn + a;
      const uint8_t* q = ldsW + wb * 2048 + lane * 16;
      const v8i aw = operand_from(*reinterpret_cast<const uint4*>(q), *reinterpret_cast<const uint4*>(q + 1024));
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = mfma_fp8_16x16x128(aw, bt[b], acc[a][b]);
    }
  }

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each block, token column i
  const int i = lane & 15, g = lane >> 4;
  const float* ws = p.w_scale + (size_t)o.e * p.Nw;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int rt = 128 * wm + 16 * b + i;                  // row within the tile
    if (rt >= rows) continue;
    const int r = o.seg0 + o.m0 + rt;                       // sorted row
    if (GATEUP) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int nb = n0 + 64 * wn + 16 * a + 4 * g;       // channel
        if (nb >= p.n_out) continue;
        const float4 sg = *reinterpret_cast<const float4*>(ws + nb);
        const float4 su = *reinterpret_cast<const float4*>(ws + p.n_out + nb);
        const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
        float gv[4], uv[4], av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          gv[v] = acc[a][b][v] * p.s_act * sgv[v];
          uv[v] = acc[a + 4][b][v] * p.s_act * suv[v];
          av[v] = act_fn(gv[v], p.act_fn) * uv[v] / p.s_a;
        }
        *reinterpret_cast<uint32_t*>(p.a_out + (size_t)r * p.n_out + nb) = pack4_e4m3(av[0], av[1], av[2], av[3]);
        if (p.dbg) {
          float* d = p.dbg + (size_t)r * 2 * p.n_out;
          *reinterpret_cast<float4*>(d + nb) = make_float4(gv[0], gv[1], gv[2], gv[3]);
          *reinterpret_cast<float4*>(d + p.n_out + nb) = make_float4(uv[0], uv[1], uv[2], uv[3]);
        }
      }
    } else {
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int nb = n0 + 128 * wn + 16 * a + 4 * g;
        if (nb >= p.Nw) continue;
        const float4 sw = *reinterpret_cast<const float4*>(ws + nb);
        float4 out;
        out.x = acc[a][b][0] * p.s_act * sw.x;
        out.y = acc[a][b][1] * p.s_act * sw.y;
        out.z = acc[a][b][2] * p.s_act * sw.z;
        out.w = acc[a][b][3] * p.s_act * sw.w;
        *reinterpret_cast<float4*>(p.partial + (size_t)r * p.n_out + nb) = out;
      }
    }
  }
}

bool prefill_available() { return true; }

size_t prefill_gemm2_partial_bytes(int T, int H) { return (size_t)2 * T * H * sizeof(float); }

void launch_moe_prefill(const MoeGemmParams& p, bool gateup, hipStream_t st) {
  // every expert's rows split into tiles of kPM; the count of tiles is at most P/kPM + E
  const int mtiles_upper = (p.P + kPM - 1) / kPM + p.E;
  const int ntiles = gateup ? (p.n_out + kPN / 2 - 1) / (kPN / 2) : (p.Nw + kPN - 1) / kPN;
  const unsigned grid = (unsigned)((size_t)mtiles_upper * ntiles);
  if (gateup)
    hipLaunchKernelGGL(moe_prefill_kernel<true>, dim3(grid), dim3(kPThreads), kPLds, st, p, mtiles_upper, ntiles);
  else
    hipLaunchKernelGGL(moe_prefill_kernel<false>, dim3(grid), dim3(kPThreads), kPLds, st, p, mtiles_upper, ntiles);
}

}  // namespace w4a8
