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
// Tile. A workgroup computes 192 sorted rows (tokens of one expert) x 256 weight rows,
// K in steps of 128, with 4 waves. Wave w owns 64 weight rows (4 blocks of 16) against
// all 192 tokens (12 blocks), so its int4 codes go from global memory straight into its
// own registers, are converted there (v_perm table lookup, exact for all 16
// two's-complement codes) and are used as MFMA operands without an LDS round trip. For
// gate|up the 64 rows are 32 gate channels and the 32 matching up channels, so
// act(gate) * up is formed in registers. Only the token tile (192 x 128 E4M3 codes per
// k-step, gathered through sorted_pair for gate|up) is shared through LDS, double
// buffered, in MFMA operand order with an XOR swizzle that keeps both the staging writes
// and the operand reads free of bank conflicts.
//
// Pipeline, per k-step s (one barrier each):
//   * store the tokens of step s+1 (loaded one step earlier) into the other LDS buffer,
//     issue the token loads of step s+2,
//   * 64 MFMAs of step s, with the conversion of step s+1's weights (loaded two steps
//     earlier) and the weight loads of step s+3 in between.
// Loads past the last k-step read in-bounds data or zeros and are never used, so the
// loop has no branches.
//
// Accumulation note: gfx950's fp8 MFMA keeps about 14 bits below the largest product of
// an instruction, so results differ from exact fp32 sums by about 1e-5 of the row scale.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

constexpr int kTB = 12;           // token blocks of 16 rows per tile
constexpr int kPM = 16 * kTB;     // sorted rows per tile
constexpr int kPN = 256;          // weight rows per tile
constexpr int kPThreads = 256;    // 4 waves, 64 weight rows each
constexpr int kTJ = kPM * 8 / kPThreads;                  // 16-byte token chunks per thread and k-step
constexpr int kPTokBytes = kTB * 2048;                    // blocks of 16 rows x 128 codes
constexpr int kPLds = 2 * kPTokBytes;                      // two token buffers
constexpr int kGroupM = 4;        // M-tiles per band of the tile order
constexpr int kWRing = 3;         // k-steps of raw weights in flight per wave
constexpr uint32_t kPOutOfRange = 0x80000000u;   // past every buffer (all are < 2^31 bytes)

__device__ __forceinline__ uint4 pf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Four two's-complement nibbles -> four exact E4M3 codes: 0..7 -> 00 38 40 44 48 4A 4C 4E,
// -8..-1 -> D0 CE CC CA C8 C4 C0 B8. Per byte, sel = nibble & 7 and sgn = nibble >> 3.
__device__ __forceinline__ uint32_t e4m3_of_nibbles(uint32_t sel, uint32_t sgn) {
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, sel);
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, sel);
  // selector 12 reads as 0x00, 13 as 0xFF: a byte mask of the sign bits
  const uint32_t msk = __builtin_amdgcn_perm(0u, 0u, sgn | 0x0C0C0C0Cu);
  return (msk & neg) | (~msk & pos);
}

// 16 bytes of packed int4 (32 K-values; in each word, byte b holds element b in its low
// nibble and element 4+b in its high nibble) -> the 8 registers of an MFMA operand, in
// natural K order.
__device__ __forceinline__ v8i int4x32_to_e4m3(uint4 q) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  v8i a;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a[2 * t] = (int)e4m3_of_nibbles(w[t] & 0x07070707u, (w[t] >> 3) & 0x01010101u);
    a[2 * t + 1] = (int)e4m3_of_nibbles((w[t] >> 4) & 0x07070707u, (w[t] >> 7) & 0x01010101u);
  }
  return a;
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

// LDS position of the 16 bytes that lane (row i, K-part g) reads in half h of a token
// block: 16-byte slot 16 g + (i ^ (2 g + 8 h)) of the half's 1 KB. Within 16 consecutive
// reading lanes the slots are distinct mod 16 (no bank conflict); so are they for 16
// consecutive staging lanes (two rows x four K-parts x two halves).
__device__ __forceinline__ int tok_slot(int i, int g, int h) { return 16 * g + (i ^ (2 * g + 8 * h)); }

template <bool GATEUP>
__global__ __launch_bounds__(kPThreads, 1) void moe_prefill_kernel(MoeGemmParams p, int mtiles_upper, int ntiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int i = lane & 15, g = lane >> 4;

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
  // first channel of the tile: gate|up -> 128 channels (gate rows + the matching up rows)
  const int n0 = GATEUP ? ntile * (kPN / 2) : ntile * kPN;

  // ---- this lane's weight rows: block a of the wave, row i of the block, K-part g
  const uint32_t row_bytes = (uint32_t)p.K / 2;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const uint8_t*>(p.w) + (size_t)o.e * p.Nw * row_bytes), (short)0,
      (int)(p.Nw * row_bytes), 0x00020000);
  uint32_t woff[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    // gate|up: blocks 0,1 gate channels n0 + 32 w + 16 (a % 2) + i, blocks 2,3 their up rows
    const int chan = GATEUP ? n0 + 32 * wave + 16 * (a & 1) + i : n0 + 64 * wave + 16 * a + i;
    const int grow = GATEUP && a >= 2 ? chan + p.n_out : chan;
    woff[a] = chan < (GATEUP ? p.n_out : p.Nw) ? (uint32_t)grow * row_bytes + 16 * g : kPOutOfRange;
  }

  // ---- token staging: chunk c = tid + 256 j is tile row c / 8, 16-byte part c % 8.
  // gate|up gathers token rows of x (T*H < 2^31 bytes); down reads the tile's own rows of
  // the sorted activation (the buffer starts at the tile, kPM*K < 2^31 bytes).
  const uint8_t* tbase = GATEUP ? p.act : p.act + (size_t)(o.seg0 + o.m0) * p.K;
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)tbase, (short)0, (int)((GATEUP ? p.P / 2 : rows) * p.K), 0x00020000);
  uint32_t toff[kTJ];
  int tdst[kTJ];
#pragma unroll
  for (int j = 0; j < kTJ; ++j) {
    const int c = tid + kPThreads * j, r = c >> 3, part = c & 7;
    uint32_t off = kPOutOfRange;
    if (r < rows) {
      const int srow = GATEUP ? (p.sorted_pair[o.seg0 + o.m0 + r] >> 1) : r;
      off = (uint32_t)srow * p.K + part * 16;
    }
    toff[j] = off;
    const int pg = part >> 1, ph = part & 1;
    tdst[j] = (r >> 4) * 2048 + ph * 1024 + tok_slot(r & 15, pg, ph) * 16;
  }
  const int rd0 = tok_slot(i, g, 0) * 16, rd1 = 1024 + tok_slot(i, g, 1) * 16;

  v4f acc[kTB][4];
#pragma unroll
  for (int bb = 0; bb < kTB; ++bb)
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[bb][a] = v4f{0.f, 0.f, 0.f, 0.f};

  const int steps = p.K / 128;
  // an out-of-range offset stays out of range after adding k (offsets < 2^31, k < 2^30)
  uint4 tq[kTJ];
  auto load_tokens = [&](int s) {
#pragma unroll
    for (int j = 0; j < kTJ; ++j) tq[j] = pf_ld16(tr, toff[j] + (uint32_t)(s * 128));
  };
  auto store_tokens = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kTJ; ++j) *reinterpret_cast<uint4*>(lds + buf * kPTokBytes + tdst[j]) = tq[j];
  };
  uint4 wq[kWRing][4];
  auto load_weights = [&](int slot, int s) {
#pragma unroll
    for (int a = 0; a < 4; ++a) wq[slot][a] = pf_ld16(wr, woff[a] + (uint32_t)(s * 64));
  };

  // ---- prologue: weights of steps 0..2 in flight, tokens of step 0 in LDS, of step 1 in flight
#pragma unroll
  for (int s = 0; s < kWRing; ++s) load_weights(s, s);
  load_tokens(0);
  store_tokens(0);
  load_tokens(1);
  v8i aop[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) aop[a] = int4x32_to_e4m3(wq[0][a]);
  __syncthreads();

  // One k-step; SLOT = s % kWRing is a constant so that the weight ring stays in
  // registers. The token blocks are walked with the next block's operand read ahead;
  // into each block's 4 MFMAs go one token store (step s+1) or one token load (step s+2),
  // one or two of the 16 words of the step s+1 weight conversion, and in the first 4 a
  // weight load of step s+3; scheduling barriers keep the compiler from hoisting every
  // LDS read to the top.
  auto kstep = [&](int s, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr int NSLOT = (SLOT + 1) % kWRing;
    const int cur = s & 1;
    const uint8_t* T = lds + cur * kPTokBytes;
    uint8_t* Tn = lds + (cur ^ 1) * kPTokBytes;
    v8i anext[4];
    v8i bcur = operand_from(*reinterpret_cast<const uint4*>(T + rd0), *reinterpret_cast<const uint4*>(T + rd1));
#pragma unroll
    for (int bb = 0; bb < kTB; ++bb) {
      v8i bnext;
      if (bb < kTB - 1)
        bnext = operand_from(*reinterpret_cast<const uint4*>(T + (bb + 1) * 2048 + rd0),
                             *reinterpret_cast<const uint4*>(T + (bb + 1) * 2048 + rd1));
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[bb][a] = mfma_fp8_16x16x128(aop[a], bcur, acc[bb][a]);
      const int j = bb >> 1;
      if ((bb & 1) == 0)
        *reinterpret_cast<uint4*>(Tn + tdst[j]) = tq[j];                     // step s+1
      else
        tq[j] = pf_ld16(tr, toff[j] + (uint32_t)((s + 2) * 128));             // step s+2
      if (bb < 4) wq[SLOT][bb] = pf_ld16(wr, woff[bb] + (uint32_t)((s + kWRing) * 64));
#pragma unroll
      for (int wi = bb; wi < 16; wi += kTB) {
        const int a = wi >> 2, tw = wi & 3;
        const uint32_t w = tw == 0 ? wq[NSLOT][a].x : tw == 1 ? wq[NSLOT][a].y : tw == 2 ? wq[NSLOT][a].z
                                                                                         : wq[NSLOT][a].w;
        anext[a][2 * tw] = (int)e4m3_of_nibbles(w & 0x07070707u, (w >> 3) & 0x01010101u);
        anext[a][2 * tw + 1] = (int)e4m3_of_nibbles((w >> 4) & 0x07070707u, (w >> 7) & 0x01010101u);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (bb < kTB - 1) bcur = bnext;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) aop[a] = anext[a];
    __syncthreads();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  static_assert(kWRing == 3, "the loop below is unrolled by the ring size");
  int s = 0;
  for (; s + 3 <= steps; s += 3) {
    kstep(s, S0{});
    kstep(s + 1, S1{});
    kstep(s + 2, S2{});
  }
  if (s < steps) kstep(s, S0{});
  if (s + 1 < steps) kstep(s + 1, S1{});

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each block, token column i
  const float* ws = p.w_scale + (size_t)o.e * p.Nw;
#pragma unroll
  for (int bb = 0; bb < kTB; ++bb) {
    const int rt = 16 * bb + i;                              // row within the tile
    if (rt >= rows) continue;
    const int r = o.seg0 + o.m0 + rt;                        // sorted row
    if (GATEUP) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int nb = n0 + 32 * wave + 16 * a + 4 * g;      // channel
        if (nb >= p.n_out) continue;
        const float4 sg = *reinterpret_cast<const float4*>(ws + nb);
        const float4 su = *reinterpret_cast<const float4*>(ws + p.n_out + nb);
        const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
        float gv[4], uv[4], av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          gv[v] = acc[bb][a][v] * p.s_act * sgv[v];
          uv[v] = acc[bb][a + 2][v] * p.s_act * suv[v];
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
      for (int a = 0; a < 4; ++a) {
        const int nb = n0 + 64 * wave + 16 * a + 4 * g;
        if (nb >= p.Nw) continue;
        const float4 sw = *reinterpret_cast<const float4*>(ws + nb);
        float4 out;
        out.x = acc[bb][a][0] * p.s_act * sw.x;
        out.y = acc[bb][a][1] * p.s_act * sw.y;
        out.z = acc[bb][a][2] * p.s_act * sw.z;
        out.w = acc[bb][a][3] * p.s_act * sw.w;
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
