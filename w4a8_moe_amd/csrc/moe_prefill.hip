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
// Conversion. Each int4 code becomes its exact E4M3 code by a table lookup on the byte
// permute unit: for the 4 low (or high) nibbles of a word, one v_perm picks the codes of
// 0..7, one the codes of -8..-1, and a third picks between them by the sign bit. The
// products are then the exact q * x, so the accumulation error is that of the fp8
// instruction on these products alone. (Offset codes q + 8, three bit operations per
// word, would need the row sums of x taken back out, and the instruction's error grows
// with the sum of |products|, about six times larger with the offset: that failed the
// output tolerance.)
//
// Tile. A workgroup computes 256 sorted rows (tokens of one expert) x 256 weight rows,
// K in steps of 128, with 4 waves. Wave w owns 64 weight rows (4 blocks of 16) against
// all 256 tokens (16 blocks), so its int4 codes go from global memory straight into its
// own registers, are converted there and are used as MFMA operands without an LDS round
// trip. For
// gate|up the 64 rows are 32 gate channels and the 32 matching up channels, so
// act(gate) * up is formed in registers. Only the token tile (256 x 128 E4M3 codes per
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

#include "common.h"
#include "kernels.h"

namespace w4a8 {

constexpr int kTB = 16;           // token blocks of 16 rows per tile
constexpr int kPM = 16 * kTB;     // sorted rows per tile
constexpr int kPN = 256;          // weight rows per tile
constexpr int kPThreads = 256;    // 4 waves, 64 weight rows each
constexpr int kTJ = kPM * 8 / kPThreads;                  // 16-byte token chunks per thread and k-step
constexpr int kPTokBytes = kTB * 2048;                    // blocks of 16 rows x 128 codes
constexpr int kPLds = 2 * kPTokBytes;                      // two token buffers
constexpr int kGroupM = 4;        // M-tiles per band of the tile order
constexpr uint32_t kPOutOfRange = 0x80000000u;   // past every buffer (all are < 2^31 bytes)

__device__ __forceinline__ uint4 pf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// per-lane offset plus a wave-uniform one (the step), added by the load itself
__device__ __forceinline__ uint4 pf_ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, __builtin_amdgcn_readfirstlane(soff), 0));
}

// Four two's-complement nibbles (sel = nibble & 7 per byte, sgn = 4 * sign bit per byte)
// -> four exact E4M3 codes: 0..7 -> 00 38 40 44 48 4A 4C 4E, -8..-1 -> D0 CE CC CA C8 C4
// C0 B8. The last permute takes byte i from the positive (selector i) or the negative
// (selector 4 + i) table.
__device__ __forceinline__ uint32_t e4m3_of_nibbles(uint32_t sel, uint32_t sgn) {
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, sel);
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, sel);
  return __builtin_amdgcn_perm(neg, pos, sgn | 0x03020100u);
}

// One packed word (byte b: element b in the low nibble, element 4+b in the high nibble)
// -> E4M3 codes of elements 0..3 (lo) and 4..7 (hi).
__device__ __forceinline__ uint32_t e4m3_of_nibbles_sel(uint32_t sel, uint32_t selsgn) {
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, sel);
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, sel);
  return __builtin_amdgcn_perm(neg, pos, selsgn);
}
__device__ __forceinline__ void int4x8_to_e4m3(uint32_t w, uint32_t& lo, uint32_t& hi, uint32_t m4 = 0x04040404u,
                                               uint32_t id = 0x03020100u) {
  const uint32_t w4 = w >> 4;
  lo = e4m3_of_nibbles_sel(w & 0x07070707u, ((w >> 1) & m4) | id);
  hi = e4m3_of_nibbles_sel(w4 & 0x07070707u, ((w4 >> 1) & m4) | id);
}

__device__ __forceinline__ v8i int4x32_to_e4m3(uint4 q) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  v8i a;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t lo, hi;
    int4x8_to_e4m3(w[t], lo, hi);
    a[2 * t] = (int)lo;
    a[2 * t + 1] = (int)hi;
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

// ACT: the gated activation (gate|up only), a template parameter so that each instance
// carries the code of one activation in its unrolled epilogue.
template <bool GATEUP, int ACT>
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

  // ---- this lane's weights: block a of the wave, the 16 bytes at lane * 16 of each of the
  //      block's tiles (row i, K-part g of a 16-row x 128-K tile)
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
    woff[a] = chan < (GATEUP ? p.n_out : p.Nw) ? (uint32_t)(grow - i) * row_bytes + 16 * lane : kPOutOfRange;
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
    for (int j = 0; j < kTJ; ++j) tq[j] = pf_ld16s(tr, toff[j], (uint32_t)(s * 128));
  };
  auto store_tokens = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kTJ; ++j) *reinterpret_cast<uint4*>(lds + buf * kPTokBytes + tdst[j]) = tq[j];
  };
  uint4 w0[4], w1[4];          // raw weights of steps s and s+1
  auto load_weights = [&](uint4 (&w)[4], int s) {
#pragma unroll
    for (int a = 0; a < 4; ++a) w[a] = pf_ld16s(wr, woff[a], (uint32_t)(s * kTileBytes));
  };

  // ---- prologue: weights of steps 0..2 in flight, tokens of step 0 in LDS, of step 1 in flight
  load_weights(w0, 0);
  load_weights(w1, 1);
  load_tokens(0);
  store_tokens(0);
  load_tokens(1);
  v8i aop[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) aop[a] = int4x32_to_e4m3(w0[a]);
  lds_barrier();

  // One k-step per iteration (a single loop body keeps every accumulator in place). The
  // token blocks are walked with the next block's operand read ahead; into each block's 4
  // MFMAs go one token store (step s+1) or one token load (step s+2) and one or two of the
  // 16 words of the step s+1 weight conversion; a weight block's raw registers are
  // reloaded with step s+2 as soon as its last word is converted. Scheduling barriers keep
  // the compiler from hoisting every LDS read to the top.
  // the two byte masks of the conversion live in registers, so that mask-and-merge is one
  // 3-input bit operation
  uint32_t km4 = 0x04040404u, kid = 0x03020100u;
  asm volatile("" : "+v"(km4), "+v"(kid));
  for (int s = 0; s < steps; ++s) {
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
        tq[j] = pf_ld16s(tr, toff[j], (uint32_t)((s + 2) * 128));             // step s+2
#pragma unroll
      for (int wi = bb; wi < 16; wi += kTB) {
        const int a = wi >> 2, tw = wi & 3;
        const uint32_t w = tw == 0 ? w1[a].x : tw == 1 ? w1[a].y : tw == 2 ? w1[a].z : w1[a].w;
        uint32_t lo, hi;
        int4x8_to_e4m3(w, lo, hi, km4, kid);
        anext[a][2 * tw] = (int)lo;
        anext[a][2 * tw + 1] = (int)hi;
      }
      // words wi are converted at bb = wi (16 blocks): block a's last word goes at bb = 4 a + 3
      static_assert(kTB == 16, "the reload points below follow the conversion order for 16 blocks");
      if ((bb & 3) == 3) w1[bb >> 2] = pf_ld16s(wr, woff[bb >> 2], (uint32_t)((s + 2) * kTileBytes));
      __builtin_amdgcn_sched_barrier(0);
      if (bb < kTB - 1) bcur = bnext;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) aop[a] = anext[a];
    lds_barrier();
  }

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each block, token column i. Every
  // value it reads is gathered before its first store (the byte stores may alias any
  // load), so the loads overlap instead of each waiting behind the stores before it.
  const float* ws = p.w_scale + (size_t)o.e * p.Nw;
  const int lim = GATEUP ? p.n_out : p.Nw;
  int nbs[4];
  float4 sc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    // gate|up: a = 0, 1 gate scales of channel nbs[a], a = 2, 3 the up scales of nbs[a - 2];
    // each folded with the activation's static scale once
    nbs[a] = GATEUP ? n0 + 32 * wave + 16 * (a & 1) + 4 * g : n0 + 64 * wave + 16 * a + 4 * g;
    const int nl = nbs[a] < lim ? nbs[a] : 0;
    const float4 w4 = *reinterpret_cast<const float4*>(ws + (GATEUP && a >= 2 ? p.n_out : 0) + nl);
    sc[a] = make_float4(w4.x * p.s_act, w4.y * p.s_act, w4.z * p.s_act, w4.w * p.s_act);
  }
  // Values are computed for every (row, channel) of the lane, uniformly; only the stores
  // are guarded (rows and channels past the tile's valid range hold zero sums).
#pragma unroll
  for (int bb = 0; bb < kTB; ++bb) {
    const int rt = 16 * bb + i;                              // row within the tile
    const bool row_ok = rt < rows;
    const size_t r = (size_t)(o.seg0 + o.m0 + (row_ok ? rt : 0));   // sorted row
    if (GATEUP) {
      uint8_t* arow = p.a_out + r * p.n_out;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int nb = nbs[a];                               // channel
        const float sgv[4] = {sc[a].x, sc[a].y, sc[a].z, sc[a].w};
        const float suv[4] = {sc[a + 2].x, sc[a + 2].y, sc[a + 2].z, sc[a + 2].w};
        float gv[4], uv[4], av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          gv[v] = acc[bb][a][v] * sgv[v];
          uv[v] = acc[bb][a + 2][v] * suv[v];
          av[v] = div_rn(act_fast<ACT>(gv[v]) * uv[v], p.s_a, p.inv_s_a);
        }
        const uint32_t codes = pack4_e4m3(av[0], av[1], av[2], av[3]);
        if (row_ok && nb < p.n_out) {
          *reinterpret_cast<uint32_t*>(arow + nb) = codes;
          if (p.dbg) {
            float* d = p.dbg + r * 2 * p.n_out;
            *reinterpret_cast<float4*>(d + nb) = make_float4(gv[0], gv[1], gv[2], gv[3]);
            *reinterpret_cast<float4*>(d + p.n_out + nb) = make_float4(uv[0], uv[1], uv[2], uv[3]);
          }
        }
      }
    } else {
      float* prow = p.partial + r * p.n_out;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int nb = nbs[a];
        const float4 out = make_float4(acc[bb][a][0] * sc[a].x, acc[bb][a][1] * sc[a].y,
                                       acc[bb][a][2] * sc[a].z, acc[bb][a][3] * sc[a].w);
        if (row_ok && nb < p.Nw) *reinterpret_cast<float4*>(prow + nb) = out;
      }
    }
  }
}

bool prefill_available() { return true; }

void launch_moe_prefill(const MoeGemmParams& p, bool gateup, hipStream_t st) {
  // every expert's rows split into tiles of kPM; the count of tiles is at most P/kPM + E
  const int mtiles_upper = (p.P + kPM - 1) / kPM + p.E;
  const int ntiles = gateup ? (p.n_out + kPN / 2 - 1) / (kPN / 2) : (p.Nw + kPN - 1) / kPN;
  const unsigned grid = (unsigned)((size_t)mtiles_upper * ntiles);
  if (!gateup)
    hipLaunchKernelGGL((moe_prefill_kernel<false, 0>), dim3(grid), dim3(kPThreads), kPLds, st, p, mtiles_upper, ntiles);
  else if (p.act_fn == 0)
    hipLaunchKernelGGL((moe_prefill_kernel<true, 0>), dim3(grid), dim3(kPThreads), kPLds, st, p, mtiles_upper, ntiles);
  else if (p.act_fn == 1)
    hipLaunchKernelGGL((moe_prefill_kernel<true, 1>), dim3(grid), dim3(kPThreads), kPLds, st, p, mtiles_upper, ntiles);
  else
    hipLaunchKernelGGL((moe_prefill_kernel<true, 2>), dim3(grid), dim3(kPThreads), kPLds, st, p, mtiles_upper, ntiles);
}

}  // namespace w4a8
