// Tiled (prefill-shaped) grouped GEMM of the routed experts: many tokens per expert,
// bound by the matrix cores.
//
// The method ("INT4 MoE weights, FP8 compute", page "ROCm: enable trillion-parameter
// MoE models with INT4-FP8 single node"; int4 weights upcast to float8 for fp8 math,
// page "[AMD][Quantization] Add int4fp8_moe online quantization on ROCm"): every product
// is an E4M3 activation times an int4 weight code, summed in fp32; the per-channel and
// static scales are applied in the epilogue. The products run on the fp16 MFMA
// (16x16x32), which forms them exactly and adds them in fp32 (common.h: the fp8 MFMA's
// sums are less precise, and their error breaks the output tolerance): int4 codes are
// widened to exact fp16 by exponent placement, E4M3 codes by the hardware conversion
// (those facing a weight's high nibble divided by 16, exact).
//
// Tile. A workgroup computes TB blocks of 16 sorted rows (tokens of one expert; 32, 64 or
// 256 rows, chosen by the rows per expert) x 256 weight rows, K in steps of 128, with NW
// waves: 4 (one per SIMD), or 8 for the gate|up 256-row tiles. Wave w owns 256 / NW weight
// rows (BPW = 16 / NW blocks of 16) against all TB token blocks, so its int4 codes go from
// global memory straight into its own registers, are widened there and used as MFMA
// operands without an LDS round trip. For gate|up the rows are gate channels and the
// matching up channels (half each), so act(gate) * up is formed in registers. Only the
// token tile (TB*16 rows x 128 K per k-step, gathered through sorted_pair for gate|up) is
// shared through LDS, double buffered: each thread widens its
// staging chunks to fp16 once, and the waves read finished MFMA operands (1 KB per token
// block and K-part, lane l's 16 bytes at 16 l: no bank conflicts on either side).
//
// Pipeline of the 256-row tiles, per k-step s (one barrier each): issue the weight loads of
// step s+2; then walk the token blocks, the next block's operands read ahead, widening the
// step's 4 BPW weight words (BPW blocks x 4 MFMAs of K = 32) K-part by K-part inside the
// first token block, storing the tokens of step s+1 (loaded one step earlier) into the other
// LDS buffer and issuing the token loads of step s+2 on the way. Loads past the last k-step
// read in-bounds data or zeros and are never used, so the loop has no branches. (The
// compiler moves a step's fresh weight loads into the ring by copies at the end of the step,
// which waits for them: in effect the weights run one step ahead, which the long steps of
// these tiles cover.)
//
// The 32- and 64-row tiles have short steps (32 or 64 MFMAs per wave), so they keep their
// loads R steps ahead in register rings without copies (the loop body unrolled by R, each
// step's slot fixed), walk the K-parts in the outer loop and widen the next part's weights
// while the current part's MFMAs run. Each accumulator sees its MFMAs in the same order in
// both pipelines, so the two give the same bits.
//
// Measured on MI355X (Grok-1-shaped prefill, 256-row tiles, rocprofv3 counters): the matrix
// cores are busy 63% of the cycles for gate|up with 8 waves (57% with 4) at 2.22 GHz, and
// 62-63% for the down projection (4 waves) at 2.26-2.31 GHz; with one wave per SIMD the
// step's other work (barrier, operand waits, prologue, epilogue) adds to the MFMA time
// rather than hiding under it, which a second wave per SIMD partly takes back.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

constexpr int kPN = 256;          // weight rows per tile
constexpr uint32_t kPOutOfRange = 0x80000000u;   // past every buffer (all are < 2^31 bytes)

// per-lane offset plus a wave-uniform one (the step), added by the load itself
template <int AUX = 0>
__device__ __forceinline__ uint4 pf_ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, __builtin_amdgcn_readfirstlane(soff), AUX));
}
#ifndef W4A8_PREFILL_NT
#define W4A8_PREFILL_NT 0
#endif
constexpr int kPfWeightAux = W4A8_PREFILL_NT ? 2 : 0;   // cache-policy bits of the weight loads

__device__ __forceinline__ uint32_t word4(const uint4& q, int m) {
  return m == 0 ? q.x : (m == 1 ? q.y : (m == 2 ? q.z : q.w));
}

struct TileOrigin {
  int e, seg0, cnt, m0;   // expert, its first sorted row, its row count, tile's first row in it
};

// Linear M-tile index -> (expert, first row). Returns false past the last tile.
__device__ __forceinline__ bool locate_mtile(const int32_t* __restrict__ offsets, int E, int pm, int mt,
                                             TileOrigin& o) {
  int before = 0;
  for (int e = 0; e < E; ++e) {
    const int s0 = offsets[e], c = offsets[e + 1] - s0;
    const int nt = (c + pm - 1) / pm;
    if (mt < before + nt) {
      o.e = e; o.seg0 = s0; o.cnt = c; o.m0 = (mt - before) * pm;
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

// TB: token blocks of 16 rows per tile. ACT: the gated activation (gate|up only), a template
// parameter so that each instance carries the code of one activation in its epilogue.
template <bool GATEUP, int ACT, int TB, int R, int NW>
__global__ __launch_bounds__(64 * NW, 1) void moe_prefill_kernel(MoeGemmParams p, int mtiles_upper, int ntiles,
                                                                   int groupm, int chunk) {
  constexpr int kThreads = 64 * NW;
  constexpr int BPW = 16 / NW;                       // 16-row weight blocks per wave
  constexpr int HB = BPW / 2;                        // gate|up: gate blocks per wave (then as many up)
  constexpr int kPM = 16 * TB;                       // sorted rows per tile
  constexpr int kTJ = kPM * 8 / kThreads;            // 16-byte token chunks per thread and k-step
  constexpr int kTokBytes = TB * 4096;               // blocks of 16 rows x 128 K, fp16
  constexpr int kTStride = TB / kTJ;                 // token blocks per staged chunk
  static_assert(TB % kTJ == 0 && (R == 0 || NW == 4), "the rings run with 4 waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int i = lane & 15, g = lane >> 4;

  // Tile order. The order walks bands of groupm M-tiles, all N-tiles of a band before the
  // next band (with a split reduction, the K-slice is the fastest index). Workgroups are
  // dispatched round-robin over the 8 XCDs (workgroup b on XCD b % 8), and XCD x takes
  // chunks x, x + 8, x + 16, ... of chunk consecutive tiles of the order (chunk: about the
  // workgroups one XCD holds at once): the workgroups resident on an XCD share a few token
  // and weight tiles in its L2, and the empty tiles at the end of the order (the M-tile
  // count is an upper bound) are spread over all XCDs. The grid is a whole number of 8
  // chunks; tiles past the order's end exit.
  const int b = blockIdx.x, xcd = b % 8, kx = b / 8;
  const int tk = ((kx / chunk) * 8 + xcd) * chunk + kx % chunk;
  if (tk >= mtiles_upper * ntiles * (GATEUP ? 1 : p.ksplit)) return;
  const int slice = GATEUP ? 0 : tk % p.ksplit;
  const int t = GATEUP ? tk : tk / p.ksplit;
  const int span = groupm * ntiles, band = t / span, rem = t % span;
  const int gm = min(groupm, mtiles_upper - band * groupm);
  const int mt = band * groupm + rem % gm, ntile = rem / gm;
  TileOrigin o;
  if (!locate_mtile(p.offsets, p.E, kPM, mt, o)) return;
  const int rows = min(kPM, o.cnt - o.m0);                  // valid sorted rows in this tile
  // first channel of the tile: gate|up -> 128 channels (gate rows + the matching up rows)
  const int n0 = GATEUP ? ntile * (kPN / 2) : ntile * kPN;

  // ---- this lane's weights: block a of the wave, the 16 bytes at lane * 16 of each of the
  //      block's tiles (row i, K-part g of a 16-row x 128-K tile)
  const uint32_t row_bytes = (uint32_t)p.K / 2;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const uint8_t*>(p.w) + (size_t)o.e * p.Nw * row_bytes), (short)0,
      (int)(p.Nw * row_bytes), 0x00020000);
  uint32_t woff[BPW];
#pragma unroll
  for (int a = 0; a < BPW; ++a) {
    // gate|up: blocks 0..HB-1 gate channels n0 + 16 HB w + 16 (a % HB) + i, the next HB their up rows
    const int chan = GATEUP ? n0 + 16 * HB * wave + 16 * (a % HB) + i : n0 + 16 * BPW * wave + 16 * a + i;
    const int grow = GATEUP && a >= HB ? chan + p.n_out : chan;
    woff[a] = chan < (GATEUP ? p.n_out : p.Nw) ? (uint32_t)(grow - i) * row_bytes + 16 * lane : kPOutOfRange;
  }

  // ---- token staging: each thread moves kTJ chunks of 16 E4M3 codes per k-step.
  // gate|up gathers token rows of x (T*H < 2^31 bytes); down reads the tile's own rows of
  // the sorted activation (the buffer starts at the tile, kPM*K < 2^31 bytes).
  const uint8_t* tbase = GATEUP ? p.act : p.act + (size_t)(o.seg0 + o.m0) * p.K;
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)tbase, (short)0, (int)((GATEUP ? p.P / 2 : rows) * p.K), 0x00020000);
  uint32_t toff[kTJ];
  int tdst[kTJ];
#pragma unroll
  for (int j = 0; j < kTJ; ++j) {
    // chunk c = tid + 256 j: row 16 (c >> 7) + c % 16, 16-byte part p = (c >> 4) & 7 (K 16 p..+16);
    // 16 consecutive lanes take 16 rows of one part, so their LDS stores are consecutive
    const int c = tid + kThreads * j, r = 16 * (c >> 7) + (c & 15), part = (c >> 4) & 7;
    uint32_t off = kPOutOfRange;
    if (r < rows) {
      const int srow = GATEUP ? (p.sorted_pair[o.seg0 + o.m0 + r] >> 1) : r;
      off = (uint32_t)srow * p.K + part * 16;
    }
    toff[j] = off;
    // part p holds K-parts m = 2 (p & 1), +1 of lane group g = p >> 1 (K 32 g + 8 m .. +8)
    tdst[j] = ((r >> 4) * 4 + 2 * (part & 1)) * 1024 + ((r & 15) + 16 * (part >> 1)) * 16;
  }
  const int rdl = lane * 16;
  v4f acc[TB][BPW];
#pragma unroll
  for (int bb = 0; bb < TB; ++bb)
#pragma unroll
    for (int a = 0; a < BPW; ++a) acc[bb][a] = v4f{0.f, 0.f, 0.f, 0.f};

  const int k0 = slice * p.kslice;                           // the slice's K range
  const int steps = (min(p.K - k0, p.kslice)) / 128;
  const uint32_t kb = (uint32_t)(k0 / 128);                 // its first k-step
  // an out-of-range offset stays out of range after adding k (offsets < 2^31, k < 2^30)
  auto store_tokens = [&](uint8_t* T, int j, const uint4& q) {
    *reinterpret_cast<v8h*>(T + tdst[j]) = e4m3x8_to_f16(q.x, q.y);
    *reinterpret_cast<v8h*>(T + tdst[j] + 1024) = e4m3x8_to_f16(q.z, q.w);
  };
  // the two nibble masks of the widening live in registers (one 3-input bit op per mask)
  uint32_t mlo = 0x0F0F0F0Fu, mhi = 0xF0F0F0F0u;
  asm volatile("" : "+v"(mlo), "+v"(mhi));
  if constexpr (R == 0) {
    uint4 tq[kTJ];
    auto load_tokens = [&](int s) {
#pragma unroll
      for (int j = 0; j < kTJ; ++j) tq[j] = pf_ld16s(tr, toff[j], (uint32_t)((kb + s) * 128));
    };
    uint4 wc[BPW], wn[BPW];      // raw weights of steps s and s+1
#pragma unroll
    for (int a = 0; a < BPW; ++a) {
      wc[a] = pf_ld16s<kPfWeightAux>(wr, woff[a], kb * kTileBytes);
      wn[a] = pf_ld16s<kPfWeightAux>(wr, woff[a], (kb + 1) * kTileBytes);
    }
    load_tokens(0);
#pragma unroll
    for (int j = 0; j < kTJ; ++j) store_tokens(lds, j, tq[j]);
    load_tokens(1);
    lds_barrier();

    for (int s = 0; s < steps; ++s) {
      const uint8_t* Tc = lds + (s & 1) * kTokBytes;
      uint8_t* Tn = lds + ((s & 1) ^ 1) * kTokBytes;
      // this step's weight operands: word m of block a -> K 32 g + 8 m .. +8 of its rows,
      // widened K-part by K-part inside the first token block, each part before its MFMAs
      // (the register allocator then keeps every accumulator in place: measured, Grok-1-shaped
      // prefill gate|up / down 39.04 / 18.48 -> 38.40 / 18.33 ms, the 8-way share's 5.26 ->
      // 4.89 ms gate|up, against widening all 16 words at the top of the step)
      v8h A[4][BPW];
      uint4 wraw[BPW];
#pragma unroll
      for (int a = 0; a < BPW; ++a) {
        wraw[a] = wc[a];
        wc[a] = wn[a];
        wn[a] = pf_ld16s<kPfWeightAux>(wr, woff[a], (uint32_t)((kb + s + 2) * kTileBytes));
      }
      // token blocks in order, each block's 16 MFMAs (4 K-parts x 4 weight blocks) together:
      // an accumulator's four MFMAs of the step are adjacent, which keeps every accumulator in
      // place (spread over the step, the register allocator rotates them through copies)
      v8h Bc[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) Bc[m] = *reinterpret_cast<const v8h*>(Tc + m * 1024 + rdl);
#pragma unroll
      for (int bb = 0; bb < TB; ++bb) {
        v8h Bn[4];
        if (bb + 1 < TB) {
#pragma unroll
          for (int m = 0; m < 4; ++m) Bn[m] = *reinterpret_cast<const v8h*>(Tc + ((bb + 1) * 4 + m) * 1024 + rdl);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (bb == 0) {
#pragma unroll
            for (int a = 0; a < BPW; ++a) A[m][a] = int4x8_to_f16(word4(wraw[a], m), mlo, mhi);
          }
#pragma unroll
          for (int a = 0; a < BPW; ++a) acc[bb][a] = mfma_f16(A[m][a], Bc[m], acc[bb][a]);
        }
        if (bb % kTStride == 0) {
          const int j = bb / kTStride;
          store_tokens(Tn, j, tq[j]);                                        // step s+1
          tq[j] = pf_ld16s(tr, toff[j], (uint32_t)((kb + s + 2) * 128));      // step s+2
        }
        __builtin_amdgcn_sched_barrier(0);
        if (bb + 1 < TB) {
#pragma unroll
          for (int m = 0; m < 4; ++m) Bc[m] = Bn[m];
        }
      }
      lds_barrier();
    }
  } else {
    // Small tiles: a k-step is short (TB * 16 MFMAs per wave), so the loads run R k-steps
    // ahead, in register rings with one fixed slot per step of an R-step loop body (a ring
    // rotated by copies would wait for each refill at the copy). Weights of step u sit in
    // wq[u % R]; tokens of step u in tq[u % R], stored to LDS during step u - 1. The weights
    // are widened one K-part at a time, the next part's while this part's MFMAs run. A body
    // past the last k-step still moves its ring (in-bounds or zero loads, never used) and
    // meets its barrier, and skips the arithmetic.
    // The prologue stages step 0's tokens, then issues the loads in the order one pass of
    // the loop body issues them (weights of a step, then the tokens one step later), so the
    // loop header sees the same loads in flight from either side and its waits stay precise.
    uint4 wq[R][BPW], tq[R][kTJ];
#pragma unroll
    for (int j = 0; j < kTJ; ++j) tq[0][j] = pf_ld16s(tr, toff[j], kb * 128);
#pragma unroll
    for (int j = 0; j < kTJ; ++j) store_tokens(lds, j, tq[0][j]);
#pragma unroll
    for (int d = 0; d < R; ++d) {
#pragma unroll
      for (int a = 0; a < BPW; ++a) {
        wq[d][a] = pf_ld16s<kPfWeightAux>(wr, woff[a], (kb + d) * kTileBytes);
        __builtin_amdgcn_sched_barrier(0);                // keep the issue order
      }
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        tq[(d + 1) % R][j] = pf_ld16s(tr, toff[j], (uint32_t)((kb + d + 1) * 128));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
    for (int s0 = 0; s0 < steps; s0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int s = s0 + u;
        const uint8_t* Tc = lds + (s & 1) * kTokBytes;
        uint8_t* Tn = lds + ((s & 1) ^ 1) * kTokBytes;
        const int un = (u + 1) % R;                          // ring slot of step s + 1
        if (s < steps) {
          v8h Ac[BPW], Bc[TB];
#pragma unroll
          for (int a = 0; a < BPW; ++a) Ac[a] = int4x8_to_f16(word4(wq[u][a], 0), mlo, mhi);
#pragma unroll
          for (int bb = 0; bb < TB; ++bb) Bc[bb] = *reinterpret_cast<const v8h*>(Tc + (bb * 4) * 1024 + rdl);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            v8h An[BPW], Bn[TB];
            if (m + 1 < 4) {
#pragma unroll
              for (int a = 0; a < BPW; ++a) An[a] = int4x8_to_f16(word4(wq[u][a], m + 1), mlo, mhi);
#pragma unroll
              for (int bb = 0; bb < TB; ++bb)
                Bn[bb] = *reinterpret_cast<const v8h*>(Tc + (bb * 4 + m + 1) * 1024 + rdl);
            }
#pragma unroll
            for (int bb = 0; bb < TB; ++bb)
#pragma unroll
              for (int a = 0; a < BPW; ++a) acc[bb][a] = mfma_f16(Ac[a], Bc[bb], acc[bb][a]);
            if (m + 1 < 4) {
#pragma unroll
              for (int a = 0; a < BPW; ++a) Ac[a] = An[a];
#pragma unroll
              for (int bb = 0; bb < TB; ++bb) Bc[bb] = Bn[bb];
            }
          }
        }
        // refill: weights of step s + R into this step's slot; tokens of step s + 1 to LDS,
        // then step s + 1 + R into their slot
#pragma unroll
        for (int a = 0; a < BPW; ++a) wq[u][a] = pf_ld16s<kPfWeightAux>(wr, woff[a], (uint32_t)((kb + s + R) * kTileBytes));
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          store_tokens(Tn, j, tq[un][j]);
          tq[un][j] = pf_ld16s(tr, toff[j], (uint32_t)((kb + s + 1 + R) * 128));
        }
        lds_barrier();
      }
    }
  }

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each block, token column i. Every
  // value it reads is gathered before its first store (the byte stores may alias any
  // load), so the loads overlap instead of each waiting behind the stores before it.
  const float* ws = p.w_scale + (size_t)o.e * p.Nw;
  const int lim = GATEUP ? p.n_out : p.Nw;
  int nbs[BPW];
  float4 sc[BPW];
#pragma unroll
  for (int a = 0; a < BPW; ++a) {
    // gate|up: a < HB gate scales of channel nbs[a], a >= HB the up scales of nbs[a - HB];
    // each folded with the activation's static scale once
    nbs[a] = GATEUP ? n0 + 16 * HB * wave + 16 * (a % HB) + 4 * g : n0 + 16 * BPW * wave + 16 * a + 4 * g;
    const int nl = nbs[a] < lim ? nbs[a] : 0;
    const float4 w4 = *reinterpret_cast<const float4*>(ws + (GATEUP && a >= HB ? p.n_out : 0) + nl);
    sc[a] = make_float4(w4.x * p.s_act, w4.y * p.s_act, w4.z * p.s_act, w4.w * p.s_act);
  }
  // Values are computed for every (row, channel) of the lane, uniformly; only the stores
  // are guarded (rows and channels past the tile's valid range hold zero sums).
#pragma unroll
  for (int bb = 0; bb < TB; ++bb) {
    const int rt = 16 * bb + i;                              // row within the tile
    const bool row_ok = rt < rows;
    const size_t r = (size_t)(o.seg0 + o.m0 + (row_ok ? rt : 0));   // sorted row
    if (GATEUP) {
      uint8_t* arow = p.a_out + r * p.n_out;
#pragma unroll
      for (int a = 0; a < HB; ++a) {
        const int nb = nbs[a];                               // channel
        const float sgv[4] = {sc[a].x, sc[a].y, sc[a].z, sc[a].w};
        const float suv[4] = {sc[a + HB].x, sc[a + HB].y, sc[a + HB].z, sc[a + HB].w};
        float gv[4], uv[4], av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          gv[v] = acc[bb][a][v] * sgv[v];
          uv[v] = acc[bb][a + HB][v] * suv[v];
          av[v] = requant_value<ACT>(gv[v], uv[v], p.s_a, p.inv_s_a);
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
      float* prow = p.partial + ((size_t)slice * p.P + r) * p.n_out;
#pragma unroll
      for (int a = 0; a < BPW; ++a) {
        const int nb = nbs[a];
        const float4 out = make_float4(acc[bb][a][0] * sc[a].x, acc[bb][a][1] * sc[a].y,
                                       acc[bb][a][2] * sc[a].z, acc[bb][a][3] * sc[a].w);
        if (row_ok && nb < p.Nw) *reinterpret_cast<float4*>(prow + nb) = out;
      }
    }
  }
}

bool prefill_available() { return true; }

// Token blocks per tile, by the mean rows per expert (P / E): 32-row tiles up to 48 rows,
// 64-row tiles up to 1536 (gate|up: up to 511), 256-row tiles above. The 32- and 64-row tiles run two
// workgroups per CU with register rings, and up to about a thousand rows per expert that
// outweighs reading each weight tile once per 64 rows instead of once per 256; the 256-row
// tiles win once an expert holds many of them (their weights then come from the caches).
// 128-row tiles were never the fastest. Measured gate|up / down, us (same GPU):
//   Mixtral-shaped   96 tokens: 32-row 143 / 79,   64-row 140 / 81
//                   192 tokens: 32-row 168 / 98,   64-row 189 / 104
//                   256 tokens: 32-row 208 / 110,  64-row 199 / 114
//                   512 tokens: 64-row 295 / 155,  128-row 408 / 206
//                  1024 tokens: 64-row 483 / 282,  256-row 716 / 324
//                  4096 tokens: 64-row 1708 / 859, 256-row 1884 / 976
//                  8192 tokens: 64-row 3428 / 1699, 256-row 3557 / 1718
//                 16384 tokens: 64-row 6814 / 3371, 256-row 6562 / 3088
//   Grok-1-shaped   2048 tokens: 64-row 3090 / 1500, 256-row 3608 / 1843
//                   4096 tokens: 64-row 5949 / 2934, 256-row 6066 / 2921
//                   8192 tokens: 64-row 11435 / 5652, 256-row 11117 / 5179
//                  32768 tokens: 64-row 44428 / 21947, 256-row 39594 / 19223
// With 8 waves per 256-row gate|up workgroup those tiles take gate|up from 512 rows per
// expert on (gate|up, us, 64-row against 256-row tiles, same GPU): Mixtral-shaped 2048
// tokens 892 / 855, 4096 tokens 1636 / 1542, 6144 tokens 2529 / 2268; Grok-1-shaped 2048
// tokens 2933 / 2880, 4096 tokens 5787 / 6032; one GPU's 8-way share of Grok-1 4096 tokens
// 718 / 700, 6144 tokens 1109 / 1084. The down projection keeps 64-row tiles up to 1536
// (Mixtral-shaped 2048 tokens 464 against 635 us with 256-row tiles).
int prefill_token_blocks(int P, int E, bool gateup) {
#ifdef W4A8_PREFILL_TB
  (void)P; (void)E; (void)gateup;
  return W4A8_PREFILL_TB;   // 2, 4 or 16
#endif
  const int mean = (P + E - 1) / E;
  return mean <= 48 ? 2 : (mean <= (gateup ? 511 : 1536) ? 4 : 16);
}

// Split of the down projection's reduction. Gate|up needs the whole K (its epilogue forms
// the activation). The down projection of a small grid (few M-tiles: batches of a few
// hundred tokens) is split into K-slices of at least 8 k-steps until about two workgroups
// per CU hold work, as long as the extra partial sums' round trip (8 bytes per row, channel
// and slice) stays under a quarter of the weight bytes; the combine adds them in slice
// order. Measured (Mixtral-shaped down + combine): 65 tokens 128 -> 91 us and 128 tokens
// 128 -> 95 us with 4 slices; 512 tokens 194 -> 228 us with 4 slices, hence the limit.
void plan_prefill(MoeGemmParams& p, bool gateup) {
  p.ksplit = 1;
  p.kslice = p.K;
  if (gateup) return;
  const int pm = 16 * prefill_token_blocks(p.P, p.E, false);
  const int est_mtiles = std::max((p.P + pm - 1) / pm, std::min(p.E, p.P));   // M-tiles holding rows
  const long tiles = (long)est_mtiles * ((p.Nw + kPN - 1) / kPN);
  const long want = 2L * device_cus();
  const int steps = p.K / 128;
  const double weight_bytes = (double)std::min(p.E, p.P) * p.Nw * (p.K / 2);
  const double slice_bytes = 8.0 * p.P * p.Nw;              // one more slice's partials, written and read
  const int by_traffic = 1 + (int)(0.25 * weight_bytes / slice_bytes);
  int ks = (int)std::min<long>((want + tiles - 1) / tiles, std::max(1, steps / 8));
  ks = std::min(ks, by_traffic);
  ks = std::max(1, std::min(ks, 16));
  const int per = (steps + ks - 1) / ks;                    // k-steps per slice
  p.kslice = per * 128;
  p.ksplit = (steps + per - 1) / per;
}

// Depth of the register rings of the 32- and 64-row tiles (0: the copy pipeline of the
// larger tiles). Measured, Mixtral-shaped gate|up at 65 tokens: 139.3 us with 32-row tiles
// and no ring, 128.6 with a ring of 4, 123.2 with 2; with 64-row tiles (256 tokens) 194.5 ->
// 187.1 us with a ring of 2 (3: 191.1, 4: 194.5). 128-row tiles were slower with a ring in
// either loop order (512 tokens: 408 us with the copies; K-parts outer 439-486 us, token
// blocks outer 464 / 484 / 486 us for rings of 2 / 3 / 4) and keep the copies; 256-row
// tiles have no registers left for one.
#ifndef W4A8_PREFILL_GROUPM_SMALL
#define W4A8_PREFILL_GROUPM_SMALL 16
#endif
#ifndef W4A8_PREFILL_GROUPM_LARGE
#define W4A8_PREFILL_GROUPM_LARGE 4
#endif
#ifndef W4A8_PREFILL_CHUNK_MUL
#define W4A8_PREFILL_CHUNK_MUL 1
#endif
#ifndef W4A8_PREFILL_RING2
#define W4A8_PREFILL_RING2 2
#endif
#ifndef W4A8_PREFILL_RING4
#define W4A8_PREFILL_RING4 2
#endif
// Waves of the 256-row tiles' gate|up workgroup: 8 (two per SIMD, 32 weight rows and 128
// accumulators per lane each) rather than 4 (one per SIMD, 64 weight rows, 256 accumulators):
// the same tile and traffic, and a second wave to issue while the other waits for the matrix
// core. Measured gate|up: Grok-1-shaped prefill 37.87 -> 37.29 ms, one GPU's 8-way share of
// Grok-1 4.92 -> 4.59 ms, Mixtral-shaped 8192 tokens 3.20 -> 2.98 ms; the down projection
// with 8 waves was mixed (Grok-1 18.18 -> 18.69 ms, the share 2.81 -> 2.78, Mixtral-shaped
// 8192 tokens 1.63 -> 1.56) and keeps 4.
#ifndef W4A8_PREFILL_NW16
#define W4A8_PREFILL_NW16 8
#endif
template <int TB>
static void launch_tb(const MoeGemmParams& p, bool gateup, hipStream_t st) {
  constexpr int kPM = 16 * TB;
  constexpr int R = TB == 2 ? W4A8_PREFILL_RING2 : (TB == 4 ? W4A8_PREFILL_RING4 : 0);
  // every expert's rows split into tiles of kPM; the count of tiles is at most P/kPM + E
  const int mtiles_upper = (p.P + kPM - 1) / kPM + p.E;
  const int ntiles = gateup ? (p.n_out + kPN / 2 - 1) / (kPN / 2) : (p.Nw + kPN - 1) / kPN;
  const size_t tiles = (size_t)mtiles_upper * ntiles * (gateup ? 1 : p.ksplit);
  // workgroups one XCD holds at once: its CUs times the workgroups per CU (two for the
  // 32- and 64-row tiles, one for the 256-row tiles)
  const int chunk = std::max(1, device_cus() / 8) * (TB <= 4 ? 2 : 1) * W4A8_PREFILL_CHUNK_MUL;
  const int groupm = TB <= 4 ? W4A8_PREFILL_GROUPM_SMALL : W4A8_PREFILL_GROUPM_LARGE;
  const unsigned grid = (unsigned)((tiles + 8 * (size_t)chunk - 1) / (8 * (size_t)chunk) * 8 * chunk);
  const size_t lds = 2 * TB * 4096;
  constexpr int NW = TB == 16 ? W4A8_PREFILL_NW16 : 4;    // gate|up waves
  const dim3 block(64 * NW);
  if (!gateup)
    hipLaunchKernelGGL((moe_prefill_kernel<false, 0, TB, R, 4>), dim3(grid), dim3(64 * 4), lds, st, p, mtiles_upper,
                       ntiles, groupm, chunk);
  else if (p.act_fn == 0)
    hipLaunchKernelGGL((moe_prefill_kernel<true, 0, TB, R, NW>), dim3(grid), block, lds, st, p, mtiles_upper,
                       ntiles, groupm, chunk);
  else if (p.act_fn == 1)
    hipLaunchKernelGGL((moe_prefill_kernel<true, 1, TB, R, NW>), dim3(grid), block, lds, st, p, mtiles_upper,
                       ntiles, groupm, chunk);
  else
    hipLaunchKernelGGL((moe_prefill_kernel<true, 2, TB, R, NW>), dim3(grid), block, lds, st, p, mtiles_upper,
                       ntiles, groupm, chunk);
}

void launch_moe_prefill(const MoeGemmParams& p, bool gateup, hipStream_t st) {
  const int tb = prefill_token_blocks(p.P, p.E, gateup);
  if (tb == 2) launch_tb<2>(p, gateup, st);
  else if (tb == 4) launch_tb<4>(p, gateup, st);
  else launch_tb<16>(p, gateup, st);
}

}  // namespace w4a8
