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
// Which matrix core: the fp16 MFMA (16x16x32) on the exact values (common.h: the fp8
// MFMA's sums are not exact; E4M3 values and int4 codes are exact in fp16).
//
// Mapping. A workgroup = 8 waves on one expert and one K-slice. The activation rows of
// the expert (at most 32 per pass: two 16-column tiles; an expert with more rows takes
// another pass over its weights, read again) for a K-chunk are staged in LDS as their
// E4M3 bytes (16 rows x 4096 K in 64 KB, so up to 16 rows the whole reduction of
// Mixtral's gate|up is one chunk, with no restaging barrier mid-stream), in the order the
// MFMA B operand is read (one ds_read_b128 per lane covers two instructions, 1 KB per
// wave without bank conflicts), and widened to fp16 in registers. Each wave owns two blocks of 16
// weight rows (gate rows n..n+15 and up rows I+n..I+n+15, or two blocks of down rows) and
// streams them with 16-byte buffer loads, kDepth k-steps (of 128) ahead, without a break
// at LDS chunk boundaries. The weights are in the tiled layout (w4_tile): one load
// instruction of a wave fetches one contiguous 1 KB tile (16 rows x 128 K), and a wave's
// whole stream over K is contiguous.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace w4a8 {

// Tuning knobs (defaults chosen by measurement on MI355X):
//   W4A8_DECODE_DEPTH     k-steps of weights in flight per wave (LDS chunks hold multiples)
//   W4A8_DECODE_NT_LOADS  stream the weights with the nontemporal hint (on by default: they are
//                         read once; whole graph-captured layer steps, us, without / with it:
//                         Mixtral-shaped 32 tokens 142.5 / 126.6, 16 tokens 140.1 / 123.4, 48 tokens
//                         151.5 / 136.0; Grok-1-shaped 438.5 / 397.8; one GPU's 8-way share 73.9 / 69.4)
//   W4A8_DECODE_BODY      k-steps per unrolled loop body
#ifndef W4A8_DECODE_DEPTH
#define W4A8_DECODE_DEPTH 4
#endif
#ifndef W4A8_DECODE_NT_LOADS
#define W4A8_DECODE_NT_LOADS 1
#endif
#ifndef W4A8_DECODE_BODY
#define W4A8_DECODE_BODY 16
#endif
constexpr int kDepth = W4A8_DECODE_DEPTH;
constexpr int kBody = W4A8_DECODE_BODY;                    // k-steps per unrolled loop body
constexpr int kWaitVmcnt0 = 0x0F70;                        // s_waitcnt vmcnt(0) (expcnt, lgkmcnt: no wait)
static_assert(kBody % kDepth == 0, "the loop body holds whole rounds");
// an LDS chunk holds at least one round of k-steps for the most column tiles (else the
// chunk loop could not advance)
static_assert(kDecodeLds / (16 * kDecodeMaxTiles) >= 128 * kDepth, "LDS chunk below one round");
constexpr int kWeightLoadAux = W4A8_DECODE_NT_LOADS ? 2 : 0;   // cache-policy bits: nt
__device__ __forceinline__ uint32_t word_of(const uint4& q, int m) {
  return m == 0 ? q.x : (m == 1 ? q.y : (m == 2 ? q.z : q.w));
}

// Raw buffer loads: an offset at or past the resource's size returns zeros and moves no
// data, so the weight stream below issues the same loads every step (no branches around
// loads, which would make the compiler drain every outstanding load before each use).
constexpr uint32_t kOutOfRange = 0x80000000u;

// A lane's fixed offset plus the k-step's (a wave-uniform scalar, added by the load): no
// per-lane arithmetic per load. Past the wave's K-range the scalar part is kOutOfRange.
__device__ __forceinline__ uint4 buf_ld16_step(__amdgpu_buffer_rsrc_t r, uint32_t voff, int step, int steps) {
  const uint32_t soff = step < steps ? (uint32_t)step * kTileBytes : kOutOfRange;
  return __builtin_bit_cast(
      uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, __builtin_amdgcn_readfirstlane(soff), kWeightLoadAux));
}


// One k-step (128 K) of one wave: 4 MFMAs of K = 32 per weight block and column tile
// (the first nt of NT tiles). B comes from the E4M3 LDS chunk: per (tile, k-step) two
// 1 KB halves, half h holding lane (c, g)'s codes 32 g + 16 h .. +16 of token column c
// (sub-steps 2h and 2h + 1), widened to fp16 in registers.
template <int NT>
__device__ __forceinline__ void mma_step(const uint4& a0, const uint4& a1, const uint8_t* lds, int s, int S, int nt,
                                         int lane, uint32_t mlo, uint32_t mhi, v4f* acc0, v4f* acc1) {
  // tile 0's two halves are read first (their latency runs under the conversions)
  uint4 b0[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) b0[h] = *reinterpret_cast<const uint4*>(lds + (s * 2 + h) * 1024 + lane * 16);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const v8h A0 = int4x8_to_f16(word_of(a0, m), mlo, mhi);
    const v8h A1 = int4x8_to_f16(word_of(a1, m), mlo, mhi);
    const uint4& bh = b0[m >> 1];
    const v8h B0 = (m & 1) ? e4m3x8_to_f16(bh.z, bh.w) : e4m3x8_to_f16(bh.x, bh.y);
    acc0[0] = mfma_f16(A0, B0, acc0[0]);
    acc1[0] = mfma_f16(A1, B0, acc1[0]);
#pragma unroll
    for (int j = 1; j < NT; ++j) {
      if (j < nt) {
        const uint2 bj = *reinterpret_cast<const uint2*>(lds + ((j * S + s) * 2 + (m >> 1)) * 1024 + lane * 16 +
                                                         (m & 1) * 8);
        const v8h b = e4m3x8_to_f16(bj.x, bj.y);
        acc0[j] = mfma_f16(A0, b, acc0[j]);
        acc1[j] = mfma_f16(A1, b, acc1[j]);
      }
    }
  }
}

// Consume one k-step from the register ring, then refill the same registers with the
// k-step kDepth ahead (out-of-range offsets past this wave's K-range move no data).
template <int NT>
__device__ __forceinline__ void stream_step(uint4& q0, uint4& q1, __amdgpu_buffer_rsrc_t wr, uint32_t off0,
                                            uint32_t off1, int ST, int ST1, int gstep, const uint8_t* lds, int s,
                                            int S, int nt, int lane, uint32_t mlo, uint32_t mhi, v4f* acc0,
                                            v4f* acc1) {
  mma_step<NT>(q0, q1, lds, s, S, nt, lane, mlo, mhi, acc0, acc1);
  __builtin_amdgcn_sched_barrier(0);                        // keep the refill after the use
  const int nxt = gstep + kDepth;
  q0 = buf_ld16_step(wr, off0, nxt, ST);
  q1 = buf_ld16_step(wr, off1, nxt, ST1);
}

// The S k-steps of one LDS chunk against the column tiles (see mma_step). Full rounds of
// kDepth k-steps issue a load for every step they consume (no branch around any load);
// only the last chunk can end with a partial round, which issues no loads. The compiler
// drains all outstanding loads at every loop header, so the k-steps run in unrolled
// bodies of kBody steps (precise waits inside), then in rounds of kDepth.
template <int NT>
__device__ __forceinline__ void stream_chunk(uint4 (&q0)[kDepth], uint4 (&q1)[kDepth], __amdgpu_buffer_rsrc_t wr,
                                             uint32_t off0, uint32_t off1, int ST, int ST1, int sg,
                                             const uint8_t* lds, int S, int nt, int lane, uint32_t mlo,
                                             uint32_t mhi, v4f* acc0, v4f* acc1) {
  static_assert(NT <= kDecodeMaxTiles, "more column tiles take passes");
  int s = 0;
  for (; s + kBody <= S; s += kBody) {
#pragma unroll
    for (int t = 0; t < kBody; ++t)
      stream_step<NT>(q0[t % kDepth], q1[t % kDepth], wr, off0, off1, ST, ST1, sg + s + t, lds, s + t, S, nt, lane,
                      mlo, mhi, acc0, acc1);
  }
  for (; s + kDepth <= S; s += kDepth) {
#pragma unroll
    for (int t = 0; t < kDepth; ++t)
      stream_step<NT>(q0[t], q1[t], wr, off0, off1, ST, ST1, sg + s + t, lds, s + t, S, nt, lane, mlo, mhi, acc0,
                      acc1);
  }
  const int rem = S - s;
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (d < rem) mma_step<NT>(q0[d], q1[d], lds, s + d, S, nt, lane, mlo, mhi, acc0, acc1);
}

// MULTI: an expert may hold more rows than MAXT column tiles; the workgroup then takes them
// in passes of 16 * MAXT rows, streaming its weights once per pass (without MULTI the
// kernel takes up to 16 * MAXT rows per expert).
template <bool GATEUP, int MAXT, bool MULTI>
__global__ __launch_bounds__(kDecodeWaves * kWave) void moe_decode_kernel(MoeGemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());   // wave-uniform (scalar) index
  int bid = blockIdx.x;
  const int group = bid % p.groups; bid /= p.groups;
  const int slice = bid % p.ksplit;
  const int e = bid / p.ksplit;
  const int k_begin = slice * p.kslice;
  const int k_end = min(p.K, k_begin + p.kslice);

  // weight row blocks of this wave: gate|up -> (cb, n_out/16 + cb); down -> (2cb, 2cb + 1)
  const int nthr = blockDim.x;                              // p.waves waves
  const int cb = group * p.waves + wave;
  const int blk0 = GATEUP ? cb : 2 * cb;
  const int blk1 = GATEUP ? (p.n_out / 16 + cb) : 2 * cb + 1;
  const bool has_work = blk0 * 16 < (GATEUP ? p.n_out : p.Nw);
  const bool has1 = GATEUP || blk1 * 16 < p.Nw;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t row_bytes = (uint32_t)p.K / 2;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const uint8_t*>(p.w) + (size_t)e * p.Nw * row_bytes), (short)0,
      (int)(p.Nw * row_bytes), 0x00020000);
  // tiled weights: the 1 KB tile (16 rows x 128 K) of a block and k-step, in lane order
  const uint32_t off0 = (uint32_t)(blk0 * 16) * row_bytes + (k_begin / 128) * kTileBytes + lane * 16;
  const uint32_t off1 = (uint32_t)((has1 ? blk1 : blk0) * 16) * row_bytes + (k_begin / 128) * kTileBytes + lane * 16;
  const int ST = has_work ? (k_end - k_begin) >> 7 : 0;    // k-steps of 128 this wave streams
  const int ST1 = has1 ? ST : 0;

  v4f acc0[MAXT], acc1[MAXT];
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    acc0[j] = v4f{0.f, 0.f, 0.f, 0.f}; acc1[j] = acc0[j];
  }
  // nibble masks held in registers (one v_bitop3 per mask and word)
  uint32_t mlo = 0x0F0F0F0Fu, mhi = 0xF0F0F0F0u;
  asm volatile("" : "+v"(mlo), "+v"(mhi));

  // prefetch the first kDepth k-steps (before the routing is read: they do not depend on
  // it); the stream runs on across chunk boundaries
  uint4 q0[kDepth], q1[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    q0[d] = buf_ld16_step(wr, off0, d, ST);
    q1[d] = buf_ld16_step(wr, off1, d, ST1);
  }
  const int seg0 = p.offsets[e];
  const int cnt_all = p.offsets[e + 1] - seg0;
  if (cnt_all <= 0) return;                                 // untouched expert: no more weight traffic
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.act, (short)0, (int)((GATEUP ? p.P / 2 : p.P) * p.K), 0x00020000);
  for (int c0 = 0;; c0 += 16 * MAXT) {
    const int cnt = MULTI ? min(cnt_all - c0, 16 * MAXT) : cnt_all;   // this pass's rows
    const int rs0 = seg0 + c0;                                // its first sorted row
    const int nt = min((cnt + 15) >> 4, MAXT);                // column tiles holding rows
    const int kc_max = ((p.lds_bytes / (16 * nt)) / (128 * kDepth)) * (128 * kDepth);   // E4M3 rows of 16*nt tokens
    // Staging sources. A thread's staging slots all sit at lane tid % 64 of their 64-slot
    // block, so it always stages column c = tid % 16 of a tile: the activation row behind
    // column c of each tile is looked up once here (a byte offset into act, or out of range
    // for a column past the expert's rows: the buffer load then returns zeros).
    uint32_t srow[MAXT];
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      const int col = j * 16 + (tid & 15);
      const int r = GATEUP ? (p.sorted_pair[rs0 + min(col, cnt - 1)] >> 1) : rs0 + min(col, cnt - 1);
      srow[j] = col < cnt ? (uint32_t)r * (uint32_t)p.K : kOutOfRange;
    }
    int sg = 0;                                               // k-steps consumed so far
    for (int kc0 = k_begin; kc0 < k_end; kc0 += kc_max) {
      const int klen = min(kc_max, k_end - kc0);
      const int S = klen >> 7;                                // k-steps in this chunk
      if (kc0 != k_begin) lds_barrier();                      // LDS reuse
      // ---- stage the activation rows of this chunk as E4M3 bytes. Unit = 16 codes of one
      //      row: (tile j, k-step s, half h, lane c + 16 g) -> 16 bytes at
      //      ((j*S + s)*2 + h)*1024 + lane*16, codes 32 g + 16 h .. +16 of the k-step.
      {
        // Buffer loads straight into LDS (no registers, so all of a wave's units are in
        // flight at once): one instruction moves a 64-unit block (tile j, k-step st, half h)
        // = v / 64, lane (c + 16 gg) to v * 16. Lanes of a column past the expert's rows
        // load out of range, which writes zeros.
        const int blocks = nt * S * 2;
        for (int blk = wave; blk < blocks; blk += nthr / kWave) {
          const int h = blk & 1, js = blk >> 1;
          const int j = js / S, st = js - j * S;
          uint32_t base = srow[0];
#pragma unroll
          for (int jj = 1; jj < MAXT; ++jj) base = j == jj ? srow[jj] : base;
          const uint32_t kk = (uint32_t)(st * 128 + (lane >> 4) * 32 + h * 16);
          const uint32_t off = base != kOutOfRange ? base + kc0 + kk : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16,
                                                   off, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);            // this wave's LDS loads (vmcnt, not lgkmcnt)
      }
      lds_barrier();
      // ---- stream the weights of this chunk
      if (has_work) {
        stream_chunk<MAXT>(q0, q1, wr, off0, off1, ST, ST1, sg, lds, S, nt, lane, mlo, mhi, acc0, acc1);
      }
      sg += S;
    }
    if (!MULTI && !has_work) return;
    if (has_work) {
      // ---- epilogue: lane holds rows 4g..4g+3 of each block, column (token row) j*16 + i
      const float* ws = p.w_scale + (size_t)e * p.Nw;
      const float k0 = p.s_act;
#pragma unroll
      for (int j = 0; j < MAXT; ++j) {
        const int col = j * 16 + i;
        if (j >= nt || col >= cnt) continue;
        const int r = rs0 + col;
        if (GATEUP) {
          const int nb = cb * 16 + 4 * g;
          const float4 sg4 = *reinterpret_cast<const float4*>(ws + nb);
          const float4 su4 = *reinterpret_cast<const float4*>(ws + p.n_out + nb);
          float gv[4], uv[4], av[4];
          const float sgv[4] = {sg4.x, sg4.y, sg4.z, sg4.w}, suv[4] = {su4.x, su4.y, su4.z, su4.w};
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            gv[v] = acc0[j][v] * k0 * sgv[v];
            uv[v] = acc1[j][v] * k0 * suv[v];
            av[v] = requant_value_rt(gv[v], uv[v], p.s_a, p.inv_s_a, p.act_fn);
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
            o.x = acc[0] * k0 * sw.x;
            o.y = acc[1] * k0 * sw.y;
            o.z = acc[2] * k0 * sw.z;
            o.w = acc[3] * k0 * sw.w;
            *reinterpret_cast<float4*>(p.partial + ((size_t)slice * p.P + r) * p.n_out + nb) = o;
          }
        }
      }
    }
    if (!MULTI || c0 + 16 * MAXT >= cnt_all) break;
    // the next pass: LDS reuse, the weight stream again from the first k-step, fresh sums
    lds_barrier();
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      q0[d] = buf_ld16_step(wr, off0, d, ST);
      q1[d] = buf_ld16_step(wr, off1, d, ST1);
    }
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      acc0[j] = v4f{0.f, 0.f, 0.f, 0.f}; acc1[j] = acc0[j];
    }
  }
}

// The streaming kernel takes up to 80 tokens, the tiled kernel above. Measured whole layer
// steps, us, streaming (two column tiles, passes of 32 rows, nontemporal weight stream)
// against tiled, with the router as drawn and with a per-expert bias (the most rows of an
// expert in brackets): 80 tokens Mixtral-shaped 158.9 against 168.3 (28), 176.3 against
// 183.8 (48); one GPU's 8-way share of Grok-1 85.8 against 99.1 (24), 101.1 against 102.7
// (37); Grok-1-shaped 490.8 against 492.8 (24), 517.6 against 527.7 (37). At 88 and 96
// tokens the biased routers (largest experts of 52 to 56 rows, two passes) make streaming
// lose by 9-12%; at 128 tokens it loses by 15-20% with either router.
constexpr int kStreamMaxTokens = 80;
bool decode_fits(int T) { return T <= kStreamMaxTokens; }

// CUs of the current device, looked up once per device. Each slot is an atomic, so calls
// from several host threads are safe (every writer stores the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Fraction of the workgroup slots busy over the rounds that `units` workgroups take.
static double round_fill(long units, long slots) {
  const long rounds = (units + slots - 1) / slots;
  return rounds > 0 ? (double)units / (double)(rounds * slots) : 1.0;
}

// Down projection: split K into slices of at most one E4M3 LDS chunk for 16 rows (4096 K),
// balanced to whole k-steps (a chunk may end with a partial round), and wmax..4 waves per
// workgroup (32 channels each): the combination that fills the rounds of workgroup slots
// best, preferring fewer slices (each adds a partial sum to the combine) and then more
// waves (more loads in flight). Returns its round fill.
static double plan_down(MoeGemmParams& p, int wmax, long experts, long slots) {
  const int step = 128;
  const int kmax = (kDecodeLds / 16) / (128 * kDepth) * (128 * kDepth);
  const int first = (p.K + kmax - 1) / kmax;
  double best = -1.0;
  for (int ks = first; ks <= 4 * first; ++ks) {
    const int kslice = ((p.K + ks - 1) / ks + step - 1) / step * step;
    if ((p.K + kslice - 1) / kslice != ks) continue;        // rounding merged two slices
    for (int w = wmax; w >= std::min(4, kDecodeWaves); --w) {
      const int groups = (p.n_out + 32 * w - 1) / (32 * w);
      const double fill = round_fill((long)groups * ks * experts, slots);
      if (fill > best + 0.02) {
        best = fill;
        p.kslice = kslice;
        p.ksplit = ks;
        p.waves = w;
        p.groups = groups;
      }
    }
  }
  return best;
}

// Above 32 tokens the kernel keeps two column tiles and takes an expert's rows in passes of
// 32 (a second pass only for an expert with more than 32 rows). Against four column tiles
// (which needed ~180 registers per lane and so 4-wave workgroups), measured gate|up / down,
// us: Mixtral-shaped 33 tokens 96.4 / 49.7 -> 86.7 / 42.3, 40 tokens 100.4 / 50.2 -> 87.8 /
// 42.9, 48 tokens 105.6 / 50.6 -> 91.1 / 49.1; Grok-1-shaped 40 tokens 299.7 / 171.8 -> 272.2
// / 161.5; one GPU's 8-way share of Grok-1 at 48 tokens 43.7 / 34.1 -> 39.6 / 28.5.
void plan_decode(MoeGemmParams& p, bool gateup) {
  // an expert never holds more rows than there are tokens (its two slots differ)
  const int T = p.P / 2;
  p.max_tiles = T <= 16 ? 1 : 2;
  p.lds_bytes = kDecodeLds;
  if (gateup) {
    // The whole reduction (the fused epilogue needs it). Waves per workgroup (16 channels
    // each): 8, 7 or 4, the count that fills the rounds of workgroup slots (two per CU)
    // best; a partly empty round leaves HBM bandwidth unused. Mixtral-shaped I = 14336 =
    // 7 * 2048: 7 waves give 1024 workgroups instead of 896 for 512 slots; one GPU's
    // 8-way share of Grok-1 (I = 4096): 4 waves give 512 instead of 256. (5 and 6 waves
    // measured 15-40% slower than these at both shapes, 7 slow at the second.)
    p.kslice = p.K;
    p.ksplit = 1;
    const long experts = std::min(p.E, 2 * T);              // experts that can hold rows
    const long slots = 2L * device_cus();
    double best = -1.0;
    for (int w : {8, 7, 4}) {
      if (w > kDecodeWaves) continue;
      const int groups = (p.n_out + 16 * w - 1) / (16 * w);
      const double fill = round_fill((long)groups * experts, slots);
      if (fill > best + 1e-9) {
        best = fill;
        p.waves = w;
        p.groups = groups;
      }
    }
  } else {
    // A grid of several rounds takes at most 6 waves when that fills as well (Grok-1 shape,
    // 8 slices: 8 waves in 3 rounds 182.6 us, 6 waves in 4 rounds 162.0 us, 4 waves 167.6
    // us; a single round keeps 8: Mixtral shape 50.0 us, 58.6 with 6).
    const long experts = std::min(p.E, 2 * T);
    const long slots = 2L * device_cus();
    const double fill = plan_down(p, kDecodeWaves, experts, slots);
    if ((long)p.groups * p.ksplit * experts > slots && p.waves > 6) {
      MoeGemmParams q = p;
      if (plan_down(q, std::min(6, kDecodeWaves), experts, slots) >= fill - 0.02) {
        p.kslice = q.kslice; p.ksplit = q.ksplit; p.waves = q.waves; p.groups = q.groups;
      }
    }
  }
}

template <bool GATEUP>
static void launch_decode_t(const MoeGemmParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)(p.groups * p.ksplit * p.E);
  const dim3 block(p.waves * kWave);
  // an expert holds at most T rows (its two slots differ); more than the column tiles
  // take passes
  const bool multi = p.P / 2 > 16 * p.max_tiles;
  if (p.max_tiles <= 1)
    hipLaunchKernelGGL((moe_decode_kernel<GATEUP, 1, false>), dim3(grid), block, p.lds_bytes, st, p);
  else if (!multi)
    hipLaunchKernelGGL((moe_decode_kernel<GATEUP, 2, false>), dim3(grid), block, p.lds_bytes, st, p);
  else
    hipLaunchKernelGGL((moe_decode_kernel<GATEUP, 2, true>), dim3(grid), block, p.lds_bytes, st, p);
}

void launch_moe_decode(const MoeGemmParams& p, bool gateup, hipStream_t st) {
  if (gateup) launch_decode_t<true>(p, st);
  else launch_decode_t<false>(p, st);
}

// ---------------------------------------------------------------------------- combine
// out[t][n] = w0 * Y0 + w1 * Y1, Y = sum over split-K slices in slice order; fp32, then
// bf16 (nearest even) or fp32. 4 channels per thread, 64 threads per workgroup (a few
// MB of partials: many small workgroups), the slices' loads issued up to 8 at a time
// before they are added (still in slice order).
constexpr int kCombineThreads = 64;

template <int BATCH>   // slices loaded per round: 1 for an unsplit reduction, else 8
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ partial, int ksplit, int P,
                                                                 int H, const int32_t* __restrict__ pair_pos,
                                                                 const float* __restrict__ topk_w, int chunks,
                                                                 int out_bf16, void* __restrict__ out) {
  const int t = blockIdx.x / chunks;
  const int n = ((blockIdx.x % chunks) * kCombineThreads + threadIdx.x) * 4;
  if (n >= H) return;
  const int r0 = pair_pos[2 * t], r1 = pair_pos[2 * t + 1];
  const float w0 = topk_w[2 * t], w1 = topk_w[2 * t + 1];
  float4 y0 = make_float4(0.f, 0.f, 0.f, 0.f), y1 = y0;
  for (int s0 = 0; s0 < ksplit; s0 += BATCH) {
    float4 a[BATCH], b[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int s = min(s0 + u, ksplit - 1);              // in range; extra loads are not added
      a[u] = *reinterpret_cast<const float4*>(partial + ((size_t)s * P + r0) * H + n);
      b[u] = *reinterpret_cast<const float4*>(partial + ((size_t)s * P + r1) * H + n);
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (s0 + u < ksplit) {
        y0.x += a[u].x; y0.y += a[u].y; y0.z += a[u].z; y0.w += a[u].w;
        y1.x += b[u].x; y1.y += b[u].y; y1.z += b[u].z; y1.w += b[u].w;
      }
    }
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
  const int chunks = (H / 4 + kCombineThreads - 1) / kCombineThreads;
  const dim3 grid((unsigned)((size_t)T * chunks));
  if (ksplit == 1)
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(kCombineThreads), 0, st, partial, ksplit, P, H, pair_pos, topk_w,
                       chunks, out_bf16 ? 1 : 0, out);
  else
    hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(kCombineThreads), 0, st, partial, ksplit, P, H, pair_pos, topk_w,
                       chunks, out_bf16 ? 1 : 0, out);
}

}  // namespace w4a8
