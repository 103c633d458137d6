// moe_route_sort kernels: top-2 routing on unquantized router logits
// (num_local_experts / num_experts_per_tok and the router gate kept out of
// quantization, config.json of the page "ROCm: enable trillion-parameter MoE models
// with INT4-FP8 single node") and the expert-contiguous, stable order of the
// (token, slot) pairs that the grouped GEMMs consume.
//
// One token per thread. Ranks inside a block come from wave ballots (no
// order-dependent atomics), so the order of pairs inside an expert's segment is the
// pair order p = 2t + slot, and every run gives the same bytes.
#include "common.h"
#include "kernels.h"

namespace w4a8 {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;

struct Top2 {
  int i0, i1;
  float w0, w1;
};

// Higher logit first; on equal logits the lower expert id first (the scan runs over
// ascending ids and only a strictly larger logit displaces).
__device__ __forceinline__ Top2 top2_of_row(const float* __restrict__ row, int E) {
  float b0 = row[0], b1 = row[1];
  int i0 = 0, i1 = 1;
  if (b1 > b0) { float tf = b0; b0 = b1; b1 = tf; i0 = 1; i1 = 0; }
  for (int e = 2; e < E; ++e) {
    const float l = row[e];
    if (l > b0) { b1 = b0; i1 = i0; b0 = l; i0 = e; }
    else if (l > b1) { b1 = l; i1 = e; }
  }
  Top2 r;
  r.i0 = i0; r.i1 = i1;
  // softmax over all experts, keep two, renormalise == 1 / (1 + exp(l1 - l0))
  r.w0 = 1.0f / (1.0f + expf(b1 - b0));
  r.w1 = 1.0f - r.w0;
  return r;
}

// Per-expert rank of this thread's token among the earlier tokens of the block that
// route to the same expert (either slot), plus each wave's per-expert totals in wt.
// Returns the in-wave ranks for the thread's two experts.
__device__ __forceinline__ void wave_ranks(bool valid, int i0, int i1, int E, int* wt /*[waves][E]*/,
                                           int& r0, int& r1) {
  const int lane = lane_id(), w = wave_id();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  r0 = r1 = 0;
  for (int e = 0; e < E; ++e) {
    const bool f = valid && (i0 == e || i1 == e);
    const uint64_t m = __ballot(f);
    const int before = __popcll(m & below);
    if (valid && i0 == e) r0 = before;
    if (valid && i1 == e) r1 = before;
    if (lane == 0) wt[w * E + e] = __popcll(m);
  }
}

// Single-block path (T <= 256): everything in one launch, no workspace. Workgroups past
// the first, when there are any, quantize x to E4M3 (fp8_quant_static's code) meanwhile.
__global__ __launch_bounds__(kRouteThreads) void route_small_kernel(
    const float* __restrict__ logits, int T, int E, int32_t* __restrict__ ids, float* __restrict__ tw,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos, const uint16_t* __restrict__ x, int64_t xn, float s_x,
    uint8_t* __restrict__ xq) {
  if (blockIdx.x > 0) {
    fp8_quant_span(x, xn, s_x, xq, (blockIdx.x - 1) * (int64_t)kRouteThreads + threadIdx.x,
                   (int64_t)(gridDim.x - 1) * kRouteThreads);
    return;
  }
  extern __shared__ int smem[];
  int* wt = smem;                              // [waves][E]
  int* off = smem + kRouteWaves * E;           // [E+1]
  const int t = threadIdx.x;
  const bool valid = t < T;
  Top2 r = {0, 1, 0.f, 0.f};
  if (valid) {
    r = top2_of_row(logits + (size_t)t * E, E);
    ids[2 * t] = r.i0; ids[2 * t + 1] = r.i1;
    tw[2 * t] = r.w0; tw[2 * t + 1] = r.w1;
  }
  int q0, q1;
  wave_ranks(valid, r.i0, r.i1, E, wt, q0, q1);
  __syncthreads();
  if (E <= kWave) {
    // wave 0, lane e: expert e's count, then an inclusive scan over the lanes
    if (t < kWave) {
      int c = 0;
      if (t < E)
        for (int w = 0; w < kRouteWaves; ++w) c += wt[w * E + t];
      int incl = c;
      for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (t >= d) incl += v;
      }
      if (t < E) {
        off[t] = incl - c;
        counts[t] = c;
        offsets[t] = incl - c;
      }
      if (t == E - 1) {
        off[E] = incl;
        offsets[E] = incl;
      }
    }
  } else if (t == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      int c = 0;
      for (int w = 0; w < kRouteWaves; ++w) c += wt[w * E + e];
      counts[e] = c;
      offsets[e] = run;
      run += c;
    }
    off[E] = run;
    offsets[E] = run;
  }
  __syncthreads();
  if (!valid) return;
  const int w = wave_id();
  int p0 = off[r.i0] + q0, p1 = off[r.i1] + q1;
  for (int v = 0; v < w; ++v) { p0 += wt[v * E + r.i0]; p1 += wt[v * E + r.i1]; }
  sorted_pair[p0] = 2 * t; pair_pos[2 * t] = p0;
  sorted_pair[p1] = 2 * t + 1; pair_pos[2 * t + 1] = p1;
}

// Multi-block path, phase 1: top-2 per token, block histogram -> cnt[b][E].
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int32_t* __restrict__ ids, float* __restrict__ tw,
    int32_t* __restrict__ cnt) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kRouteThreads + threadIdx.x;
  if (t < T) {
    Top2 r = top2_of_row(logits + (size_t)t * E, E);
    ids[2 * t] = r.i0; ids[2 * t + 1] = r.i1;
    tw[2 * t] = r.w0; tw[2 * t + 1] = r.w1;
    atomicAdd(&hist[r.i0], 1);                 // integer counts: order-independent
    atomicAdd(&hist[r.i1], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) cnt[(size_t)blockIdx.x * E + e] = hist[e];
}

// Phase 2 (one block): counts, offsets, and each block's base position per expert.
// Thread (s, e) owns expert e over a segment of consecutive blocks (256 / E segments),
// so the serial walk per thread is nb / (256 / E) blocks and each step's loads, over
// consecutive e, are contiguous. Integer sums: the result does not depend on the split.
__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(
    int nb, int E, const int32_t* __restrict__ cnt, int32_t* __restrict__ base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  extern __shared__ int sm[];
  int* part = sm;                              // [S][E]: segment sums, then exclusive scans
  int* tot = sm + kRouteThreads;               // [E]
  int* off = tot + E;                          // [E]
  const int S = kRouteThreads / E;             // E <= 256, so S >= 1
  const int L = (nb + S - 1) / S;              // blocks per segment
  const int t = threadIdx.x, s = t / E, e = t - s * E;
  const bool act = s < S;
  const int b0 = s * L, b1 = min(nb, b0 + L);
  if (act) {
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += cnt[(size_t)b * E + e];
    part[t] = sum;
  }
  __syncthreads();
  if (t < E) {
    int run = 0;
    for (int q = 0; q < S; ++q) { const int v = part[q * E + t]; part[q * E + t] = run; run += v; }
    tot[t] = run;
    counts[t] = run;
  }
  __syncthreads();
  if (t < kWave) {
    // wave 0: exclusive scan of the totals over the experts, 64 at a time
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
      const int v = c0 + t < E ? tot[c0 + t] : 0;
      int incl = v;
      for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (t >= d) incl += u;
      }
      if (c0 + t < E) { off[c0 + t] = carry + incl - v; offsets[c0 + t] = carry + incl - v; }
      carry += __shfl(incl, kWave - 1);
    }
    if (t == 0) offsets[E] = carry;
  }
  __syncthreads();
  if (act) {
    int run = off[e] + part[t];
    for (int b = b0; b < b1; ++b) {
      base[(size_t)b * E + e] = run;
      run += cnt[(size_t)b * E + e];
    }
  }
}

// Phase 3: stable scatter of the block's pairs.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    int T, int E, const int32_t* __restrict__ ids, const int32_t* __restrict__ base,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  extern __shared__ int wt[];                  // [waves][E]
  const int t = blockIdx.x * kRouteThreads + threadIdx.x;
  const bool valid = t < T;
  int i0 = 0, i1 = 1;
  if (valid) { i0 = ids[2 * t]; i1 = ids[2 * t + 1]; }
  int q0, q1;
  wave_ranks(valid, i0, i1, E, wt, q0, q1);
  __syncthreads();
  if (!valid) return;
  const int w = wave_id();
  const int32_t* bb = base + (size_t)blockIdx.x * E;
  int p0 = bb[i0] + q0, p1 = bb[i1] + q1;
  for (int v = 0; v < w; ++v) { p0 += wt[v * E + i0]; p1 += wt[v * E + i1]; }
  sorted_pair[p0] = 2 * t; pair_pos[2 * t] = p0;
  sorted_pair[p1] = 2 * t + 1; pair_pos[2 * t + 1] = p1;
}

size_t route_workspace_bytes(int T, int E) {
  if (T <= kRouteThreads) return 0;
  const size_t nb = (size_t)(T + kRouteThreads - 1) / kRouteThreads;
  return 2 * nb * (size_t)E * sizeof(int32_t);
}

void launch_route_sort(const float* logits, int T, int E, int32_t* ids, float* tw, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws, hipStream_t st,
                       const uint16_t* x, int64_t xn, float s_x, uint8_t* xq) {
  if (T <= kRouteThreads) {
    // with x: the quantization rides along in extra workgroups of the same launch
    const unsigned grid = 1 + (x && xn > 0 ? (unsigned)fp8_quant_blocks(xn) : 0u);
    const size_t lds = (size_t)(kRouteWaves * E + E + 1) * sizeof(int);
    hipLaunchKernelGGL(route_small_kernel, dim3(grid), dim3(kRouteThreads), lds, st, logits, T, E, ids, tw,
                       counts, offsets, sorted_pair, pair_pos, x, xn, s_x, xq);
    return;
  }
  if (x && xn > 0) launch_fp8_quant(x, xn, s_x, xq, st);
  const int nb = (T + kRouteThreads - 1) / kRouteThreads;
  int32_t* cnt = static_cast<int32_t*>(ws);
  int32_t* base = cnt + (size_t)nb * E;
  hipLaunchKernelGGL(route_topk_kernel, dim3(nb), dim3(kRouteThreads), E * sizeof(int), st, logits, T, E,
                     ids, tw, cnt);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), (kRouteThreads + 2 * E) * sizeof(int), st,
                     nb, E, cnt, base, counts, offsets);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(kRouteThreads), kRouteWaves * E * sizeof(int), st,
                     T, E, ids, base, sorted_pair, pair_pos);
}

}  // namespace w4a8
