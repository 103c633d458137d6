"""Benchmark of the W4A8 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one forward of the layer over one batch of synthetic tokens: one moe_layer_w4a8
call (the launches of moe_route_sort_quant, moe_gemm1_w4a8 and moe_gemm2_w4a8: routing and
x -> E4M3, gate|up, down + combine; checked byte-equal to those three calls); four
consecutive steps are captured in one HIP graph,
as a model's decode graph holds its consecutive layers, and exactly K steps are timed. Inputs
(packed weights, scales, x, logits) are resident in HBM before the timed region. The
packed weights are rotated over several copies when one copy would fit in the 256 MB
Infinity Cache, so that the HBM stream is measured. w4_pack + w4_tile (load time), the block-FP8
GEMV and the per-tensor FP8 (W8A8) linear are timed separately and reported in the same JSON line.

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense OCP-FP8 MFMA, published
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA, published
METRIC = "MoE layer tokens/s + % HBM peak (decode T=32), % fp8 MFMA peak (prefill)"
ACT_NAMES = {synth.ACT_SILU: "silu", synth.ACT_GELU_ERF: "gelu_erf", synth.ACT_GELU_TANH: "gelu_tanh"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # layer steps timed (prefill: at most 10). A timed run carries about 0.7 ms of fixed wall-clock
    # cost (the first graph launch, the closing synchronization): measured on one GPU, ms per
    # Mixtral-shaped step, 64 steps 0.138-0.144, 320 steps 0.131, 1024 steps 0.127, against
    # 0.125 per call timed with events inside one graph; Grok-1-shaped 0.410 / 0.410 / 0.407.
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_decode", choices=sorted(synth.MOE_CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block-gemv", action="store_true",
                    help="skip timing the block-FP8 GEMVs and the per-tensor FP8 linears")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the default decode workload, skip the prefill layer's line")
    ap.add_argument("--no-grok-decode", action="store_true",
                    help="with the default decode workload, skip the Grok-1-shaped decode layer's line")
    ap.add_argument("--no-tp8", action="store_true",
                    help="with the default decode workload, skip one GPU's 8-way share of the Grok-1 layer")
    ap.add_argument("--no-token-sweep", action="store_true",
                    help="with the default decode workload, skip the 32..1024-token sweep of the two GEMMs")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run a 1 GiB device-to-device copy (a known-size reference for HBM counters)")
    return ap.parse_args()


def static_scales(name):
    d = json.load(open(os.path.join(ROOT, "tests", "golden", "static_scales.json")))[name]
    return np.float32(float.fromhex(d["s_x_hex"])), np.float32(float.fromhex(d["s_a_hex"]))


def bf16_dev(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


# consecutive layer steps captured in one HIP graph: the 32 MoE layers of one Mixtral-8x7B
# decode forward (Grok-1 has 64). Measured on one GPU, 64 steps timed, ms per Mixtral- /
# Grok-1-shaped step: 32 steps per graph 0.142-0.147 / 0.410, 4 steps 0.149-0.153 / 0.422,
# 1 step 0.155 / 0.431.
STEPS_PER_GRAPH = 32

COUNTER_FILES = {"mixtral_decode": "moe_decode_mixtral_T32.json", "grok_decode": "moe_decode_grok_T32.json",
                 "grok_prefill": "moe_prefill_grok_T32768.json"}


def sources_sha256(paths):
    """sha256 over the kernel's source files, in order (a changed kernel voids its counters)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def counter_traffic(workload):
    """HBM bytes per gate|up launch from the committed rocprofv3 counters, or None when
    they were taken on another workload or on different kernel sources."""
    path = os.path.join(ROOT, "profiles", COUNTER_FILES.get(workload, "-"))
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("workload") != workload or sources_sha256(d["sources"]) != d["sources_sha256"]:
        return None
    return int(d["traffic_bytes_per_launch"])


def moe_bytes(cfg, counts):
    """Algorithmic HBM bytes of the layer and of the gate|up call (touched experts only)."""
    touched = int(np.count_nonzero(counts))
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    P = 2 * T
    w13 = touched * (2 * I * H // 2 + 2 * I * 4)
    w2 = touched * (H * I // 2 + H * 4)
    gemm1 = w13 + T * H + P * I                      # packed w13 + scales, x codes in, a codes out
    layer = w13 + w2 + T * H * 2 + T * E * 4 + T * H * (4 if cfg.out_f32 else 2)
    return layer, gemm1, touched


def gemm1_flops(cfg):
    """Multiply-add work of the gate|up call: every one of the 2T sorted rows against the
    2I weight rows of its expert, K = H."""
    return 2.0 * (2 * cfg.T) * (2 * cfg.I) * cfg.H


def cpu_baseline(cfg, s_x, s_a):
    """The oracle on the whole decode layer of the workload (every token, every expert):
    each expert's weights are packed by the oracle (timed apart, beside the GPU's w4_pack),
    and the timed part is the oracle's layer forward, which unpacks each expert's int4 rows
    in chunks and sums exactly in fp64."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    packed13, packed2, pack_s, pack_n = {}, {}, 0.0, 0
    for e in range(cfg.E):
        w13 = synth.moe_expert_weights(cfg, "w13", e)
        w2 = synth.moe_expert_weights(cfg, "w2", e)
        t0 = time.perf_counter()
        packed13[e] = oracle.w4_pack(w13)
        packed2[e] = oracle.w4_pack(w2)
        pack_s += time.perf_counter() - t0
        pack_n += w13.size + w2.size
        del w13, w2
    # whole layer forwards, repeated until about 10 s of host time (at most 3)
    runs, total = 0, 0.0
    while runs < 3 and (runs == 0 or total < 10.0):
        t0 = time.perf_counter()
        oracle.moe_forward(x, logits, s_x, lambda e: packed13[e], lambda e: packed2[e], cfg.act, s_a, cfg.out_f32,
                           E=cfg.E)
        total += time.perf_counter() - t0
        runs += 1
    dt = total / runs
    return {"oracle_w4_pack": {"weights": int(pack_n), "s": round(pack_s, 3),
                               "GB/s": round(pack_n * 3.5 / pack_s / 1e9, 3)},
            "value": float(cfg.T / dt), "unit": "tokens/s",
            "cores": int(max(1, blas_threads)), "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{cfg.T} of {cfg.T} tokens: the whole {cfg.name} layer (all {cfg.E} experts, fp64 oracle "
                      f"forward with per-expert chunked int4 unpacking and exact sums), {runs} runs, "
                      f"{total:.2f} s"}


def graph_call_us(torch, fn, iters):
    """Average GPU time of fn(i), i < iters, captured back to back in one graph and replayed
    between two HIP events on the current stream (the library launches on it)."""
    for i in range(5):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(st)
    g.replay()
    ev[1].record(st)
    torch.cuda.synchronize()
    del g
    return ev[0].elapsed_time(ev[1]) * 1e3 / iters


def bench_block_gemv(torch, W, dev, reps=16, iters=50):
    """block-FP8 GEMV at the projection shapes; weights rotated over `reps` copies."""
    out = {}
    for cfg in synth.BLOCK_CONFIGS.values():
        w = bf16_dev(torch, synth.block_weights(cfg), dev)
        q, S = W.fp8_block_quant(w)
        del w
        qs = [q.clone() for _ in range(reps)]
        x = bf16_dev(torch, synth.block_activations(cfg), dev)
        y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=dev)
        us = graph_call_us(torch, lambda i: W.fp8_block_linear(x, qs[i % reps], S, out=y), iters)
        nbytes = cfg.N * cfg.K + S.numel() * 4 + cfg.M * cfg.K * 2 + cfg.M * cfg.N * 2
        out[cfg.name] = {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1),
                         "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del qs
    return out


def bench_fp8_linear(torch, W, dev, reps=16, iters=50):
    """Per-tensor FP8 (W8A8) linear at the Grok-1 attention projection shapes: the call
    (x quantized to E4M3 and the GEMV, one launch) timed on the library's stream; weights rotated over
    `reps` copies (>= 590 MB, past the Infinity Cache)."""
    out = {}
    d = json.load(open(os.path.join(ROOT, "tests", "golden", "static_scales.json")))
    for cfg in synth.LINEAR_CONFIGS.values():
        s_x = float.fromhex(d[cfg.name]["s_x_hex"])
        w = bf16_dev(torch, synth.block_weights(cfg), dev)
        q, s = W.fp8_tensor_quant(w)
        s_w = float(s.item())
        del w
        qs = [q.clone() for _ in range(reps)]
        x = bf16_dev(torch, synth.block_activations(cfg), dev)
        y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(256, W.workspace_bytes(W.OP_FP8_LINEAR, cfg.M, cfg.N, cfg.K, 0)), dtype=torch.uint8,
                         device=dev)
        us = graph_call_us(torch, lambda i: W.fp8_linear_w8a8(x, s_x, qs[i % reps], s_w, out=y, ws=ws), iters)
        nbytes = cfg.N * cfg.K + cfg.M * cfg.K * 2 + cfg.M * cfg.N * 2     # weights, bf16 x in, bf16 y out
        out[cfg.name] = {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1),
                         "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del qs
    return out


def bench_kv_store(torch, W, dev, T=32, D=1024, slots_total=65536, iters=100):
    """FP8 KV cache store at the Grok-1 decode step (32 tokens, 8 key/value heads of 128),
    into a 64K-slot cache; the scales are the min_kv_scale floor (1.0)."""
    rng = np.random.default_rng(9)
    k = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(dev).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(dev).to(torch.bfloat16)
    slots = torch.from_numpy(rng.choice(slots_total, T, replace=False).astype(np.int32)).to(dev)
    kc = torch.zeros((slots_total, D), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    for _ in range(5):
        W.fp8_kv_cache_store(k, v, slots, 1.0, 1.0, kc, vc)
    torch.cuda.synchronize()
    # a few microseconds of GPU work: timed as `iters` calls captured in one graph, so the
    # Python binding's launch overhead stays out of the figure
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            W.fp8_kv_cache_store(k, v, slots, 1.0, 1.0, kc, vc)
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(st)
    g.replay()
    ev[1].record(st)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / iters
    return {"us": round(us, 3), "tokens": T, "row_elements": D, "timed": f"{iters} calls in one HIP graph"}


SWEEP_TOKENS = (32, 48, 80, 81, 128, 256, 512, 1024)


def token_sweep(torch, W, base, iters=20):
    """The two grouped GEMMs of the Mixtral-shaped layer at batch sizes around the switch
    from the streaming kernel (up to 80 tokens) to the tiled one: per T, each call's
    average time over back-to-back launches, its HBM rate (touched experts' weights and
    scales, activations in and out) and its matrix rate (routed rows only). The weights
    are rotated over two copies so that they stream from HBM."""
    import dataclasses
    dev = torch.device("cuda:0")
    s_x, s_a = static_scales(base.name)
    w13b = bf16_dev(torch, synth.moe_weights(base, "w13"), dev)
    w13, s13 = W.w4_pack(w13b, tiled=True)
    del w13b
    w2b = bf16_dev(torch, synth.moe_weights(base, "w2"), dev)
    w2, s2 = W.w4_pack(w2b, tiled=True)
    del w2b
    W13, W2 = [w13, w13.clone()], [w2, w2.clone()]
    H, I, E = base.H, base.I, base.E
    st = torch.cuda.current_stream()
    out = {}
    for T in SWEEP_TOKENS:
        cfg = dataclasses.replace(base, T=T)
        x = bf16_dev(torch, synth.activations(dataclasses.replace(base, T=max(T, 32)))[:T], dev)
        logits = torch.from_numpy(synth.router_logits(dataclasses.replace(base, T=max(T, 32)))[:T]).to(dev)
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        ro = W.route_outputs(T, E, dev)
        W.moe_route_sort_quant(logits, x, s_x, out=ro, xq=xq)
        a = torch.empty((2 * T, I), dtype=torch.uint8, device=dev)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ws2 = torch.empty(max(256, W.workspace_bytes(W.OP_GEMM2, T, H, I, E)), dtype=torch.uint8, device=dev)

        def g1(i):
            W.moe_gemm1_w4a8(xq, s_x, W13[i % 2], s13, ro["offsets"], ro["sorted_pair"], cfg.act, s_a, out=a)

        def g2(i):
            W.moe_gemm2_w4a8(a, s_a, W2[i % 2], s2, ro["offsets"], ro["pair_pos"], ro["weights"], "bf16", ws=ws2,
                             out=y)
        res = {}
        for name, fn in (("gate_up", g1), ("down_combine", g2)):
            for i in range(3):
                fn(i)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(st)
            for i in range(iters):
                fn(i)
            ev[1].record(st)
            torch.cuda.synchronize()
            res[name] = ev[0].elapsed_time(ev[1]) * 1e3 / iters
        counts = ro["counts"].cpu().numpy()
        _, g1_bytes, touched = moe_bytes(cfg, counts)
        g2_bytes = touched * (H * I // 2 + H * 4) + 2 * T * I + T * H * 2
        out[str(T)] = {"kernel": "tiled" if W.moe_kernel(T) == W.KERNEL_TILED else "streaming",
                       "gate_up_us": round(res["gate_up"], 2), "down_combine_us": round(res["down_combine"], 2),
                       "gate_up_GB/s": round(g1_bytes / res["gate_up"] / 1e3, 1),
                       "gate_up_TFLOP/s": round(gemm1_flops(cfg) / res["gate_up"] / 1e6, 1),
                       "down_GB/s": round(g2_bytes / res["down_combine"] / 1e3, 1),
                       "tokens_per_s_two_gemms": round(T / ((res["gate_up"] + res["down_combine"]) * 1e-6), 1)}
    del W13, W2
    return out


def copy_bandwidth(torch, dev, nbytes=1 << 30, iters=10):
    """A plain device-to-device copy of 1 GiB (read + write bytes per second): the
    measured reference beside the 8 TB/s published peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(st)
    for _ in range(iters):
        dst.copy_(src)
    ev[1].record(st)
    torch.cuda.synchronize()
    s = ev[0].elapsed_time(ev[1]) * 1e-3 / iters
    del src, dst
    return 2 * nbytes / s / 1e9


def measure_layer(torch, W, cfg, steps, warmup):
    """One workload: pack, graph-captured steps, the timed region, per-call durations.
    Returns the JSON fields of the workload and the routing ids (for the CPU baseline)."""
    dev = torch.device("cuda:0")
    s_x, s_a = static_scales(cfg.name)
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E

    # ---- load: bf16 weights -> w4_pack + w4_tile on the GPU (timed separately), rotation copies
    w13b = bf16_dev(torch, synth.moe_weights(cfg, "w13"), dev)
    w2b = bf16_dev(torch, synth.moe_weights(cfg, "w2"), dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    w13, s13 = W.w4_pack(w13b, tiled=True)
    w2, s2 = W.w4_pack(w2b, tiled=True)
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1)
    # bf16 in, packed words out, then the words read and written again by the tiling
    pack_bytes = (w13b.numel() + w2b.numel()) * 3.5 + (s13.numel() + s2.numel()) * 4
    del w13b, w2b
    packed_bytes = (w13.numel() + w2.numel()) * 4
    copies = max(1, int(np.ceil(768e6 / packed_bytes))) if packed_bytes < 768e6 else 1
    W13 = [w13] + [w13.clone() for _ in range(copies - 1)]
    W2 = [w2] + [w2.clone() for _ in range(copies - 1)]

    x = bf16_dev(torch, synth.activations(cfg), dev)
    logits = torch.from_numpy(synth.router_logits(cfg)).to(dev)
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    a = torch.empty((2 * T, I), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32 if cfg.out_f32 else torch.bfloat16, device=dev)
    ws1 = torch.empty(max(256, W.workspace_bytes(W.OP_GEMM1, T, H, I, E)), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(max(256, W.workspace_bytes(W.OP_GEMM2, T, H, I, E)), dtype=torch.uint8, device=dev)
    ro = W.route_outputs(T, E, dev)
    od = "f32" if cfg.out_f32 else "bf16"

    def route_quant():
        W.moe_route_sort_quant(logits, x, s_x, out=ro, xq=xq)

    def gemm1(i):
        W.moe_gemm1_w4a8(xq, s_x, W13[i % copies], s13, ro["offsets"], ro["sorted_pair"], cfg.act, s_a, ws=ws1,
                         out=a)

    def gemm2(i):
        W.moe_gemm2_w4a8(a, s_a, W2[i % copies], s2, ro["offsets"], ro["pair_pos"], ro["weights"], od, ws=ws2,
                         out=out)

    wsl = torch.empty(max(256, W.workspace_bytes(W.OP_LAYER, T, H, I, E)), dtype=torch.uint8, device=dev)
    out1 = torch.empty_like(out)

    def step(i):
        W.moe_layer_w4a8(logits, x, s_x, W13[i % copies], s13, W2[i % copies], s2, cfg.act, s_a, od, ws=wsl,
                         out=out1)

    # the one call and the three calls it stands for give the same bytes
    route_quant(); gemm1(0); gemm2(0); step(0)
    torch.cuda.synchronize()
    if not torch.equal(out, out1):
        raise RuntimeError("moe_layer_w4a8 differs from the three calls")

    # eager reference step, then captured HIP graphs (launch overhead of the Python binding
    # stays out of the timed region): per weight copy, one of a single step and one of
    # STEPS_PER_GRAPH consecutive steps (the weight copies alternating inside), as a model's
    # decode graph holds its consecutive layers; every replay must match the eager step
    step(0)
    torch.cuda.synchronize()
    ref_out = out1.clone()
    counts = ro["counts"].cpu().numpy()
    ids = ro["ids"].cpu().numpy()
    graphs1, graphsN, graphsR = [], [], []
    rest = steps % STEPS_PER_GRAPH
    for c in range(copies):
        full = STEPS_PER_GRAPH if steps >= STEPS_PER_GRAPH else 0
        for n, dst in ((1, graphs1), (full, graphsN), (rest, graphsR)):
            if n == 0:
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(n):
                    step(c + k)
            dst.append(g)
    for i in range(warmup):
        graphs1[i % copies].replay()
    torch.cuda.synchronize()
    for g in graphs1[:1] + graphsN[:1] + graphsR[:1]:
        out1.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out1, ref_out):
            raise RuntimeError("graph replay differs from the eager step")

    # ---- timed region: exactly K steps (graphs of STEPS_PER_GRAPH steps, then one graph of
    #      the remaining K mod STEPS_PER_GRAPH steps), wall clock between two synchronizations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    done = 0
    while done + STEPS_PER_GRAPH <= steps:
        graphsN[done % copies].replay()
        done += STEPS_PER_GRAPH
    if done < steps:
        graphsR[done % copies].replay()
        done += rest
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps

    # ---- per-call duration: one call's launches back to back in a graph, between two HIP
    #      events on the stream the library launches on

    def per_launch_us(fn, n=min(256, max(20, steps))):
        # n calls captured back to back in one graph (so a short call is timed on the GPU, not
        # behind the Python binding's launch cost), replayed between two events on the stream
        return graph_call_us(torch, fn, n)

    per_call = {"route_sort_quant": per_launch_us(lambda i: route_quant()),
                "gemm1": per_launch_us(gemm1), "gemm2_combine": per_launch_us(gemm2),
                "moe_layer_w4a8": per_launch_us(step)}
    layer_bytes, gemm1_bytes, touched = moe_bytes(cfg, counts)
    layer_us = ms_per_step * 1e3
    tiled = W.moe_kernel(T) == W.KERNEL_TILED
    if tiled:
        # many tokens per expert: the tiled kernel is bound by the matrix cores; the products
        # run on the 16-bit matrix instruction (exact E4M3 x int4 values in fp16),
        # so the kernel's roofline is the fp16 dense peak; the fp8 peak's fraction is context
        tf = gemm1_flops(cfg) / (per_call["gemm1"] * 1e-6) / 1e12
        roofline = {"kernel": "moe_gemm1_w4a8 (moe_prefill_kernel<gate|up>, fp16 MFMA)", "bound": "mfma",
                    "achieved": round(tf, 1), "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / FP16_PEAK_TFLOPS, 4), "traffic": counter_traffic(cfg.name),
                    "flops_per_launch": gemm1_flops(cfg), "bytes_per_launch": int(gemm1_bytes),
                    "frac_of_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
        layer_flops = 2 * gemm1_flops(cfg) * 0.75         # gate|up + down (half the width of gate|up)
        layer_tf = layer_flops / (layer_us * 1e-6) / 1e12
        layer_frac = {"layer_mfma_frac": round(layer_tf / FP16_PEAK_TFLOPS, 4),
                      "layer_fp8_peak_frac": round(layer_tf / FP8_PEAK_TFLOPS, 4)}
    else:
        g1_gbs = gemm1_bytes / per_call["gemm1"] / 1e3
        roofline = {"kernel": "moe_gemm1_w4a8 (moe_decode_kernel<gate|up>)", "bound": "hbm",
                    "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(g1_gbs / HBM_PEAK_GBS, 4), "traffic": counter_traffic(cfg.name),
                    "bytes_per_launch": int(gemm1_bytes)}
        layer_frac = {"layer_hbm_frac": round(layer_bytes / (layer_us * 1e3) / HBM_PEAK_GBS, 4)}
    result = {
        "metric": METRIC,
        "value": round(T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "intermediate": I, "experts": E, "top_k": 2,
                   "activation": ACT_NAMES[cfg.act], "out": "fp32" if cfg.out_f32 else "bf16",
                   "weight_copies_rotated": copies, "experts_touched": touched,
                   "steps_per_graph": min(STEPS_PER_GRAPH, steps)},
        **layer_frac,
        "layer_bytes": int(layer_bytes),
        "calls_us": {k: round(v, 2) for k, v in per_call.items()},
        "roofline": roofline,
        "w4_pack+w4_tile": {"ms": round(pack_ms, 3), "GB/s": round(pack_bytes / pack_ms / 1e6, 1)},
    }
    return result, ids


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the layer on one GPU (one GPU's share of the model); "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    import w4a8_moe_amd as W

    cfg = synth.MOE_CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    result, ids = measure_layer(torch, W, cfg, args.steps, args.warmup)
    if args.workload == "mixtral_decode" and not args.no_prefill:
        # the metric's second half: the Grok-1-shaped prefill layer, bound by the matrix cores
        torch.cuda.empty_cache()
        pf, _ = measure_layer(torch, W, synth.GROK_PREFILL, min(args.steps, 10), min(args.warmup, 2))
        result["prefill"] = {k: pf[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "config",
                                                 "layer_mfma_frac", "layer_fp8_peak_frac", "calls_us", "roofline")}
        torch.cuda.empty_cache()
    if args.workload == "mixtral_decode" and not args.no_grok_decode:
        # the largest single-GPU decode layer: Grok-1-shaped, 2.42 GB of int4 weights per step
        gd, _ = measure_layer(torch, W, synth.GROK_DECODE, args.steps, args.warmup)
        result["grok_decode"] = {k: gd[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "config",
                                                     "layer_hbm_frac", "layer_bytes", "calls_us", "roofline")}
        torch.cuda.empty_cache()
    if args.workload == "mixtral_decode" and not args.no_tp8:
        # one GPU's 8-way tensor-parallel share of the Grok-1 layer (intermediate 4096 of 32768),
        # decode and prefill: 302 MB of int4 weights, where a launch's fixed costs weigh most
        share = {}
        for c in (synth.GROK_TP8_DECODE, synth.GROK_TP8_PREFILL):
            decode = W.moe_kernel(c.T) == W.KERNEL_STREAM
            m, _ = measure_layer(torch, W, c, args.steps if decode else min(args.steps, 10),
                                 args.warmup if decode else min(args.warmup, 2))
            share[c.name] = {k: m[k] for k in ("value", "unit", "ms_per_step", "steps", "config", "layer_hbm_frac",
                                               "layer_mfma_frac", "layer_fp8_peak_frac", "calls_us", "roofline")
                             if k in m}
            torch.cuda.empty_cache()
        result["grok_tp8"] = share
    if args.workload == "mixtral_decode" and not args.no_token_sweep:
        result["token_sweep"] = token_sweep(torch, W, synth.MIXTRAL_DECODE)
        torch.cuda.empty_cache()
    if result["roofline"]["bound"] == "hbm":
        cb = copy_bandwidth(torch, dev)
        result["hbm_copy_ref"] = {"GB/s": round(cb, 1), "of_peak": round(cb / HBM_PEAK_GBS, 4),
                                  "gemm1_frac_of_copy": round(result["roofline"]["achieved"] / cb, 4)}
    if args.copy_ref:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_ref_bytes"] = 1 << 30
    if not args.no_block_gemv:
        result["block_fp8_gemv"] = bench_block_gemv(torch, W, dev)
        result["fp8_linear_w8a8"] = bench_fp8_linear(torch, W, dev)
        result["fp8_kv_cache_store"] = bench_kv_store(torch, W, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, *static_scales(cfg.name))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
