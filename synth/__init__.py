"""Seeded synthetic inputs for the W4A8 MoE layer and the block-FP8 linear.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds none of the method's arithmetic: only workload shapes, random
draws, and the rounding of those draws to bf16 (the storage type of the inputs).

Every tensor is drawn from ``numpy.random.default_rng([cfg, tensor, index, chunk])``
so that any row block can be regenerated on its own (the oracle checks sampled
rows of full-size layers without materialising the whole layer).

bf16 values are carried as ``uint16`` bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

# tensor ids used in the seed tuple
T_W13, T_W2, T_X, T_LOGITS, T_BIAS, T_BLOCK_W, T_BLOCK_X = range(7)

# rows generated per seed chunk for the expert weights
CHUNK_ROWS = 2048

ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic MoE layer workload."""
    name: str
    T: int            # tokens
    H: int            # hidden size (K of gate|up, N of down)
    I: int            # intermediate size per expert
    E: int            # experts
    act: int          # gated activation
    w_sigma: float    # expert weights ~ N(0, w_sigma), bf16
    logit_sigma: float
    out_f32: bool     # output dtype: fp32 (True) or bf16
    w_cfg: int        # seed id of the weights
    x_cfg: int        # seed id of the activations and router logits
    expert_bias: bool = False  # per-expert logit bias ~ N(0, 1) (unequal loads)
    x_sigma: float = 1.0


@dataclass(frozen=True)
class BlockConfig:
    """One synthetic block-FP8 dense decode GEMV workload."""
    name: str
    M: int
    N: int
    K: int
    w_sigma: float = 0.02
    x_sigma: float = 1.0
    cfg: int = 5
    sub: int = 0      # distinguishes the two projection shapes in the seed


# Workloads. Shapes: Grok-1 (hidden 6144, intermediate 32768, 8 experts, top-2) as
# printed in the config.json of the page "ROCm: enable trillion-parameter MoE models
# with INT4-FP8 single node"; Mixtral-8x7B (named on the page "[AMD][Quantization] Add
# int4fp8_moe online quantization on ROCm") with its published hidden 4096 /
# intermediate 14336; prefill of 32 sequences x 1024 tokens from the bench command on
# the first page; block-FP8 projection shapes [16384,2560] and [13312,2560] from the
# page "qwen4_exp: serve the block-FP8 dense projections natively (+25% decode)".
TINY = MoEConfig("tiny", T=16, H=256, I=512, E=4, act=ACT_SILU, w_sigma=0.02,
                 logit_sigma=1.0, out_f32=True, w_cfg=1, x_cfg=1)
MIXTRAL_DECODE = MoEConfig("mixtral_decode", T=32, H=4096, I=14336, E=8, act=ACT_SILU,
                           w_sigma=0.02, logit_sigma=1.5, out_f32=False, w_cfg=2, x_cfg=2)
GROK_DECODE = MoEConfig("grok_decode", T=32, H=6144, I=32768, E=8, act=ACT_GELU_ERF,
                        w_sigma=0.015, logit_sigma=1.5, out_f32=False, w_cfg=3, x_cfg=3)
GROK_PREFILL = MoEConfig("grok_prefill", T=32768, H=6144, I=32768, E=8, act=ACT_GELU_ERF,
                         w_sigma=0.015, logit_sigma=1.5, out_f32=False, w_cfg=3, x_cfg=4,
                         expert_bias=True)
# One GPU's share of the Grok-1 layer under 8-way tensor parallelism (the page "ROCm:
# enable trillion-parameter MoE models with INT4-FP8 single node" serves it with --tp 8):
# each GPU holds I / 8 = 4096 gate and up channels and the matching K-slice of the down
# projection, while routing is replicated, so the tokens and router logits are those of
# the full layer (same activation seeds). The weights are a layer of their own with the
# share's shape (seed 6).
GROK_TP8_DECODE = MoEConfig("grok_tp8_decode", T=32, H=6144, I=4096, E=8, act=ACT_GELU_ERF,
                            w_sigma=0.015, logit_sigma=1.5, out_f32=False, w_cfg=6, x_cfg=3)
GROK_TP8_PREFILL = MoEConfig("grok_tp8_prefill", T=32768, H=6144, I=4096, E=8, act=ACT_GELU_ERF,
                             w_sigma=0.015, logit_sigma=1.5, out_f32=False, w_cfg=6, x_cfg=4,
                             expert_bias=True)
BLOCK_QKVZ_M1 = BlockConfig("block_qkvz_m1", M=1, N=16384, K=2560, sub=0)
BLOCK_QKVZ_M8 = BlockConfig("block_qkvz_m8", M=8, N=16384, K=2560, sub=0)
BLOCK_QKV_M1 = BlockConfig("block_qkv_m1", M=1, N=13312, K=2560, sub=1)
BLOCK_QKV_M8 = BlockConfig("block_qkv_m8", M=8, N=13312, K=2560, sub=1)
BLOCK_QKVZ_M32 = BlockConfig("block_qkvz_m32", M=32, N=16384, K=2560, sub=0)   # small-batch decode
BLOCK_QKV_M32 = BlockConfig("block_qkv_m32", M=32, N=13312, K=2560, sub=1)

# Per-tensor FP8 (W8A8) dense projections of the Grok-1 attention block (page "ROCm:
# enable trillion-parameter MoE models with INT4-FP8 single node": hidden 6144, 48 query
# heads and 8 key/value heads of 128): the fused q|k|v projection [6144 + 2 * 1024, 6144]
# and the output projection [6144, 6144], decode rows M in {1, 8, 32} (32: the batch of the
# page's bench command).
FP8_QKV_M1 = BlockConfig("fp8_qkv_m1", M=1, N=8192, K=6144, cfg=7, sub=0)
FP8_QKV_M8 = BlockConfig("fp8_qkv_m8", M=8, N=8192, K=6144, cfg=7, sub=0)
FP8_O_M1 = BlockConfig("fp8_o_m1", M=1, N=6144, K=6144, cfg=7, sub=1)
FP8_O_M8 = BlockConfig("fp8_o_m8", M=8, N=6144, K=6144, cfg=7, sub=1)
FP8_QKV_M32 = BlockConfig("fp8_qkv_m32", M=32, N=8192, K=6144, cfg=7, sub=0)   # the page's decode batch of 32
FP8_O_M32 = BlockConfig("fp8_o_m32", M=32, N=6144, K=6144, cfg=7, sub=1)

MOE_CONFIGS = {c.name: c for c in (TINY, MIXTRAL_DECODE, GROK_DECODE, GROK_PREFILL, GROK_TP8_DECODE,
                                   GROK_TP8_PREFILL)}
BLOCK_CONFIGS = {c.name: c for c in (BLOCK_QKVZ_M1, BLOCK_QKVZ_M8, BLOCK_QKVZ_M32, BLOCK_QKV_M1, BLOCK_QKV_M8,
                                     BLOCK_QKV_M32)}
LINEAR_CONFIGS = {c.name: c for c in (FP8_QKV_M1, FP8_QKV_M8, FP8_QKV_M32, FP8_O_M1, FP8_O_M8, FP8_O_M32)}


def custom_moe(name, T, H, I, E, act=ACT_SILU, w_sigma=0.02, logit_sigma=1.0,
               out_f32=True, w_cfg=100, x_cfg=100, expert_bias=False):
    """A MoE workload of arbitrary shape (parity tests at small sizes)."""
    return MoEConfig(name, T=T, H=H, I=I, E=E, act=act, w_sigma=w_sigma,
                     logit_sigma=logit_sigma, out_f32=out_f32, w_cfg=w_cfg, x_cfg=x_cfg,
                     expert_bias=expert_bias)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    This is the storage rounding of the drawn inputs. Inputs here are finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    r = u + bias
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _normal_bf16(seed, n, sigma) -> np.ndarray:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(n, dtype=np.float32)
    z *= np.float32(sigma)
    return f32_to_bf16_bits(z)


def expert_weight_rows(cfg_id: int, tensor: int, e: int, K: int, sigma: float,
                       row0: int, row1: int) -> np.ndarray:
    """Rows [row0, row1) of expert e's bf16 weight matrix (uint16 [row1-row0, K])."""
    out = np.empty((row1 - row0, K), np.uint16)
    c0, c1 = row0 // CHUNK_ROWS, (row1 - 1) // CHUNK_ROWS
    for c in range(c0, c1 + 1):
        chunk = _normal_bf16([cfg_id, tensor, e, c], CHUNK_ROWS * K, sigma).reshape(CHUNK_ROWS, K)
        lo = max(row0, c * CHUNK_ROWS)
        hi = min(row1, (c + 1) * CHUNK_ROWS)
        out[lo - row0:hi - row0] = chunk[lo - c * CHUNK_ROWS:hi - c * CHUNK_ROWS]
    return out


def _matrix_jobs(out2d, cfg_id, tensor, idx, N, K, sigma):
    """Chunked fill jobs for one [N, K] bf16 matrix seeded by (cfg_id, tensor, idx)."""
    def make(c):
        def work():
            lo, hi = c * CHUNK_ROWS, min(N, (c + 1) * CHUNK_ROWS)
            chunk = _normal_bf16([cfg_id, tensor, idx, c], CHUNK_ROWS * K, sigma)
            out2d[lo:hi] = chunk.reshape(CHUNK_ROWS, K)[:hi - lo]
        return work
    return [make(c) for c in range((N + CHUNK_ROWS - 1) // CHUNK_ROWS)]


def _run(jobs):
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda f: f(), jobs))


def expert_weights(cfg_id: int, tensor: int, E: int, N: int, K: int, sigma: float,
                   experts=None, out: np.ndarray | None = None) -> np.ndarray:
    """bf16 weights [E, N, K] (uint16), generated in row chunks on a thread pool.

    Rows past N in the last chunk are drawn and discarded, so the values of a row
    depend only on (cfg_id, tensor, expert, row, K, sigma).
    """
    if out is None:
        out = np.empty((E, N, K), np.uint16)
    experts = range(E) if experts is None else experts
    jobs = []
    for e in experts:
        jobs += _matrix_jobs(out[e], cfg_id, tensor, e, N, K, sigma)
    _run(jobs)
    return out


def activations(cfg: MoEConfig) -> np.ndarray:
    """Token activations x, bf16 bits [T, H]."""
    T, H = cfg.T, cfg.H
    rows_per = max(1, (1 << 22) // H)
    out = np.empty((T, H), np.uint16)
    jobs = list(range((T + rows_per - 1) // rows_per))

    def work(c):
        lo, hi = c * rows_per, min(T, (c + 1) * rows_per)
        out[lo:hi] = _normal_bf16([cfg.x_cfg, T_X, 0, c], (hi - lo) * H, cfg.x_sigma).reshape(hi - lo, H)

    _run([lambda c=c: work(c) for c in jobs])
    return out


def router_logits(cfg: MoEConfig) -> np.ndarray:
    """Router logits, float32 [T, E]; N(0, logit_sigma) plus an optional per-expert bias."""
    rng = np.random.default_rng([cfg.x_cfg, T_LOGITS, 0, 0])
    z = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32) * np.float32(cfg.logit_sigma)
    if cfg.expert_bias:
        b = np.random.default_rng([cfg.x_cfg, T_BIAS, 0, 0]).standard_normal(cfg.E, dtype=np.float32)
        z = z + b[None, :]
    return z.astype(np.float32)


def moe_weights(cfg: MoEConfig, which: str, experts=None) -> np.ndarray:
    """bf16 expert weights: ``"w13"`` = [E, 2I, H] (gate rows then up rows), ``"w2"`` = [E, H, I]."""
    if which == "w13":
        return expert_weights(cfg.w_cfg, T_W13, cfg.E, 2 * cfg.I, cfg.H, cfg.w_sigma, experts)
    if which == "w2":
        return expert_weights(cfg.w_cfg, T_W2, cfg.E, cfg.H, cfg.I, cfg.w_sigma, experts)
    raise ValueError(which)


def moe_expert_weights(cfg: MoEConfig, which: str, e: int) -> np.ndarray:
    """bf16 weights of one expert: [2I, H] for ``"w13"``, [H, I] for ``"w2"``."""
    if which == "w13":
        tensor, N, K = T_W13, 2 * cfg.I, cfg.H
    elif which == "w2":
        tensor, N, K = T_W2, cfg.H, cfg.I
    else:
        raise ValueError(which)
    out = np.empty((N, K), np.uint16)
    _run(_matrix_jobs(out, cfg.w_cfg, tensor, e, N, K, cfg.w_sigma))
    return out


def moe_weight_rows(cfg: MoEConfig, which: str, e: int, rows) -> np.ndarray:
    """Selected rows of one expert's bf16 weight matrix (uint16 [len(rows), K])."""
    rows = np.asarray(rows, np.int64)
    if which == "w13":
        tensor, K = T_W13, cfg.H
    elif which == "w2":
        tensor, K = T_W2, cfg.I
    else:
        raise ValueError(which)
    out = np.empty((len(rows), K), np.uint16)
    for c in np.unique(rows // CHUNK_ROWS):
        sel = np.nonzero(rows // CHUNK_ROWS == c)[0]
        chunk = expert_weight_rows(cfg.w_cfg, tensor, e, K, cfg.w_sigma,
                                   int(c) * CHUNK_ROWS, int(c + 1) * CHUNK_ROWS)
        out[sel] = chunk[rows[sel] - int(c) * CHUNK_ROWS]
    return out


def block_weights(cfg: BlockConfig) -> np.ndarray:
    """bf16 dense weight [N, K] of a block-FP8 projection (before block quantization)."""
    out = np.empty((cfg.N, cfg.K), np.uint16)
    _run(_matrix_jobs(out, cfg.cfg, T_BLOCK_W, cfg.sub, cfg.N, cfg.K, cfg.w_sigma))
    return out


def block_activations(cfg: BlockConfig) -> np.ndarray:
    """bf16 decode activations [M, K]."""
    return _normal_bf16([cfg.cfg, T_BLOCK_X, cfg.sub, cfg.M], cfg.M * cfg.K, cfg.x_sigma).reshape(cfg.M, cfg.K)


def custom_block(name, M, N, K, cfg=50, sub=0, w_sigma=0.02):
    return BlockConfig(name, M=M, N=N, K=K, cfg=cfg, sub=sub, w_sigma=w_sigma)
