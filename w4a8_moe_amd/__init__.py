"""Python binding of libw4a8moe (ctypes): argument marshalling only.

Every step runs in the HIP library; PyTorch supplies device memory and the stream.
The library is loaded from this directory (``libw4a8moe.so``, built in-tree by
``w4a8_moe_amd.build``); if it is missing it is built once, and if that fails the
import of a function raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a8moe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "libw4a8moe.h")

# constants mirrored from include/libw4a8moe.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_ARG, ERR_HIP = 0, -1, -2, -3, -4, -5, -6, -7
ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2
DT_F32, DT_BF16, DT_E4M3 = 0, 1, 2
OP_ROUTE_SORT, OP_GEMM1, OP_GEMM1_BF16, OP_GEMM2, OP_BLOCK_LINEAR = 1, 2, 3, 4, 5
OP_TENSOR_QUANT, OP_FP8_LINEAR, OP_LAYER = 6, 7, 8

_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "w4_pack": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "w4_tile": (_I32, [_P, _I32, _I32, _I32, _P, _P]),
    "fp8_quant_static": (_I32, [_P, _I64, _F32, _P, _P]),
    "moe_route_sort": (_I32, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_sort_quant": (_I32, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _F32, _P, _P, _SZ, _P]),
    "moe_gemm1_w4a8": (_I32, [_P, _I32, _F32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P,
                              _P, _SZ, _P]),
    "moe_gemm2_w4a8": (_I32, [_P, _F32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "moe_gemm2_w4a8_noalloc": (_I32, [_P, _F32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P]),
    "moe_gemm2_w4a8_noalloc_max_workspace": (_SZ, []),
    "moe_layer_w4a8": (_I32, [_P, _P, _F32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F32, _I32, _P, _P, _SZ,
                              _P]),
    "fp8_block_quant": (_I32, [_P, _I32, _I32, _P, _P, _P]),
    "fp8_block_linear": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "fp8_tensor_quant": (_I32, [_P, _I64, _P, _P, _P, _SZ, _P]),
    "fp8_linear_w8a8": (_I32, [_P, _F32, _P, _F32, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "fp8_kv_cache_store": (_I32, [_P, _P, _P, _I32, _I32, _F32, _F32, _P, _P, _I32, _P]),
    "w4a8_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "w4a8_status_str": (ctypes.c_char_p, [_I32]),
    "w4a8_moe_kernel": (_I32, [_I32]),
}


class W4A8Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: status {status} ({status_str(status)})")
        self.status = status


def lib():
    """The loaded library (building it in-tree first if it is not there)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from .build import build
                build()
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def header_functions():
    """Names of the functions declared in include/libw4a8moe.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)) - {"if"})


def status_str(status: int) -> str:
    return lib().w4a8_status_str(status).decode()


def workspace_bytes(op, a, b, c, E) -> int:
    return int(lib().w4a8_workspace_bytes(op, a, b, c, E))


KERNEL_STREAM, KERNEL_TILED = 0, 1


def moe_kernel(T) -> int:
    """KERNEL_STREAM or KERNEL_TILED: the kernel the MoE GEMM calls use for T tokens."""
    return int(lib().w4a8_moe_kernel(T))


# ------------------------------------------------------------------ torch wrappers
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, status):
    if status != OK:
        raise W4A8Error(fn, status)


def _need(t, dtype, shape, name):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    return t


def _workspace(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def w4_pack(w, tiled=False):
    """bf16 [E, N, K] -> (packed int32 [E, N, K/8], scale fp32 [E, N]); with tiled=True the
    words come in the layout the MoE GEMMs read, int32 [E, N/16, K/128, 256] (w4_tile)."""
    torch = _torch()
    E, N, K = w.shape
    _need(w, torch.bfloat16, (E, N, K), "w")
    packed = torch.empty((E, N, K // 8), dtype=torch.int32, device=w.device)
    scale = torch.empty((E, N), dtype=torch.float32, device=w.device)
    _check("w4_pack", lib().w4_pack(_ptr(w), E, N, K, _ptr(packed), _ptr(scale), _stream(w.device)))
    if tiled:
        packed = w4_tile(packed)
    return packed, scale


def w4_tile(packed, out=None):
    """packed int32 [E, N, K/8] (w4_pack) -> the tiled layout int32 [E, N/16, K/128, 256]."""
    torch = _torch()
    E, N, K8 = packed.shape
    K = K8 * 8
    _need(packed, torch.int32, (E, N, K8), "packed")
    shape = (E, N // 16, K // 128, 256)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=packed.device)
    _need(out, torch.int32, shape, "tiled")
    _check("w4_tile", lib().w4_tile(_ptr(packed), E, N, K, _ptr(out), _stream(packed.device)))
    return out


def fp8_quant_static(x, s, out=None):
    """bf16 tensor -> uint8 E4M3 codes of the same shape, e4m3(x / s)."""
    torch = _torch()
    _need(x, torch.bfloat16, tuple(x.shape), "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, tuple(x.shape), "out")
    _check("fp8_quant_static", lib().fp8_quant_static(_ptr(x), x.numel(), float(s), _ptr(out), _stream(x.device)))
    return out


def route_outputs(T, E, device):
    """Preallocated outputs (and workspace) of moe_route_sort."""
    torch = _torch()
    return dict(ids=torch.empty((T, 2), dtype=torch.int32, device=device),
                weights=torch.empty((T, 2), dtype=torch.float32, device=device),
                counts=torch.empty(E, dtype=torch.int32, device=device),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=device),
                sorted_pair=torch.empty(2 * T, dtype=torch.int32, device=device),
                pair_pos=torch.empty(2 * T, dtype=torch.int32, device=device),
                ws=_workspace(workspace_bytes(OP_ROUTE_SORT, T, 0, 0, E), device))


def moe_route_sort(logits, out=None):
    """fp32 [T, E] -> dict(ids, weights, counts, offsets, sorted_pair, pair_pos, ws)."""
    torch = _torch()
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    dev = logits.device
    o = out if out is not None else route_outputs(T, E, dev)
    ids, w, counts, offsets, sp, pos, ws = (o["ids"], o["weights"], o["counts"], o["offsets"], o["sorted_pair"],
                                            o["pair_pos"], o["ws"])
    if ws.numel() < workspace_bytes(OP_ROUTE_SORT, T, 0, 0, E):
        raise ValueError("route workspace too small")
    _check("moe_route_sort", lib().moe_route_sort(_ptr(logits), T, E, _ptr(ids), _ptr(w), _ptr(counts),
                                                  _ptr(offsets), _ptr(sp), _ptr(pos), _ptr(ws), ws.numel(),
                                                  _stream(dev)))
    return o


def moe_route_sort_quant(logits, x, s_x, out=None, xq=None):
    """moe_route_sort(logits) and fp8_quant_static(x, s_x) in one call (one launch up to
    256 tokens): the dict of moe_route_sort plus "xq", the E4M3 codes of x."""
    torch = _torch()
    T, E = logits.shape
    H = x.shape[1]
    _need(logits, torch.float32, (T, E), "logits")
    _need(x, torch.bfloat16, (T, H), "x")
    dev = logits.device
    o = out if out is not None else route_outputs(T, E, dev)
    if xq is None:
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    _need(xq, torch.uint8, (T, H), "xq")
    ids, w, counts, offsets, sp, pos, ws = (o["ids"], o["weights"], o["counts"], o["offsets"], o["sorted_pair"],
                                            o["pair_pos"], o["ws"])
    if ws.numel() < workspace_bytes(OP_ROUTE_SORT, T, 0, 0, E):
        raise ValueError("route workspace too small")
    _check("moe_route_sort_quant",
           lib().moe_route_sort_quant(_ptr(logits), T, E, _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets), _ptr(sp),
                                      _ptr(pos), _ptr(x), H, float(s_x), _ptr(xq), _ptr(ws), ws.numel(),
                                      _stream(dev)))
    o["xq"] = xq
    return o


def moe_gemm1_w4a8(x, s_x, w13, s_w13, offsets, sorted_pair, act, s_a, debug=False, ws=None, out=None):
    """x bf16 [T, H] or uint8 E4M3 codes [T, H]; returns a_fp8 uint8 [2T, I] (and fp32 [2T, 2I] if debug)."""
    torch = _torch()
    T, H = x.shape
    if w13.dim() != 4:
        raise ValueError("w13: expected the tiled layout [E, 2I/16, H/128, 256] (w4_tile)")
    E, NB, KT, _ = w13.shape
    I = NB * 8
    dt = DT_BF16 if x.dtype == torch.bfloat16 else DT_E4M3
    _need(x, torch.bfloat16 if dt == DT_BF16 else torch.uint8, (T, H), "x")
    _need(w13, torch.int32, (E, 2 * I // 16, H // 128, 256), "w13 (tiled)")
    _need(s_w13, torch.float32, (E, 2 * I), "s_w13")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(sorted_pair, torch.int32, (2 * T,), "sorted_pair")
    dev = x.device
    a = out if out is not None else torch.empty((2 * T, I), dtype=torch.uint8, device=dev)
    _need(a, torch.uint8, (2 * T, I), "a_fp8")
    dbg = torch.empty((2 * T, 2 * I), dtype=torch.float32, device=dev) if debug else None
    nws = workspace_bytes(OP_GEMM1_BF16 if dt == DT_BF16 else OP_GEMM1, T, H, I, E)
    if ws is None or ws.numel() < nws:
        ws = _workspace(nws, dev)
    _check("moe_gemm1_w4a8", lib().moe_gemm1_w4a8(_ptr(x), dt, float(s_x), _ptr(w13), _ptr(s_w13), _ptr(offsets),
                                                  _ptr(sorted_pair), T, H, I, E, int(act), float(s_a), _ptr(a),
                                                  _ptr(dbg), _ptr(ws), ws.numel(), _stream(dev)))
    return (a, dbg) if debug else a


def moe_gemm2_w4a8(a, s_a, w2, s_w2, offsets, pair_pos, topk_w, out_dtype="bf16", ws=None, out=None):
    """a uint8 E4M3 [2T, I] -> out [T, H] (bf16 or fp32)."""
    torch = _torch()
    P, I = a.shape
    T = P // 2
    if w2.dim() != 4:
        raise ValueError("w2: expected the tiled layout [E, H/16, I/128, 256] (w4_tile)")
    E, HB, _, _ = w2.shape
    H = HB * 16
    _need(a, torch.uint8, (2 * T, I), "a_fp8")
    _need(w2, torch.int32, (E, H // 16, I // 128, 256), "w2 (tiled)")
    _need(s_w2, torch.float32, (E, H), "s_w2")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(pair_pos, torch.int32, (2 * T,), "pair_pos")
    _need(topk_w, torch.float32, (T, 2), "topk_w")
    dt = DT_BF16 if out_dtype in ("bf16", torch.bfloat16) else DT_F32
    dev = a.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if dt == DT_BF16 else torch.float32, device=dev)
    nws = workspace_bytes(OP_GEMM2, T, H, I, E)
    if ws is None or ws.numel() < nws:
        ws = _workspace(nws, dev)
    _check("moe_gemm2_w4a8", lib().moe_gemm2_w4a8(_ptr(a), float(s_a), _ptr(w2), _ptr(s_w2), _ptr(offsets),
                                                  _ptr(pair_pos), _ptr(topk_w), T, H, I, E, dt, _ptr(out),
                                                  _ptr(ws), ws.numel(), _stream(dev)))
    return out


def moe_gemm2_w4a8_noalloc(a, s_a, w2, s_w2, offsets, pair_pos, topk_w, out_dtype="bf16", out=None):
    """moe_gemm2_w4a8 with the library's own scratch in place of a workspace (the call
    allocates nothing on the device; ``out`` is allocated here only when not given)."""
    torch = _torch()
    P, I = a.shape
    T = P // 2
    if w2.dim() != 4:
        raise ValueError("w2: expected the tiled layout [E, H/16, I/128, 256] (w4_tile)")
    E, HB, _, _ = w2.shape
    H = HB * 16
    _need(a, torch.uint8, (2 * T, I), "a_fp8")
    _need(w2, torch.int32, (E, H // 16, I // 128, 256), "w2 (tiled)")
    _need(s_w2, torch.float32, (E, H), "s_w2")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(pair_pos, torch.int32, (2 * T,), "pair_pos")
    _need(topk_w, torch.float32, (T, 2), "topk_w")
    dt = DT_BF16 if out_dtype in ("bf16", torch.bfloat16) else DT_F32
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if dt == DT_BF16 else torch.float32, device=a.device)
    _check("moe_gemm2_w4a8_noalloc", lib().moe_gemm2_w4a8_noalloc(
        _ptr(a), float(s_a), _ptr(w2), _ptr(s_w2), _ptr(offsets), _ptr(pair_pos), _ptr(topk_w), T, H, I, E, dt,
        _ptr(out), _stream(a.device)))
    return out


def noalloc_max_workspace():
    return int(lib().moe_gemm2_w4a8_noalloc_max_workspace())


def moe_layer_w4a8(logits, x, s_x, w13, s_w13, w2, s_w2, act, s_a, out_dtype="bf16", ws=None, out=None):
    """The whole layer in one library call: logits fp32 [T, E], x bf16 [T, H], w13 and w2
    in the tiled layout -> out [T, H] (bf16 or fp32). ``ws`` (uint8, at least
    workspace_bytes(OP_LAYER, T, H, I, E)) is allocated here when not given."""
    torch = _torch()
    T, H = x.shape
    if w13.dim() != 4 or w2.dim() != 4:
        raise ValueError("w13, w2: expected the tiled layout (w4_tile)")
    E = w13.shape[0]
    I = w13.shape[1] * 16 // 2
    _need(logits, torch.float32, (T, E), "logits")
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w13, torch.int32, (E, 2 * I // 16, H // 128, 256), "w13 (tiled)")
    _need(s_w13, torch.float32, (E, 2 * I), "s_w13")
    _need(w2, torch.int32, (E, H // 16, I // 128, 256), "w2 (tiled)")
    _need(s_w2, torch.float32, (E, H), "s_w2")
    dt = DT_BF16 if out_dtype in ("bf16", torch.bfloat16) else DT_F32
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16 if dt == DT_BF16 else torch.float32, device=dev)
    nws = workspace_bytes(OP_LAYER, T, H, I, E)
    if ws is None or ws.numel() < nws:
        ws = _workspace(nws, dev)
    _check("moe_layer_w4a8", lib().moe_layer_w4a8(_ptr(logits), _ptr(x), float(s_x), _ptr(w13), _ptr(s_w13),
                                                  _ptr(w2), _ptr(s_w2), T, H, I, E, int(act), float(s_a), dt,
                                                  _ptr(out), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def fp8_block_quant(w):
    """bf16 [N, K] -> (uint8 E4M3 [N, K], fp32 scales [ceil(N/128), ceil(K/128)])."""
    torch = _torch()
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    S = torch.empty(((N + 127) // 128, (K + 127) // 128), dtype=torch.float32, device=w.device)
    _check("fp8_block_quant", lib().fp8_block_quant(_ptr(w), N, K, _ptr(q), _ptr(S), _stream(w.device)))
    return q, S


def fp8_block_linear(x, w, s, out=None):
    """bf16 x [M, K], E4M3 w [N, K], scales [ceil(N/128), K/128] -> bf16 y [M, N]."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w, torch.uint8, (N, K), "w")
    _need(s, torch.float32, ((N + 127) // 128, K // 128), "s")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check("fp8_block_linear", lib().fp8_block_linear(_ptr(x), _ptr(w), _ptr(s), M, N, K, _ptr(y), None, 0,
                                                      _stream(x.device)))
    return y


def fp8_tensor_quant(w):
    """bf16 weight (any shape) -> (uint8 E4M3 codes of the same shape, fp32 scale [1] on the
    device): one scale fp32(max|w| / 448) for the tensor."""
    torch = _torch()
    _need(w, torch.bfloat16, tuple(w.shape), "w")
    q = torch.empty(tuple(w.shape), dtype=torch.uint8, device=w.device)
    s = torch.empty(4, dtype=torch.float32, device=w.device)         # 16 bytes: the scale in [0]
    nws = workspace_bytes(OP_TENSOR_QUANT, 0, 0, 0, 0)
    ws = _workspace(nws, w.device)
    _check("fp8_tensor_quant", lib().fp8_tensor_quant(_ptr(w), w.numel(), _ptr(q), _ptr(s), _ptr(ws), ws.numel(),
                                                      _stream(w.device)))
    return q, s[:1]


def fp8_linear_w8a8(x, s_x, w, s_w, out=None, ws=None):
    """bf16 x [M, K] with its static scale s_x, E4M3 w [N, K] with its tensor scale s_w
    (host floats) -> bf16 y [M, N]."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w, torch.uint8, (N, K), "w")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    nws = workspace_bytes(OP_FP8_LINEAR, M, N, K, 0)
    if nws > 0 and (ws is None or ws.numel() < nws):
        ws = _workspace(nws, x.device)
    _check("fp8_linear_w8a8", lib().fp8_linear_w8a8(_ptr(x), float(s_x), _ptr(w), float(s_w), M, N, K, _ptr(y),
                                                    _ptr(ws) if nws > 0 else None, ws.numel() if nws > 0 else 0,
                                                    _stream(x.device)))
    return y


def fp8_kv_cache_store(k, v, slots, s_k, s_v, k_cache, v_cache):
    """bf16 k, v [T, D], int32 slots [T], static scales (host floats), uint8 E4M3 caches
    [num_slots, D] updated in place: row slots[t] gets e4m3(k[t] / s_k), e4m3(v[t] / s_v)."""
    torch = _torch()
    T, D = k.shape
    S = k_cache.shape[0]
    _need(k, torch.bfloat16, (T, D), "k")
    _need(v, torch.bfloat16, (T, D), "v")
    _need(slots, torch.int32, (T,), "slots")
    _need(k_cache, torch.uint8, (S, D), "k_cache")
    _need(v_cache, torch.uint8, (S, D), "v_cache")
    _check("fp8_kv_cache_store", lib().fp8_kv_cache_store(_ptr(k), _ptr(v), _ptr(slots), T, D, float(s_k), float(s_v),
                                                          _ptr(k_cache), _ptr(v_cache), S, _stream(k.device)))
    return k_cache, v_cache


def moe_layer(x, s_x, logits, w13, s_w13, w2, s_w2, act, s_a, out_dtype="bf16"):
    """The whole layer: route+sort, gate|up, down+combine (x bf16 or E4M3 codes; w13 and w2
    in the tiled layout)."""
    if x.dtype == _torch().bfloat16:
        r = moe_route_sort_quant(logits, x, s_x)
        x = r["xq"]
    else:
        r = moe_route_sort(logits)
    a = moe_gemm1_w4a8(x, s_x, w13, s_w13, r["offsets"], r["sorted_pair"], act, s_a)
    return moe_gemm2_w4a8(a, s_a, w2, s_w2, r["offsets"], r["pair_pos"], r["weights"], out_dtype)
