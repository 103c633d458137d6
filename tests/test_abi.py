"""The C-ABI library loads, exports every declared entry point, and rejects bad arguments
on the host before any HIP call (no GPU needed: every call below fails validation)."""
import ctypes

import pytest

import w4a8_moe_amd as W

A = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)
U = 0x10008          # a fake, misaligned address


@pytest.fixture(scope="module")
def L():
    return W.lib()


def test_exports_every_declared_function(L):
    names = W.header_functions()
    assert set(names) == {"w4_pack", "w4_tile", "fp8_quant_static", "moe_route_sort", "moe_route_sort_quant", "moe_gemm1_w4a8", "moe_gemm2_w4a8",
                          "moe_gemm2_w4a8_noalloc", "moe_gemm2_w4a8_noalloc_max_workspace", "moe_layer_w4a8",
                          "fp8_block_quant", "fp8_block_linear", "fp8_tensor_quant", "fp8_linear_w8a8",
                          "fp8_kv_cache_store",
                          "w4a8_workspace_bytes", "w4a8_status_str", "w4a8_moe_kernel"}
    for n in names:
        assert hasattr(L, n), n


def test_kernel_choice(L):
    # up to 80 tokens the streaming kernel, above it the tiled one
    assert [W.moe_kernel(t) for t in (0, 1, 32, 33, 64, 72, 80)] == [W.KERNEL_STREAM] * 7
    assert [W.moe_kernel(t) for t in (81, 1024, 32768)] == [W.KERNEL_TILED] * 3


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert W.status_str(code) and W.status_str(code) != "unknown status"
    assert W.status_str(-99) == "unknown status"


def test_route_sort_quant_validation(L):
    def call(T=32, E=8, H=256, s=0.5, logits=A, x=A, xq=A, ws=None, nws=0):
        return L.moe_route_sort_quant(logits, T, E, A, A, A, A, A, A, x, H, s, xq, ws, nws, None)
    assert call(T=-1) == W.ERR_SHAPE
    assert call(E=1) == W.ERR_SHAPE
    assert call(H=0) == W.ERR_SHAPE
    assert call(T=1 << 20, H=4096) == W.ERR_SHAPE              # T*H >= 2^31
    assert call(s=0.0) == W.ERR_ARG
    assert call(s=float("inf")) == W.ERR_ARG
    assert call(x=None) == W.ERR_NULL
    assert call(xq=None) == W.ERR_NULL
    assert call(x=U) == W.ERR_ALIGN
    assert call(xq=U) == W.ERR_ALIGN
    assert call(T=300) == W.ERR_WORKSPACE                      # several blocks need a workspace


def test_w4_tile_validation(L):
    B = A + (1 << 20)
    assert L.w4_tile(None, 1, 16, 128, A, None) == W.ERR_NULL
    assert L.w4_tile(A, 1, 16, 128, None, None) == W.ERR_NULL
    assert L.w4_tile(A, 1, 24, 128, B, None) == W.ERR_SHAPE           # N % 16
    assert L.w4_tile(A, 1, 16, 192, B, None) == W.ERR_SHAPE           # K % 128
    assert L.w4_tile(A, 0, 16, 128, B, None) == W.ERR_SHAPE
    assert L.w4_tile(A, 1, 0, 128, B, None) == W.ERR_SHAPE
    assert L.w4_tile(U, 1, 16, 128, B, None) == W.ERR_ALIGN
    assert L.w4_tile(A, 1, 16, 128, U, None) == W.ERR_ALIGN
    assert L.w4_tile(A, 1, 16, 128, A, None) == W.ERR_ARG             # in place
    assert L.w4_tile(A, 1, 16, 128, A + 512, None) == W.ERR_ARG       # overlapping


def test_w4_pack_validation(L):
    assert L.w4_pack(None, 1, 16, 64, A, A, None) == W.ERR_NULL
    assert L.w4_pack(A, 1, 16, 60, A, A, None) == W.ERR_SHAPE          # K % 8
    assert L.w4_pack(A, 0, 16, 64, A, A, None) == W.ERR_SHAPE
    assert L.w4_pack(A, 1, 16, 4, A, A, None) == W.ERR_SHAPE
    assert L.w4_pack(U, 1, 16, 64, A, A, None) == W.ERR_ALIGN
    assert L.w4_pack(A, 1, 16, 64, A, U, None) == W.ERR_ALIGN


def test_fp8_quant_validation(L):
    assert L.fp8_quant_static(A, 16, 0.0, A, None) == W.ERR_ARG
    assert L.fp8_quant_static(A, 16, float("nan"), A, None) == W.ERR_ARG
    assert L.fp8_quant_static(A, 16, float("inf"), A, None) == W.ERR_ARG
    assert L.fp8_quant_static(A, -1, 1.0, A, None) == W.ERR_SHAPE
    assert L.fp8_quant_static(None, 16, 1.0, A, None) == W.ERR_NULL
    assert L.fp8_quant_static(A, 16, 1.0, U, None) == W.ERR_ALIGN
    assert L.fp8_quant_static(None, 0, 1.0, None, None) == W.OK        # empty: nothing enqueued


def test_route_sort_validation(L):
    f = L.moe_route_sort
    assert f(A, 8, 1, A, A, A, A, A, A, None, 0, None) == W.ERR_SHAPE         # E < 2
    assert f(A, 8, 257, A, A, A, A, A, A, None, 0, None) == W.ERR_SHAPE       # E > 256
    assert f(A, -1, 8, A, A, A, A, A, A, None, 0, None) == W.ERR_SHAPE
    assert f(A, (1 << 22) + 1, 8, A, A, A, A, A, A, None, 0, None) == W.ERR_SHAPE
    assert f(None, 8, 8, A, A, A, A, A, A, None, 0, None) == W.ERR_NULL
    assert f(A, 8, 8, A, A, A, A, U, A, None, 0, None) == W.ERR_ALIGN
    need = W.workspace_bytes(W.OP_ROUTE_SORT, 5000, 0, 0, 8)
    assert need > 0 and W.workspace_bytes(W.OP_ROUTE_SORT, 256, 0, 0, 8) == 0
    assert f(A, 5000, 8, A, A, A, A, A, A, A, need - 1, None) == W.ERR_WORKSPACE
    assert f(A, 5000, 8, A, A, A, A, A, A, None, need, None) == W.ERR_NULL


def _g1(L, **kw):
    a = dict(x=A, x_dtype=W.DT_E4M3, s_x=0.01, w13=A, s_w13=A, offsets=A, sorted_pair=A, T=32, H=256, I=512,
             E=8, act=W.ACT_SILU, s_a=0.01, a_fp8=A, dbg=None, ws=None, ws_bytes=0)
    a.update(kw)
    return L.moe_gemm1_w4a8(a["x"], a["x_dtype"], a["s_x"], a["w13"], a["s_w13"], a["offsets"], a["sorted_pair"],
                            a["T"], a["H"], a["I"], a["E"], a["act"], a["s_a"], a["a_fp8"], a["dbg"], a["ws"],
                            a["ws_bytes"], None)


def test_gemm1_validation(L):
    assert _g1(L, H=200) == W.ERR_SHAPE
    assert _g1(L, I=100) == W.ERR_SHAPE
    assert _g1(L, E=1) == W.ERR_SHAPE
    assert _g1(L, T=-3) == W.ERR_SHAPE
    assert _g1(L, act=7) == W.ERR_ARG
    assert _g1(L, x_dtype=W.DT_F32) == W.ERR_ARG
    assert _g1(L, s_x=0.0) == W.ERR_ARG
    assert _g1(L, s_a=-1.0) == W.ERR_ARG
    assert _g1(L, w13=None) == W.ERR_NULL
    assert _g1(L, a_fp8=U) == W.ERR_ALIGN
    assert _g1(L, dbg=U) == W.ERR_ALIGN
    need = W.workspace_bytes(W.OP_GEMM1_BF16, 32, 256, 512, 8)
    assert need >= 32 * 256 and W.workspace_bytes(W.OP_GEMM1, 32, 256, 512, 8) == 0
    assert _g1(L, x_dtype=W.DT_BF16, ws=A, ws_bytes=need - 1) == W.ERR_WORKSPACE
    assert _g1(L, T=0) == W.OK                                   # empty: nothing enqueued


def _g2(L, **kw):
    a = dict(a=A, s_a=0.01, w2=A, s_w2=A, offsets=A, pair_pos=A, topk_w=A, T=32, H=256, I=512, E=8,
             dt=W.DT_BF16, out=A, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return L.moe_gemm2_w4a8(a["a"], a["s_a"], a["w2"], a["s_w2"], a["offsets"], a["pair_pos"], a["topk_w"],
                            a["T"], a["H"], a["I"], a["E"], a["dt"], a["out"], a["ws"], a["ws_bytes"], None)


def test_gemm2_validation(L):
    assert _g2(L, I=384 + 64) == W.ERR_SHAPE
    assert _g2(L, dt=W.DT_E4M3) == W.ERR_ARG
    assert _g2(L, s_a=float("nan")) == W.ERR_ARG
    assert _g2(L, topk_w=None) == W.ERR_NULL
    assert _g2(L, out=U) == W.ERR_ALIGN
    need = W.workspace_bytes(W.OP_GEMM2, 32, 256, 512, 8)
    assert need >= 2 * 32 * 256 * 4
    assert _g2(L, ws_bytes=need - 1) == W.ERR_WORKSPACE
    assert _g2(L, ws=None, ws_bytes=need) == W.ERR_NULL
    assert _g2(L, T=0) == W.OK


def test_gemm2_noalloc_validation(L):
    """The allocation-free down call rejects what the workspace call rejects, and a batch
    whose split-K partials exceed the library's array, all before any HIP call."""
    assert W.noalloc_max_workspace() == 32 << 20

    def g(T=32, H=256, I=512, E=8, dt=W.DT_BF16, s_a=0.5, out=A, topk_w=A):
        return L.moe_gemm2_w4a8_noalloc(A, s_a, A, A, A, A, topk_w, T, H, I, E, dt, out, None)
    assert g(I=384 + 64) == W.ERR_SHAPE
    assert g(dt=W.DT_E4M3) == W.ERR_ARG
    assert g(s_a=0.0) == W.ERR_ARG
    assert g(topk_w=None) == W.ERR_NULL
    assert g(out=U) == W.ERR_ALIGN
    assert g(T=0) == W.OK
    # 2 T H 4 bytes of partials at least: 4096 tokens x 6144 channels is 192 MiB
    assert W.workspace_bytes(W.OP_GEMM2, 4096, 6144, 32768, 8) > 32 << 20
    assert g(T=4096, H=6144, I=32768) == W.ERR_WORKSPACE


def test_layer_validation(L):
    """The one-call layer rejects bad arguments before any HIP call; its workspace holds at
    least the routing outputs, x codes, intermediate codes and the down projection's sums."""
    def g(T=32, H=256, I=512, E=8, act=W.ACT_SILU, s_x=0.5, s_a=0.5, dt=W.DT_BF16, out=A, ws=A, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = W.workspace_bytes(W.OP_LAYER, T, H, I, E)
        return L.moe_layer_w4a8(A, A, s_x, A, A, A, A, T, H, I, E, act, s_a, dt, out, ws, ws_bytes, None)
    assert g(I=384 + 64) == W.ERR_SHAPE
    assert g(E=1) == W.ERR_SHAPE
    assert g(act=7) == W.ERR_ARG
    assert g(dt=W.DT_E4M3) == W.ERR_ARG
    assert g(s_x=float("inf")) == W.ERR_ARG
    assert g(s_a=-1.0) == W.ERR_ARG
    assert g(out=None) == W.ERR_NULL
    assert g(ws=None) == W.ERR_NULL
    assert g(out=U) == W.ERR_ALIGN
    assert g(T=0) == W.OK
    for T, H, I, E in ((32, 256, 512, 8), (1, 4096, 14336, 8), (64, 6144, 32768, 8), (300, 256, 512, 4)):
        need = W.workspace_bytes(W.OP_LAYER, T, H, I, E)
        assert need >= 2 * T * (12 + I + 4 * H) + T * H
        assert g(T=T, H=H, I=I, E=E, ws_bytes=need - 1) == W.ERR_WORKSPACE
    assert W.workspace_bytes(W.OP_LAYER, 32, 256, 384 + 64, 8) == 0


def test_block_validation(L):
    assert L.fp8_block_quant(None, 128, 128, A, A, None) == W.ERR_NULL
    assert L.fp8_block_quant(A, 128, 100, A, A, None) == W.ERR_SHAPE
    assert L.fp8_block_quant(A, 128, 128, U, A, None) == W.ERR_ALIGN
    f = L.fp8_block_linear
    assert f(A, A, A, 0, 256, 256, A, None, 0, None) == W.ERR_SHAPE
    assert f(A, A, A, 65, 256, 256, A, None, 0, None) == W.ERR_SHAPE
    assert f(A, A, A, 1, 250, 256, A, None, 0, None) == W.ERR_SHAPE
    assert f(A, A, A, 1, 256, 200, A, None, 0, None) == W.ERR_SHAPE
    assert f(A, A, U, 1, 256, 256, A, None, 0, None) == W.ERR_ALIGN
    assert f(None, A, A, 1, 256, 256, A, None, 0, None) == W.ERR_NULL


def test_workspace_bad_args(L):
    assert W.workspace_bytes(99, 1, 1, 1, 1) == 0
    assert W.workspace_bytes(W.OP_GEMM2, 32, 100, 512, 8) == 0


def test_fp8_tensor_quant_validation(L):
    nws = W.workspace_bytes(W.OP_TENSOR_QUANT, 0, 0, 0, 0)
    assert nws == 1024 * 4
    assert L.fp8_tensor_quant(A, 0, A, A, A, nws, None) == W.ERR_SHAPE
    assert L.fp8_tensor_quant(None, 16, A, A, A, nws, None) == W.ERR_NULL
    assert L.fp8_tensor_quant(A, 16, A, None, A, nws, None) == W.ERR_NULL
    assert L.fp8_tensor_quant(A, 16, A, A, None, nws, None) == W.ERR_NULL
    assert L.fp8_tensor_quant(U, 16, A, A, A, nws, None) == W.ERR_ALIGN
    assert L.fp8_tensor_quant(A, 16, A, A, A, nws - 1, None) == W.ERR_WORKSPACE


def test_fp8_linear_w8a8_validation(L):
    def call(M=8, N=256, K=512, s_x=0.01, s_w=0.001, x=A, w=A, y=A, ws=A, nws=None):
        if nws is None:
            nws = W.workspace_bytes(W.OP_FP8_LINEAR, M, N, K, 0)
        return L.fp8_linear_w8a8(x, s_x, w, s_w, M, N, K, y, ws, nws, None)
    assert W.workspace_bytes(W.OP_FP8_LINEAR, 8, 256, 6144, 0) == 8 * 6144
    assert W.workspace_bytes(W.OP_FP8_LINEAR, 2, 256, 6144, 0) == 0      # quantized inside the kernel
    assert call(ws=None) == W.ERR_NULL
    assert call(ws=U) == W.ERR_ALIGN
    assert call(nws=16) == W.ERR_WORKSPACE
    assert call(M=0) == W.ERR_SHAPE
    assert call(M=65) == W.ERR_SHAPE
    assert call(N=24) == W.ERR_SHAPE                            # N % 16
    assert call(K=192) == W.ERR_SHAPE                           # K % 128
    assert W.workspace_bytes(W.OP_FP8_LINEAR, 2, 256, 65536, 0) == 2 * 65536   # past the fused size
    assert call(s_x=0.0) == W.ERR_ARG
    assert call(s_w=-1.0) == W.ERR_ARG
    assert call(s_w=float("nan")) == W.ERR_ARG
    assert call(x=None) == W.ERR_NULL
    assert call(w=None) == W.ERR_NULL
    assert call(y=U) == W.ERR_ALIGN
    assert call(x=U) == W.ERR_ALIGN


def test_kv_cache_store_validation(L):
    def call(T=4, D=128, s_k=1.0, s_v=1.0, k=A, v=A, slots=A, kc=A, vc=A, S=16):
        return L.fp8_kv_cache_store(k, v, slots, T, D, s_k, s_v, kc, vc, S, None)
    assert call(T=-1) == W.ERR_SHAPE
    assert call(D=12) == W.ERR_SHAPE
    assert call(S=0) == W.ERR_SHAPE
    assert call(s_k=0.0) == W.ERR_ARG
    assert call(s_v=float("inf")) == W.ERR_ARG
    assert call(T=0, k=None) == W.OK                           # nothing to store
    assert call(slots=None) == W.ERR_NULL
    assert call(vc=U) == W.ERR_ALIGN


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so, before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
