"""Helpers for the GPU parity tests: device transfer and the comparison rules."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def torch():
    import torch as _t
    return _t


def dev():
    return torch().device("cuda:0")


def bf16_dev(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).to(dev())


def f32_dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def u8_dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def host(t):
    tt = torch()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits):
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def static_scales(name):
    d = json.load(open(os.path.join(GOLDEN, "static_scales.json")))[name]
    return np.float32(float.fromhex(d["s_x_hex"])), np.float32(float.fromhex(d["s_a_hex"]))


def same_codes(a, b):
    """E4M3 codes equal, with +0 and -0 identified."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    return (a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))


def assert_gateup_close(h_gpu, h_ref):
    """fp32 gate|up: |h_gpu - h_ref| <= 1e-4 * max_n |h_ref[r, :]| for every row r."""
    h_gpu = np.asarray(h_gpu, np.float64)
    rowmax = np.max(np.abs(h_ref), axis=1, keepdims=True)
    err = np.abs(h_gpu - h_ref)
    bad = err > 1e-4 * rowmax
    worst = float(np.max(err / np.maximum(rowmax, 1e-30)))
    print(f"gate|up: max |err| / row max = {worst:.3g} (bar 1e-4)")
    assert not bad.any(), f"{bad.sum()} gate|up values off; worst ratio {worst:.3g}"
    return worst


def assert_final_close(out_gpu, out_ref):
    """Final outputs: |d| <= 1e-2 max|ref| everywhere and <= 0.1% of elements above 1e-3 max|ref|."""
    out_gpu = np.asarray(out_gpu, np.float64)
    out_ref = np.asarray(out_ref, np.float64)
    m = np.max(np.abs(out_ref))
    d = np.abs(out_gpu - out_ref)
    assert d.max() <= 1e-2 * m, f"max err {d.max():.4g} > 1e-2 * {m:.4g}"
    frac = np.mean(d > 1e-3 * m)
    print(f"final: max |err| / max|ref| = {d.max() / m:.3g}, {frac:.4%} of {d.size} elements above 1e-3 max|ref|")
    assert frac <= 1e-3, f"{frac:.4%} of elements above 1e-3 max|ref|"


def assert_codes_consistent(c_gpu, c_ref, h_gpu, act, s_a, I, max_frac=1e-2, a_ref=None):
    """Requantized codes. The oracle's epilogue (activation, division by s_a, E4M3
    rounding) applied to the GPU's own gate|up values must give the GPU's codes, every one;
    against the oracle's codes, differences may only come from the gate|up differences
    (checked separately to the 1e-4 bar), on at most max_frac of the codes: a differing
    code must be one that a value between the two activations rounds to (the rounding is
    monotone), or, without the oracle's activation a_ref, a neighbour of the oracle's."""
    from oracle import activation, quantize_static
    h = np.asarray(h_gpu, np.float64)
    a_own = activation(h[:, :I], act) * h[:, I:]
    own = quantize_static(a_own.astype(np.float32), s_a)
    own_eq = same_codes(own, c_gpu)
    # the kernel takes every decision near a rounding boundary in double precision, with the
    # oracle's formulas, from the same gate|up values: the codes are the same, all of them
    assert own_eq.all(), f"{int((~own_eq).sum())} codes differ from the oracle's epilogue on the GPU's own gate|up"
    eq = same_codes(c_gpu, c_ref)
    frac = 1.0 - eq.mean()
    print(f"a codes: {frac:.4%} differ from the oracle's")
    if eq.all():
        return
    assert frac <= max_frac, f"{frac:.4%} of codes differ"
    if a_ref is None:
        _assert_adjacent(np.asarray(c_gpu)[~eq], np.asarray(c_ref)[~eq])
        return
    from oracle import e4m3_decode
    d = ~eq
    a1 = a_own[d].astype(np.float32)
    a2 = np.asarray(a_ref, np.float64)[d].astype(np.float32)
    lo = e4m3_decode(quantize_static(np.minimum(a1, a2), s_a))
    hi = e4m3_decode(quantize_static(np.maximum(a1, a2), s_a))
    got = e4m3_decode(np.asarray(c_gpu, np.uint8)[d])
    ok = (got >= lo) & (got <= hi)
    assert ok.all(), f"{(~ok).sum()} codes not explained by the gate|up difference"


def _assert_adjacent(c1, c2):
    cg = np.asarray(c1, np.int64)
    cr = np.asarray(c2, np.int64)
    mg, mr = cg & 0x7F, cr & 0x7F
    adjacent = ((cg >> 7) == (cr >> 7)) & (np.abs(mg - mr) == 1) | ((mg == 0) & (mr == 1)) | ((mr == 0) & (mg == 1))
    assert adjacent.all(), "a code flip is not between neighbouring codes"


def tile_words(packed):
    """The GEMMs' tiled weight layout, from its definition: int32 [E, N, K/8] -> [E, N/16,
    K/128, 256] where 16-byte unit i + 16 g of tile (nb, ks) is bytes 64 ks + 16 g .. +16
    of row 16 nb + i."""
    packed = np.asarray(packed)
    E, N, K8 = packed.shape
    x = packed.reshape(E, N // 16, 16, K8 // 16, 4, 4)        # e, nb, i, ks, g, word
    return np.ascontiguousarray(x.transpose(0, 1, 3, 4, 2, 5)).reshape(E, N // 16, K8 // 16, 256)


def rows_of_tiled(tiled_e, rows):
    """Rows (in w4_pack's row layout, int32 [len(rows), K/8]) of one expert's tiled words
    [N/16, K/128, 256]."""
    rows = np.asarray(rows)
    if isinstance(tiled_e, np.ndarray):
        t, nb, i = tiled_e, rows // 16, rows % 16
    else:                                                       # a device tensor: gather there
        t = tiled_e
        nb, i = (torch().from_numpy(v).to(t.device) for v in (rows // 16, rows % 16))
    NB, KT, _ = t.shape
    x = t.reshape(NB, KT, 4, 16, 4)                             # nb, ks, g, i, word
    got = x[nb, :, :, i, :].reshape(len(rows), KT * 16)
    return got if isinstance(got, np.ndarray) else host(got)
