"""Harness helpers: which tokens the oracle checks on full-size layers.

Not part of the method. A full prefill layer (tens of TFLOP in fp64) is out of reach
on the host, so parity there is checked on a seeded subset of tokens that always
includes the tokens whose pairs sit at the start, the end and every 128-row boundary
of each expert's segment of the sorted pair order (where any row tiling of that
segment has its edges), topped up with random tokens.
"""
import numpy as np


def prefill_token_subset(offsets, sorted_pair, T, n_tokens=1024, seed=0, edge=8, stride=128):
    offsets = np.asarray(offsets, dtype=np.int64)
    sorted_pair = np.asarray(sorted_pair, dtype=np.int64)
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        rows.extend(range(lo, min(hi, lo + edge)))
        rows.extend(range(max(lo, hi - edge), hi))
        for b in range(lo + stride, hi, stride):
            rows.extend((b - 1, b))
    toks = np.unique(sorted_pair[np.array(rows, dtype=np.int64)] // 2) if rows else np.zeros(0, np.int64)
    rng = np.random.default_rng([seed, T, n_tokens])
    if toks.size > n_tokens:
        toks = np.sort(rng.choice(toks, n_tokens, replace=False))
    need = n_tokens - toks.size
    if need > 0:
        rest = np.setdiff1d(np.arange(T), toks)
        extra = rng.choice(rest, min(need, rest.size), replace=False)
        toks = np.sort(np.concatenate([toks, extra]))
    return toks.astype(np.int64)
