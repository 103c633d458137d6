"""Top-2 routing on router logits and the expert-contiguous sort of (token, slot) pairs.

Page A, ``config.json``: ``num_local_experts`` 8, ``num_experts_per_tok`` 2; the
router gates ``model.layers.*.block_sparse_moe.gate`` are in ``ignored_layers``
(kept unquantized), so the logits arrive as floating point.

Readings (pages silent):

* weights: softmax over all E logits, keep the top 2, renormalise to sum 1
  (equivalently w0 = 1 / (1 + exp(l1 - l0)), w1 = 1 - w0 in exact arithmetic);
* selection on the raw logits: higher logit first, on equal logits the lower expert
  id first; slot 0 is the winner;
* pair p = 2 t + slot. The sort is stable: within an expert's segment the pairs
  keep increasing p.
"""
import numpy as np


def route_top2(logits):
    """logits float32 [T, E] -> (ids int32 [T, 2], weights float64 [T, 2])."""
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    if E < 2:
        raise ValueError("top-2 routing needs E >= 2")
    if not np.all(np.isfinite(l)):
        raise ValueError("non-finite logits")
    # order by (logit descending, expert id ascending): a stable sort of -logit
    order = np.argsort(-l, axis=1, kind="stable")
    ids = order[:, :2].astype(np.int32)
    m = np.max(l, axis=1, keepdims=True)
    p = np.exp(l - m)
    p /= np.sum(p, axis=1, keepdims=True)                      # softmax over all E
    top = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = top / np.sum(top, axis=1, keepdims=True)               # renormalise the top 2
    return ids, w


def route_sort(ids, E):
    """ids int32 [T, 2] -> counts [E], offsets [E+1], sorted_pair [2T], pair_pos [2T] (int32).

    counts = histogram of the experts of all pairs; offsets = exclusive prefix sum
    (offsets[E] = 2T); sorted_pair = the pair ids ordered by expert, stable in p;
    pair_pos = the inverse permutation (position of pair p in sorted order).
    """
    ids = np.asarray(ids, dtype=np.int64)
    expert_of_pair = ids.reshape(-1)                           # index p = 2t + slot
    P = expert_of_pair.size
    counts = np.bincount(expert_of_pair, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    sorted_pair = np.argsort(expert_of_pair, kind="stable")
    pair_pos = np.empty(P, dtype=np.int64)
    pair_pos[sorted_pair] = np.arange(P)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_pair.astype(np.int32), pair_pos.astype(np.int32))
