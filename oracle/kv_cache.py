"""FP8 KV cache with static scales (the KV8 of the W4A8KV8 model): the cache store.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page A's quantization_config: ``kv_cache_scheme`` static; ``export.kv_cache_group``
["*k_proj", "*v_proj"] (the outputs of the key and value projections are the two cached
groups); ``export.min_kv_scale`` 1.0.

Readings (the pages give no arithmetic):

* one static per-tensor scale per group and layer, calibrated like the activations' and
  floored at min_kv_scale: s = max(fp32(fp32(max|v|) / 448), 1.0);
* the store quantizes each token's key and value rows with their group's scale,
  e4m3(fp32(v / s)) (nearest even, saturating), and writes them to the token's cache slot;
  a negative slot marks a padding token that is not stored; slots of one call are distinct;
* the cache is [num_slots, D] E4M3 codes per group, D = key/value heads x head dim; rows of
  slots not written keep their contents.
"""
import numpy as np

from .bf16 import bf16_to_f32
from .fp8 import E4M3_MAX, e4m3_encode

MIN_KV_SCALE = 1.0


def kv_scale(max_abs, min_scale=MIN_KV_SCALE) -> np.float32:
    """Static KV scale: fp32(fp32(max|v|) / 448), floored at min_kv_scale."""
    s = np.float32(np.float32(max_abs) / np.float32(E4M3_MAX))
    return np.float32(max(s, np.float32(min_scale)))


def kv_cache_store(k_bits, v_bits, slots, s_k, s_v, k_cache, v_cache):
    """bf16 k, v [T, D], int slots [T], scales; caches uint8 [num_slots, D] ->
    (new k cache, new v cache): copies of the caches with each token's rows written."""
    kc, vc = np.array(k_cache, dtype=np.uint8, copy=True), np.array(v_cache, dtype=np.uint8, copy=True)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    assert len(np.unique(slots[keep])) == int(keep.sum()), "slots of one call are distinct"
    for bits, s, cache in ((k_bits, s_k, kc), (v_bits, s_v, vc)):
        s = np.float32(s)
        with np.errstate(over="ignore"):
            q = e4m3_encode((bf16_to_f32(bits) / s).astype(np.float32))   # correctly rounded quotient
        cache[slots[keep]] = q[keep]
    return kc, vc
