"""Cache updates of one decode step, as plain array assignments (test oracle only).

* :func:`kv_write` — the new token's key and value go to the slot the host chose for it; a
  token maps to (page, slot within page) ("vLLM의 핵심 이해: PagedAttention", section 6,
  TokenTable / SlotAllocator), written here as the flat slot ``block * BS + offset``. A
  negative slot means "no write".
* :func:`copy_blocks` — copy-on-write: before writing into a shared block that is still
  filling, that block's contents are copied into a private block ("serving-paged-attention",
  section "공유는 표를 베끼는 일이 된다"). Every pair copies from the state before the call,
  for K and V and (for an 8-bit cache) their per-(block, head) scales.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def kv_write(k: np.ndarray, v: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
             slot_mapping: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the ``[NB, Hkv, BS, D]`` caches with token t written to its slot."""
    kc, vc = k_cache.copy(), v_cache.copy()
    bs = kc.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        kc[slot // bs, :, slot % bs, :] = k[t]
        vc[slot // bs, :, slot % bs, :] = v[t]
    return kc, vc


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, block_mapping: np.ndarray,
                k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None):
    """Return copies with ``cache[dst] = old_cache[src]`` for every (src, dst) pair.

    Returns ``(k_cache, v_cache, k_scale, v_scale)``; the scales are ``None`` when not given.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
        if ks is not None:
            ks[dst] = k_scale[src]
        if vs is not None:
            vs[dst] = v_scale[src]
    return kc, vc, ks, vs
