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

from .fp8 import E4M3_TABLE, float_to_e4m3

E4M3_MAX = np.float32(448.0)


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


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                block_mapping: np.ndarray, src_scales=None, dst_scales=None):
    """Preemption by swap moves whole blocks to another pool and back ("serving-paged-
    attention", section "그래도 넘칠 때 — 선점"): ``dst[d] = src[s]`` for every (s, d) pair,
    with the per-(block, head) scales of an 8-bit pool. Returns new ``(dst_k, dst_v, dst_scales)``
    (``dst_scales`` a (k, v) pair or None)."""
    dk, dv = dst_k.copy(), dst_v.copy()
    ds = None if dst_scales is None else (dst_scales[0].copy(), dst_scales[1].copy())
    for s, d in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        dk[d] = src_k[s]
        dv[d] = src_v[s]
        if ds is not None:
            ds[0][d] = src_scales[0][s]
            ds[1][d] = src_scales[1][s]
    return dk, dv, ds


def kv_write_fp8(k: np.ndarray, v: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray,
                 k_scale: np.ndarray, v_scale: np.ndarray, slot_mapping: np.ndarray):
    """Slot-mapped append into an E4M3 cache with one fp32 scale per (block, KV head).

    The pages give no scale policy for appending to an 8-bit cache; the one computed here keeps
    each scale an upper bound of its block's content over 448, the rule the input quantizer
    uses. For each token, in the order of the call, and KV head, all in float32:

    * ``s_prev`` = the block's scale, or 0 when the token lands at offset 0 (a fresh block);
    * ``a`` = max |x| over the token's row; ``s = a / 448`` if ``a > s_prev * 448``, else
      ``s = s_prev``; a fresh all-zero row gets ``s = 1``;
    * if ``s`` changed and the block already holds tokens, each stored code ``c`` at offsets
      before the token is re-encoded as ``enc(f32(f32(dec(c) * s_prev) / s))``;
    * the token itself is stored as ``enc(f32(x) / s)``; ``enc`` clamps to [-448, 448] and rounds
      to nearest-even (:func:`oracle.fp8.float_to_e4m3`).

    Returns new ``(k_codes, v_codes, k_scale, v_scale)``.
    """
    kc, vc = k_codes.copy(), v_codes.copy()
    ks, vs = k_scale.copy(), v_scale.copy()
    bs = kc.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = int(slot // bs), int(slot % bs)
        for codes, scales, rows in ((kc, ks, k), (vc, vs, v)):
            for h in range(codes.shape[1]):
                x = np.asarray(rows[t, h], dtype=np.float16).astype(np.float32)
                s_prev = np.float32(0.0) if off == 0 else np.float32(scales[blk, h])
                a = np.float32(np.max(np.abs(x)))
                s = np.float32(a / E4M3_MAX) if a > np.float32(s_prev * E4M3_MAX) else s_prev
                if s == 0:
                    s = np.float32(1.0)
                if s != s_prev and off > 0:
                    old = E4M3_TABLE[codes[blk, h, :off]].astype(np.float32)
                    y = (old * s_prev).astype(np.float32) / s
                    codes[blk, h, :off] = float_to_e4m3(np.clip(y, -E4M3_MAX, E4M3_MAX))
                codes[blk, h, off] = float_to_e4m3(np.clip(x / s, -E4M3_MAX, E4M3_MAX))
                scales[blk, h] = s
    return kc, vc, ks, vs
