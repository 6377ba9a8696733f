"""8-bit KV input preparation: fp16 values -> OCP FP8 E4M3 codes + per-(block, KV head) scales.

The pages only say that an 8-bit KV cache halves the bytes per value and doubles the number of
requests that fit ("serving-paged-attention", section "실무에서 만지는 지점"; the talk summary's
paragraph on KV quantization). The format is fixed here as OCP E4M3 (bias 7, largest finite
448, no infinities, S.1111.111 = NaN) with one fp32 scale per (physical block, KV head),
separately for K and V: ``s = amax / 448`` (``s = 1`` when the tile is all zero) and
``code = round-to-nearest-even(clamp(x / s, -448, 448))``. The cast is torch's
``float8_e4m3fn`` conversion, applied after the clamp so nothing saturates to NaN.

Only inputs are made here. The attention kernels dequantize ``code * scale``; the oracle is fed
the same codes and scales.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F


def quantize_tile(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Quantize one tile (any shape, fp16/fp32, NaN entries ignored and emitted as NaN codes)."""
    xf = np.asarray(x, dtype=np.float32)
    live = ~np.isnan(xf)
    amax = float(np.max(np.abs(xf[live]))) if live.any() else 0.0
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(np.where(live, xf, 0.0) / s, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[~live] = E4M3_NAN_CODE
    return codes, s


def quantize_pool(cache: np.ndarray, live_blocks: np.ndarray, chunk: int = 2048) -> tuple[np.ndarray, np.ndarray]:
    """Quantize a ``[NB, Hkv, BS, D]`` fp16 pool tile by tile (same rule as :func:`quantize_tile`).

    Blocks not in ``live_blocks`` become all-NaN codes with a NaN scale (they are never read).
    Works on ``chunk`` blocks at a time. Returns ``(codes uint8 [NB, Hkv, BS, D], scales float32
    [NB, Hkv])``.
    """
    nb, hkv = cache.shape[:2]
    codes = np.full(cache.shape, E4M3_NAN_CODE, dtype=np.uint8)
    scales = np.full((nb, hkv), np.nan, dtype=np.float32)
    live_blocks = np.asarray(live_blocks, dtype=np.int64)
    for i in range(0, len(live_blocks), chunk):
        ids = live_blocks[i: i + chunk]
        x = torch.from_numpy(cache[ids]).float()  # [n, Hkv, BS, D]
        live = ~torch.isnan(x)
        xz = torch.where(live, x, torch.zeros((), dtype=torch.float32))
        amax = xz.abs().amax(dim=(2, 3))
        s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones((), dtype=torch.float32))
        y = (xz / s[:, :, None, None]).clamp(-E4M3_MAX, E4M3_MAX)
        c = y.to(torch.float8_e4m3fn).view(torch.uint8)
        c[~live] = E4M3_NAN_CODE
        codes[ids] = c.numpy()
        scales[ids] = s.numpy()
    return codes, scales
