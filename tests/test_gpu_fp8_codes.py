"""GPU pin of the in-kernel E4M3 decode for every finite code.

An 8-bit KV cache holds OCP E4M3 codes with one fp32 scale per (block, KV head)
("serving-paged-attention", section "실무에서 만지는 지점": the cache may be kept in 8 bits). The
random N(0, 1) pools of the other tests would hide one wrong code (a subnormal, or one near
±448) inside the attention tolerance, so this test isolates the decode: every sequence has a
single cached token, whose softmax weight is exactly 1, so the output row is that token's
dequantized V row, code * scale, rounded to fp16. The keys are code 0 (score 0, weight
2^0 = 1 exactly) and every other slot of the blocks holds the NaN code, which masking must keep
out. Each of the 254 finite codes appears in a V row, under V scales 1 and 2^-3 (all products
are exact in fp16), and the output is compared value for value with the oracle's E4M3 table
(+0 and -0 compare equal: the kernels add the product to a +0 accumulator).

Covered: the vector-ALU decode kernel (G = 1 and 3 query heads per KV head), the matrix-core
decode kernel (G = 4 and 8 in a padded 16-row tile, G = 32) and the prefill kernel (one-token
chunks),
for D 64 / 128 and block sizes 8 / 16.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_helpers import dev, log

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)  # 254 codes


def codes_case(d, bs, hkv, v_scale_value, seed):
    """One single-token sequence per V row; KV head h of sequence b holds a rotation of the
    finite codes so that every code appears in every head."""
    rng = np.random.default_rng(seed)
    rows = -(-len(FINITE) // d)
    padded = np.concatenate([FINITE, np.zeros(rows * d - len(FINITE), np.uint8)])
    seqs = rows
    nb = seqs + 3
    blocks = rng.permutation(nb)[:seqs]
    k_cache = np.full((nb, hkv, bs, d), NAN_CODE, np.uint8)
    v_cache = np.full((nb, hkv, bs, d), NAN_CODE, np.uint8)
    v_rows = np.zeros((seqs, hkv, d), np.uint8)
    for b in range(seqs):
        for h in range(hkv):
            row = np.roll(padded, 37 * h)[b * d:(b + 1) * d]
            v_rows[b, h] = row
            v_cache[blocks[b], h, 0] = row
            k_cache[blocks[b], h, 0] = 0
    k_scale = np.ones((nb, hkv), np.float32)
    v_scale = np.full((nb, hkv), v_scale_value, np.float32)
    tables = np.stack([blocks, blocks], 1).astype(np.int32)  # second entry never read
    lens = np.ones(seqs, np.int32)
    return dict(k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
                tables=tables, lens=lens, v_rows=v_rows, seqs=seqs)


def expected(c, hq, hkv, v_scale_value):
    g = hq // hkv
    vals = oracle.E4M3_TABLE[c["v_rows"]] * float(v_scale_value)  # [S, Hkv, D], float64, exact
    out = np.repeat(vals, g, axis=1).astype(np.float16)  # rounding is exact: checked below
    assert np.array_equal(out.astype(np.float64), np.repeat(vals, g, axis=1))
    return out


def check(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.float().cpu().numpy()
    w = want.astype(np.float32)
    bad = np.argwhere(g != w)
    log(f"{what}: {g.size} elements, {len(bad)} mismatches")
    assert len(bad) == 0, f"{what}: first mismatches at {bad[:5].tolist()}: got {g[tuple(bad[0])]}, want {w[tuple(bad[0])]}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [8, 16])
@pytest.mark.parametrize("g", [1, 3, 4, 8, 32])
@pytest.mark.parametrize("v_scale_value", [1.0, 0.125])
def test_decode_dequantizes_every_code(d, bs, g, v_scale_value):
    import paged_kv_cache_287_amd as pa

    hkv = 2
    hq = g * hkv
    c = codes_case(d, bs, hkv, v_scale_value, seed=900 + d + bs + g)
    rng = np.random.default_rng(901)
    q = dev(rng.standard_normal((c["seqs"], hq, d), dtype=np.float32).astype(np.float16))
    out = torch.full_like(q, float("nan"))
    log(f"[e4m3 codes] decode D={d} BS={bs} G={g} v_scale={v_scale_value}")
    pa.pa_decode(out, q, dev(c["k_cache"]), dev(c["v_cache"]), dev(c["tables"]), dev(c["lens"]),
                 float(1.0 / np.sqrt(d)), k_scale=dev(c["k_scale"]), v_scale=dev(c["v_scale"]))
    torch.cuda.synchronize()
    check(out, expected(c, hq, hkv, v_scale_value), f"decode D{d} BS{bs} G{g} s={v_scale_value}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 32])
@pytest.mark.parametrize("v_scale_value", [1.0, 0.125])
def test_prefill_dequantizes_every_code(d, g, v_scale_value):
    import paged_kv_cache_287_amd as pa

    hkv, bs = 2, 16
    hq = g * hkv
    c = codes_case(d, bs, hkv, v_scale_value, seed=950 + d + g)
    rng = np.random.default_rng(951)
    s = c["seqs"]
    q = dev(rng.standard_normal((s, hq, d), dtype=np.float32).astype(np.float16))
    out = torch.full_like(q, float("nan"))
    qs = dev(np.arange(s + 1, dtype=np.int32))
    log(f"[e4m3 codes] prefill D={d} G={g} v_scale={v_scale_value}")
    pa.pa_prefill(out, q, dev(c["k_cache"]), dev(c["v_cache"]), dev(c["tables"]), dev(c["lens"]),
                  qs, float(1.0 / np.sqrt(d)), max_query_len=1, max_context_len=bs,
                  k_scale=dev(c["k_scale"]), v_scale=dev(c["v_scale"]))
    torch.cuda.synchronize()
    check(out, expected(c, hq, hkv, v_scale_value), f"prefill D{d} G{g} s={v_scale_value}")
