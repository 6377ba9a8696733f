"""Pins for the float64 oracle: each check compares it with something other than itself.

* torch's own attention routine (scaled_dot_product_attention, float64 on the CPU) over the
  generator's contiguous logical K/V, i.e. unpaged attention;
* torch's float8_e4m3fn decoding for all 256 codes;
* closed forms (hand-computable softmax weights, L = 1, q = 0, identical keys);
* brute-force scalar loops with math.fsum on the tiny workload;
* invariants the pages state: physical relabelling changes nothing, copy-on-write leaves the
  other sequences' view unchanged, shared-prefix tables point at one copy;
* the pages' printed capacity numbers (tests/golden/pages_facts.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.attention import attend
from workloads.configs import scatter_sequence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def sdpa_reference(q: np.ndarray, logical_k, logical_v, scale) -> np.ndarray:
    """torch SDPA in float64 over contiguous K/V, KV heads repeated per group (unpaged)."""
    s_, hq, d = q.shape
    out = np.zeros((s_, hq, d))
    for b, (kk, vv) in enumerate(zip(logical_k, logical_v)):
        hkv = kk.shape[1]
        g = hq // hkv
        qt = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]  # [1, Hq, 1, D]
        kt = torch.from_numpy(np.asarray(kk, dtype=np.float64)).permute(1, 0, 2)  # [Hkv, L, D]
        vt = torch.from_numpy(np.asarray(vv, dtype=np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(g, dim=0)[None]
        vt = vt.repeat_interleave(g, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(np.float32(scale)))
        out[b] = o[0, :, 0, :].numpy()
    return out


def run_oracle(case, **kw):
    return oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                         case.scale, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                         v_scale=case.v_scale, **kw)


# ------------------------------------------------------------------------------------------
# E4M3 decoding
# ------------------------------------------------------------------------------------------
def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3_to_float(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    assert np.isnan(mine).sum() == 2 and np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


def test_e4m3_closed_forms():
    t = oracle.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0  # largest finite
    assert t[0x38] == 1.0
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0


# ------------------------------------------------------------------------------------------
# attention: closed forms
# ------------------------------------------------------------------------------------------
def test_attend_hand_computed_weights():
    # scores 0 and ln 3 -> weights 1/4 and 3/4
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o = attend(q, k, v, 1.0)
    assert np.allclose(o, [[0.25, 0.75]], rtol=0, atol=1e-15)
    # the scale multiplies the scores before the softmax
    o2 = attend(q, k, v, 0.5)  # scores 0, ln(3)/2 -> weights 1/(1+sqrt3), sqrt3/(1+sqrt3)
    r3 = math.sqrt(3.0)
    assert np.allclose(o2, [[1 / (1 + r3), r3 / (1 + r3)]], rtol=0, atol=1e-15)


def test_single_token_returns_its_value():
    case = workloads.random_case(11, [1, 1, 1], 8, 2, 64, 16)
    out = run_oracle(case)
    for b in range(3):
        for h in range(8):
            assert np.array_equal(out[b, h], case.logical_v[b][0, h // 4].astype(np.float64))


def test_zero_query_and_identical_keys_give_mean_value():
    case = workloads.random_case(12, [37, 200], 4, 4, 128, 16)
    case.q[:] = 0
    out = run_oracle(case)
    for b in range(2):
        mean = case.logical_v[b].astype(np.float64).mean(axis=0)  # [Hkv, D]
        assert np.allclose(out[b], mean, rtol=0, atol=1e-14)
    case = workloads.random_case(13, [50], 2, 1, 64, 8)
    L = 50
    same_k = np.repeat(case.logical_k[0][:1], L, axis=0)
    scatter_sequence(case.k_cache, case.block_tables[0], same_k)
    out = run_oracle(case)
    mean = case.logical_v[0].astype(np.float64).mean(axis=0)
    assert np.allclose(out[0], np.repeat(mean, 2, axis=0), rtol=0, atol=1e-14)


def test_empty_sequence_gives_zero():
    case = workloads.random_case(14, [0, 5], 4, 2, 64, 16)
    out = run_oracle(case)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


# ------------------------------------------------------------------------------------------
# attention: against torch's independent routine (unpaged, contiguous K/V)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("lens,hq,hkv,d,bs", [
    ([1, 15, 16, 33], 4, 2, 64, 16),
    ([100, 7, 300], 8, 8, 128, 8),     # MHA
    ([64, 513, 2], 32, 8, 128, 32),    # GQA 4
    ([129, 40], 32, 1, 128, 64),       # MQA
    ([17, 250], 6, 2, 64, 16),         # GQA 3
])
def test_decode_equals_unpaged_sdpa(lens, hq, hkv, d, bs):
    case = workloads.random_case(21, lens, hq, hkv, d, bs)
    out = run_oracle(case)
    ref = sdpa_reference(case.q, case.logical_k, case.logical_v, case.scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_tiny_workload_equals_unpaged_sdpa():
    case = workloads.tiny()
    out = run_oracle(case)
    ref = sdpa_reference(case.q, case.logical_k, case.logical_v, case.scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_tiny_workload_brute_force_fsum():
    case = workloads.tiny()
    out = run_oracle(case)
    s_, hq, d = case.q.shape
    g = hq // case.num_kv_heads
    for b in range(s_):
        L = int(case.context_lens[b])
        for h in range(hq):
            kvh = h // g
            q = [float(x) for x in case.q[b, h]]
            scores = []
            for t in range(L):
                blk = int(case.block_tables[b, t // 16])
                kt = case.k_cache[blk, kvh, t % 16]
                scores.append(0.125 * math.fsum(q[i] * float(kt[i]) for i in range(d)))
            m = max(scores)
            w = [math.exp(x - m) for x in scores]
            den = math.fsum(w)
            for i in range(d):
                num = math.fsum(w[t] * float(case.v_cache[int(case.block_tables[b, t // 16]), kvh, t % 16, i])
                                for t in range(L))
                assert abs(out[b, h, i] - num / den) <= 1e-13


def _flat_slot_view(pool64: np.ndarray, table_row, length, bs):
    """Alternative indexing route: the pool as a flat token-slot array [NB*BS, Hkv, D]."""
    flat = pool64.transpose(0, 2, 1, 3).reshape(-1, pool64.shape[1], pool64.shape[3])
    t = np.arange(length)
    return flat[np.asarray(table_row, dtype=np.int64)[t // bs] * bs + t % bs]


@pytest.mark.parametrize("hkv", [8, 1])
def test_fp8_decode_equals_sdpa_on_torch_dequantized_cache(hkv):
    case = workloads.random_case(31, [40, 333, 16], 32, hkv, 128, 16)
    tables = [row[: -(-int(L) // 16)] for row, L in zip(case.block_tables, case.context_lens)]
    live = np.unique(np.concatenate(tables).astype(np.int64))
    kc, ks = workloads.quantize_pool(case.k_cache, live)
    vc, vs = workloads.quantize_pool(case.v_cache, live)
    out = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                        kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)

    def deq(codes, scales):
        x = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return x * scales.astype(np.float64)[:, :, None, None]

    kd, vd = deq(kc, ks), deq(vc, vs)
    lk = [_flat_slot_view(kd, case.block_tables[b], int(L), 16) for b, L in enumerate(case.context_lens)]
    lv = [_flat_slot_view(vd, case.block_tables[b], int(L), 16) for b, L in enumerate(case.context_lens)]
    ref = sdpa_reference(case.q, lk, lv, case.scale)
    assert np.max(np.abs(out - ref)) < 1e-12
    # quantization error against the fp16 cache is small but non-zero (reported, not gated)
    out16 = run_oracle(case)
    err = np.max(np.abs(out - out16))
    assert 0 < err < 0.1


# ------------------------------------------------------------------------------------------
# invariants from the pages
# ------------------------------------------------------------------------------------------
def relabel(case, seed):
    """Move every physical block p to pi(p) and rewrite the tables accordingly."""
    rng = np.random.default_rng(seed)
    pi = rng.permutation(case.num_blocks)
    kc = np.empty_like(case.k_cache)
    vc = np.empty_like(case.v_cache)
    kc[pi] = case.k_cache
    vc[pi] = case.v_cache
    ks = vs = None
    if case.k_scale is not None:
        ks = np.empty_like(case.k_scale)
        vs = np.empty_like(case.v_scale)
        ks[pi] = case.k_scale
        vs[pi] = case.v_scale
    return kc, vc, ks, vs, pi[case.block_tables].astype(np.int32)


@pytest.mark.parametrize("kv_dtype", ["f16", "fp8_e4m3"])
def test_physical_relabelling_changes_nothing(kv_dtype):
    case = workloads.random_case(41, [5, 77, 160, 1], 8, 2, 128, 16, kv_dtype=kv_dtype)
    out = run_oracle(case)
    kc, vc, ks, vs, tables = relabel(case, 99)
    out2 = oracle.decode(case.q, kc, vc, tables, case.context_lens, case.scale, kv_dtype=kv_dtype,
                         k_scale=ks, v_scale=vs)
    assert np.array_equal(out, out2)


def test_unused_slots_are_poisoned_and_ignored():
    case = workloads.tiny()
    # the generator leaves every unattended slot NaN; the oracle output stays finite
    assert np.isnan(case.k_cache[case.pad_block]).all()
    out = run_oracle(case)
    assert np.isfinite(out).all()


@pytest.fixture(scope="module")
def prefix_case():
    return workloads.shared_prefix(False)


@pytest.fixture(scope="module")
def fork_case():
    return workloads.shared_prefix(True)


def test_shared_prefix_tables_alias_one_copy(prefix_case):
    case = prefix_case
    pre = case.step.pre_block_tables
    lens = case.step.pre_context_lens
    assert pre.shape[0] == 100
    first = pre[:, :32]
    assert (first == first[0]).all()  # every table starts with the same 32 physical ids
    private = sum(-(-int(L) // 16) - 32 for L in lens)
    used = set()
    for row, L in zip(pre, lens):
        used.update(int(x) for x in row[: -(-int(L) // 16)])
    assert len(used) == 32 + private
    # the shared block-aligned prefix never needs a copy in this step
    assert case.step.block_mapping.shape == (0, 2)


def _apply_step(case):
    st = case.step
    kc, vc, _, _ = oracle.copy_blocks(case.k_cache, case.v_cache, st.block_mapping)
    return oracle.kv_write(st.new_k, st.new_v, kc, vc, st.slot_mapping)


def test_slot_mapped_append_round_trips_through_tables(prefix_case):
    case = prefix_case
    kc, vc = _apply_step(case)
    for b in range(case.num_seqs):
        L = int(case.context_lens[b])
        kk = oracle.gather_sequence(kc, case.block_tables[b], L)
        vv = oracle.gather_sequence(vc, case.block_tables[b], L)
        assert np.array_equal(kk, case.logical_k[b].astype(np.float64))
        assert np.array_equal(vv, case.logical_v[b].astype(np.float64))


def test_append_writes_only_its_slots(prefix_case):
    case = prefix_case
    kc, vc = _apply_step(case)
    changed = np.any(kc.view(np.uint16) != case.k_cache.view(np.uint16), axis=(1, 3))  # [NB, BS]
    expect = np.zeros_like(changed)
    for s in case.step.slot_mapping:
        expect[s // 16, s % 16] = True
    assert np.array_equal(changed, expect)


def test_copy_on_write_isolation(fork_case):
    case = fork_case
    st = case.step
    assert len(st.block_mapping) > 50  # most last blocks are partially filled and shared
    pre = oracle.decode(case.q, case.k_cache, case.v_cache, st.pre_block_tables,
                        st.pre_context_lens, case.scale)
    kc, vc = _apply_step(case)
    # the view through the old tables is untouched by the copies and the appends
    again = oracle.decode(case.q, kc, vc, st.pre_block_tables, st.pre_context_lens, case.scale)
    assert np.array_equal(pre, again)
    # siblings now differ only by their own new token, and each matches unpaged attention
    post = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale)
    ref = sdpa_reference(case.q, case.logical_k, case.logical_v, case.scale)
    assert np.max(np.abs(post - ref)) < 1e-12
    copied, _, _, _ = oracle.copy_blocks(case.k_cache, case.v_cache, st.block_mapping)
    for src, dst in st.block_mapping:
        assert src != dst
        assert np.array_equal(copied[dst].view(np.uint16), case.k_cache[src].view(np.uint16))


def test_copy_blocks_copies_from_pre_call_state_including_scales():
    rng = np.random.default_rng(5)
    kc = rng.standard_normal((6, 2, 4, 8)).astype(np.float16)
    vc = rng.standard_normal((6, 2, 4, 8)).astype(np.float16)
    ks = rng.random((6, 2)).astype(np.float32)
    vs = rng.random((6, 2)).astype(np.float32)
    pairs = np.array([[0, 3], [1, 4]], dtype=np.int32)
    k2, v2, ks2, vs2 = oracle.copy_blocks(kc, vc, pairs, ks, vs)
    for s, d in pairs:
        assert np.array_equal(k2[d], kc[s]) and np.array_equal(v2[d], vc[s])
        assert ks2[d].tolist() == ks[s].tolist() and vs2[d].tolist() == vs[s].tolist()
    for untouched in (0, 1, 2, 5):
        assert np.array_equal(k2[untouched], kc[untouched])


# ------------------------------------------------------------------------------------------
# the pages' capacity numbers
# ------------------------------------------------------------------------------------------
def test_capacity_numbers_from_pages():
    facts = json.load(open(GOLDEN))
    f = facts["kv_bytes_per_token_8b"]
    per_tok = oracle.kv_cache_bytes(f["layers"], f["kv_heads"], f["head_dim"], 1, f["bytes_per_value"])
    assert per_tok == f["bytes"] == 128 * 1024
    r = facts["kv_bytes_4096_token_request"]
    per_req = oracle.kv_cache_bytes(f["layers"], f["kv_heads"], f["head_dim"], r["tokens"], f["bytes_per_value"])
    assert per_req == r["bytes"] == 512 * 2 ** 20
    m = facts["max_requests_80gb_card"]
    free = (m["card_gib"] - m["weights_gib"]) * 2 ** 30
    assert m["free_gib"] * 2 ** 30 == free
    assert oracle.max_concurrent_requests(free, int(per_req)) == m["requests"]
    w = facts["naive_reservation_waste"]
    frac = oracle.naive_waste_fraction(w["max_tokens"], w["average_tokens"])
    assert int(100 * frac) == w["printed_percent"]
    e = facts["eight_bit_kv_capacity"]
    b16 = oracle.kv_cache_bytes(32, 8, 128, 4096, e["bytes_per_value_before"])
    b8 = oracle.kv_cache_bytes(32, 8, 128, 4096, e["bytes_per_value_after"])
    assert oracle.max_concurrent_requests(free, int(b8)) == e["requests_factor"] * m["requests"]
    # with one fp32 scale per (block, head) for K and V, the gain is just under 2 at BS 16
    b8s = b8 + 2 * 32 * 8 * (4096 // 16) * 4
    assert 1.99 < b16 / b8s < 2.0


def test_paged_waste_bound_from_pages():
    facts = json.load(open(GOLDEN))
    p = facts["paged_waste_bound"]
    bs = p["block_size"]
    assert max(oracle.paged_waste_slots(L, bs) for L in range(1, 5000)) == p["max_waste_tokens"]
    ex = facts["four_slot_page_example"]
    assert -(-ex["tokens"] // ex["slots_per_page"]) == ex["pages"]
    assert oracle.paged_waste_slots(ex["tokens"], ex["slots_per_page"]) == ex["idle_slots_without_sharing"]
    assert facts["default_block_size"]["tokens"] == 16


# ------------------------------------------------------------------------------------------
# E4M3 encoding and the 8-bit append policy
# ------------------------------------------------------------------------------------------
def test_e4m3_encoder_matches_torch_including_ties():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(50000) * 60, rng.standard_normal(20000) * 0.02,
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11]])
    x = np.clip(x, -448, 448).astype(np.float32)
    vals = oracle.E4M3_TABLE[:0x7F]
    ties = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    for arr in (x, ties, -ties):
        ref = torch.from_numpy(arr).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.float_to_e4m3(arr), ref)
    # round trip of every finite code
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.float_to_e4m3(oracle.e4m3_to_float(codes).astype(np.float32)), codes)


def _fp8_pool(nb=8, hkv=2, bs=16, d=64):
    codes = np.full((nb, hkv, bs, d), 0x7F, dtype=np.uint8)
    scales = np.full((nb, hkv), np.nan, dtype=np.float32)
    return codes, codes.copy(), scales, scales.copy()


def test_fp8_append_first_token_equals_tile_quantizer():
    rng = np.random.default_rng(8)
    kc, vc, ks, vs = _fp8_pool()
    k = (rng.standard_normal((1, 2, 64)) * 3).astype(np.float16)
    v = rng.standard_normal((1, 2, 64)).astype(np.float16)
    kc2, vc2, ks2, vs2 = oracle.kv_write_fp8(k, v, kc, vc, ks, vs, np.array([3 * 16], np.int64))
    for h in range(2):
        codes, s = workloads.quantize_tile(k[0, h])
        assert np.array_equal(kc2[3, h, 0], codes) and ks2[3, h] == s
        codes, s = workloads.quantize_tile(v[0, h])
        assert np.array_equal(vc2[3, h, 0], codes) and vs2[3, h] == s
    assert np.array_equal(kc2[[0, 1, 2, 4, 5, 6, 7]], kc[[0, 1, 2, 4, 5, 6, 7]])


def test_fp8_append_without_growth_equals_whole_block_quantization():
    # the largest token first: later appends never rescale, and the block equals quantizing
    # the whole block at once with the same amax / 448 rule
    rng = np.random.default_rng(9)
    kc, vc, ks, vs = _fp8_pool()
    rows = rng.standard_normal((10, 2, 64)).astype(np.float32)
    rows[0] *= 8
    rows = rows.astype(np.float16)
    for t in range(10):
        prev = kc.copy()
        kc, vc, ks, vs = oracle.kv_write_fp8(rows[t:t + 1], rows[t:t + 1], kc, vc, ks, vs,
                                             np.array([5 * 16 + t], np.int64))
        assert np.array_equal(kc[5, :, :t], prev[5, :, :t])  # earlier codes untouched
    for h in range(2):
        codes, s = workloads.quantize_tile(rows[:, h])
        assert np.array_equal(kc[5, h, :10], codes) and ks[5, h] == s


def test_fp8_append_growth_rescales_and_keeps_the_bound():
    # Each stored value is rounded once when written and once more every time its block's
    # scale grows afterwards; one E4M3 rounding errs by at most 2^-4 of the value (normal
    # range) or 2^-10 of the scale (subnormal range).
    rng = np.random.default_rng(10)
    kc, vc, ks, vs = _fp8_pool()
    ks[2] = 1e30  # a stale scale from an earlier use of the block is ignored at offset 0
    rows = (rng.standard_normal((16, 2, 64)) * np.geomspace(0.01, 50, 16)[:, None, None]).astype(np.float16)
    rescales = np.zeros((16, 2), dtype=np.int64)  # later rescales seen by each stored token
    for t in range(16):
        before = ks[2].copy()
        kc, vc, ks, vs = oracle.kv_write_fp8(rows[t:t + 1], rows[t:t + 1], kc, vc, ks, vs,
                                             np.array([2 * 16 + t], np.int64))
        if t > 0:
            rescales[:t] += (ks[2] != before)[None, :]
        x = rows[: t + 1].astype(np.float64)  # [t+1, 2, 64]
        for h in range(2):
            amax = np.abs(x[:, h]).max()
            assert ks[2, h] >= np.float32(amax / 448) * (1 - 1e-7)
            back = oracle.e4m3_to_float(kc[2, h, : t + 1]) * ks[2, h]
            err = np.abs(back - x[:, h])
            n = (1 + rescales[: t + 1, h])[:, None]
            assert (err <= n * (2.0 ** -4 * 1.1 * np.abs(x[:, h]) + 2.0 ** -10 * ks[2, h])).all()
    assert rescales.max() >= 5  # the growth did force repeated re-encoding
    assert ks[2, 0] == np.float32(np.float32(np.abs(rows[:, 0].astype(np.float32)).max()) / np.float32(448))


def test_swap_round_trip_restores_blocks_and_attention():
    # swap a sequence's blocks out to a host pool, then back in at other device ids: the
    # blocks come back bit for bit and attention through the re-pointed table is unchanged
    case = workloads.random_case(61, [40, 130, 7], 8, 2, 64, 16, pool_factor=3.0)
    ref = run_oracle(case)
    b = 1
    n = -(-int(case.context_lens[b]) // 16)
    old_ids = case.block_tables[b, :n].copy()
    host_k = np.zeros((n,) + case.k_cache.shape[1:], np.float16)
    host_v = np.zeros_like(host_k)
    hk, hv, _ = oracle.swap_blocks(case.k_cache, case.v_cache, host_k, host_v,
                                   np.stack([old_ids, np.arange(n)], 1))
    used = set(int(x) for r, L in zip(case.block_tables, case.context_lens) for x in r[: -(-int(L) // 16)])
    free = [i for i in range(case.num_blocks) if i not in used and i != case.pad_block][:n]
    kc, vc, _ = oracle.swap_blocks(hk, hv, case.k_cache, case.v_cache, np.stack([np.arange(n), free], 1))
    for i, (o, f) in enumerate(zip(old_ids, free)):
        assert np.array_equal(kc[f].view(np.uint16), case.k_cache[o].view(np.uint16))
    tables = case.block_tables.copy()
    tables[b, :n] = free
    out = oracle.decode(case.q, kc, vc, tables, case.context_lens, case.scale)
    assert np.array_equal(out, ref)


# ------------------------------------------------------------------------------------------
# paged prefill (causal chunk attention)
# ------------------------------------------------------------------------------------------
def test_prefill_equals_causal_sdpa_and_decode_on_last_token():
    case = workloads.random_case(71, [40, 130, 17], 8, 2, 64, 16)
    n = [13, 130, 1]  # chunk lengths: partial, whole prompt, a single (decode) token
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    rng = np.random.default_rng(72)
    q = rng.standard_normal((qs[-1], 8, 64)).astype(np.float16)
    out = oracle.prefill(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, qs,
                         case.scale)
    for b in range(3):
        L = int(case.context_lens[b])
        kt = torch.from_numpy(case.logical_k[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(4, 0)
        vt = torch.from_numpy(case.logical_v[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(4, 0)
        qt = torch.from_numpy(q[qs[b]:qs[b + 1]].astype(np.float64)).permute(1, 0, 2)  # [H, n, D]
        pos = torch.arange(L - n[b], L)[:, None]
        mask = torch.arange(L)[None, :] <= pos  # [n, L] causal with the chunk at the end
        ref = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=mask,
                                                               scale=float(np.float32(case.scale)))
        assert np.max(np.abs(out[qs[b]:qs[b + 1]] - ref[0].permute(1, 0, 2).numpy())) < 1e-12
    # the last query of each chunk sees the whole context: it is a decode step
    last = q[qs[1:] - 1]
    dec = oracle.decode(last, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale)
    assert np.array_equal(out[qs[1:] - 1], dec)
