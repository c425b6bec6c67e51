"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle fails at least one of
them: a dropped scale or a sign error (library attention, worked example), a
wrong block/offset split or layout index (library attention on randomly placed
blocks, worked example, block-size repacking), a wrong grouped-query mapping
(library attention with grouped heads, repeated-head equivalence, worked
example head 1), a wrong decoder or rounding (exhaustive decoder checks,
library rounding), reads of unused memory (NaN poison everywhere unused).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers: build paged inputs from contiguous per-sequence K/V (test-side)
# ---------------------------------------------------------------------------

def _to_storage(x64, dtype):
    """float64 array -> (storage array, exact float64 values of the stored elements)."""
    if dtype == "f32":
        st = x64.astype(np.float32)
        return st, st.astype(np.float64)
    if dtype == "f16":
        st = x64.astype(np.float16)
        return st, st.astype(np.float64)
    t = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16)
    st = t.view(torch.int16).numpy().view(np.uint16)
    return st.copy(), t.to(torch.float64).numpy()


def _nan_storage(dtype):
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.uint16(0x7FC0)


def make_paged_case(rng, ctxs, Hq, Hkv, D, bs, dtype, free_blocks=3, table_pad=1):
    """Random q, contiguous K/V per sequence, scattered into a NaN-poisoned pool.

    Returns storage arrays for the oracle plus exact float64 contiguous copies
    for the library reference.
    """
    S = len(ctxs)
    nblk = [(c + bs - 1) // bs for c in ctxs]
    NB = sum(nblk) + free_blocks
    MB = max(max(nblk), 1) + table_pad
    perm = rng.permutation(NB)
    tables = np.full((S, MB), -1, dtype=np.int32)
    k_pool = np.full((NB, bs, Hkv, D), _nan_storage(dtype))
    v_pool = np.full((NB, bs, Hkv, D), _nan_storage(dtype))
    q_st, q64 = _to_storage(rng.standard_normal((S, Hq, D)), dtype)
    k64s, v64s = [], []
    used = 0
    for s, c in enumerate(ctxs):
        k_st, k64 = _to_storage(rng.standard_normal((c, Hkv, D)), dtype)
        v_st, v64 = _to_storage(rng.standard_normal((c, Hkv, D)), dtype)
        k64s.append(k64)
        v64s.append(v64)
        for j in range(nblk[s]):
            tables[s, j] = perm[used]
            used += 1
        for t in range(c):
            b = tables[s, t // bs]
            k_pool[b, t % bs] = k_st[t]
            v_pool[b, t % bs] = v_st[t]
    return dict(q=q_st, q64=q64, k_pool=k_pool, v_pool=v_pool, tables=tables,
                ctx=np.array(ctxs, dtype=np.int32), k64=k64s, v64=v64s, NB=NB, MB=MB)


def library_attention(q64, k64s, v64s, scale):
    """torch's scaled_dot_product_attention in float64 on contiguous K/V (grouped heads)."""
    S, Hq, D = q64.shape
    out = np.zeros((S, Hq, D))
    for s in range(S):
        if k64s[s].shape[0] == 0:
            continue
        q = torch.from_numpy(q64[s]).unsqueeze(0).unsqueeze(2)          # [1, Hq, 1, D]
        k = torch.from_numpy(k64s[s]).permute(1, 0, 2).unsqueeze(0)      # [1, Hkv, L, D]
        v = torch.from_numpy(v64s[s]).permute(1, 0, 2).unsqueeze(0)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k.contiguous(), v.contiguous(), scale=scale, enable_gqa=True)
        out[s] = o[0, :, 0, :].numpy()
    return out


# ---------------------------------------------------------------------------
# element decoders and rounding
# ---------------------------------------------------------------------------

def test_f16_decoder_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode_elements(bits.view(np.float16), "f16")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_bf16_decoder_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.decode_elements(bits, "bf16")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_single_value_decoders():
    assert oracle.f16_bits_to_f64(0x3C00) == 1.0
    assert oracle.f16_bits_to_f64(0x0001) == 2.0 ** -24
    assert oracle.f16_bits_to_f64(0x7BFF) == 65504.0
    assert oracle.bf16_bits_to_f64(0x3F80) == 1.0
    assert oracle.bf16_bits_to_f64(0xC000) == -2.0
    assert oracle.bf16_bits_to_f64(0x0001) == 2.0 ** -133


def _rounding_probe(rng, n):
    mant = rng.uniform(-1, 1, n)
    expo = rng.integers(-140, 130, n)
    x = np.ldexp(mant, expo)
    return np.concatenate([x, rng.standard_normal(n), [0.0, -0.0, 1.0, 65504.0, 65520.0, 1e300, -1e300]])


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(11)
    x = _rounding_probe(rng, 200000)
    ref = x.astype(np.float16).astype(np.float64)
    got = oracle.round_to_dtype(x, "f16")
    assert np.array_equal(ref, got)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(12)
    x = _rounding_probe(rng, 200000)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    got = oracle.round_to_dtype(x, "f32")
    assert np.array_equal(ref, got)


def test_round_bf16_matches_torch():
    # torch rounds float32 -> bfloat16 to nearest even; inputs exact in float32
    # make that a single rounding, so it is the same map as double -> bf16.
    rng = np.random.default_rng(13)
    x = _rounding_probe(rng, 200000)
    with np.errstate(over="ignore"):
        x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_dtype(x, "bf16")
    assert np.array_equal(ref, got)


def test_round_bf16_ties_to_even():
    one = 1.0
    half_ulp = 2.0 ** -8                      # bf16 has 7 fraction bits
    got = oracle.round_to_dtype(np.array([one + half_ulp, one + 3 * half_ulp, one + half_ulp * 1.0001]), "bf16")
    assert got[0] == 1.0                      # tie -> even (1.0)
    assert got[1] == 1.0 + 4 * half_ulp       # tie -> even (1 + 2^-6)
    assert got[2] == 1.0 + 2 * half_ulp       # above the tie -> up


# ---------------------------------------------------------------------------
# attention: library routine, worked example, closed forms, invariances
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (8, 2)])
@pytest.mark.parametrize("bs", [1, 8, 16])
def test_matches_library_attention(dtype, Hq, Hkv, bs):
    rng = np.random.default_rng(100 + Hq * 7 + Hkv * 3 + bs)
    D = 16
    ctxs = [1, bs, bs + 1, 3 * bs - 1, 37]
    c = make_paged_case(rng, ctxs, Hq, Hkv, D, bs, dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], scale, dtype)
    ref = library_attention(c["q64"], c["k64"], c["v64"], scale)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_worked_example():
    g = _golden("attention_worked_example.json")
    bs, NB, D, Hkv = g["block_size"], g["num_blocks"], g["head_dim"], g["num_kv_heads"]
    k_pool = np.full((NB, bs, Hkv, D), np.nan, dtype=np.float32)
    v_pool = np.full((NB, bs, Hkv, D), np.nan, dtype=np.float32)
    table = g["block_table"]
    for t in range(g["context_len"]):
        k_pool[table[t // bs], t % bs, 0] = g["k_logical"][t]
        v_pool[table[t // bs], t % bs, 0] = g["v_logical"][t]
    q = np.array([g["q"]], dtype=np.float32)
    got = oracle.paged_decode(q, k_pool, v_pool, np.array([table], dtype=np.int32),
                              np.array([g["context_len"]], dtype=np.int32), g["scale"], "f32")
    np.testing.assert_allclose(got[0], np.array(g["expected"]), rtol=0, atol=g["tolerance_abs"])
    # closed forms, recomputed here from the derivation
    e = math.e
    Z1 = math.exp(5) + math.exp(-2) + math.exp(7)
    assert abs(got[0, 0, 0] - 4 / (2 + e)) < 1e-14
    assert abs(got[0, 0, 1] - e / (2 + e)) < 1e-14
    assert abs(got[0, 1, 0] - (math.exp(5) + 3 * math.exp(7)) / Z1) < 1e-14
    assert abs(got[0, 1, 1] - math.exp(-2) / Z1) < 1e-14


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_context_one_returns_first_value_exactly(dtype):
    rng = np.random.default_rng(7)
    c = make_paged_case(rng, [1, 1, 1], 4, 2, 32, 16, dtype)
    got = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], 0.17, dtype)
    for s in range(3):
        for h in range(4):
            assert np.array_equal(got[s, h], c["v64"][s][0, h // 2])


def test_context_zero_gives_zeros():
    rng = np.random.default_rng(8)
    c = make_paged_case(rng, [0, 5, 0], 2, 2, 16, 8, "f32")
    got = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], 0.25, "f32")
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.all(np.isfinite(got[1])) and np.any(got[1] != 0)


@pytest.mark.parametrize("mode", ["identical_keys", "zero_scale"])
def test_equal_scores_give_mean_of_values(mode):
    rng = np.random.default_rng(9)
    ctxs = [1, 7, 16, 33]
    c = make_paged_case(rng, ctxs, 2, 1, 32, 8, "f32")
    scale = 0.0 if mode == "zero_scale" else 0.3
    if mode == "identical_keys":
        key = rng.standard_normal(32).astype(np.float32)
        for s, L in enumerate(ctxs):
            for t in range(L):
                c["k_pool"][c["tables"][s, t // 8], t % 8, 0] = key
    got = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], scale, "f32")
    for s in range(len(ctxs)):
        mean = c["v64"][s][:, 0, :].mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(got[s, h], mean, rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(10)
    c = make_paged_case(rng, [40], 1, 1, 16, 16, "f32")
    j = 23
    q = np.zeros((1, 1, 16), dtype=np.float32)
    q[0, 0, 3] = 1.0
    key = np.zeros(16, dtype=np.float32)
    key[3] = 200.0                             # score 200 vs |score| <= ~4 elsewhere
    for t in range(40):
        if t != j:
            c["k_pool"][c["tables"][0, t // 16], t % 16, 0, 3] = np.float32(rng.uniform(-1, 1))
    c["k_pool"][c["tables"][0, j // 16], j % 16, 0] = key
    got = oracle.paged_decode(q, c["k_pool"], c["v_pool"], c["tables"], c["ctx"], 1.0, "f32")
    np.testing.assert_allclose(got[0, 0], c["v64"][0][j, 0], rtol=0, atol=1e-70)


def test_shift_of_all_keys_leaves_output_unchanged():
    # adding the same vector to every key shifts every score by q.c*scale
    rng = np.random.default_rng(14)
    ctxs = [5, 30, 64]
    c = make_paged_case(rng, ctxs, 2, 2, 16, 16, "f32")
    # keys on a 2^-8 grid so that adding +-0.5 below is exact in f32
    c["k_pool"] = (np.round(c["k_pool"] * 256) / 256).astype(np.float32)
    base = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], 0.25, "f32")
    shift = np.float32(0.5) * np.sign(rng.standard_normal((2, 16))).astype(np.float32)
    k2 = c["k_pool"].copy()
    for s, L in enumerate(ctxs):
        for t in range(L):
            k2[c["tables"][s, t // 16], t % 16] += shift   # exact in f32 (+-0.5 on N(0,1) values)
    got = oracle.paged_decode(c["q"], k2, c["v_pool"], c["tables"], c["ctx"], 0.25, "f32")
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-12)


def test_linear_in_values():
    rng = np.random.default_rng(15)
    c = make_paged_case(rng, [9, 21], 2, 1, 8, 8, "f32")
    a = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], 0.4, "f32")
    v2 = (c["v_pool"] * np.float32(2.0)).astype(np.float32)
    b = oracle.paged_decode(c["q"], c["k_pool"], v2, c["tables"], c["ctx"], 0.4, "f32")
    np.testing.assert_array_equal(b, 2.0 * a)


def _repage(case, bs_new, rng, dtype):
    """Rebuild the same logical sequences at another block size and placement."""
    bs_old = case["k_pool"].shape[1]
    ctxs = list(case["ctx"])
    S = len(ctxs)
    Hkv, D = case["k_pool"].shape[2:]
    nblk = [(c + bs_new - 1) // bs_new for c in ctxs]
    NB = sum(nblk) + 2
    MB = max(nblk) + 1
    perm = rng.permutation(NB)
    tables = np.full((S, MB), -1, dtype=np.int32)
    k_pool = np.full((NB, bs_new, Hkv, D), _nan_storage(dtype))
    v_pool = np.full((NB, bs_new, Hkv, D), _nan_storage(dtype))
    used = 0
    for s, c in enumerate(ctxs):
        for j in range(nblk[s]):
            tables[s, j] = perm[used]
            used += 1
        for t in range(c):
            src_b = case["tables"][s, t // bs_old]
            k_pool[tables[s, t // bs_new], t % bs_new] = case["k_pool"][src_b, t % bs_old]
            v_pool[tables[s, t // bs_new], t % bs_new] = case["v_pool"][src_b, t % bs_old]
    return k_pool, v_pool, tables


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_block_size_and_placement_do_not_change_bits(dtype):
    rng = np.random.default_rng(16)
    ctxs = [1, 8, 17, 100, 255]
    c = make_paged_case(rng, ctxs, 4, 2, 64, 16, dtype)
    scale = float(np.float32(1 / 8))
    ref = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], scale, dtype)
    for bs_new in (8, 16, 32):
        kp, vp, tb = _repage(c, bs_new, rng, dtype)
        got = oracle.paged_decode(c["q"], kp, vp, tb, c["ctx"], scale, dtype)
        assert np.array_equal(got, ref), f"block_size {bs_new} changed the result"


def test_grouped_heads_equal_repeated_kv_heads():
    rng = np.random.default_rng(17)
    ctxs = [3, 40, 77]
    Hq, Hkv, G = 8, 2, 4
    c = make_paged_case(rng, ctxs, Hq, Hkv, 32, 16, "f16")
    gqa = oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"], 0.2, "f16")
    # MHA pool where kv head h holds kv head h // G of the grouped pool
    k_mha = np.repeat(c["k_pool"], G, axis=2)
    v_mha = np.repeat(c["v_pool"], G, axis=2)
    mha = oracle.paged_decode(c["q"], k_mha, v_mha, c["tables"], c["ctx"], 0.2, "f16")
    assert np.array_equal(gqa, mha)


def test_rejects_out_of_range_tables_and_lengths():
    rng = np.random.default_rng(18)
    c = make_paged_case(rng, [20, 5], 2, 2, 8, 8, "f32")
    bad = c["tables"].copy()
    bad[0, 1] = c["NB"]                         # past the pool
    with pytest.raises(ValueError):
        oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], bad, c["ctx"], 1.0, "f32")
    bad = c["tables"].copy()
    bad[1, 0] = -1                              # a used entry that is unmapped
    with pytest.raises(ValueError):
        oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], bad, c["ctx"], 1.0, "f32")
    ctx = c["ctx"].copy()
    ctx[0] = c["MB"] * 8 + 1                    # longer than the table can map
    with pytest.raises(ValueError):
        oracle.paged_decode(c["q"], c["k_pool"], c["v_pool"], c["tables"], ctx, 1.0, "f32")


# ---------------------------------------------------------------------------
# append (reshape_and_cache)
# ---------------------------------------------------------------------------

def test_append_lands_where_the_pages_table_example_says():
    g = _golden("pages_worked_numbers.json")["block_table_example"]
    bs = g["block_size"]
    NB, Hkv, D = 10, 2, 4
    for tok in g["tokens"]:
        # the slot follows from the table by hand; the oracle only sees the slot
        assert tok["slot"] == tok["block"] * bs + tok["offset"]
        assert g["block_table"][tok["t"] // bs] == tok["block"]
        k_cache = np.full((NB, bs, Hkv, D), 0x5A5A, dtype=np.uint16)
        v_cache = np.full((NB, bs, Hkv, D), 0xA5A5, dtype=np.uint16)
        k = np.arange(Hkv * D, dtype=np.uint16).reshape(1, Hkv, D) + 1
        v = k + 100
        oracle.reshape_and_cache(k, v, k_cache, v_cache, np.array([tok["slot"]]), "bf16")
        assert np.array_equal(k_cache[tok["block"], tok["offset"]], k[0])
        assert np.array_equal(v_cache[tok["block"], tok["offset"]], v[0])
        mask = np.ones((NB, bs), dtype=bool)
        mask[tok["block"], tok["offset"]] = False
        assert np.all(k_cache[mask] == 0x5A5A) and np.all(v_cache[mask] == 0xA5A5)


def test_append_skips_negative_slots_and_rejects_overflow():
    NB, bs, Hkv, D = 4, 8, 1, 4
    k_cache = np.zeros((NB, bs, Hkv, D), dtype=np.float32)
    v_cache = np.zeros((NB, bs, Hkv, D), dtype=np.float32)
    k = np.ones((3, Hkv, D), dtype=np.float32)
    v = 2 * k
    oracle.reshape_and_cache(k, v, k_cache, v_cache, np.array([-1, 9, -5]), "f32")
    assert np.count_nonzero(k_cache) == D and np.all(k_cache[1, 1] == 1)
    assert np.count_nonzero(v_cache) == D and np.all(v_cache[1, 1] == 2)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(k, v, k_cache, v_cache, np.array([0, NB * bs, 1]), "f32")


def test_append_then_decode_sees_new_token():
    # decode after append attends over the appended token as the last position
    rng = np.random.default_rng(19)
    c = make_paged_case(rng, [17], 1, 1, 8, 16, "f32", table_pad=0)
    L = 17
    new_k = rng.standard_normal((1, 1, 8)).astype(np.float32)
    new_v = rng.standard_normal((1, 1, 8)).astype(np.float32)
    slot = int(c["tables"][0, L // 16]) * 16 + L % 16
    kp, vp = c["k_pool"].copy(), c["v_pool"].copy()
    oracle.reshape_and_cache(new_k, new_v, kp, vp, np.array([slot]), "f32")
    got = oracle.paged_decode(c["q"], kp, vp, c["tables"], np.array([L + 1], dtype=np.int32), 0.3, "f32")
    k64 = np.concatenate([c["k64"][0], new_k.astype(np.float64)])
    v64 = np.concatenate([c["v64"][0], new_v.astype(np.float64)])
    ref = library_attention(c["q64"], [k64], [v64], 0.3)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
