"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/), closed forms, library routines that implement
the same definition independently (torch's float8_e4m3fn / bfloat16 casts,
numpy's float16 cast, torch's scaled_dot_product_attention), invariants and
brute force on small inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_size_examples.json")


# ----------------------------------------------------------------- P1 sizes
def test_kv_size_worked_examples(oracle):
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        b = oracle.kv_bytes(ex["layers"], ex["kv_heads"], ex["head_dim"], ex["seq_len"], ex["batch"],
                            ex["bytes_per_elem"])
        assert abs(b / ex["unit_bytes"] - ex["printed"]) <= ex["abs_tol"], (ex["name"], b)


def test_kv_size_linear_and_fractions(oracle):
    g = json.load(open(GOLDEN))
    bpe = g["bytes_per_element"]
    base = oracle.kv_bytes(80, 8, 128, 32768, 1, bpe["FP16"])
    # linear in every factor
    assert oracle.kv_bytes(80, 8, 128, 65536, 1, 2) == 2 * base
    assert oracle.kv_bytes(80, 8, 128, 32768, 3, 2) == 3 * base
    # FP8 = half, INT4 = a quarter, INT2 = an eighth of 16-bit storage
    frac = g["fraction_of_bf16"]
    assert oracle.kv_bytes(80, 8, 128, 32768, 1, bpe["FP8"]) / base == frac["FP8"]
    assert oracle.kv_bytes(80, 8, 128, 32768, 1, bpe["INT4"]) / base == frac["INT4"]
    assert oracle.kv_bytes(80, 8, 128, 32768, 1, bpe["INT2"]) / base == 0.125


# ----------------------------------------------------------------- bf16 / fp16
def test_bf16_rne_matches_torch(oracle):
    rng = np.random.default_rng(7)
    # random magnitudes plus exact ties (low 16 bits = 0x8000) and near-ties
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]            # finite only
    ties = (bits & 0xFFFF0000) | 0x8000
    near = (bits & 0xFFFF0000) | 0x7FFF
    allb = np.concatenate([bits, ties, near]).astype(np.uint32)
    f = allb.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    L = oracle.lib()
    got = np.array([L.kvqo_bf16_rne(float(x)) for x in f[:20000]], dtype=np.uint16)
    assert np.array_equal(got, ref[:20000])
    got_t = np.array([L.kvqo_bf16_rne(float(x)) for x in f[len(bits):len(bits) + 20000]], dtype=np.uint16)
    assert np.array_equal(got_t, ref[len(bits):len(bits) + 20000])


def test_bf16_directed_rounding_brackets(oracle):
    """up(f) is the smallest bf16 >= f and down(f) the largest bf16 <= f."""
    L = oracle.lib()
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) < 0xFE]
    for x in bits.view(np.float32)[:5000]:
        x = float(x)
        up, dn = L.kvqo_bf16_up(x), L.kvqo_bf16_down(x)
        vu, vd = float(L.kvqo_bf16_value(up)), float(L.kvqo_bf16_value(dn))
        assert vd <= x <= vu
        if vu != x:
            # the two results are adjacent bf16 values: nothing representable in between
            assert vd != x
            assert abs(int(up) - int(dn)) == 1 or (up & 0x7FFF) == 0 or (dn & 0x7FFF) == 0
    # exact values are fixed points; zero stays zero
    for x in (0.0, 1.0, -2.5, 448.0, 3.0 / 256):
        assert L.kvqo_bf16_up(x) == L.kvqo_bf16_down(x) == L.kvqo_bf16_rne(x)


def test_f16_rne_matches_numpy(oracle):
    rng = np.random.default_rng(9)
    vals = np.concatenate([
        rng.standard_normal(20000) * 3.0,
        rng.standard_normal(5000) * 1e-5,                # subnormal range
        np.ldexp(rng.integers(0, 2**12, 5000).astype(np.float64) + 0.5, -24),  # exact ties in subnormals
        np.array([65504.0, 65519.9, 65520.0, -0.0, 0.0]),
    ])
    bf16 = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_to_f16_bits(bf16)
    ref = oracle.bf16_value(bf16).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    L = oracle.lib()
    for v in vals[-5000:]:
        assert L.kvqo_f16_rne(float(v)) == np.float16(v).view(np.uint16)


# ----------------------------------------------------------------- P2 E4M3 decode
def test_e4m3_decode_table_matches_torch(oracle):
    tab = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]


def test_e4m3_decode_landmarks(oracle):
    g = json.load(open(GOLDEN))["e4m3"]
    tab = oracle.e4m3_table()
    assert tab[0x7E] == g["max_finite"] and tab[0xFE] == -g["max_finite"]
    assert tab[0x08] == g["min_normal"]
    assert tab[0x01] == g["min_subnormal"]
    assert tab[0x00] == 0.0 and math.copysign(1, tab[0x80]) == -1.0
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0)                        # strictly increasing codes 0..0x7E
    assert np.array_equal(tab[0x80:0xFF], -pos)            # sign-magnitude
    # 3 mantissa bits: 8 equally spaced values per binade
    for e in range(1, 15):
        seg = pos[e * 8:(e + 1) * 8]
        assert np.allclose(np.diff(seg), seg[0] / 8)


# ----------------------------------------------------------------- P3 E4M3 encode
def test_e4m3_roundtrip(oracle):
    tab = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    enc = oracle.e4m3_encode(tab[codes].astype(np.float32))
    assert np.array_equal(enc, codes)


def _nearest_e4m3(y: np.ndarray, tab: np.ndarray) -> np.ndarray:
    """Independent search: nearest finite E4M3 value, ties to even code, saturating."""
    codes = np.array([c for c in range(0x7F)], dtype=np.int64)            # 0..0x7E
    vals = tab[codes]
    a = np.abs(y.astype(np.float64))
    a = np.minimum(a, 448.0)
    dist = np.abs(a[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer the even mantissa (even code)
    pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 10**6).min(axis=1)
    single = np.where(cand, codes[None, :], 10**6).min(axis=1)
    pick = np.where(cand.sum(axis=1) > 1, pick, single)
    sign = np.signbit(y).astype(np.int64) * 0x80
    return (pick | sign).astype(np.uint8)


def test_e4m3_encode_brute_force(oracle):
    tab = oracle.e4m3_table()
    rng = np.random.default_rng(11)
    pos = tab[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    m32 = mids.astype(np.float32)
    ulp_up = np.nextafter(m32, np.float32(np.inf))
    ulp_dn = np.nextafter(m32, np.float32(-np.inf))
    samples = np.concatenate([
        m32, ulp_up, ulp_dn, pos.astype(np.float32),
        (rng.standard_normal(50000) * 60).astype(np.float32),
        np.ldexp(rng.random(50000), rng.integers(-14, 10, 50000)).astype(np.float32),
        np.array([448.0, 464.0, 1e30, np.inf, 447.99, 2.0**-10, 2.0**-10 * 1.0000001], dtype=np.float32),
    ])
    samples = np.concatenate([samples, -samples])
    got = oracle.e4m3_encode(samples)
    ref = _nearest_e4m3(samples, tab)
    assert np.array_equal(got, ref)


def test_e4m3_encode_matches_torch_exhaustive_range(oracle):
    """All float32 bit patterns with |y| in [2^-12, 448) vs torch's float8_e4m3fn cast.

    torch rounds to nearest-even; it produces NaN (not saturation) above the
    largest finite value, so that region is checked by the brute-force test.
    """
    lo = np.array([2.0**-12], dtype=np.float32).view(np.uint32)[0]
    hi = np.array([448.0], dtype=np.float32).view(np.uint32)[0]
    step = 1 << 24
    for start in range(int(lo), int(hi), step):
        n = min(step, int(hi) - start)
        got = oracle.e4m3_encode_range(start, n)
        y = torch.arange(start, start + n, dtype=torch.int64).to(torch.int32).view(torch.float32)
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, ref), start
        neg = torch.neg(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got | 0x80, neg), start


def test_e4m3_encode_monotone(oracle):
    y = np.linspace(-500, 500, 200001).astype(np.float32)
    tab = oracle.e4m3_table()
    v = tab[oracle.e4m3_encode(y)]
    assert np.all(np.diff(v) >= 0)


# ----------------------------------------------------------------- P4 FP8 quantizer
def _bf16(x) -> np.ndarray:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_fp8_quantizer_bounds(oracle):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    x[:, [3, 50, 77, 120]] *= 20.0
    xb = _bf16(x)
    codes, s, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_TOKEN_HEAD, xb)
    xv = oracle.bf16_value(xb).astype(np.float64)
    sv = oracle.bf16_value(s).astype(np.float64)[:, None]
    xh = oracle.dequantize_rows(oracle.FP8, codes, s)
    assert np.all(np.abs(xv) / sv <= 448.0)                # per-row scale: nothing saturates
    err = np.abs(xv - xh)
    assert np.all(err <= np.maximum(2.0**-4 * np.abs(xv), 2.0**-10 * sv))
    # the scale is the bf16 ceiling of amax/448 (outward rounding: >= exact ratio, < one bf16 step above)
    amax = np.abs(xv).max(axis=1, keepdims=True)
    assert np.all(sv >= amax / 448.0)
    assert np.all(sv <= amax / 448.0 * (1 + 2.0**-7))


def test_fp8_exactly_representable_rows_roundtrip(oracle):
    rng = np.random.default_rng(13)
    tab = oracle.e4m3_table()
    for _ in range(200):
        s = 2.0 ** int(rng.integers(-12, 4))
        c = rng.integers(0, 0x7F, 128).astype(np.uint8) | (rng.integers(0, 2, 128).astype(np.uint8) << 7)
        c[0] = 0x7E                                        # the row max is 448*s
        x = (s * tab[c]).astype(np.float32)
        codes, sc, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_TOKEN_HEAD, _bf16(x)[None])
        assert oracle.bf16_value(sc)[0] == s
        assert np.array_equal(codes[0], c)


def test_fp8_zero_row_and_static_saturation(oracle):
    codes, s, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_TOKEN_HEAD, np.zeros((1, 128), np.uint16))
    assert s[0] == 0 and not codes.any()
    x = _bf16(np.array([[1000.0, -1000.0, 0.5] + [0.0] * 125], dtype=np.float32))
    c, _, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_TENSOR, x, _bf16(np.float32(1.0)))
    assert c[0, 0] == 0x7E and c[0, 1] == 0xFE and c[0, 2] == 0x30


def test_per_token_beats_static_per_head_on_outliers(oracle):
    """Per-(token, head) scales lose less than one static per-head scale when a
    few tokens carry large values (the failure mode the formats notes of the
    molayo1419.me page describe for per-head / per-tensor scaling)."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal((512, 128)).astype(np.float32)
    x[::37] *= 50.0                                        # a few outlier tokens
    xb = _bf16(x)
    xv = oracle.bf16_value(xb).astype(np.float64)
    c1, s1, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_TOKEN_HEAD, xb)
    e1 = np.abs(oracle.dequantize_rows(oracle.FP8, c1, s1) - xv).mean()
    stat = oracle.lib().kvqo_bf16_up(float(np.abs(xv).max() / 448.0))
    c2, s2, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_HEAD, xb, np.uint16(stat))
    e2 = np.abs(oracle.dequantize_rows(oracle.FP8, c2, s2) - xv).mean()
    assert e1 < e2


# ----------------------------------------------------------------- P5 INT8 / INT4
def test_int8_error_bound_and_nearest_code(oracle):
    rng = np.random.default_rng(15)
    x = (rng.standard_normal((3000, 128)) * 1.5).astype(np.float32)
    x[::7] += 5.0
    xb = _bf16(x)
    codes, s, z = oracle.quantize_rows(oracle.INT8, oracle.PER_TOKEN_HEAD, xb)
    xv = oracle.bf16_value(xb).astype(np.float64)
    sv = oracle.bf16_value(s).astype(np.float64)[:, None]
    zv = oracle.bf16_value(z).astype(np.float64)[:, None]
    xh = oracle.dequantize_rows(oracle.INT8, codes, s, z)
    assert np.allclose(xh, codes * sv + zv, rtol=0, atol=0)
    assert np.all(np.abs(xv - xh) <= sv * (0.5 + 2.0**-12))
    # z is the row minimum and maps to code 0; the bf16 ceiling of the step is at
    # most 2^-7 above (max - min)/255, so the maximum lands on 253, 254 or 255
    assert np.array_equal(zv[:, 0], xv.min(axis=1))
    assert np.all(codes[np.arange(len(x)), xv.argmin(axis=1)] == 0)
    assert np.all(codes[np.arange(len(x)), xv.argmax(axis=1)] >= 253)
    # brute force over all 256 codes: the chosen one is (one of) the nearest
    grid = np.arange(256, dtype=np.float64)
    for r in range(0, 3000, 97):
        d = np.abs(xv[r][:, None] - (grid[None, :] * sv[r] + zv[r]))
        chosen = d[np.arange(128), codes[r]]
        assert np.all(chosen <= d.min(axis=1) + sv[r] * 2.0**-12)


def test_int8_constant_row(oracle):
    xb = _bf16(np.full((1, 128), 0.75, np.float32))
    codes, s, z = oracle.quantize_rows(oracle.INT8, oracle.PER_TOKEN_HEAD, xb)
    assert s[0] == 0 and not codes.any()
    assert oracle.dequantize_rows(oracle.INT8, codes, s, z)[0, 0] == 0.75


@pytest.mark.parametrize("levels", [15, 3])
def test_int4_int2_asym_bound(oracle, levels):
    """4-bit (15 steps) and the KIVI 2-bit setting ([ryotta] section 3.1: 3 steps)."""
    rng = np.random.default_rng(16 + levels)
    for _ in range(300):
        x = (rng.standard_normal(32) * rng.choice([1, 20])).astype(np.float16).astype(np.float32)
        c, s, z = oracle.uint_asym(x, levels)
        sv, zv = float(oracle.bf16_value([s])[0]), float(oracle.bf16_value([z])[0])
        assert zv <= x.min() and c.max() <= levels
        assert np.all(np.abs(x - (c * sv + zv)) <= sv * (0.5 + 2.0**-12))
        grid = np.arange(levels + 1) * sv + zv
        d = np.abs(x[:, None].astype(np.float64) - grid[None, :])
        assert np.all(d[np.arange(32), c] <= d.min(axis=1) + sv * 2.0**-12)
        # the minimum maps to code 0 and (the step being at most 2^-7 above
        # (max - z) / levels) the maximum to the top code
        assert c[np.argmin(x)] == 0 and c[np.argmax(x)] == levels


def test_int2_grid_values_roundtrip(oracle):
    """Values on the 2-bit grid {z, z+s, z+2s, z+3s} with bf16-exact z and s
    quantize back to their own codes and dequantize exactly."""
    for z, s in ((-1.5, 0.25), (0.0, 2.0**-5), (3.0, 1.0), (-40.0, 12.0)):
        codes = np.array([0, 1, 2, 3, 3, 2, 1, 0] * 4, dtype=np.float64)
        x = (z + codes * s).astype(np.float32)
        c, sb, zb = oracle.uint_asym(x, 3)
        assert float(oracle.bf16_value([zb])[0]) == z and float(oracle.bf16_value([sb])[0]) == s
        assert np.array_equal(c, codes.astype(np.uint8))


def test_kivi_window_rule(oracle):
    # tokens leave the fp16 window in whole 32-token groups once more than 128 are held
    assert oracle.kivi_quantized_count(131072, 128, 32) == 130944
    assert 131072 - oracle.kivi_quantized_count(131072, 128, 32) == 128
    assert oracle.kivi_quantized_count(127, 128, 32) == 0
    assert oracle.kivi_quantized_count(159, 128, 32) == 0
    assert oracle.kivi_quantized_count(160, 128, 32) == 32
    for T in range(0, 1000, 7):
        nq = oracle.kivi_quantized_count(T, 128, 32)
        assert nq % 32 == 0 and (T < 128 or 128 <= T - nq < 160)


@pytest.mark.parametrize("bits", [4, 2])
def test_kivi_groups_per_channel_and_per_token(oracle, bits):
    """K statistics run along tokens (one (s, z) per channel per group); V along channels."""
    rng = np.random.default_rng(17)
    T, n = 200, 128
    levels = (1 << bits) - 1
    k = (rng.standard_normal((T, n)) * np.where(np.arange(n) % 31 == 0, 20, 1)).astype(np.float16)
    v = rng.standard_normal((T, n)).astype(np.float16)
    st = oracle.kivi_stream(k.view(np.uint16), v.view(np.uint16), 128, 32, bits)
    assert st["nq"] == 64 and st["k_s"].shape == (2, n) and st["v_s"].shape == (64,)
    assert st["k_codes"].max() == levels and st["v_codes"].max() == levels
    kh, vh = oracle.kivi_dequant(st, 32)
    ks = np.repeat(oracle.bf16_value(st["k_s"]), 32, axis=0)
    assert np.all(np.abs(kh[:64] - k[:64].astype(np.float64)) <= ks * (0.5 + 2.0**-12))
    vs = oracle.bf16_value(st["v_s"])[:, None]
    assert np.all(np.abs(vh[:64] - v[:64].astype(np.float64)) <= vs * (0.5 + 2.0**-12))
    assert np.array_equal(kh[64:], k[64:].astype(np.float64))         # window kept exactly
    # an outlier channel gets its own, larger step; ordinary channels are not widened by it
    assert ks[0, 0] > 5 * np.median(ks[0])
    # brute force per K channel of the first group: each code is a nearest of the 2^b levels
    k0 = k[:32].astype(np.float64)
    kz = oracle.bf16_value(st["k_z"][0]).astype(np.float64)
    grid = kz[None, :, None] + np.arange(levels + 1)[None, None, :] * ks[0][None, :, None]
    dist = np.abs(k0[:, :, None] - grid)
    chosen = np.take_along_axis(dist, st["k_codes"][:32, :, None].astype(np.int64), axis=2)[..., 0]
    assert np.all(chosen <= dist.min(axis=2) + ks[0][None, :] * 2.0**-12)


def test_kivi_2bit_error_exceeds_4bit(oracle):
    """Fewer levels, larger steps: on the same rows the 2-bit steps are about
    5x (15/3) the 4-bit ones and the mean error grows accordingly."""
    rng = np.random.default_rng(18)
    k = rng.standard_normal((192, 128)).astype(np.float16)
    v = rng.standard_normal((192, 128)).astype(np.float16)
    e = {}
    for bits in (4, 2):
        st = oracle.kivi_stream(k.view(np.uint16), v.view(np.uint16), 128, 32, bits)
        kh, vh = oracle.kivi_dequant(st, 32)
        e[bits] = (np.abs(kh[:64] - k[:64]).mean(), np.abs(vh[:64] - v[:64]).mean(),
                   np.median(oracle.bf16_value(st["k_s"])), np.median(oracle.bf16_value(st["v_s"])))
    assert 4.5 <= e[2][2] / e[4][2] <= 5.5 and 4.5 <= e[2][3] / e[4][3] <= 5.5
    assert e[2][0] > 3 * e[4][0] and e[2][1] > 3 * e[4][1]


# ----------------------------------------------------------------- P6 attention
def _sdpa(q, k, v, scale):
    """torch reference in fp64; GQA by repeating KV heads."""
    Hq, d = q.shape
    T, n_kv, _ = k.shape
    G = Hq // n_kv
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)      # [Hq][T][d]
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    qq = torch.from_numpy(q)[:, None, :]                                    # [Hq][1][d]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return o[:, 0, :].numpy()


def test_attention_matches_torch_sdpa(oracle):
    rng = np.random.default_rng(18)
    for (T, Hq, n_kv, d) in [(1, 4, 4, 8), (3, 8, 2, 4), (37, 8, 2, 16), (300, 16, 4, 32)]:
        q = rng.standard_normal((Hq, d))
        k = rng.standard_normal((T, n_kv, d)) * 2
        v = rng.standard_normal((T, n_kv, d))
        scale = float(np.float32(1 / math.sqrt(d)))
        out, lse = oracle.attention(q, k, v, scale)
        assert np.allclose(out, _sdpa(q, k, v, scale), rtol=1e-12, atol=1e-12)
        G = Hq // n_kv
        sc = np.einsum("hd,thd->ht", q, np.repeat(k, G, axis=1)) * scale
        assert np.allclose(lse, np.log(np.exp(sc).sum(axis=1)), rtol=1e-12, atol=1e-12)


def test_attention_special_cases(oracle):
    rng = np.random.default_rng(19)
    d = 128
    v = rng.standard_normal((1, 2, d))
    q = rng.standard_normal((8, d))
    k = rng.standard_normal((1, 2, d))
    out, _ = oracle.attention(q, k, v, 0.088)
    assert np.array_equal(out[:4], np.repeat(v[0, :1], 4, 0)) and np.array_equal(out[4:], np.repeat(v[0, 1:], 4, 0))
    # q = 0 -> plain mean of the values
    k = rng.standard_normal((50, 2, d)); v = rng.standard_normal((50, 2, d))
    out, lse = oracle.attention(np.zeros((2, d)), k, v, 0.1)
    assert np.allclose(out, v.mean(axis=0), atol=1e-14) and np.allclose(lse, math.log(50))
    # two tokens: p0 = 1 / (1 + exp(s1 - s0))
    k2 = rng.standard_normal((2, 1, d)); v2 = rng.standard_normal((2, 1, d)); q2 = rng.standard_normal((1, d))
    s0, s1 = 0.05 * (q2[0] @ k2[0, 0]), 0.05 * (q2[0] @ k2[1, 0])
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out, _ = oracle.attention(q2, k2, v2, 0.05)
    assert np.allclose(out[0], p0 * v2[0, 0] + (1 - p0) * v2[1, 0], atol=1e-14)
    # one dominant score picks its value row
    k3 = np.zeros((5, 1, d)); k3[2, 0, 0] = 1e4
    out, _ = oracle.attention(np.eye(1, d), k3, v2.repeat(3, 0)[:5], 1.0)
    assert np.array_equal(out[0], v2.repeat(3, 0)[2, 0])
    # empty context
    out, lse = oracle.attention(q, np.zeros((0, 2, d)), np.zeros((0, 2, d)), 0.1)
    assert not out.any() and np.all(np.isneginf(lse))


def test_attention_gqa_equals_expanded_mha(oracle):
    rng = np.random.default_rng(20)
    q = rng.standard_normal((16, 32)); k = rng.standard_normal((40, 2, 32)); v = rng.standard_normal((40, 2, 32))
    a, la = oracle.attention(q, k, v, 0.2)
    b, lb = oracle.attention(q, np.repeat(k, 8, axis=1), np.repeat(v, 8, axis=1), 0.2)
    assert np.allclose(a, b, atol=1e-14) and np.allclose(la, lb, atol=1e-13)


def test_lse_merge_reproduces_unsplit(oracle):
    rng = np.random.default_rng(21)
    d, T = 64, 500
    q = rng.standard_normal((1, d)); k = rng.standard_normal((T, 1, d)) * 3; v = rng.standard_normal((T, 1, d))
    full, lfull = oracle.attention(q, k, v, 0.125)
    for _ in range(10):
        cuts = np.sort(rng.choice(np.arange(1, T), size=rng.integers(1, 8), replace=False))
        bounds = [0] + list(cuts) + [T]
        os_, ls = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            o, l = oracle.attention(q, k[a:b], v[a:b], 0.125)
            os_.append(o[0]); ls.append(l[0])
        m, lm = oracle.lse_merge(np.array(os_), np.array(ls))
        assert np.allclose(m, full[0], atol=1e-12) and abs(lm - lfull[0]) < 1e-12


def test_decode_reference_context_one_returns_value_row(oracle):
    rng = np.random.default_rng(22)
    kb = _bf16(rng.standard_normal((1, 2, 128))); vb = _bf16(rng.standard_normal((1, 2, 128)))
    qb = _bf16(rng.standard_normal((8, 128)))
    for dt in (oracle.FP8, oracle.INT8):
        r = oracle.decode_reference(qb, kb, vb, dt)
        assert np.array_equal(r["out"][:4], np.repeat(r["v_hat"][0, :1], 4, 0))


# --------------------------------------------------- verification (K+1 queries)
def test_verify_reference_matches_masked_sdpa(oracle):
    """Causal attention of the n_new newest positions against torch's
    scaled_dot_product_attention with an explicit boolean mask, on the same
    dequantized cache."""
    rng = np.random.default_rng(23)
    for dt in (oracle.FP8, oracle.INT8):
        for (T, n_new, Hq, n_kv) in [(1, 1, 4, 1), (9, 4, 8, 2), (70, 3, 16, 2), (33, 16, 2, 2)]:
            kb = _bf16(rng.standard_normal((T, n_kv, 128)) * 1.5)
            vb = _bf16(rng.standard_normal((T, n_kv, 128)))
            qb = _bf16(rng.standard_normal((n_new, Hq, 128)))
            r = oracle.verify_reference(qb, kb, vb, dt, softmax_scale=0.0883)
            G = Hq // n_kv
            q = torch.from_numpy(oracle.bf16_value(qb).astype(np.float64)).permute(1, 0, 2)      # [Hq][n_new][d]
            k = torch.from_numpy(np.repeat(r["k_hat"], G, axis=1)).permute(1, 0, 2)              # [Hq][T][d]
            v = torch.from_numpy(np.repeat(r["v_hat"], G, axis=1)).permute(1, 0, 2)
            i = torch.arange(n_new)[:, None]
            t = torch.arange(T)[None, :]
            mask = t < (T - n_new + 1 + i)                                                         # [n_new][T]
            # (the oracle takes the softmax scale as an fp32 value, as the kernels do)
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                                 scale=float(np.float32(0.0883)))
            assert np.allclose(r["out"], o.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12), (dt, T, n_new)


def test_verify_reference_special_cases(oracle):
    rng = np.random.default_rng(24)
    T, n_new, Hq, n_kv = 30, 4, 8, 2
    kb = _bf16(rng.standard_normal((T, n_kv, 128))); vb = _bf16(rng.standard_normal((T, n_kv, 128)))
    qb = _bf16(rng.standard_normal((n_new, Hq, 128)))
    for dt in (oracle.FP8, oracle.INT8):
        r = oracle.verify_reference(qb, kb, vb, dt)
        # the newest position sees the whole cache: plain one-query decode
        d = oracle.decode_reference(qb[-1], kb, vb, dt)
        assert np.array_equal(r["out"][-1], d["out"]) and np.array_equal(r["lse"][-1], d["lse"])
        # one new position is the decode step itself
        r1 = oracle.verify_reference(qb[:1], kb, vb, dt)
        d1 = oracle.decode_reference(qb[0], kb, vb, dt)
        assert np.array_equal(r1["out"][0], d1["out"]) and np.array_equal(r1["lse"][0], d1["lse"])
        # causality: changing the rows position i must not see leaves row i as it was
        kb2, vb2 = kb.copy(), vb.copy()
        kb2[T - 2:] = _bf16(rng.standard_normal((2, n_kv, 128)) * 4)
        vb2[T - 2:] = _bf16(rng.standard_normal((2, n_kv, 128)) * 4)
        r2 = oracle.verify_reference(qb, kb2, vb2, dt)
        assert np.array_equal(r2["out"][:2], r["out"][:2]) and np.array_equal(r2["lse"][:2], r["lse"][:2])
        assert not np.allclose(r2["out"][2:], r["out"][2:])
    # identical keys: uniform weights over exactly the visible prefix
    k1 = np.tile(_bf16(rng.standard_normal((1, 1, 128))), (T, 1, 1))
    r = oracle.verify_reference(qb[:, :2], k1, vb[:, :1], oracle.FP8)
    for i in range(n_new):
        n_vis = T - n_new + 1 + i
        assert np.allclose(r["out"][i], r["v_hat"][:n_vis, 0].mean(axis=0), atol=1e-12)
    # fewer cached tokens than new positions: the first rows see nothing
    r = oracle.verify_reference(qb, kb[:2], vb[:2], oracle.FP8)
    assert not r["out"][:2].any() and np.all(np.isneginf(r["lse"][:2]))
    assert np.all(np.isfinite(r["lse"][2:]))


# ----------------------------------------------------------------- E5M2
def test_e5m2_decode_matches_torch(oracle):
    tab = oracle.e5m2_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    # landmarks: largest finite 57344 (0x7B), +inf 0x7C, smallest normal 2^-14, smallest subnormal 2^-16
    assert tab[0x7B] == 57344.0 and np.isposinf(tab[0x7C]) and np.isneginf(tab[0xFC])
    assert tab[0x04] == 2.0**-14 and tab[0x01] == 2.0**-16 and tab[0x80] == 0.0 and np.signbit(tab[0x80])
    assert set(np.flatnonzero(nan)) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}


def test_e5m2_encode_matches_torch_below_saturation(oracle):
    """torch's float8_e5m2 cast rounds to nearest-even; below 57344 it never
    overflows, so there the two must agree on every input (a float32 sweep of
    stride 2^9 in the bit pattern over [2^-20, 57344), both signs)."""
    lo = int(np.array([2.0**-20], np.float32).view(np.uint32)[0])
    hi = int(np.array([57344.0], np.float32).view(np.uint32)[0])
    bits = np.arange(lo, hi, 1 << 9, dtype=np.uint32)
    for sign in (0, 0x80000000):
        y = (bits | np.uint32(sign)).view(np.float32)
        got = oracle.e5m2_encode(y)
        ref = torch.from_numpy(y.copy()).to(torch.float8_e5m2).view(torch.uint8).numpy()
        assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


def test_e5m2_encode_brute_force_ties_and_saturation(oracle):
    tab = oracle.e5m2_table()
    finite = np.flatnonzero(np.isfinite(tab) & (np.arange(256) < 0x80))   # non-negative finite codes
    vals = tab[finite]
    order = np.argsort(vals, kind="stable")
    fv, fc = vals[order], finite[order]
    fv, keep = np.unique(fv, return_index=True)
    fc = fc[keep]
    mids = (fv[:-1] + fv[1:]) / 2
    probes = np.concatenate([fv, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                             np.nextafter(mids.astype(np.float32), np.float32(0))]).astype(np.float32)
    probes = probes[probes < 57344.0]
    got = oracle.e5m2_encode(probes)
    for y, c in zip(probes.astype(np.float64), got):
        d = np.abs(fv - y)
        best = np.flatnonzero(d == d.min())
        if len(best) == 1:
            assert c == fc[best[0]], (y, c)
        else:                                              # a tie: the even mantissa wins
            cand = fc[best]
            assert c in cand and (c & 1) == 0, (y, c, cand)
    # every finite code round-trips; saturation and specials
    for c in range(256):
        if np.isfinite(tab[c]):
            assert oracle.e5m2_encode(np.array([tab[c]], np.float32))[0] == (0x80 if c == 0x80 else c)
    sat = oracle.e5m2_encode(np.array([57344.0, 61440.0, 1e9, np.inf, -1e30, -np.inf, np.nan], np.float32))
    assert list(sat[:6]) == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB] and sat[6] == 0x7F


def test_e5m2_quantizer_bounds(oracle):
    rng = np.random.default_rng(25)
    x = rng.standard_normal((1500, 128)).astype(np.float32)
    x[:, [3, 50]] *= 20.0
    xb = _bf16(x)
    codes, s, z = oracle.quantize_rows(oracle.E5M2, oracle.PER_TOKEN_HEAD, xb)
    assert z is None
    xv = oracle.bf16_value(xb).astype(np.float64)
    sv = oracle.bf16_value(s).astype(np.float64)[:, None]
    xh = oracle.dequantize_rows(oracle.E5M2, codes, s)
    assert np.all(np.abs(xv) / sv <= 57344.0)              # per-row scale: nothing saturates
    # two mantissa bits: relative error <= 2^-3 for normals, absolute <= 2^-17 s in the subnormal range
    assert np.all(np.abs(xv - xh) <= np.maximum(2.0**-3 * np.abs(xv), 2.0**-17 * sv))
    amax = np.abs(xv).max(axis=1, keepdims=True)
    assert np.all(sv >= amax / 57344.0) and np.all(sv <= amax / 57344.0 * (1 + 2.0**-7))
    # E4M3 keeps one more mantissa bit: smaller error on the same rows
    c4, s4, _ = oracle.quantize_rows(oracle.FP8, oracle.PER_TOKEN_HEAD, xb)
    e4 = np.abs(xv - oracle.dequantize_rows(oracle.FP8, c4, s4)).mean()
    assert e4 < np.abs(xv - xh).mean()
    # static scale: elements beyond 57344 s saturate to the largest code
    cs, _, _ = oracle.quantize_rows(oracle.E5M2, oracle.PER_HEAD, _bf16(np.array([[1e4, -3e5, 0.5]], np.float32)),
                                    static_scale=_bf16(np.array([1.0], np.float32))[0])
    assert list(cs[0]) == [oracle.e5m2_encode(np.array([1e4], np.float32))[0], 0xFB,
                           oracle.e5m2_encode(np.array([0.5], np.float32))[0]]


# ----------------------------------------------------------------- FP8-domain QK (query in E4M3)
def _torch_fp8_query(q: torch.Tensor) -> torch.Tensor:
    """The per-row E4M3 rule through torch's own casts: scale = smallest bf16
    >= amax / 448 (float32 division), codes = float8_e4m3fn cast of q / scale."""
    qf = q.float()
    s32 = qf.abs().amax(dim=-1, keepdim=True) / 448.0
    sb = s32.to(torch.bfloat16)
    up = (sb.view(torch.int16) + 1).view(torch.bfloat16)          # next bf16 above (positive values)
    sb = torch.where(sb.float() < s32, up, sb).float()
    codes = torch.where(sb > 0, qf / torch.where(sb > 0, sb, torch.ones_like(sb)), torch.zeros_like(qf))
    return codes.to(torch.float8_e4m3fn).double() * sb.double()


def test_fp8_query_matches_torch_casts(oracle):
    g = torch.Generator().manual_seed(21)
    q = (torch.randn(64, 128, generator=g) * torch.logspace(-3, 2, 64)[:, None]).to(torch.bfloat16)
    q[3] = 0.0                                                      # zero row: scale 0, q^ = 0
    qb = q.view(torch.int16).numpy().view(np.uint16)
    got = oracle.fp8_query(qb)
    assert np.array_equal(got, _torch_fp8_query(q).numpy())
    assert not got[3].any()
    qf = q.double().numpy()
    s = np.abs(qf).max(axis=1, keepdims=True) / 448.0
    # half an E4M3 step: 2^-4 relative for normals, 2^-10 of the scale below 2^-6 s (scale <= 2^-7 above s)
    assert np.all(np.abs(got - qf) <= np.maximum(2.0**-4 * np.abs(qf), 2.0**-10 * s * (1 + 2.0**-7)) + 1e-30)


def test_fp8_domain_reference_exact_for_representable_query(oracle):
    """A query already on the E4M3 grid of its own scale (one element at code
    0x7E = 448) quantizes to itself: the FP8-domain reference equals the plain one."""
    rng = np.random.default_rng(22)
    Hq, n_kv, T, d = 8, 2, 40, 128
    table = oracle.e4m3_table()
    finite = np.array([c for c in range(256) if np.isfinite(table[c])])
    codes = rng.choice(finite, size=(Hq, d))
    codes[:, 5] = 0x7E
    s = 2.0 ** rng.integers(-8, 0, size=(Hq, 1))
    q = torch.from_numpy(table[codes] * s).to(torch.bfloat16)
    assert np.array_equal(q.double().numpy(), table[codes] * s)     # exact in bf16
    qb = q.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.fp8_query(qb), table[codes] * s)
    k = torch.randn(T, n_kv, d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    v = torch.randn(T, n_kv, d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a = oracle.decode_reference(qb, k, v, oracle.FP8)
    b = oracle.decode_reference(qb, k, v, oracle.FP8, q8=True)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])
    # an arbitrary bf16 query is not on the grid: the two references differ
    q2 = torch.randn(Hq, d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c = oracle.decode_reference(q2, k, v, oracle.FP8)
    e = oracle.decode_reference(q2, k, v, oracle.FP8, q8=True)
    assert np.abs(c["out"] - e["out"]).max() > 1e-4


# ---------------------------------------------------------------- FP8 score-V product
# attention_fp8pv: the score-V product of FP8-domain attention ("FP8 KV Cache부터
# INT4 Weight-Only까지", core concept 3).  Reading: each token's weight relative
# to its 32-token block's integer log2 reference, times its V scale, held as an
# E4M3 code under the smallest power-of-two block scale that fits 448.

def _softmax_weights(scores):
    m = scores.max()
    w = np.exp(scores - m)
    return w / w.sum()


def _log2_scores_as_keys(lam, d, ln2_32):
    """Keys whose score against q = e_0 at softmax scale ln2_32 (a float32
    value, as the oracle takes it) is lam_t ln 2: channel 0 holds lam ln2 /
    ln2_32."""
    T, n_kv = lam.shape
    k = np.zeros((T, n_kv, d))
    k[:, :, 0] = lam * math.log(2.0) / ln2_32
    return k


LN2_32 = float(np.float32(math.log(2.0)))


def test_fp8pv_exact_when_every_weight_is_representable(oracle):
    """Scores on an integer log2 grid and power-of-two V scales make every
    P / S a power of two within 2^-4..256 (12 binades of scores and scales
    below the block's top), exactly representable in E4M3: the result is then
    the plain softmax attention (the pinned fp64 oracle) over x^ = vs * vcode,
    to rounding."""
    rng = np.random.default_rng(5)
    T, Hq, n_kv, d = 150, 4, 2, 6
    lam = rng.integers(-8, 3, size=(T, n_kv)).astype(np.float64)         # log2 scores
    lam[32:64] -= 5.0                                                    # a block with a lower reference
    k = _log2_scores_as_keys(lam, d, LN2_32)
    q = np.zeros((Hq, d))
    q[:, 0] = 1.0
    vs = np.ldexp(1.0, rng.integers(-8, -5, size=(T, n_kv)))
    vcode = rng.standard_normal((T, n_kv, d))
    out, lse, allow = oracle.attention_fp8pv(q, k, vcode, vs, LN2_32)
    ref, ref_lse = oracle.attention(q, k, vcode * vs[:, :, None], LN2_32)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-12)
    # every weight sits on a representable value, far from a rounding boundary
    assert not allow.any()


def test_fp8pv_within_half_an_e4m3_step_of_exact_attention(oracle):
    """Random scores and scales: each weight is off by at most half an E4M3
    step (2^-4 relative; 2^-10 S absolute in the subnormal range, S <= 2^-7
    of the block's largest weight times 448 / 256), so the output is within
    2^-4 sum_t p_t |x^_t| + 2^-14.8 max_t |x^_t| of the exact softmax attention
    (p from a plain softmax here); and the error is not zero."""
    rng = np.random.default_rng(6)
    T, Hq, n_kv, d = 333, 8, 2, 16
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((T, n_kv, d)) * 1.5
    vcode = rng.standard_normal((T, n_kv, d))
    vs = np.abs(rng.standard_normal((T, n_kv))) * 0.02 + 1e-3
    scale = float(np.float32(0.4))
    out, lse, _ = oracle.attention_fp8pv(q, k, vcode, vs, scale)
    x = vcode * vs[:, :, None]
    G = Hq // n_kv
    worst = 0.0
    for h in range(Hq):
        g = h // G
        sc = scale * (k[:, g, :] @ q[h])
        p = _softmax_weights(sc)
        exact = p @ x[:, g, :]
        bound = 2.0**-4 * (p @ np.abs(x[:, g, :])) + 2.0**-14.8 * np.abs(x[:, g, :]).max()
        err = np.abs(out[h] - exact)
        assert np.all(err <= bound * (1 + 1e-9)), h
        worst = max(worst, float((err / bound).max()))
        m = sc.max()
        assert abs(lse[h] - (m + math.log(np.exp(sc - m).sum()))) < 1e-12
    assert 0.05 < worst <= 1.0


def test_fp8pv_weights_match_torch_e4m3_cast(oracle):
    """Weights read back through one-hot V rows (vcode_t = e_t, d = T): each
    token's weight times the softmax denominator is 2^(mu - M) S times the
    E4M3 value of P / S, with the E4M3 rounding done by torch's float8_e4m3fn
    cast, bit for bit, for two 32-token blocks and a partial third."""
    rng = np.random.default_rng(7)
    T = 77
    lam = rng.uniform(-9.0, 4.0, size=(T, 1))
    lam[40] = 7.3                                            # block 1 peaks higher
    k = _log2_scores_as_keys(lam, T, LN2_32)
    q = np.zeros((1, T))
    q[0, 0] = 1.0
    vs = rng.uniform(0.004, 0.03, size=(T, 1))
    vcode = np.eye(T).reshape(T, 1, T)
    out, _, _ = oracle.attention_fp8pv(q, k, vcode, vs, LN2_32)
    lam = (LN2_32 * k[:, 0, 0]) / math.log(2.0)              # the log2 score as the oracle forms it
    M = max(math.ceil(lam[b:b + 32].max()) for b in range(0, T, 32))
    L = np.exp2(lam - M).sum()
    for b in range(0, T, 32):
        blk = slice(b, min(b + 32, T))
        mu = math.ceil(lam[blk].max())
        P = np.exp2(lam[blk] - mu) * vs[blk, 0]
        E = math.ceil(math.log2(P.max() / 448.0))
        S = 2.0**E
        assert P.max() <= 448.0 * S and P.max() > 224.0 * S
        codes = torch.from_numpy(P / S).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        want = codes * S * 2.0**(mu - M)
        got = out[0, blk] * L
        assert np.allclose(got, want, rtol=1e-12, atol=0), b


def test_fp8pv_integer_shift_invariance_and_block_alignment(oracle):
    """Adding an integer to every log2 score moves each block reference by the
    same integer: the output is unchanged (to the rounding of forming the
    scores).  Blocks start at token 0 of the context: dropping the first token
    shifts every block boundary, which regroups the tokens whose weights fall
    in E4M3's subnormal range under other block scales and changes the result,
    while the plain attention moves only by that token's (vanishing) weight."""
    rng = np.random.default_rng(8)
    T, Hq, n_kv, d = 200, 2, 1, 8
    lam = rng.uniform(-16, 6, size=(T, n_kv))
    vcode = rng.standard_normal((T, n_kv, d))
    vs = rng.uniform(0.005, 0.05, size=(T, n_kv))
    q = np.zeros((Hq, d))
    q[:, 0] = 1.0
    a, _, _ = oracle.attention_fp8pv(q, _log2_scores_as_keys(lam, d, LN2_32), vcode, vs, LN2_32)
    b, _, _ = oracle.attention_fp8pv(q, _log2_scores_as_keys(lam + 3.0, d, LN2_32), vcode, vs, LN2_32)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-16)
    lam[0] = -60.0                                            # token 0 carries no weight
    k = _log2_scores_as_keys(lam, d, LN2_32)
    c, _, _ = oracle.attention_fp8pv(q, k, vcode, vs, LN2_32)
    e, _, _ = oracle.attention_fp8pv(q, k[1:], vcode[1:], vs[1:], LN2_32)
    ref, _ = oracle.attention(q, k, vcode * vs[:, :, None], LN2_32)
    ref1, _ = oracle.attention(q, k[1:], vcode[1:] * vs[1:, :, None], LN2_32)
    assert np.abs(ref - ref1).max() < 1e-15
    assert np.abs(c - e).max() > 1e-10
