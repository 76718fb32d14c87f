"""Planted mistakes in the oracle must fail its pins.

Each mutant is the oracle with one function replaced by a plausible wrong
version: a wrong rounding, an off-by-one, a swapped operand, a dropped term.
Every pin listed for it has to reject it, so the pins in test_oracle_pins.py
are shown to be able to catch that class of error.  The mistakes are planted
on the CPU, in Python stand-ins; the oracle itself is unchanged.
"""
import numpy as np
import pytest
import torch

from tests import test_oracle_pins as P


class Mutant:
    """The oracle module with some attributes overridden."""

    def __init__(self, base, **override):
        self._base = base
        self._over = override

    def __getattr__(self, name):
        return self._over[name] if name in self._over else getattr(self._base, name)


def rejects(pin, mutant, *args):
    with pytest.raises(AssertionError):
        pin(mutant, *args)


def _np_attention(q, k, v, scale, kv_of=None, drop_last=False, scale_twice=False):
    """fp64 softmax attention with a selectable mistake."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Hq, d = q.shape
    T, n_kv = k.shape[0], (k.shape[1] if k.ndim == 3 else 1)
    if drop_last and T > 0:
        k, v, T = k[:-1], v[:-1], T - 1
    out = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    if T == 0:
        return out, lse
    G = Hq // n_kv
    s = scale * scale if scale_twice else scale
    for h in range(Hq):
        g = kv_of(h, G, n_kv) if kv_of else h // G
        sc = s * (k[:, g, :] @ q[h])
        m = sc.max()
        w = np.exp(sc - m)
        out[h] = w @ v[:, g, :] / w.sum()
        lse[h] = m + np.log(w.sum())
    return out, lse


def test_attention_mutants_are_caught(oracle):
    wrong_gqa = Mutant(oracle, attention=lambda q, k, v, s: _np_attention(q, k, v, s, kv_of=lambda h, G, n: h % n))
    rejects(P.test_attention_matches_torch_sdpa, wrong_gqa)
    rejects(P.test_attention_gqa_equals_expanded_mha, wrong_gqa)
    off_by_one = Mutant(oracle, attention=lambda q, k, v, s: _np_attention(q, k, v, s, drop_last=True))
    rejects(P.test_attention_matches_torch_sdpa, off_by_one)
    rejects(P.test_attention_special_cases, off_by_one)
    scale_twice = Mutant(oracle, attention=lambda q, k, v, s: _np_attention(q, k, v, s, scale_twice=True))
    rejects(P.test_attention_matches_torch_sdpa, scale_twice)
    # the stand-in itself, without a mistake, passes: the pins reject the mistakes, not the stand-in
    P.test_attention_matches_torch_sdpa(Mutant(oracle, attention=lambda q, k, v, s: _np_attention(q, k, v, s)))


def test_lse_merge_mutant_is_caught(oracle):
    def unweighted(o, l):
        o = np.asarray(o, np.float64)
        l = np.asarray(l, np.float64)
        m = l.max()
        return o.mean(axis=0), m + np.log(np.exp(l - m).sum())
    rejects(P.test_lse_merge_reproduces_unsplit, Mutant(oracle, lse_merge=unweighted))


def test_quantizer_step_mutant_is_caught(oracle):
    """An off-by-one in the number of steps (range / (levels + 1)) clamps the
    maximum a whole step short."""
    def one_step_too_many(x, levels):
        return oracle.uint_asym(x, levels + 1)[0].clip(0, levels), *oracle.uint_asym(x, levels + 1)[1:]
    m = Mutant(oracle, uint_asym=one_step_too_many)
    for levels in (15, 3):
        rejects(P.test_int4_int2_asym_bound, m, levels)


def test_kivi_scale_zero_swap_is_caught(oracle):
    def swapped(st, group):
        st = dict(st)
        st["k_s"], st["k_z"] = st["k_z"], st["k_s"]
        return oracle.kivi_dequant(st, group)
    m = Mutant(oracle, kivi_dequant=swapped)
    for bits in (4, 2):
        rejects(P.test_kivi_groups_per_channel_and_per_token, m, bits)


def test_query_scale_rounding_mutant_is_caught(oracle):
    """The FP8-domain query with its scale rounded to nearest instead of up."""
    def nearest_scale(q_bf16):
        q = torch.from_numpy(np.asarray(q_bf16, np.uint16).view(np.int16)).view(torch.bfloat16).float()
        s = (q.abs().amax(dim=-1, keepdim=True) / 448.0).to(torch.bfloat16).float()
        c = torch.where(s > 0, q / torch.where(s > 0, s, torch.ones_like(s)), torch.zeros_like(q))
        return (c.clamp(-448, 448).to(torch.float8_e4m3fn).double() * s.double()).numpy()
    rejects(P.test_fp8_query_matches_torch_casts, Mutant(oracle, fp8_query=nearest_scale))


def test_encoder_tie_mutant_is_caught(oracle):
    """E4M3 encoding with ties away from zero instead of to the even mantissa."""
    tab = oracle.e4m3_table()
    pos = tab[:0x7F]

    def ties_away(y):
        y = np.asarray(y, np.float32).astype(np.float64)
        a = np.minimum(np.abs(y), 448.0)
        d = np.abs(a[:, None] - pos[None, :])
        best = d.min(axis=1, keepdims=True)
        code = np.where(d == best, np.arange(0x7F)[None, :], -1).max(axis=1)   # larger magnitude on ties
        return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)
    rejects(P.test_e4m3_encode_brute_force, Mutant(oracle, e4m3_encode=ties_away))


def _np_attention_fp8pv(oracle, q, k, vcode, vs, scale, block=32, s_nearest=False, vs_after=False,
                        truncate=False, drop_ref=False):
    """The FP8 score-V reading in numpy (for planting mistakes): per block of
    `block` tokens from token 0, P = 2^(lam - ceil(max lam)) vs, the smallest
    power-of-two S with max P <= 448 S, E4M3 of P / S (torch's cast), weights
    2^(mu - M) S e4m3."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    vcode = np.asarray(vcode, np.float64)
    vs = np.asarray(vs, np.float64)
    Hq, d = q.shape
    T, n_kv = k.shape[0], k.shape[1]
    G = Hq // n_kv
    s32 = float(np.float32(scale))
    out = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        g = h // G
        lam = s32 * (k[:, g, :] @ q[h]) / np.log(2.0)
        M = max(np.ceil(lam[b:b + block].max()) for b in range(0, T, block))
        w = np.zeros(T)
        for b in range(0, T, block):
            blk = slice(b, min(b + block, T))
            mu = np.ceil(lam[blk].max())
            P = np.exp2(lam[blk] - mu) * (1.0 if vs_after else vs[blk, g])
            E = np.log2(P.max() / 448.0)
            E = np.round(E) if s_nearest else np.ceil(E)
            S = 2.0**E
            y = torch.from_numpy(P / S)
            e = y.to(torch.float8_e4m3fn).to(torch.float64).numpy()
            if truncate:                         # toward zero instead of to nearest
                grid = oracle.e4m3_table()[:127]
                e = grid[np.searchsorted(grid, (P / S), side="right") - 1]
            w[blk] = e * S * (1.0 if drop_ref else 2.0**(mu - M))
            if vs_after:
                w[blk] *= vs[blk, g]
        L = np.exp2(lam - M).sum()
        out[h] = w @ vcode[:, g, :] / L
        lse[h] = M * np.log(2.0) + np.log(L)
    return out, lse, np.zeros((Hq, d))


def test_fp8pv_mutants_are_caught(oracle):
    std = lambda **kw: Mutant(oracle, attention_fp8pv=lambda q, k, v, s, sc: _np_attention_fp8pv(  # noqa: E731
        oracle, q, k, v, s, sc, **kw))
    # the stand-in without a mistake passes
    P.test_fp8pv_exact_when_every_weight_is_representable(std())
    P.test_fp8pv_weights_match_torch_e4m3_cast(std())
    P.test_fp8pv_within_half_an_e4m3_step_of_exact_attention(std())
    # blocks of 16 tokens: other block scales for the subnormal-range weights
    rejects(P.test_fp8pv_weights_match_torch_e4m3_cast, std(block=16))
    # block scale rounded to the nearest power of two: the top weights saturate
    rejects(P.test_fp8pv_exact_when_every_weight_is_representable, std(s_nearest=True))
    rejects(P.test_fp8pv_weights_match_torch_e4m3_cast, std(s_nearest=True))
    # the V scale applied after the probabilities are rounded to E4M3
    rejects(P.test_fp8pv_weights_match_torch_e4m3_cast, std(vs_after=True))
    # E4M3 rounding toward zero instead of to nearest (within a full step, so
    # the half-step bound on the aggregate output need not see it; the
    # per-weight cast does)
    rejects(P.test_fp8pv_weights_match_torch_e4m3_cast, std(truncate=True))
    # the factor 2^(mu - M) dropped: the blocks' weights lose their relative size
    rejects(P.test_fp8pv_exact_when_every_weight_is_representable, std(drop_ref=True))
    rejects(P.test_fp8pv_within_half_an_e4m3_step_of_exact_attention, std(drop_ref=True))
