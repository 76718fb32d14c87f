"""Python view of the CPU oracle (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It wraps ``libkvq_oracle.so`` (plain C,
``oracle/kvq_oracle.c``) with numpy marshalling and composes its functions
into the reference for one decode step:

  quantize on store -> dequantize -> softmax attention in fp64

following the pipeline that "KV Cache 압축" (ryotta.opik.net) §5.1 lists and
the store-time quantization with BF16 scales kept next to the codes that
"KV 캐시 양자화(KV cache quantization) ..." (molayo1419.me) describes in its
"what it is" section.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq_oracle.so")

FP8, INT8, E5M2 = 1, 2, 4       # dtype codes (FP8 = E4M3)
PER_TENSOR, PER_HEAD, PER_TOKEN_HEAD = 0, 1, 2

_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        L.kvqo_bf16_value.restype = ctypes.c_float
        L.kvqo_bf16_value.argtypes = [ctypes.c_uint16]
        for f in ("kvqo_bf16_rne", "kvqo_bf16_up", "kvqo_bf16_down"):
            getattr(L, f).restype = ctypes.c_uint16
            getattr(L, f).argtypes = [ctypes.c_float]
        L.kvqo_f16_value.restype = ctypes.c_double
        L.kvqo_f16_value.argtypes = [ctypes.c_uint16]
        L.kvqo_f16_rne.restype = ctypes.c_uint16
        L.kvqo_f16_rne.argtypes = [ctypes.c_double]
        L.kvqo_bf16_to_f16_array.argtypes = [_P, ctypes.c_int64, _P]
        L.kvqo_e4m3_value.restype = ctypes.c_double
        L.kvqo_e4m3_value.argtypes = [ctypes.c_uint8]
        L.kvqo_e4m3_encode.restype = ctypes.c_uint8
        L.kvqo_e4m3_encode.argtypes = [ctypes.c_float]
        L.kvqo_e4m3_encode_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _P]
        L.kvqo_e4m3_encode_array.argtypes = [_P, ctypes.c_int64, _P]
        L.kvqo_e5m2_value.restype = ctypes.c_double
        L.kvqo_e5m2_value.argtypes = [ctypes.c_uint8]
        L.kvqo_e5m2_encode.restype = ctypes.c_uint8
        L.kvqo_e5m2_encode.argtypes = [ctypes.c_float]
        L.kvqo_e5m2_encode_array.argtypes = [_P, ctypes.c_int64, _P]
        L.kvqo_e5m2_encode_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _P]
        L.kvqo_fp8_row.argtypes = [_P, ctypes.c_int, _P, _P]
        L.kvqo_fp8_row_static.argtypes = [_P, ctypes.c_int, ctypes.c_uint16, _P]
        L.kvqo_int8_row.argtypes = [_P, ctypes.c_int, _P, _P, _P]
        L.kvqo_uint_asym.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P, _P]
        L.kvqo_quantize_rows.argtypes = [ctypes.c_int, ctypes.c_int, _P, ctypes.c_int64, ctypes.c_int,
                                         _P, _P, _P, _P]
        L.kvqo_dequantize_rows.argtypes = [ctypes.c_int, ctypes.c_int, _P, ctypes.c_int64, ctypes.c_int,
                                           _P, _P, _P]
        L.kvqo_kivi_quantized_count.restype = ctypes.c_int64
        L.kvqo_kivi_quantized_count.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
        L.kvqo_kivi_k.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P, _P]
        L.kvqo_kivi_v.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P, _P, _P]
        L.kvqo_attention.argtypes = [_P, _P, _P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_double, _P, _P]
        L.kvqo_attention_fp8pv.argtypes = [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, ctypes.c_int, ctypes.c_double, _P, _P, _P]
        L.kvqo_e4m3_encode_f64.restype = ctypes.c_uint8
        L.kvqo_e4m3_encode_f64.argtypes = [ctypes.c_double]
        L.kvqo_lse_merge.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, _P, _P]
        L.kvqo_kv_bytes.restype = ctypes.c_double
        L.kvqo_kv_bytes.argtypes = [ctypes.c_double] * 6
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ---------------------------------------------------------------- formats
def bf16_value(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_table() -> np.ndarray:
    """fp64 value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    L = lib()
    return np.array([L.kvqo_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().kvqo_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e5m2_table() -> np.ndarray:
    """fp64 value of each of the 256 E5M2 codes (+-inf at 0x7C / 0xFC, NaN for 0x7D-0x7F / 0xFD-0xFF)."""
    L = lib()
    return np.array([L.kvqo_e5m2_value(c) for c in range(256)], dtype=np.float64)


def e5m2_encode(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().kvqo_e5m2_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e5m2_encode_range(first_bits: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint8)
    lib().kvqo_e5m2_encode_range(first_bits, count, _ptr(out))
    return out


def e4m3_encode_range(first_bits: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint8)
    lib().kvqo_e4m3_encode_range(first_bits, count, _ptr(out))
    return out


def f16_value(bits) -> np.ndarray:
    return _c(bits, np.uint16).view(np.float16).astype(np.float64)


def f16_rne(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, dtype=np.float64)
    return np.array([L.kvqo_f16_rne(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def bf16_to_f16_bits(x_bf16) -> np.ndarray:
    """fp16 bits (nearest-even) of bf16 values."""
    x = _c(x_bf16, np.uint16)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().kvqo_bf16_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


# ---------------------------------------------------------------- quantizers
def quantize_rows(dtype: int, mode: int, x_bf16, static_scale=None):
    """Quantize rows of bf16 bits [..., n] -> (codes u8, scale bf16 bits, zero bf16 bits or None)."""
    x = _c(x_bf16, np.uint16)
    n = x.shape[-1]
    rows = x.size // n
    codes = np.empty(x.shape, dtype=np.uint8)
    scale = np.empty(x.shape[:-1], dtype=np.uint16)
    zero = np.empty(x.shape[:-1], dtype=np.uint16) if dtype == INT8 else None
    ss = None
    if mode != PER_TOKEN_HEAD:
        ss = _c(np.broadcast_to(np.asarray(static_scale, dtype=np.uint16), x.shape[:-1]), np.uint16)
    lib().kvqo_quantize_rows(dtype, mode, _ptr(x), rows, n, _ptr(ss), _ptr(codes), _ptr(scale), _ptr(zero))
    return codes, scale, zero


def dequantize_rows(dtype: int, codes, scale, zero=None) -> np.ndarray:
    c = _c(codes, np.uint8)
    n = c.shape[-1]
    s = _c(np.broadcast_to(np.asarray(scale, dtype=np.uint16), c.shape[:-1]), np.uint16)
    z = None if zero is None else _c(np.broadcast_to(np.asarray(zero, dtype=np.uint16), c.shape[:-1]), np.uint16)
    out = np.empty(c.shape, dtype=np.float64)
    lib().kvqo_dequantize_rows(dtype, 2, _ptr(c), c.size // n, n, _ptr(s), _ptr(z), _ptr(out))
    return out


def uint_asym(x, levels: int):
    """Asymmetric quantizer over a 1-D float32 vector -> (codes, s bits, z bits)."""
    x = _c(x, np.float32)
    codes = np.empty(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint16)
    z = np.zeros(1, dtype=np.uint16)
    lib().kvqo_uint_asym(_ptr(x), x.size, 1, levels, _ptr(codes), 1, _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0])


# ---------------------------------------------------------------- KIVI
def kivi_quantized_count(T: int, resid: int, group: int) -> int:
    return int(lib().kvqo_kivi_quantized_count(T, resid, group))


def kivi_stream(x16_k, x16_v, resid: int, group: int, bits: int = 4):
    """KIVI state of one (sequence, KV head): fp16 bits [T][n] for K and V,
    quantized to `bits` (4 or 2) bits.

    Returns dict with nq, K codes/s/z (per channel per group), V codes/s/z
    (per token), and the fp16 residual rows [nq, T).
    """
    k = _c(x16_k, np.uint16)
    v = _c(x16_v, np.uint16)
    T, n = k.shape
    nq = kivi_quantized_count(T, resid, group)
    kc = np.zeros((nq, n), dtype=np.uint8)
    ks = np.zeros((nq // group, n), dtype=np.uint16)
    kz = np.zeros((nq // group, n), dtype=np.uint16)
    vc = np.zeros((nq, n), dtype=np.uint8)
    vs = np.zeros(nq, dtype=np.uint16)
    vz = np.zeros(nq, dtype=np.uint16)
    L = lib()
    if nq:
        L.kvqo_kivi_k(_ptr(k), nq, n, group, bits, _ptr(kc), _ptr(ks), _ptr(kz))
        L.kvqo_kivi_v(_ptr(v), nq, n, bits, _ptr(vc), _ptr(vs), _ptr(vz))
    return dict(nq=nq, k_codes=kc, k_s=ks, k_z=kz, v_codes=vc, v_s=vs, v_z=vz,
                k_res=k[nq:].copy(), v_res=v[nq:].copy())


def kivi_dequant(st, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 K^, V^ [T][n] of one KIVI stream."""
    nq = st["nq"]
    kc = st["k_codes"].astype(np.float64)
    ks = np.repeat(bf16_value(st["k_s"]).astype(np.float64), group, axis=0)
    kz = np.repeat(bf16_value(st["k_z"]).astype(np.float64), group, axis=0)
    vc = st["v_codes"].astype(np.float64)
    vs = bf16_value(st["v_s"]).astype(np.float64)[:, None]
    vz = bf16_value(st["v_z"]).astype(np.float64)[:, None]
    kq = kc * ks[:nq] + kz[:nq]
    vq = vc * vs + vz
    k = np.concatenate([kq, f16_value(st["k_res"])], axis=0)
    v = np.concatenate([vq, f16_value(st["v_res"])], axis=0)
    return k, v


# ---------------------------------------------------------------- attention
def attention(q, k, v, softmax_scale: float):
    """q [Hq][d], k/v [T][n_kv][d] (fp64) -> (out [Hq][d], lse [Hq])."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    Hq, d = q.shape
    T, n_kv, _ = k.shape if k.ndim == 3 else (0, 1, d)
    out = np.empty((Hq, d), dtype=np.float64)
    lse = np.empty(Hq, dtype=np.float64)
    lib().kvqo_attention(_ptr(q), _ptr(k), _ptr(v), T, Hq, n_kv, d,
                         float(np.float32(softmax_scale)), _ptr(out), _ptr(lse))
    return out, lse


FP8_PV_BLOCK = 32      # tokens per probability block of the FP8 score-V product


# Relative score uncertainty (of sum_i |q_i k_i|, times the softmax scale) of
# the evaluations the FP8 score-V reference is compared with, for its
# allowance: float32 accumulation of exact products, and the FP8 matrix core's
# alignment within one 128-term dot product (FP8-domain QK).
SCORE_REL_FP32 = 2.0**-20
SCORE_REL_FP8_DOT = 2.0**-12


def attention_fp8pv(q, k, vcode, vs, softmax_scale: float, block: int = FP8_PV_BLOCK,
                    score_rel: float = SCORE_REL_FP32):
    """Attention with the score-V product in the FP8 domain (kvq_oracle.c,
    kvqo_attention_fp8pv; "FP8 KV Cache부터 INT4 Weight-Only까지", core concept
    3): each token's weight relative to its 32-token block's integer log2
    reference, times its V scale, held as an E4M3 code under a power-of-two
    block scale.  q [Hq][d], k [T][n_kv][d] (fp64, dequantized), vcode
    [T][n_kv][d] (decoded V codes without their scale), vs [T][n_kv] (V scales).
    Returns (out [Hq][d], lse [Hq], allowance [Hq][d]); allowance bounds what
    an evaluation with float32 probabilities and scores off by up to score_rel
    * softmax_scale * sum_i |q_i k_i| may differ by at the E4M3 rounding
    boundaries it meets."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    vcode = _c(vcode, np.float64)
    vs = _c(vs, np.float64)
    Hq, d = q.shape
    T, n_kv = (k.shape[0], k.shape[1]) if k.ndim == 3 else (0, 1)
    out = np.empty((Hq, d), dtype=np.float64)
    lse = np.empty(Hq, dtype=np.float64)
    allow = np.empty((Hq, d), dtype=np.float64)
    lib().kvqo_attention_fp8pv(_ptr(q), _ptr(k), _ptr(vcode), _ptr(vs), T, Hq, n_kv, d,
                               float(np.float32(softmax_scale)), int(block), float(score_rel), _ptr(out), _ptr(lse),
                               _ptr(allow))
    return out, lse, allow


def v_code_values(dtype: int, codes) -> np.ndarray:
    """Decoded FP8 codes (E4M3 or E5M2) without their scale, fp64."""
    tab = e5m2_table() if dtype == E5M2 else e4m3_table()
    return tab[np.asarray(codes, dtype=np.uint8)]


def lse_merge(o_parts, lse_parts):
    o = _c(o_parts, np.float64)
    l = _c(lse_parts, np.float64)
    P, d = o.shape
    out = np.empty(d, dtype=np.float64)
    lo = np.empty(1, dtype=np.float64)
    lib().kvqo_lse_merge(_ptr(o), _ptr(l), P, d, _ptr(out), _ptr(lo))
    return out, float(lo[0])


def kv_bytes(layers, n_kv_heads, head_dim, seq_len, batch, bytes_per_elem) -> float:
    return float(lib().kvqo_kv_bytes(layers, n_kv_heads, head_dim, seq_len, batch, bytes_per_elem))


# ---------------------------------------------------------------- one decode step
def fp8_query(q_bf16) -> np.ndarray:
    """FP8-domain attention's query: every query row (one position and head,
    [..., d] bf16 bits) quantized to E4M3 by the per-(token, head) rule the K
    rows use (scale = BF16 ceiling of amax / 448, codes of q / scale), returned
    dequantized in fp64.  Some backends compute attention itself in FP8
    ("FP8 KV Cache부터 INT4 Weight-Only까지", core concept 3); the query
    quantizer is the pages' per-token FP8 rule applied to q (a reading: the
    pages give no query rule)."""
    c, s, _ = quantize_rows(FP8, PER_TOKEN_HEAD, q_bf16)
    return dequantize_rows(FP8, c, s)


def _attend(q, res, dtype: int, scale: float, pv8: bool, n_vis=None, score_rel: float = SCORE_REL_FP32):
    """Attention of q over the first n_vis cached tokens of a quantized_cache
    result: plain (fp64 on the dequantized cache) or FP8 score-V (pv8).
    Returns (out, lse, allowance or None)."""
    T = res["k_hat"].shape[0]
    n = T if n_vis is None else n_vis
    if not pv8:
        out, lse = attention(q, res["k_hat"][:n], res["v_hat"][:n], scale)
        return out, lse, None
    vcode = v_code_values(dtype, res["v_codes"][:n])
    vs = bf16_value(res["v_scale"][:n]).astype(np.float64)
    return attention_fp8pv(q, res["k_hat"][:n], vcode, vs, scale, score_rel=score_rel)


def decode_reference(q_bf16, k_bf16, v_bf16, dtype: int, mode: int = PER_TOKEN_HEAD,
                     static_kv=None, softmax_scale: Optional[float] = None, q8: bool = False,
                     pv8: bool = False):
    """Reference for one sequence.

    q_bf16 [Hq][d], k_bf16 / v_bf16 [T][n_kv][d] (bf16 bits).  ``static_kv`` =
    (k_scale, v_scale) bf16 bits broadcastable to [n_kv] for static modes.
    q8: FP8-domain QK, i.e. attention of fp8_query(q) instead of q.
    pv8: FP8 score-V product (attention_fp8pv; FP8 caches); adds "allow", for
    an evaluation whose scores carry the uncertainty of its QK (FP8 matrix
    core with q8, float32 accumulation otherwise).
    Returns dict: K/V codes, scales, zeros, and fp64 out [Hq][d], lse [Hq].
    """
    q = fp8_query(q_bf16) if q8 else bf16_value(q_bf16).astype(np.float64)
    d = q.shape[-1]
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else softmax_scale
    res = quantized_cache(k_bf16, v_bf16, dtype, mode, static_kv)
    res["out"], res["lse"], allow = _attend(q, res, dtype, scale, pv8,
                                            score_rel=SCORE_REL_FP8_DOT if q8 else SCORE_REL_FP32)
    if allow is not None:
        res["allow"] = allow
    return res


def quantized_cache(k_bf16, v_bf16, dtype: int, mode: int = PER_TOKEN_HEAD, static_kv=None):
    """Store-time quantization of one sequence's K/V rows [T][n_kv][d] (bf16
    bits) and their dequantized fp64 values: dict of K/V codes, scales, zeros
    and k_hat / v_hat."""
    k_bf16 = _c(k_bf16, np.uint16)
    v_bf16 = _c(v_bf16, np.uint16)
    T, n_kv, _ = k_bf16.shape
    res = {}
    for name, x, idx in (("k", k_bf16, 0), ("v", v_bf16, 1)):
        ss = None
        if mode != PER_TOKEN_HEAD:
            ss = np.broadcast_to(np.asarray(static_kv[idx], dtype=np.uint16), (n_kv,))
            ss = np.broadcast_to(ss, (T, n_kv))
        c, s, z = quantize_rows(dtype, mode, x, ss)
        res[name + "_codes"], res[name + "_scale"], res[name + "_zero"] = c, s, z
        res[name + "_hat"] = dequantize_rows(dtype, c, s, z)
    return res


# ---------------------------------------------------------------- verification step
def verify_reference(q_bf16, k_bf16, v_bf16, dtype: int, mode: int = PER_TOKEN_HEAD,
                     static_kv=None, softmax_scale: Optional[float] = None, q8: bool = False,
                     pv8: bool = False):
    """Reference for one sequence in a speculative-decoding verification pass.

    The target model scores the K+1 newest positions of the sequence in one
    pass over the quantized cache, dequantizing as it reads ("KV 캐시 양자화
    (KV cache quantization) ...", molayo1419.me, section on the interaction
    with speculative decoding).  q_bf16 [n_new][Hq][d] holds the queries of
    those positions, whose own K/V rows are the last n_new of k_bf16 / v_bf16
    [T][n_kv][d].  Position i (0 = oldest of the new ones) attends causally:
    to cache positions t < T - n_new + 1 + i.  A position that sees no token
    (T < n_new) gets out = 0 and lse = -inf.  q8: FP8-domain QK (fp8_query).
    pv8: FP8 score-V product over each position's visible tokens (blocks from
    token 0), adding "allow" [n_new][Hq][d].
    Returns the dict of quantized_cache plus fp64 out [n_new][Hq][d] and lse
    [n_new][Hq].
    """
    q = fp8_query(q_bf16) if q8 else bf16_value(q_bf16).astype(np.float64)
    n_new, Hq, d = q.shape
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else softmax_scale
    res = quantized_cache(k_bf16, v_bf16, dtype, mode, static_kv)
    T = res["k_hat"].shape[0]
    out = np.zeros((n_new, Hq, d), dtype=np.float64)
    lse = np.full((n_new, Hq), -np.inf, dtype=np.float64)
    allow = np.zeros((n_new, Hq, d), dtype=np.float64)
    for i in range(n_new):
        n_vis = max(0, T - n_new + 1 + i)
        out[i], lse[i], a = _attend(q[i], res, dtype, scale, pv8, n_vis,
                                    score_rel=SCORE_REL_FP8_DOT if q8 else SCORE_REL_FP32)
        if a is not None:
            allow[i] = a
    res["out"], res["lse"] = out, lse
    if pv8:
        res["allow"] = allow
    return res
