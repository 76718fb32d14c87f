"""GPU parity of the FP8 score-V product (kvq_cache.attn_flags with
KVQ_ATTN_FP8_PV): probabilities held as E4M3 codes under power-of-two scales
of 32-token blocks and PV on the scaled FP8 matrix cores, alone and together
with FP8-domain QK, over E4M3 and E5M2 caches.

The oracle is oracle.attention_fp8pv on the same quantized cache (the reading
of "FP8 KV Cache부터 INT4 Weight-Only까지", core concept 3, written out in
kvq_oracle.c).  The bar is the decode bar plus two terms that the arithmetic
fixes:
  - the oracle's allowance: one E4M3 step for every weight whose P / S lies
    within 2^-18 of a rounding boundary (the kernel forms P in float32 and may
    round it to the neighbouring code) and one subnormal step where the block
    scale itself sits on such a boundary;
  - the FP8 matrix core's alignment within one dot product, measured at up to
    2^-12.7 of the sum of |products| (scaled 16x16x128 with row scales, a probe
    on the MI355X): 2^-12 * sum_t p_t |x^_t| per output element.
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| + allowance + 2^-12 sum_t p_t |x^_t|.
Against the exact attention the output is within half an E4M3 step per
weight: 2e-3 + 1e-2 |exact| + 2^-4 sum_t p_t |x^_t| (checked too)."""
import math
import sys

import numpy as np
import pytest
import torch

from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import quantized_kv_cache_08_amd as kvq  # noqa: E402
import synthetic  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import kvq_harness as H  # noqa: E402

ATOL, RTOL = 2e-3, 1e-2
MFMA_REL = 2.0**-12
HALF_STEP = 2.0**-4
LENS = np.array([1, 5, 17, 31, 32, 33, 96, 250, 700], dtype=np.int64)
QK, PV = kvq.KVQ_ATTN_FP8_QK, kvq.KVQ_ATTN_FP8_PV


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def workload(base: str, **kw) -> synthetic.Workload:
    d = dict(synthetic.WORKLOADS[base].__dict__)
    d.update(kw)
    return synthetic.Workload(**d)


def abs_weighted(q_hat, k_hat, v_hat, scale):
    """sum_t p_t |x^_t| per query head and channel (exact softmax weights)."""
    a, _ = O.attention(q_hat, k_hat, np.abs(v_hat), scale)
    return a


def check(bt: H.Built, out, lse, seqs, mode=kvq.KVQ_SCALE_PER_TOKEN_HEAD, static_kv=None):
    """Each sequence against the FP8 score-V oracle and, with the half-step
    bound, against the exact attention; returns the largest |gpu - exact| over
    the plain decode bar (> 0: the flag changes the result)."""
    q8 = bool(bt.cache.attn_flags & QK)
    scale = 1.0 / math.sqrt(bt.w.head_dim)
    over = -1.0
    for b in seqs:
        ref = H.oracle_seq(bt, b, mode, static_kv)
        qb = H.u16(synthetic.gen_q(bt.w, "cpu", batch=len(bt.lens))[b])
        qh = O.fp8_query(qb) if q8 else O.bf16_value(qb).astype(np.float64)
        aw = abs_weighted(qh, ref["k_hat"], ref["v_hat"], scale)
        got = out[b].cpu().numpy().astype(np.float64)
        bar = ATOL + RTOL * np.abs(ref["out"]) + ref["allow"] + MFMA_REL * aw
        err = np.abs(got - ref["out"])
        i = np.unravel_index(np.argmax(err - bar), err.shape)
        assert np.all(err <= bar), f"seq {b}: diff {err[i]:.3e} > bar {bar[i]:.3e} at {i}"
        exact, exact_lse = O.attention(qh, ref["k_hat"], ref["v_hat"], scale)
        bar_x = ATOL + RTOL * np.abs(exact) + (HALF_STEP + MFMA_REL) * aw
        assert np.all(np.abs(got - exact) <= bar_x), f"seq {b}: beyond half an E4M3 step of exact attention"
        over = max(over, float((np.abs(got - exact) - (ATOL + RTOL * np.abs(exact))).max()))
        if lse is not None and not q8:
            dl = np.abs(lse[b].cpu().numpy().astype(np.float64) - exact_lse)
            assert dl.max() <= 1e-3, f"seq {b}: lse diff {dl.max():.3e}"
    return over


@pytest.mark.parametrize("dtype", ["fp8", "e5m2"])
@pytest.mark.parametrize("flags", [PV, QK | PV])
def test_fp8pv_ragged_batch_partitions(dtype, flags):
    """Lengths around the 32-token block; partitions of 1 and 3 blocks put
    segment starts on many block boundaries; all plans agree with the oracle."""
    w = workload("tiny", dtype=dtype, batch=len(LENS), context=int(LENS.max()))
    say("fp8pv ragged", dtype, flags)
    bt = H.build(w, lens=LENS)
    bt.cache.attn_flags = flags
    for part in (0, 1, 3):
        say("  partition blocks", part)
        out, lse = H.run_decode(bt, part)
        check(bt, out, lse, range(len(LENS)))


@pytest.mark.parametrize("dtype", ["fp8", "e5m2"])
def test_fp8pv_groups_and_page_sizes(dtype):
    for heads, ps in (((8, 2), 32), ((16, 2), 16), ((2, 2), 16), ((32, 2), 16), ((4, 1), 32)):
        w = workload("tiny", dtype=dtype, batch=3, num_q_heads=heads[0], num_kv_heads=heads[1], page_size=ps)
        say("fp8pv", dtype, "heads", heads, "page", ps)
        bt = H.build(w, lens=np.array([31, 300, 64]))
        bt.cache.attn_flags = QK | PV
        out, lse = H.run_decode(bt)
        check(bt, out, lse, range(3))


def test_fp8pv_static_scale_modes():
    w = workload("tiny", batch=2)
    lens = np.array([96, 250])
    for mode in (kvq.KVQ_SCALE_PER_TENSOR, kvq.KVQ_SCALE_PER_HEAD):
        if mode == kvq.KVQ_SCALE_PER_TENSOR:
            host = np.array([0.05, 0.01], dtype=np.float32)
            static_kv = tuple(H.u16(torch.tensor(v).to(torch.bfloat16)) for v in host)
        else:
            host = np.array([[0.04, 0.06], [0.009, 0.012]], dtype=np.float32)
            static_kv = tuple(H.u16(torch.from_numpy(r).to(torch.bfloat16)) for r in host)
        ss = torch.from_numpy(host).to(torch.bfloat16).cuda().contiguous()
        say("fp8pv static mode", mode)
        bt = H.build(w, lens=lens, mode=mode, static_scales=ss)
        bt.cache.attn_flags = QK | PV
        out, lse = H.run_decode(bt)
        check(bt, out, lse, range(2), mode=mode, static_kv=static_kv)


def test_fp8pv_rescales_of_the_running_state():
    """Softmax scale 0.25: the chunk maxima rise past the rescale headroom many
    times within one segment; the integer running maximum keeps every rescale
    a power of two."""
    w = workload("tiny", batch=2, num_q_heads=16, num_kv_heads=2, context=1000)
    lens = np.array([700, 1000])
    say("fp8pv rescale")
    bt = H.build(w, lens=lens)
    bt.cache.attn_flags = PV
    out, lse = H.run_decode(bt, partition_pages=1024, softmax_scale=0.25)
    for b in range(2):
        ref = H.oracle_seq(bt, b, softmax_scale=0.25)
        qh = O.bf16_value(H.u16(synthetic.gen_q(w, "cpu", batch=2)[b])).astype(np.float64)
        aw = abs_weighted(qh, ref["k_hat"], ref["v_hat"], 0.25)
        err = np.abs(out[b].cpu().numpy().astype(np.float64) - ref["out"])
        assert np.all(err <= ATOL + RTOL * np.abs(ref["out"]) + ref["allow"] + MFMA_REL * aw)


def test_fp8pv_verification_pass():
    w = workload("tiny", batch=len(LENS), context=int(LENS.max()))
    say("fp8pv verify")
    bt = H.build(w, lens=LENS)
    bt.cache.attn_flags = QK | PV
    B, q_len, Hq, d = len(LENS), 4, w.num_q_heads, w.head_dim
    q = synthetic.gen_q(w, "cuda", batch=B * q_len).reshape(B, q_len, Hq, d)
    ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, q_len, Hq, bt.max_ctx), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, q_len, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, q_len, Hq), float("nan"), device="cuda")
    kvq.verify_attention(bt.cache, q, bt.block_table, bt.context_lens, bt.max_ctx, d ** -0.5, ws, out, lse)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qc = synthetic.gen_q(w, "cpu", batch=B * q_len).reshape(B, q_len, Hq, d)
    for b in range(B):
        T = int(LENS[b])
        k, v = synthetic.gen_kv(w, b, 0, T, "cpu")
        ref = O.verify_reference(H.u16(qc[b]), H.u16(k), H.u16(v), O.FP8, q8=True, pv8=True)
        qh = O.fp8_query(H.u16(qc[b]))
        for i in range(q_len):
            n_vis = T - q_len + 1 + i
            if n_vis <= 0:
                assert not out[b, i].any()
                continue
            aw = abs_weighted(qh[i], ref["k_hat"][:n_vis], ref["v_hat"][:n_vis], d ** -0.5)
            err = np.abs(out[b, i] - ref["out"][i])
            bar = ATOL + RTOL * np.abs(ref["out"][i]) + ref["allow"][i] + MFMA_REL * aw
            assert np.all(err <= bar), f"seq {b} position {i}"


def test_fp8pv_mixed_small_shuffled_pool():
    w = workload("mixed", batch=24, context=4096)
    say("fp8pv mixed small")
    bt = H.build(w)
    bt.cache.attn_flags = QK | PV
    out, lse = H.run_decode(bt)
    check(bt, out, lse, range(24))


def test_fp8pv_llama8b_shape_every_sequence():
    """The 8B-shaped batch (B 32, context 8192) in the benchmark's launch
    configuration (the fp8attn workload), every sequence; the flag moves the
    output off the plain decode bar of the exact attention somewhere."""
    w = synthetic.WORKLOADS["fp8attn"]
    say("fp8pv llama8b shape")
    bt = H.build(w)
    bt.cache.attn_flags = QK | PV
    out, lse = H.run_decode(bt)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    over = check(bt, out, lse, range(w.batch))
    say("fp8pv llama8b largest excess over the plain bar vs exact attention", over)
